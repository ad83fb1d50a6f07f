// SSM heads of the hybrid-head mixer: causal depthwise conv1d (width 4) and
// the selective scan of Hymba blog (juejin.cn, "NVIDIA提出Hymba网络"),
// "数学表示" §4, Eq. (2), in its recurrent form
//     h_t = exp(delta_t A) h_{t-1} + (delta_t x_t) B_t,   y_t = C_t . h_t,
// with the skip D x_t and the gate SiLU(z_t); 16 states per channel
// (Hymba-1.5B-Base model card, "模型架构").
//
// Layout: x, delta, z, y are [B, T, Di] (channel fastest); B_t, C_t [B, T, 16]
// are shared by every channel of a token.  One lane owns one channel and keeps
// its 16 states in registers, so the state update needs no cross-lane work;
// B_t and C_t are the same for the whole wave (scalar loads).  exp(delta A) is
// computed as exp2(delta * A log2(e)).
//
// The time axis is cut into chunks so that B * ceil(Di/64) * chunks waves fill
// the chip.  Three kernels:
//   scan_chunk_agg   per chunk but the last: end state from a zero start, and
//                    the chunk's total delta (its decay is exp(A * sum delta));
//   scan_carry       per (b, state, channel): walks the chunks in order and
//                    replaces each chunk's aggregate by its incoming state;
//   scan_chunk_final per chunk: the recurrence from the incoming state, writing
//                    y (and the final states for the last chunk).
// With the fused conv the short convolution is recomputed from x (3-token halo)
// inside both chunk kernels and never goes to memory.
#include "hm_common.h"

#include "ssm_dev.h"

namespace {

// ---------------------------------------------------------------- standalone conv
template <typename Tact>
__global__ __launch_bounds__(256) void conv1d_kernel(const Tact* __restrict__ x,
                                                     const float* __restrict__ w,
                                                     const float* __restrict__ bias,
                                                     const float* __restrict__ st_in,
                                                     Tact* __restrict__ y,
                                                     float* __restrict__ st_out, int T, int Di,
                                                     int silu, int tchunk) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= Di) return;
  const int b = blockIdx.z;
  const int t0 = blockIdx.y * tchunk, t1 = min(T, t0 + tchunk);
  const float w0 = w[c * 4 + 0], w1 = w[c * 4 + 1], w2 = w[c * 4 + 2], w3 = w[c * 4 + 3];
  const float bb = bias ? bias[c] : 0.f;
  const Tact* xc = x + (size_t)b * T * Di + c;
  const float* sin_c = st_in ? st_in + ((size_t)b * Di + c) * 3 : nullptr;
  float h0 = conv_in(xc, (long long)t0 - 3, Di, sin_c);
  float h1 = conv_in(xc, (long long)t0 - 2, Di, sin_c);
  float h2 = conv_in(xc, (long long)t0 - 1, Di, sin_c);
  Tact* yc = y + (size_t)b * T * Di + c;
  for (int t = t0; t < t1; ++t) {
    const float xt = ldx(xc + (size_t)t * Di);
    float u = bb + w0 * h0 + w1 * h1 + w2 * h2 + w3 * xt;
    if (silu) u = siluf_(u);
    ActIO<Tact>::st(yc + (size_t)t * Di, u);
    h0 = h1;
    h1 = h2;
    h2 = xt;
  }
  if (st_out && blockIdx.y == gridDim.y - 1) {
    float* so = st_out + ((size_t)b * Di + c) * 3;
    for (int e = 0; e < 3; ++e) so[e] = conv_in(xc, (long long)T - 3 + e, Di, sin_c);
  }
}

// ---------------------------------------------------------------- kernels
template <typename Tact, bool CONV, bool FINAL, bool VEC>
__global__ __launch_bounds__(64) void scan_chunk(
    const Tact* __restrict__ x, const Tact* __restrict__ dl, const float* __restrict__ A,
    const Tact* __restrict__ Bm, const Tact* __restrict__ Cm, const float* __restrict__ D,
    const Tact* __restrict__ z, const float* __restrict__ cw, const float* __restrict__ cb,
    const float* __restrict__ cst_in, float* __restrict__ cst_out, float* __restrict__ E,
    float* __restrict__ S, Tact* __restrict__ y, float* __restrict__ h_out, int T, int Di, int L,
    int nC) {
  __shared__ ScanLds<Tact, FINAL> sm;
  scan_chunk_body<Tact, CONV, FINAL, VEC>(&sm, nullptr, blockIdx.x, blockIdx.y, blockIdx.z, x, dl,
                                          A, Bm, Cm, D, z, cw, cb, cst_in, cst_out, E, S, y, h_out,
                                          T, Di, L, nC);
}

constexpr int kRanges = 8;

__global__ __launch_bounds__(64 * kRanges) void scan_carry(const float* __restrict__ A,
                                                           const float* __restrict__ h0,
                                                           float* __restrict__ E,
                                                           const float* __restrict__ S, int Bsz,
                                                           int Di, int nC) {
  scan_carry_body<kRanges>(blockIdx.x, blockIdx.y, blockIdx.z, A, h0, E, S, Di, nC);
}

template <typename Tact, bool CONV>
hm_status launch_scan(const void* x, const float* cw, const float* cb, const float* cst_in,
                      float* cst_out, const void* delta, const float* A, const void* Bm,
                      const void* Cm, const float* D, const void* z, const float* h0, void* y,
                      float* h_out, int B, int T, int Di, void* workspace, hipStream_t st) {
  const int L = scan_chunk_len(B, T, Di);
  const int nC = (T + L - 1) / L;
  float* E = (float*)workspace;
  float* S = E + (size_t)B * nC * kNS * Di;
  const dim3 blk(64);
  const int gx = (Di + 63) / 64;
  // 16-byte staging needs 16-byte aligned rows and 16-byte aligned bases
  const int vec = ((size_t)Di * sizeof(Tact)) % 16 == 0 && hm::aligned16(x) &&
                  hm::aligned16(delta) && (z == nullptr || hm::aligned16(z)) &&
                  hm::aligned16(Bm) && hm::aligned16(Cm);
  if (nC > 1) {
    if (vec)
      hipLaunchKernelGGL((scan_chunk<Tact, CONV, false, true>), dim3(gx, nC - 1, B), blk, 0, st,
                         (const Tact*)x, (const Tact*)delta, A, (const Tact*)Bm, (const Tact*)Cm,
                         D, (const Tact*)z, cw, cb, cst_in, cst_out, E, S, (Tact*)y, h_out, T, Di,
                         L, nC);
    else
      hipLaunchKernelGGL((scan_chunk<Tact, CONV, false, false>), dim3(gx, nC - 1, B), blk, 0, st,
                         (const Tact*)x, (const Tact*)delta, A, (const Tact*)Bm, (const Tact*)Cm,
                         D, (const Tact*)z, cw, cb, cst_in, cst_out, E, S, (Tact*)y, h_out, T, Di,
                         L, nC);
    hm_status s = hm::check_launch("scan_chunk<aggregate>");
    if (s != HM_OK) return s;
  }
  hipLaunchKernelGGL(scan_carry, dim3(gx, kNS, B), dim3(64 * kRanges), 0, st, A, h0, E, (const float*)S,
                     B, Di, nC);
  hm_status s = hm::check_launch("scan_carry");
  if (s != HM_OK) return s;
  if (vec)
    hipLaunchKernelGGL((scan_chunk<Tact, CONV, true, true>), dim3(gx, nC, B), blk, 0, st,
                       (const Tact*)x, (const Tact*)delta, A, (const Tact*)Bm, (const Tact*)Cm, D,
                       (const Tact*)z, cw, cb, cst_in, cst_out, E, S, (Tact*)y, h_out, T, Di, L,
                       nC);
  else
    hipLaunchKernelGGL((scan_chunk<Tact, CONV, true, false>), dim3(gx, nC, B), blk, 0, st,
                       (const Tact*)x, (const Tact*)delta, A, (const Tact*)Bm, (const Tact*)Cm, D,
                       (const Tact*)z, cw, cb, cst_in, cst_out, E, S, (Tact*)y, h_out, T, Di, L,
                       nC);
  return hm::check_launch("scan_chunk<final>");
}

}  // namespace

namespace hm {

hm_status conv_scan_impl(const void* x, const float* conv_w, const float* conv_b,
                         const float* conv_state_in, float* conv_state_out,
                         const void* delta, const float* A, const void* Bm, const void* Cm,
                         const float* D, const void* z, const float* h0, void* y,
                         float* h_out, int B, int T, int Di, int K, int N, hm_dtype dtype,
                         void* workspace, size_t workspace_bytes, hipStream_t st,
                         bool fuse_conv, bool dry) {
  HM_PTR(x);
  HM_PTR(delta);
  HM_PTR(A);
  HM_PTR(Bm);
  HM_PTR(Cm);
  HM_PTR(y);
  HM_OPT_PTR(D);
  HM_OPT_PTR(z);
  HM_OPT_PTR(h0);
  HM_OPT_PTR(h_out);
  HM_REQUIRE(B > 0 && T > 0 && Di > 0, HM_ERR_INVALID, "B, T and Di must be positive");
  HM_REQUIRE(N == kNS, HM_ERR_UNSUPPORTED, "only N = 16 states are supported");
  HM_REQUIRE(dtype == HM_BF16 || dtype == HM_F32, HM_ERR_UNSUPPORTED, "dtype must be f32 or bf16");
  HM_REQUIRE((double)B * T * Di < 4.0e9 && B <= 65535, HM_ERR_UNSUPPORTED, "tensor too large");
  HM_REQUIRE(y != x && y != delta && y != z && y != Bm && y != Cm, HM_ERR_INVALID,
             "y must not alias an input");
  HM_REQUIRE(h_out == nullptr || h_out != h0, HM_ERR_INVALID, "h_out must not alias h0");
  if (fuse_conv) {
    HM_REQUIRE(K == kConvK, HM_ERR_UNSUPPORTED, "only conv width K = 4 is supported");
    HM_PTR(conv_w);
    HM_PTR(conv_b);
    HM_OPT_PTR(conv_state_in);
    HM_OPT_PTR(conv_state_out);
    HM_REQUIRE(conv_state_out == nullptr || conv_state_out != conv_state_in, HM_ERR_INVALID,
               "conv_state_out must not alias conv_state_in");
  }
  const size_t need = hm_selective_scan_workspace(B, T, Di, N);
  HM_REQUIRE(workspace != nullptr && workspace_bytes >= need && aligned16(workspace),
             HM_ERR_WORKSPACE, "workspace smaller than hm_selective_scan_workspace()");
  if (dry) return HM_OK;
  if (dtype == HM_BF16) {
    // long scans with aligned bf16 rows: two launches (the final pass
    // composes its own incoming states) instead of aggregate, carry and final
    if (fuse_conv && Di % 8 == 0 && aligned16(x) && aligned16(delta) && aligned16(Bm) &&
        aligned16(Cm) && (z == nullptr || aligned16(z)) && conv_scan_two_launch_pays(B, T, Di))
      return conv_scan_two_launch_bf16(x, conv_w, conv_b, conv_state_in, conv_state_out, delta,
                                       A, Bm, Cm, D, z, h0, y, h_out, B, T, Di, workspace, st);
    if (fuse_conv)
      return launch_scan<bf16_t, true>(x, conv_w, conv_b, conv_state_in, conv_state_out, delta,
                                       A, Bm, Cm, D, z, h0, y, h_out, B, T, Di, workspace, st);
    return launch_scan<bf16_t, false>(x, nullptr, nullptr, nullptr, nullptr, delta, A, Bm, Cm, D,
                                      z, h0, y, h_out, B, T, Di, workspace, st);
  }
  if (fuse_conv)
    return launch_scan<float, true>(x, conv_w, conv_b, conv_state_in, conv_state_out, delta, A,
                                    Bm, Cm, D, z, h0, y, h_out, B, T, Di, workspace, st);
  return launch_scan<float, false>(x, nullptr, nullptr, nullptr, nullptr, delta, A, Bm, Cm, D, z,
                                   h0, y, h_out, B, T, Di, workspace, st);
}

}  // namespace hm

extern "C" {

size_t hm_selective_scan_workspace(int B, int T, int Di, int N) {
  if (B <= 0 || T <= 0 || Di <= 0 || N != kNS) return 0;
  const int L = scan_chunk_len(B, T, Di);
  const size_t nC = (size_t)(T + L - 1) / L;
  return (size_t)B * nC * (kNS + 1) * Di * sizeof(float);
}

hm_status hm_selective_scan(const void* x, const void* delta, const float* A, const void* Bm,
                            const void* Cm, const float* D, const void* z, const float* h0,
                            void* y, float* h_out, int B, int T, int Di, int N, hm_dtype dtype,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return hm::conv_scan_impl(x, nullptr, nullptr, nullptr, nullptr, delta, A, Bm, Cm, D, z, h0,
                            y, h_out, B, T, Di, kConvK, N, dtype, workspace, workspace_bytes,
                            (hipStream_t)stream, false, false);
}

hm_status hm_conv_selective_scan(const void* x, const float* conv_w, const float* conv_b,
                                 const float* conv_state_in, float* conv_state_out,
                                 const void* delta, const float* A, const void* Bm,
                                 const void* Cm, const float* D, const void* z, const float* h0,
                                 void* y, float* h_out, int B, int T, int Di, int K, int N,
                                 hm_dtype dtype, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return hm::conv_scan_impl(x, conv_w, conv_b, conv_state_in, conv_state_out, delta, A, Bm, Cm,
                            D, z, h0, y, h_out, B, T, Di, K, N, dtype, workspace, workspace_bytes,
                            (hipStream_t)stream, true, false);
}

hm_status hm_causal_conv1d(const void* x, const float* w, const float* bias,
                           const float* state_in, void* y, float* state_out, int B, int T,
                           int Di, int K, int apply_silu, hm_dtype dtype, void* stream) {
  HM_PTR(x);
  HM_PTR(w);
  HM_PTR(y);
  HM_OPT_PTR(bias);
  HM_OPT_PTR(state_in);
  HM_OPT_PTR(state_out);
  HM_REQUIRE(B > 0 && T > 0 && Di > 0, HM_ERR_INVALID, "B, T and Di must be positive");
  HM_REQUIRE(K == kConvK, HM_ERR_UNSUPPORTED, "only conv width K = 4 is supported");
  HM_REQUIRE(dtype == HM_BF16 || dtype == HM_F32, HM_ERR_UNSUPPORTED, "dtype must be f32 or bf16");
  HM_REQUIRE(y != x, HM_ERR_INVALID, "y must not alias x");
  HM_REQUIRE(state_out == nullptr || state_out != state_in, HM_ERR_INVALID,
             "state_out must not alias state_in");
  HM_REQUIRE((double)B * T * Di < 4.0e9 && B <= 65535 && T <= (1 << 22), HM_ERR_UNSUPPORTED,
             "tensor too large");
  const int tchunk = 64;
  const dim3 grid((Di + 255) / 256, (T + tchunk - 1) / tchunk, B);
  hipStream_t st = (hipStream_t)stream;
  if (dtype == HM_BF16)
    hipLaunchKernelGGL(conv1d_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)x, w, bias,
                       state_in, (bf16_t*)y, state_out, T, Di, apply_silu, tchunk);
  else
    hipLaunchKernelGGL(conv1d_kernel<float>, grid, dim3(256), 0, st, (const float*)x, w, bias,
                       state_in, (float*)y, state_out, T, Di, apply_silu, tchunk);
  return hm::check_launch("conv1d_kernel");
}

}  // extern "C"
