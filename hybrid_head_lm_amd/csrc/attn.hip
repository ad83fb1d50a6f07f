// Attention heads of the hybrid-head mixer over X~ = [meta tokens; tokens].
//
// What is computed: Hymba blog (juejin.cn, "NVIDIA提出Hymba网络"), "数学表示" §3,
// Eq. (1), softmax(Q K^T) V with the standard 1/sqrt(Dh) scale; sliding-window
// layers with meta tokens visible to every later token ("Hymba简介",
// "Hymba 的整体架构"); GQA and rotary embeddings (Hymba-1.5B-Base model card,
// "模型架构").
//
// bf16 path (Dh = 64), two kernels:
//   attn_prep_bf16  one pass over K and V: K rotated and written as bf16 rows
//                   [B, Hkv, Tpad, 64]; V written as transposed 64x64 tiles
//                   [B, Hkv, Tpad/64, 64 (d), 64 (key)] so both MFMA operands
//                   load as 16-byte rows.
//   attn_fwd_bf16   flash attention: a workgroup of 4 waves owns 128 query rows
//                   of one head (32 per wave); 64-key tiles of K and V^T are
//                   staged through LDS (double buffered) and shared by the 4
//                   waves; each wave computes S^T = K Q^T with
//                   v_mfma_f32_32x32x16_bf16 (keys on MFMA rows, its 32 queries
//                   on columns, so every lane owns one query and its softmax
//                   state), an online softmax in float32 (exp2 with the scale and
//                   log2(e) folded into Q), and O^T += V^T P^T with the same
//                   MFMA.  Only key tiles with a visible pair are visited: the
//                   meta tiles and the causal window; the element mask is
//                   applied only on tiles that are not fully visible.
// float32 path (Dh in {16, 32, 64}): a pre-pass rotates K, then one thread per
// query row runs the online softmax over its visible keys.
#include <cmath>

#include "attn_dev.h"

namespace {

// ---------------------------------------------------------------- bf16 kernels
__global__ __launch_bounds__(64) void attn_prep_bf16(
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, bf16_t* __restrict__ Kr,
    bf16_t* __restrict__ Vt, int T, int Tpad, int Hkv, long long pos0, double rstep) {
  attn_prep_bf16_body(blockIdx.x, blockIdx.y, blockIdx.z, k, v, nullptr, nullptr, 0, Kr, Vt, T,
                      Tpad, Hkv, pos0, rstep);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void attn_fwd_bf16(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ Kr, const bf16_t* __restrict__ Vt,
    bf16_t* __restrict__ o, int T, int Tpad, int Hq, int Hkv, int M, int W, long long pos0,
    float qscale, double rstep, int n_qt, int n_groups) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages][2][8192];
  attn_fwd_bf16_body(smem, blockIdx.x, q, Kr, Vt, o, T, Tpad, Hq, Hkv, M, W, pos0, qscale, rstep,
                     n_qt, n_groups, T, 0);
}

// ---------------------------------------------------------------- float32 path
template <int DH>
__global__ __launch_bounds__(256) void attn_prep_f32(const float* __restrict__ k,
                                                     const float* __restrict__ v,
                                                     float* __restrict__ Kr,
                                                     float* __restrict__ Vc, int B, int T,
                                                     int Hkv, long long pos0, double log2_base) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)B * T * Hkv * (DH / 2);
  if (idx >= total) return;
  const int d = idx % (DH / 2);
  const int g = (idx / (DH / 2)) % Hkv;
  const int t = (idx / ((DH / 2) * Hkv)) % T;
  const int b = idx / ((long long)(DH / 2) * Hkv * T);
  const size_t row = (((size_t)b * T + t) * Hkv + g) * DH;
  float sn, cs;
  rope_sincos(pos0 + t, d, DH, log2_base, &sn, &cs);
  const float x1 = k[row + d], x2 = k[row + d + DH / 2];
  float* dst = Kr + (((size_t)b * Hkv + g) * T + t) * DH;
  dst[d] = x1 * cs - x2 * sn;
  dst[d + DH / 2] = x2 * cs + x1 * sn;
  Vc[row + d] = v[row + d];
  Vc[row + d + DH / 2] = v[row + d + DH / 2];
}

template <int DH>
__global__ __launch_bounds__(128) void attn_fwd_f32(const float* __restrict__ q,
                                                    const float* __restrict__ Kr,
                                                    const float* __restrict__ v,
                                                    float* __restrict__ o, int B, int T, int Hq,
                                                    int Hkv, int M, int W, long long pos0,
                                                    float scale, double log2_base) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)B * Hq * T) return;
  const int i = idx % T;
  const int h = (idx / T) % Hq;
  const int b = idx / ((long long)T * Hq);
  const int g = h / (Hq / Hkv);
  float qr[DH];
  const float* src = q + (((size_t)b * T + i) * Hq + h) * DH;
#pragma unroll
  for (int d = 0; d < DH / 2; ++d) {
    float sn, cs;
    rope_sincos(pos0 + i, d, DH, log2_base, &sn, &cs);
    const float x1 = src[d], x2 = src[d + DH / 2];
    qr[d] = (x1 * cs - x2 * sn) * scale;
    qr[d + DH / 2] = (x2 * cs + x1 * sn) * scale;
  }
  float acc[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) acc[d] = 0.f;
  float m = -1e30f, l = 0.f;
  const float* kb = Kr + ((size_t)b * Hkv + g) * T * DH;
  auto visit = [&](int j) {
    const float* kr = kb + (size_t)j * DH;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < DH; ++d) s += qr[d] * kr[d];
    const float mn = fmaxf(m, s);
    const float alpha = expf(m - mn);
    const float p = expf(s - mn);
    l = l * alpha + p;
    const float* vr = v + (((size_t)b * T + j) * Hkv + g) * DH;
#pragma unroll
    for (int d = 0; d < DH; ++d) acc[d] = acc[d] * alpha + p * vr[d];
    m = mn;
  };
  const int me = M < i + 1 ? M : i + 1;
  for (int j = 0; j < me; ++j) visit(j);
  int js = (W > 0) ? (i - W + 1 > M ? i - W + 1 : M) : M;
  if (js < me) js = me;
  for (int j = js; j <= i; ++j) visit(j);
  float* dst = o + (((size_t)b * T + i) * Hq + h) * DH;
  const float inv = 1.f / l;
#pragma unroll
  for (int d = 0; d < DH; ++d) dst[d] = acc[d] * inv;
}

// ---------------------------------------------------------------- index exports
__global__ void debug_mask_kernel(int T, int M, int W, unsigned char* out) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)T * T) return;
  out[idx] = hm_visible((int)(idx / T), (int)(idx % T), M, W) ? 1 : 0;
}

__global__ void debug_tile_kernel(int T, int M, int W, int bm, int bn, int* out) {
  const int a = blockIdx.x * blockDim.x + threadIdx.x;
  const int nq = (T + bm - 1) / bm, nk = (T + bn - 1) / bn;
  if (a >= nq) return;
  int* row = out + (size_t)a * nk;
  for (int c = 0; c < nk; ++c) row[c] = 0;
  const int i0 = a * bm, i1 = min(i0 + bm, T);
  const KvRanges rg = hm_kv_ranges(i0, i1, M, W, bn);
  const int nt = rg.e0 + (rg.e1 - rg.b1);
  for (int it = 0; it < nt; ++it) {
    const int tile = it < rg.e0 ? it : rg.b1 + (it - rg.e0);
    row[tile] = hm_tile_class(i0, i1, tile * bn, min(tile * bn + bn, T), M, W);
  }
}

}  // namespace

namespace hm {

// Shapes and options shared by the prepare and attend halves.
static hm_status attn_check(int B, int T, int Hkv, int Dh, float rope_base, long long pos0,
                            hm_dtype dtype) {
  HM_REQUIRE(B > 0 && T > 0 && Hkv > 0 && Dh > 0, HM_ERR_INVALID,
             "B, T, Hkv and Dh must be positive");
  HM_REQUIRE(pos0 >= 0, HM_ERR_INVALID, "pos0 must be >= 0");
  HM_REQUIRE(rope_base > 1.0f && std::isfinite(rope_base), HM_ERR_INVALID, "rope_base must be > 1");
  HM_REQUIRE(dtype == HM_BF16 || dtype == HM_F32, HM_ERR_UNSUPPORTED, "dtype must be f32 or bf16");
  if (dtype == HM_BF16)
    HM_REQUIRE(Dh == 64, HM_ERR_UNSUPPORTED, "bf16 attention supports Dh = 64 only");
  else
    HM_REQUIRE(Dh == 16 || Dh == 32 || Dh == 64, HM_ERR_UNSUPPORTED,
               "f32 attention supports Dh in {16, 32, 64}");
  HM_REQUIRE(B <= 65535 && Hkv <= 65535 && T <= (1 << 24), HM_ERR_UNSUPPORTED, "tensor too large");
  return HM_OK;
}

hm_status attn_kv_prepare_impl(const void* k, const void* v, void* kv, size_t kv_bytes, int B,
                               int T, int Hkv, int Dh, float rope_base, long long pos0,
                               hm_dtype dtype, hipStream_t st, bool dry) {
  HM_PTR(k);
  HM_PTR(v);
  HM_PTR(kv);
  hm_status s = attn_check(B, T, Hkv, Dh, rope_base, pos0, dtype);
  if (s != HM_OK) return s;
  HM_REQUIRE((double)B * T * Hkv * Dh < 4.0e9, HM_ERR_UNSUPPORTED, "tensor too large");
  HM_REQUIRE(kv_bytes >= hm_attn_kv_bytes(B, T, Hkv, Dh, dtype), HM_ERR_WORKSPACE,
             "kv buffer smaller than hm_attn_kv_bytes()");
  HM_REQUIRE(kv != k && kv != v, HM_ERR_INVALID, "kv must not alias k or v");
  if (dry) return HM_OK;
  const double l2b = log2((double)rope_base);
  if (dtype == HM_BF16) {
    const double rstep = exp2(-l2b / 32.0);   // theta_{d+1} / theta_d for Dh = 64
    const int Tpad = (T + 63) / 64 * 64;
    bf16_t* Kr = (bf16_t*)kv;
    bf16_t* Vt = Kr + (size_t)B * Hkv * Tpad * 64;
    hipLaunchKernelGGL(attn_prep_bf16, dim3(Tpad / 16, Hkv, B), dim3(64), 0, st,
                       (const bf16_t*)k, (const bf16_t*)v, Kr, Vt, T, Tpad, Hkv, pos0, rstep);
    return check_launch("attn_prep_bf16");
  }
  float* Kr = (float*)kv;
  float* Vc = Kr + (size_t)B * Hkv * T * Dh;
  const long long np = (long long)B * T * Hkv * (Dh / 2);
  const dim3 grid((unsigned)((np + 255) / 256));
  switch (Dh) {
    case 16:
      hipLaunchKernelGGL(attn_prep_f32<16>, grid, dim3(256), 0, st, (const float*)k,
                         (const float*)v, Kr, Vc, B, T, Hkv, pos0, l2b);
      break;
    case 32:
      hipLaunchKernelGGL(attn_prep_f32<32>, grid, dim3(256), 0, st, (const float*)k,
                         (const float*)v, Kr, Vc, B, T, Hkv, pos0, l2b);
      break;
    default:
      hipLaunchKernelGGL(attn_prep_f32<64>, grid, dim3(256), 0, st, (const float*)k,
                         (const float*)v, Kr, Vc, B, T, Hkv, pos0, l2b);
      break;
  }
  return check_launch("attn_prep_f32");
}

hm_status attn_with_kv_impl(const void* q, const void* kv, size_t kv_bytes, void* o, int B,
                            int T, int Hq, int Hkv, int Dh, int n_meta, int window,
                            float rope_base, long long pos0, float scale, hm_dtype dtype,
                            hipStream_t st, bool dry) {
  HM_PTR(q);
  HM_PTR(kv);
  HM_PTR(o);
  hm_status s = attn_check(B, T, Hkv, Dh, rope_base, pos0, dtype);
  if (s != HM_OK) return s;
  HM_REQUIRE(Hq > 0 && Hq % Hkv == 0, HM_ERR_INVALID, "Hq must be a positive multiple of Hkv");
  HM_REQUIRE(n_meta >= 0 && n_meta <= T, HM_ERR_INVALID, "need 0 <= n_meta <= T");
  HM_REQUIRE(std::isfinite(scale), HM_ERR_INVALID, "scale must be finite");
  HM_REQUIRE(o != q && o != kv, HM_ERR_INVALID, "o must not alias q or kv");
  HM_REQUIRE((double)B * T * Hq * Dh < 4.0e9 && (double)B * Hq * ((T + kBM - 1) / kBM) < 2.0e9,
             HM_ERR_UNSUPPORTED, "tensor too large");
  HM_REQUIRE(kv_bytes >= hm_attn_kv_bytes(B, T, Hkv, Dh, dtype), HM_ERR_WORKSPACE,
             "kv buffer smaller than hm_attn_kv_bytes()");
  if (dry) return HM_OK;
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)Dh);
  const double l2b = log2((double)rope_base);
  if (dtype == HM_BF16) {
    const double rstep = exp2(-l2b / 32.0);   // theta_{d+1} / theta_d for Dh = 64
    const int Tpad = (T + 63) / 64 * 64;
    const bf16_t* Kr = (const bf16_t*)kv;
    const bf16_t* Vt = Kr + (size_t)B * Hkv * Tpad * 64;
    const int n_qt = (T + kBM - 1) / kBM;
    const int n_groups = B * Hkv * n_qt;
    const int grid = 8 * ((n_groups + 7) / 8) * (Hq / Hkv);
    hipLaunchKernelGGL(attn_fwd_bf16, dim3(grid), dim3(256), 0, st, (const bf16_t*)q, Kr, Vt,
                       (bf16_t*)o, T, Tpad, Hq, Hkv, n_meta, window, pos0, sc * kLog2e, rstep,
                       n_qt, n_groups);
    return check_launch("attn_fwd_bf16");
  }
  const float* Kr = (const float*)kv;
  const float* Vc = Kr + (size_t)B * Hkv * T * Dh;
  const long long nq = (long long)B * Hq * T;
  const dim3 grid((unsigned)((nq + 127) / 128));
  switch (Dh) {
    case 16:
      hipLaunchKernelGGL(attn_fwd_f32<16>, grid, dim3(128), 0, st, (const float*)q, Kr, Vc,
                         (float*)o, B, T, Hq, Hkv, n_meta, window, pos0, sc, l2b);
      break;
    case 32:
      hipLaunchKernelGGL(attn_fwd_f32<32>, grid, dim3(128), 0, st, (const float*)q, Kr, Vc,
                         (float*)o, B, T, Hq, Hkv, n_meta, window, pos0, sc, l2b);
      break;
    default:
      hipLaunchKernelGGL(attn_fwd_f32<64>, grid, dim3(128), 0, st, (const float*)q, Kr, Vc,
                         (float*)o, B, T, Hq, Hkv, n_meta, window, pos0, sc, l2b);
      break;
  }
  return check_launch("attn_fwd_f32");
}

hm_status swa_meta_attn_impl(const void* q, const void* k, const void* v, void* o, int B,
                             int T, int Hq, int Hkv, int Dh, int n_meta, int window,
                             float rope_base, long long pos0, float scale, hm_dtype dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t st,
                             bool dry) {
  HM_REQUIRE(o != k && o != v, HM_ERR_INVALID, "o must not alias k or v");
  HM_REQUIRE(workspace != nullptr && aligned16(workspace), HM_ERR_WORKSPACE,
             "workspace must be a non-NULL 16-byte aligned buffer");
  // validate both halves before launching either
  hm_status s = attn_kv_prepare_impl(k, v, workspace, workspace_bytes, B, T, Hkv, Dh, rope_base,
                                     pos0, dtype, st, true);
  if (s != HM_OK) return s;
  s = attn_with_kv_impl(q, workspace, workspace_bytes, o, B, T, Hq, Hkv, Dh, n_meta, window,
                        rope_base, pos0, scale, dtype, st, true);
  if (s != HM_OK || dry) return s;
  s = attn_kv_prepare_impl(k, v, workspace, workspace_bytes, B, T, Hkv, Dh, rope_base, pos0, dtype,
                           st, false);
  if (s != HM_OK) return s;
  return attn_with_kv_impl(q, workspace, workspace_bytes, o, B, T, Hq, Hkv, Dh, n_meta, window,
                           rope_base, pos0, scale, dtype, st, false);
}

}  // namespace hm

extern "C" {

size_t hm_attn_kv_bytes(int B, int T, int Hkv, int Dh, hm_dtype dtype) {
  if (B <= 0 || T <= 0 || Hkv <= 0 || Dh <= 0) return 0;
  if (dtype == HM_BF16) {
    const size_t Tpad = (size_t)(T + 63) / 64 * 64;
    return 2 * (size_t)B * Hkv * Tpad * 64 * sizeof(bf16_t);
  }
  return 2 * (size_t)B * Hkv * T * Dh * sizeof(float);
}

size_t hm_swa_meta_attn_workspace(int B, int T, int Hkv, int Dh, hm_dtype dtype) {
  return hm_attn_kv_bytes(B, T, Hkv, Dh, dtype);
}

hm_status hm_attn_kv_prepare(const void* k, const void* v, void* kv, size_t kv_bytes, int B,
                             int T, int Hkv, int Dh, float rope_base, long long pos0,
                             hm_dtype dtype, void* stream) {
  return hm::attn_kv_prepare_impl(k, v, kv, kv_bytes, B, T, Hkv, Dh, rope_base, pos0, dtype,
                                  (hipStream_t)stream, false);
}

hm_status hm_attn_with_kv(const void* q, const void* kv, size_t kv_bytes, void* o, int B, int T,
                          int Hq, int Hkv, int Dh, int n_meta, int window, float rope_base,
                          long long pos0, float scale, hm_dtype dtype, void* stream) {
  return hm::attn_with_kv_impl(q, kv, kv_bytes, o, B, T, Hq, Hkv, Dh, n_meta, window, rope_base,
                               pos0, scale, dtype, (hipStream_t)stream, false);
}

hm_status hm_swa_meta_attn(const void* q, const void* k, const void* v, void* o, int B, int T,
                           int Hq, int Hkv, int Dh, int n_meta, int window, float rope_base,
                           long long pos0, float scale, hm_dtype dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return hm::swa_meta_attn_impl(q, k, v, o, B, T, Hq, Hkv, Dh, n_meta, window, rope_base, pos0,
                                scale, dtype, workspace, workspace_bytes, (hipStream_t)stream,
                                false);
}

hm_status hm_debug_attn_mask(int T, int n_meta, int window, unsigned char* out_dev,
                             void* stream) {
  HM_REQUIRE(out_dev != nullptr, HM_ERR_INVALID, "out_dev is NULL");
  HM_REQUIRE(T > 0 && T <= 65536 && n_meta >= 0 && n_meta <= T, HM_ERR_INVALID,
             "need 0 < T <= 65536 and 0 <= n_meta <= T");
  const long long n = (long long)T * T;
  hipLaunchKernelGGL(debug_mask_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, T, n_meta, window, out_dev);
  return hm::check_launch("debug_mask_kernel");
}

hm_status hm_debug_tile_plan(int T, int n_meta, int window, int bm, int bn, int* out_dev,
                             int cap, void* stream) {
  HM_REQUIRE(out_dev != nullptr, HM_ERR_INVALID, "out_dev is NULL");
  HM_REQUIRE(T > 0 && n_meta >= 0 && n_meta <= T && bm > 0 && bn > 0, HM_ERR_INVALID,
             "need T > 0, 0 <= n_meta <= T, bm > 0, bn > 0");
  const long long nq = (T + bm - 1) / bm, nk = (T + bn - 1) / bn;
  HM_REQUIRE((long long)cap >= nq * nk, HM_ERR_INVALID,
             "out_dev holds fewer than ceil(T/bm)*ceil(T/bn) ints");
  hipLaunchKernelGGL(debug_tile_kernel, dim3((unsigned)((nq + 63) / 64)), dim3(64), 0,
                     (hipStream_t)stream, T, n_meta, window, bm, bn, out_dev);
  return hm::check_launch("debug_tile_kernel");
}

void hm_debug_attn_tiles(int* bm_workgroup, int* bm_wave, int* bn) {
  if (bm_workgroup) *bm_workgroup = kBM;
  if (bm_wave) *bm_wave = kWR;
  if (bn) *bn = kBN;
}

}  // extern "C"
