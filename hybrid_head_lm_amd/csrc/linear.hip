// Projections around the mixer (Hymba blog, juejin.cn "NVIDIA提出Hymba网络",
// "数学表示" §2: X~ times W_in_proj gives Q, K, V, the SSM input and the gate G;
// §5: W_out_proj maps the fused output back).  y = x W^T with the weight in
// nn.Linear layout [N, K], bf16 operands, float32 accumulation, bf16 results.
//
// Problems of at least 192 tiles of 256 x 256 run the 4-wave 256 x 256 kernel
// of linear_w4.hip; smaller ones run the kernel here.
// One workgroup of 4 waves per 128 x 128 output tile; 64-wide K steps of x and
// W go HBM -> LDS with global_load_lds (double buffered, 2 x 32 KB, so two
// workgroups share a CU); each wave owns a 64 x 64 quarter as 2 x 2 blocks of
// v_mfma_f32_32x32x16_bf16.  LDS rows are 128 bytes (64 bf16 of K) with the
// 16-byte chunk c of row r in slot c ^ ((r >> 1) & 7): the 16 lanes of an
// operand read take one chunk of 16 consecutive rows from 16 different bank
// groups.  The output columns may be split into segments written to separate
// tensors (the in-projection's Q, K, V, x and z), each with its own epilogue:
// a bias, an activation (SiLU for the FFN's hidden layer, softplus for the
// SSM step sizes) and a residual added last (the block's skip connections).
#include <algorithm>
#include <cmath>

#include "linear_dev.h"

namespace {

using namespace hm_lin;

constexpr int kGM = 128, kGN = 128, kGK = 64;   // workgroup tile (rows, columns, K step)
constexpr int kBigTilesMin = 192;               // 256 x 256 tiles from this many on

HM_DEV int lin_slot(int row, int c) { return c ^ ((row >> 1) & 7); }
HM_DEV int lin_off(int row, int c) { return row * 128 + (lin_slot(row, c) << 4); }

__global__ __launch_bounds__(256) void linear_bf16(const bf16_t* __restrict__ x,
                                                   const bf16_t* __restrict__ w, int M, int N,
                                                   int K, LinOut out, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2][2][kGM * 128];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * kGM, n0 = tn * kGN;

  // This thread's 16-byte chunks of each K step: LDS rows 32 i + 8 wave + lane/8,
  // slot lane & 7 (global_load_lds writes lane L of a wave at base + 16 L); rows
  // past M or N read the last row (their results are not stored).
  const bf16_t* asrc[4];
  const bf16_t* wsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * i + 8 * wave + (lane >> 3);
    const int c = lin_slot(row, lane & 7);   // the slot map is an involution in c
    asrc[i] = x + (size_t)std::min(m0 + row, M - 1) * K + c * 8;
    wsrc[i] = w + (size_t)std::min(n0 + row, N - 1) * K + c * 8;
  }
  auto issue = [&](int kt, int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_global_load_lds((const void*)(asrc[i] + (size_t)kt * kGK),
                                       (lin_lds_t*)(smem[s][0] + (32 * i + 8 * wave) * 128), 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(wsrc[i] + (size_t)kt * kGK),
                                       (lin_lds_t*)(smem[s][1] + (32 * i + 8 * wave) * 128), 16,
                                       0, 0);
    }
  };

  f32x16_v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int wr = wave >> 1, wc = wave & 1;     // this wave's 64 x 64 quarter
  const int r32 = lane & 31, hk = lane >> 5;
  const int nk = K / kGK;

  // K step kt+1 is issued right after the barrier of step kt (which frees the
  // buffer of step kt-1) and loads while step kt is computed.
  issue(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    if (kt + 1 < nk) issue(kt + 1, (kt + 1) & 1);
    const unsigned char* sa = smem[kt & 1][0];
    const unsigned char* sw = smem[kt & 1][1];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_v af[2], bw[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *(const bf16x8_v*)(sa + lin_off(64 * wr + 32 * i + r32, 2 * ks + hk));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bw[j] = *(const bf16x8_v*)(sw + lin_off(64 * wc + 32 * j + r32, 2 * ks + hk));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bw[j], acc[i][j], 0, 0, 0);
    }
  }

  // Output through LDS (the operand stages are idle now): element r of block
  // (i, j) is row 32 i + 8 (r / 4) + 4 hk + r % 4 and column 32 j + lane % 32
  // of the wave's quarter.  The tile is staged as float32, column c of row r
  // at c ^ (32 ((r >> 2) & 1)) so that the two row groups of a block write
  // disjoint banks; then every thread takes 16-byte chunks (8 columns of one
  // row, one segment): bias, activation, residual, bf16.
  float* stg = (float*)&smem[0][0][0];
  __syncthreads();   // every wave is done with the operand stages
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int sr = 64 * wr + 32 * i + 8 * (r >> 2) + 4 * hk + (r & 3);
        stg[sr * 128 + ((64 * wc + 32 * j + r32) ^ (hk << 5))] = acc[i][j][r];
      }
  __syncthreads();
#pragma unroll 2
  for (int it = 0; it < 8; ++it) {
    const int q = it * 256 + tid, sr = q >> 4, c = q & 15;
    const int row = m0 + sr, col = n0 + 8 * c;
    if (row >= M || col >= N) continue;
    const float* sp8 = stg + sr * 128 + ((8 * c) ^ (((sr >> 2) & 1) << 5));
    store_chunk8(out, row, col, *(const float4*)sp8, *(const float4*)(sp8 + 4));
  }
}

}  // namespace

namespace hm {

using namespace hm_lin;

// Validates the arguments, then one launch.
hm_status linear_launch(const void* x, const void* w, int M, int N, int K, int n_seg,
                        void* const* outs, const int* seg_cols, const hm_linear_epilogue* ep,
                        hipStream_t st, bool dry) {
  HM_PTR(x);
  HM_PTR(w);
  HM_REQUIRE(M > 0 && N > 0 && K > 0, HM_ERR_INVALID, "M, N and K must be positive");
  HM_REQUIRE(K % kGK == 0, HM_ERR_UNSUPPORTED, "K must be a multiple of 64");
  HM_REQUIRE((double)M * K < 2.0e9 && (double)N * K < 2.0e9 && (double)M * N < 2.0e9,
             HM_ERR_UNSUPPORTED, "matrix too large");
  HM_REQUIRE(n_seg >= 1 && n_seg <= kMaxSeg, HM_ERR_INVALID, "need 1 <= n_seg <= 8");
  HM_REQUIRE(outs != nullptr && seg_cols != nullptr, HM_ERR_INVALID,
             "outs and seg_cols are required (host arrays of n_seg entries)");
  LinOut o{};
  o.n = n_seg;
  o.col0[0] = 0;
  for (int s = 0; s < n_seg; ++s) {
    HM_REQUIRE(seg_cols[s] > 0 && seg_cols[s] % 16 == 0, HM_ERR_INVALID,
               "segment widths must be positive multiples of 16");
    HM_PTR(outs[s]);
    HM_REQUIRE(outs[s] != x && outs[s] != w, HM_ERR_INVALID, "outputs must not alias x or w");
    for (int t = 0; t < s; ++t)
      HM_REQUIRE(outs[t] != outs[s], HM_ERR_INVALID, "segment outputs must be distinct");
    o.p[s] = (bf16_t*)outs[s];
    o.col0[s + 1] = o.col0[s] + seg_cols[s];
    if (ep) {
      HM_REQUIRE(ep[s].act == HM_ACT_NONE || ep[s].act == HM_ACT_SILU ||
                     ep[s].act == HM_ACT_SOFTPLUS,
                 HM_ERR_INVALID, "unknown activation");
      HM_REQUIRE(ep[s].residual == nullptr || (ep[s].residual != x && ep[s].residual != w),
                 HM_ERR_INVALID, "a residual must not alias x or w");
      HM_OPT_PTR(ep[s].residual);
      HM_OPT_PTR(ep[s].bias);
      for (int t = 0; t < n_seg; ++t)
        HM_REQUIRE(ep[s].residual == nullptr || t == s || ep[s].residual != outs[t],
                   HM_ERR_INVALID, "a residual may only alias its own segment's output");
      o.bias[s] = ep[s].bias;
      o.res[s] = (const bf16_t*)ep[s].residual;
      o.act[s] = ep[s].act;
    }
  }
  HM_REQUIRE(o.col0[n_seg] == N, HM_ERR_INVALID, "segment widths must sum to N");
  if (dry) return HM_OK;
  // 256 x 256 tiles (linear_w4.hip) once they fill most CUs; else 128 x 128
  // tiles (two workgroups per CU).
  const int big_m = (M + 255) / 256, big_n = (N + 255) / 256;
  if (big_m * big_n >= kBigTilesMin) {
    launch_w4((const bf16_t*)x, (const bf16_t*)w, M, N, K, o, st);
    return check_launch("linear_bf16_w4");
  }
  const int tiles_m = (M + kGM - 1) / kGM, tiles_n = (N + kGN - 1) / kGN;
  hipLaunchKernelGGL(linear_bf16, dim3(tiles_m * tiles_n), dim3(256), 0, st, (const bf16_t*)x,
                     (const bf16_t*)w, M, N, K, o, tiles_n);
  return check_launch("linear_bf16");
}

}  // namespace hm

extern "C" {

hm_status hm_linear_bf16(const void* x, const void* w, int M, int N, int K, int n_seg,
                         void* const* outs, const int* seg_cols, void* stream) {
  return hm::linear_launch(x, w, M, N, K, n_seg, outs, seg_cols, nullptr, (hipStream_t)stream);
}

hm_status hm_linear_bf16_ex(const void* x, const void* w, int M, int N, int K, int n_seg,
                            void* const* outs, const int* seg_cols,
                            const hm_linear_epilogue* epilogues, void* stream) {
  return hm::linear_launch(x, w, M, N, K, n_seg, outs, seg_cols, epilogues, (hipStream_t)stream);
}

}  // extern "C"
