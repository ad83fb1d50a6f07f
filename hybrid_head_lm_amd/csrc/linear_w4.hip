// Projection GEMM for large problems (y = x W^T, bf16 operands, float32
// accumulation; the in- and out-projections and the feed-forward network of a
// Hymba block): one workgroup of 4 waves per 256 x 256 output tile, each wave
// owning a 128 x 128 quarter as 8 x 8 blocks of v_mfma_f32_16x16x32_bf16 with
// its 256 accumulators in AGPRs (this file is compiled without the VGPR-only
// MFMA form).  Per 32 of K a wave reads 16 operand fragments (16 KB) for 64
// MFMAs, half the LDS operand bytes per flop of the 128 x 128 kernel.
// 64-wide K steps go HBM -> LDS with global_load_lds through two 64 KB
// stages (one workgroup per CU); LDS rows are 128 bytes with the 16-byte chunk
// c of row r in slot c ^ ((r >> 1) & 7), so the 16 lanes of an operand read
// (16 consecutive rows, one chunk) hit 16 different bank groups.  Tiles are
// dealt to the XCDs in contiguous ranges (workgroup b runs on XCD b % 8), in
// groups of 4 tile rows.
// The finished tile leaves through LDS in two halves of 128 rows as 16-byte
// row chunks, the residual added after the activation.
#include "linear_dev.h"

namespace {

using namespace hm_lin;

constexpr int kTM = 256, kTN = 256, kTK = 64;
constexpr int kGroupM = 4;

HM_DEV int w4_off(int row, int c) { return row * 128 + ((c ^ ((row >> 1) & 7)) << 4); }

__global__ __launch_bounds__(256) void linear_bf16_w4(const bf16_t* __restrict__ x,
                                                      const bf16_t* __restrict__ w, int M, int N,
                                                      int K, LinOut out, int tiles_m,
                                                      int tiles_n) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2][2][kTM * 128];
  const int per_xcd = (tiles_m * tiles_n + 7) / 8;
  const int t = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (t >= tiles_m * tiles_n) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Grouped order inside an XCD's range: groups of kGroupM tile rows are walked
  // column by column, so that the 32 tiles an XCD runs at once cover 4 rows x 8
  // columns (12 operand panels in its L2 instead of ~23 for row-major order).
  // Measured on the block's shapes: fetched bytes 2.1 -> 1.0 GB (in-projection)
  // and 4.7 -> 1.9 GB (FFN up), 2-5% faster.
  const int gsz = kGroupM * tiles_n, grp0 = (t / gsz) * kGroupM;
  const int gm = min(kGroupM, tiles_m - grp0), tl = t % gsz;
  const int m0 = (grp0 + tl % gm) * kTM, n0 = (tl / gm) * kTN;

  // This thread's 16-byte chunks of each K step: wave v fills LDS rows
  // 64 v .. 64 v + 63 of x's and of W's tile, 8 rows per instruction, lane L
  // at row 8 i + L / 8, slot L % 8, which holds chunk (L % 8) ^ ((row / 2) % 8)
  // (the slot map is an involution in the chunk).  Rows past M or N read the
  // last row (their results are not stored).  Element offsets fit 32 bits
  // (M K and N K stay below 2^31).
  const int lrow = 64 * wave + (lane >> 3);
  auto issue = [&](int kt, int s) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = lrow + 8 * i;
      const unsigned c8 = (unsigned)(((lane & 7) ^ ((row >> 1) & 7)) * 8 + kt * kTK);
      const unsigned ao = (unsigned)min(m0 + row, M - 1) * (unsigned)K + c8;
      const unsigned wo = (unsigned)min(n0 + row, N - 1) * (unsigned)K + c8;
      __builtin_amdgcn_global_load_lds((const void*)(x + ao),
                                       (lin_lds_t*)(smem[s][0] + (64 * wave + 8 * i) * 128), 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(w + wo),
                                       (lin_lds_t*)(smem[s][1] + (64 * wave + 8 * i) * 128), 16,
                                       0, 0);
    }
  };

  f32x4_v acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  const int wr = wave >> 1, wc = wave & 1;
  const int r16 = lane & 15, kq = lane >> 4;
  const int nk = K / kTK;

  // Software pipeline over half K steps (32 of K, 64 MFMAs a wave): the
  // fragments of the next half step are read from LDS while the MFMAs of the
  // current one run.  In K step kt a wave reads the second half's fragments,
  // multiplies the first half, waits for K step kt + 1's loads (16 per thread
  // per step) and meets the other waves at the barrier: past it every wave
  // has read K step kt, so its buffer takes K step kt + 2, and the first half
  // of K step kt + 1 is read while the second half of K step kt is multiplied.
  bf16x8_v fa[2][8], fb[2][8];
  auto frags = [&](int hb, int kt, int ks) {
    const unsigned char* sa = smem[kt & 1][0];
    const unsigned char* sw = smem[kt & 1][1];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      fa[hb][i] = *(const bf16x8_v*)(sa + w4_off(128 * wr + 16 * i + r16, 4 * ks + kq));
#pragma unroll
    for (int j = 0; j < 8; ++j)
      fb[hb][j] = *(const bf16x8_v*)(sw + w4_off(128 * wc + 16 * j + r16, 4 * ks + kq));
  };
  auto mfmas = [&](int hb) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[hb][i], fb[hb][j], acc[i][j], 0, 0, 0);
  };
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  if (nk > 1)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(16));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();
  frags(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    frags(1, kt, 1);
    mfmas(0);
    if (kt + 1 < nk) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    if (kt + 2 < nk) issue(kt + 2, kt & 1);
    if (kt + 1 < nk) frags(0, kt + 1, 0);
    mfmas(1);
  }

  // Output.  Element r of block (i, j) is row 16 i + 4 (lane / 16) + r and
  // column 16 j + lane % 16 of the wave's quarter.  Half h of the tile (rows
  // 128 h .. 128 h + 127, the quarters of waves with wr == h) is staged as
  // float32 in a 128 x 256 tile, column c of row r at c ^ (16 ((r >> 2) & 3))
  // so that the four row groups of a block write disjoint banks; then every
  // thread takes 16-byte chunks (8 columns of one row, one segment): bias,
  // activation, residual, bf16.
  float* stg = (float*)&smem[0][0][0];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    __syncthreads();   // the operand stages (h == 0) or the previous half are no longer read
    if (wr == h) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int sr = 16 * i + 4 * kq + r;
            stg[sr * 256 + ((128 * wc + 16 * j + r16) ^ (kq << 4))] = acc[i][j][r];
          }
    }
    __syncthreads();
#pragma unroll 2
    for (int it = 0; it < 16; ++it) {
      const int q = it * 256 + tid, sr = q >> 5, c = q & 31;
      const int row = m0 + 128 * h + sr;
      const int col = n0 + 8 * c;
      if (row >= M || col >= N) continue;
      const float* sp8 = stg + sr * 256 + ((8 * c) ^ (((sr >> 2) & 3) << 4));
      store_chunk8(out, row, col, *(const float4*)sp8, *(const float4*)(sp8 + 4));
    }
  }
}

}  // namespace

namespace hm_lin {

void launch_w4(const bf16_t* x, const bf16_t* w, int M, int N, int K, const LinOut& out,
               hipStream_t st) {
  const int tm = (M + kTM - 1) / kTM, tn = (N + kTN - 1) / kTN;
  const int grid = 8 * ((tm * tn + 7) / 8);
  hipLaunchKernelGGL(linear_bf16_w4, dim3(grid), dim3(256), 0, st, x, w, M, N, K, out, tm, tn);
}

}  // namespace hm_lin
