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
#include <math.h>

#include <cmath>

#include "hm_common.h"

namespace {

constexpr int kBM = 128;     // query rows per workgroup
constexpr int kWR = 32;      // query rows per wave
constexpr int kBN = 64;      // keys per tile
constexpr int kLdsRow = 72;  // padded LDS row (bf16 elements): 144 B keeps 16-B reads conflict-free

// Swap bits 2 and 3 of a row index inside a 32-row block.  K rows are stored in
// LDS in this order so that the 32x32 MFMA output gives each lane half 8
// consecutive keys per 16-key step (the order V^T is read in for O += P V).
HM_DEV int swap_b23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// ---------------------------------------------------------------- bf16 pre-pass
__global__ __launch_bounds__(256) void attn_prep_bf16(
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, bf16_t* __restrict__ Kr,
    bf16_t* __restrict__ Vt, int T, int Tpad, int Hkv, long long pos0, double log2_base) {
  __shared__ __attribute__((aligned(16))) bf16_t sv[64 * kLdsRow];
  const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x;
  const int j0 = tile * 64;
  {  // K rows: thread -> (row t/4, dims 8c..8c+7 and their rotation partners +32)
    const int r = t >> 2, c = t & 3;
    const int j = j0 + r;
    uint4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (j < T) {
      const bf16_t* src = k + (((size_t)b * T + j) * Hkv + g) * 64;
      uint4 xl = *(const uint4*)(src + 8 * c);
      uint4 xh = *(const uint4*)(src + 32 + 8 * c);
      const bf16_t* pl = (const bf16_t*)&xl;
      const bf16_t* ph = (const bf16_t*)&xh;
      bf16_t ol[8], oh[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float sn, cs;
        rope_sincos(pos0 + j, 8 * c + e, 64, log2_base, &sn, &cs);
        const float x1 = bf2f(pl[e]), x2 = bf2f(ph[e]);
        ol[e] = f2bf(x1 * cs - x2 * sn);
        oh[e] = f2bf(x2 * cs + x1 * sn);
      }
      lo = *(const uint4*)ol;
      hi = *(const uint4*)oh;
    }
    bf16_t* dst = Kr + (((size_t)b * Hkv + g) * Tpad + j) * 64;
    *(uint4*)(dst + 8 * c) = lo;
    *(uint4*)(dst + 32 + 8 * c) = hi;
  }
  // V: 64 keys x 64 dims through LDS, written out transposed (zero past T).
  for (int ci = t; ci < 512; ci += 256) {
    const int r = ci >> 3, c = ci & 7;
    const int j = j0 + r;
    uint4 val = {0u, 0u, 0u, 0u};
    if (j < T) val = *(const uint4*)(v + (((size_t)b * T + j) * Hkv + g) * 64 + 8 * c);
    *(uint4*)(sv + r * kLdsRow + 8 * c) = val;
  }
  __syncthreads();
  bf16_t* vt = Vt + (((size_t)b * Hkv + g) * (Tpad / 64) + tile) * 4096;
  for (int ci = t; ci < 512; ci += 256) {
    const int d = ci >> 3, c = ci & 7;
    bf16_t tmp[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) tmp[e] = sv[(8 * c + e) * kLdsRow + d];
    *(uint4*)(vt + d * 64 + 8 * c) = *(const uint4*)tmp;
  }
}

// ---------------------------------------------------------------- bf16 flash kernel
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ Kr, const bf16_t* __restrict__ Vt,
    bf16_t* __restrict__ o, int T, int Tpad, int Hq, int Hkv, int M, int W, long long pos0,
    float qscale, double log2_base, int n_qt, int n_items) {
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][kBN * kLdsRow];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][64 * kLdsRow];

  // Work item.  Items are ordered (b, kv group) -> query tile (heaviest
  // first) -> head within the group, and each XCD (blockIdx % 8) takes one
  // contiguous eighth of that list, so the workgroups that read the same K/V
  // share an L2.
  const int xcd = blockIdx.x & 7, kk = blockIdx.x >> 3;
  const int per = n_items >> 3, rem = n_items & 7;
  if (kk >= per + (xcd < rem ? 1 : 0)) return;
  const int item = xcd * per + (xcd < rem ? xcd : rem) + kk;
  const int grp = Hq / Hkv;
  const int hh = item % grp;
  const int qt = n_qt - 1 - (item / grp) % n_qt;
  const int pair = item / (grp * n_qt);       // b * Hkv + g
  const int g = pair % Hkv, b = pair / Hkv;
  const int h = g * grp + hh;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, gq = lane >> 5;
  const int i0 = qt * kBM, i1 = min(i0 + kBM, T);
  const int wi0 = i0 + wave * kWR, wi1 = min(wi0 + kWR, T);
  const int qrow = min(wi0 + n, T - 1);

  // Q fragment (B operand of S^T = K Q^T): lane holds query qrow, dims
  // 16 s + 8 gq + e.  Rotated in float32, scaled by scale*log2(e), rounded to bf16.
  bf16x8_v qf[4];
  {
    const bf16_t* src = q + (((size_t)b * T + qrow) * Hq + h) * 64;
    float xs[4][8];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 raw = *(const uint4*)(src + 16 * s + 8 * gq);
      const bf16_t* p = (const bf16_t*)&raw;
#pragma unroll
      for (int e = 0; e < 8; ++e) xs[s][e] = bf2f(p[e]);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float sn, cs;
        rope_sincos(pos0 + qrow, 16 * s + 8 * gq + e, 64, log2_base, &sn, &cs);
        const float x1 = xs[s][e], x2 = xs[s + 2][e];
        xs[s][e] = (x1 * cs - x2 * sn) * qscale;
        xs[s + 2][e] = (x2 * cs + x1 * sn) * qscale;
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s][e] = (__bf16)xs[s][e];
  }

  const KvRanges rg = hm_kv_ranges(i0, i1, M, W, kBN);
  const int nt0 = rg.e0;
  const int ntiles = nt0 + (rg.e1 - rg.b1);

  const bf16_t* Kbase = Kr + (size_t)pair * Tpad * 64;
  const bf16_t* Vbase = Vt + (size_t)pair * (Tpad / 64) * 4096;

  uint4 rk[2], rv[2];
  auto gload = [&](int tile) {
    const bf16_t* kp = Kbase + (size_t)tile * 4096;
    const bf16_t* vp = Vbase + (size_t)tile * 4096;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int c = threadIdx.x + 256 * r;
      rk[r] = *(const uint4*)(kp + c * 8);
      rv[r] = *(const uint4*)(vp + c * 8);
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int c = threadIdx.x + 256 * r;
      const int row = c >> 3, col = c & 7;
      *(uint4*)(&sK[buf][swap_b23(row) * kLdsRow + col * 8]) = rk[r];
      *(uint4*)(&sV[buf][row * kLdsRow + col * 8]) = rv[r];
    }
  };

  f32x16_v acc[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  float m_run = -1e30f, l_run = 0.f;
  const float NEG_INF = -__builtin_huge_valf();

  if (ntiles > 0) gload(0 < nt0 ? 0 : rg.b1);
  for (int it = 0; it < ntiles; ++it) {
    const int tile = it < nt0 ? it : rg.b1 + (it - nt0);
    const int buf = it & 1;
    swrite(buf);
    __syncthreads();
    if (it + 1 < ntiles) gload(it + 1 < nt0 ? it + 1 : rg.b1 + (it + 1 - nt0));
    const int j0 = tile * kBN;
    const int cls = hm_tile_class(wi0, wi1, j0, min(j0 + kBN, T), M, W);
    if (cls != 0) {
      f32x16_v S[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) S[kb][i] = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8_v a = *(const bf16x8_v*)(&sK[buf][(kb * 32 + n) * kLdsRow + 16 * s + 8 * gq]);
          S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], S[kb], 0, 0, 0);
        }
      }
      if (cls == 1 || j0 + kBN > T) {
        const int qi = wi0 + n;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = j0 + 32 * kb + 16 * (i >> 3) + 8 * gq + (i & 7);
            if (!hm_visible(qi, key, M, W)) S[kb][i] = NEG_INF;
          }
      }
      float mx = S[0][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, S[0][i]);
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[1][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      float ls = 0.f;
      bf16x8_v pf[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(S[kb][i] - m_new);
          ls += p;
          pf[2 * kb + (i >> 3)][i & 7] = (__bf16)p;
        }
      l_run = l_run * alpha + ls;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8_v a = *(const bf16x8_v*)(&sV[buf][(db * 32 + n) * kLdsRow + 16 * s + 8 * gq]);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[s], acc[db], 0, 0, 0);
        }
      }
    }
  }

  const float l = l_run + __shfl_xor(l_run, 32);
  const int qi = wi0 + n;
  if (qi < T) {
    const float inv = 1.f / l;
    bf16_t* dst = o + (((size_t)b * T + qi) * Hq + h) * 64;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + 8 * r4 + 4 * gq;
        uint2 pk;
        pk.x = pack_bf16x2(acc[db][4 * r4 + 0] * inv, acc[db][4 * r4 + 1] * inv);
        pk.y = pack_bf16x2(acc[db][4 * r4 + 2] * inv, acc[db][4 * r4 + 3] * inv);
        *(uint2*)(dst + d) = pk;
      }
  }
}

// ---------------------------------------------------------------- float32 path
template <int DH>
__global__ __launch_bounds__(256) void attn_prep_f32(const float* __restrict__ k,
                                                     float* __restrict__ Kr, int B, int T,
                                                     int Hkv, long long pos0, double log2_base) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long total = (long long)B * T * Hkv * (DH / 2);
  if (idx >= total) return;
  const int d = idx % (DH / 2);
  const int g = (idx / (DH / 2)) % Hkv;
  const int t = (idx / ((DH / 2) * Hkv)) % T;
  const int b = idx / ((long long)(DH / 2) * Hkv * T);
  const float* src = k + (((size_t)b * T + t) * Hkv + g) * DH;
  float sn, cs;
  rope_sincos(pos0 + t, d, DH, log2_base, &sn, &cs);
  const float x1 = src[d], x2 = src[d + DH / 2];
  float* dst = Kr + (((size_t)b * Hkv + g) * T + t) * DH;
  dst[d] = x1 * cs - x2 * sn;
  dst[d + DH / 2] = x2 * cs + x1 * sn;
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
  out[idx] = hm_visible(idx / T, idx % T, M, W) ? 1 : 0;
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

hm_status swa_meta_attn_impl(const void* q, const void* k, const void* v, void* o, int B,
                             int T, int Hq, int Hkv, int Dh, int n_meta, int window,
                             float rope_base, long long pos0, float scale, hm_dtype dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t st,
                             bool dry) {
  HM_PTR(q);
  HM_PTR(k);
  HM_PTR(v);
  HM_PTR(o);
  HM_REQUIRE(B > 0 && T > 0 && Hq > 0 && Hkv > 0 && Dh > 0, HM_ERR_INVALID,
             "B, T, Hq, Hkv and Dh must be positive");
  HM_REQUIRE(Hq % Hkv == 0, HM_ERR_INVALID, "Hq must be a multiple of Hkv");
  HM_REQUIRE(n_meta >= 0 && n_meta <= T, HM_ERR_INVALID, "need 0 <= n_meta <= T");
  HM_REQUIRE(pos0 >= 0, HM_ERR_INVALID, "pos0 must be >= 0");
  HM_REQUIRE(rope_base > 1.0f && std::isfinite(rope_base), HM_ERR_INVALID, "rope_base must be > 1");
  HM_REQUIRE(std::isfinite(scale), HM_ERR_INVALID, "scale must be finite");
  HM_REQUIRE(o != q && o != k && o != v, HM_ERR_INVALID, "o must not alias an input");
  HM_REQUIRE(dtype == HM_BF16 || dtype == HM_F32, HM_ERR_UNSUPPORTED, "dtype must be f32 or bf16");
  if (dtype == HM_BF16)
    HM_REQUIRE(Dh == 64, HM_ERR_UNSUPPORTED, "bf16 attention supports Dh = 64 only");
  else
    HM_REQUIRE(Dh == 16 || Dh == 32 || Dh == 64, HM_ERR_UNSUPPORTED,
               "f32 attention supports Dh in {16, 32, 64}");
  HM_REQUIRE((double)B * T * Hq * Dh < 4.0e9 && B <= 65535 && Hkv <= 65535, HM_ERR_UNSUPPORTED,
             "tensor too large");
  const size_t need = hm_swa_meta_attn_workspace(B, T, Hkv, Dh, dtype);
  HM_REQUIRE(workspace != nullptr && workspace_bytes >= need && aligned16(workspace),
             HM_ERR_WORKSPACE, "workspace smaller than hm_swa_meta_attn_workspace()");
  if (dry) return HM_OK;

  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)Dh);
  const double l2b = log2((double)rope_base);
  if (dtype == HM_BF16) {
    const int Tpad = (T + 63) / 64 * 64;
    bf16_t* Kr = (bf16_t*)workspace;
    bf16_t* Vt = Kr + (size_t)B * Hkv * Tpad * 64;
    hipLaunchKernelGGL(attn_prep_bf16, dim3(Tpad / 64, Hkv, B), dim3(256), 0, st,
                       (const bf16_t*)k, (const bf16_t*)v, Kr, Vt, T, Tpad, Hkv, pos0, l2b);
    hm_status s = check_launch("attn_prep_bf16");
    if (s != HM_OK) return s;
    const int n_qt = (T + kBM - 1) / kBM;
    const int n_items = B * Hq * n_qt;
    const int grid = (n_items + 7) / 8 * 8;
    hipLaunchKernelGGL(attn_fwd_bf16, dim3(grid), dim3(256), 0, st, (const bf16_t*)q,
                       (const bf16_t*)Kr, (const bf16_t*)Vt, (bf16_t*)o, T, Tpad, Hq, Hkv,
                       n_meta, window, pos0, sc * kLog2e, l2b, n_qt, n_items);
    return check_launch("attn_fwd_bf16");
  }
  float* Kr = (float*)workspace;
  const long long np = (long long)B * T * Hkv * (Dh / 2);
  const long long nq = (long long)B * Hq * T;
#define HM_F32_CASE(DHV)                                                                    \
  case DHV:                                                                                 \
    hipLaunchKernelGGL(attn_prep_f32<DHV>, dim3((unsigned)((np + 255) / 256)), dim3(256), 0, \
                       st, (const float*)k, Kr, B, T, Hkv, pos0, l2b);                       \
    hipLaunchKernelGGL(attn_fwd_f32<DHV>, dim3((unsigned)((nq + 127) / 128)), dim3(128), 0, \
                       st, (const float*)q, (const float*)Kr, (const float*)v, (float*)o, B, \
                       T, Hq, Hkv, n_meta, window, pos0, sc, l2b);                           \
    break;
  switch (Dh) {
    HM_F32_CASE(16)
    HM_F32_CASE(32)
    HM_F32_CASE(64)
  }
#undef HM_F32_CASE
  return check_launch("attn_fwd_f32");
}

}  // namespace hm

extern "C" {

size_t hm_swa_meta_attn_workspace(int B, int T, int Hkv, int Dh, hm_dtype dtype) {
  if (B <= 0 || T <= 0 || Hkv <= 0 || Dh <= 0) return 0;
  if (dtype == HM_BF16) {
    const size_t Tpad = (size_t)(T + 63) / 64 * 64;
    return 2 * (size_t)B * Hkv * Tpad * 64 * sizeof(bf16_t);
  }
  return (size_t)B * Hkv * T * Dh * sizeof(float);
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
                             long long cap, void* stream) {
  HM_REQUIRE(out_dev != nullptr, HM_ERR_INVALID, "out_dev is NULL");
  HM_REQUIRE(T > 0 && n_meta >= 0 && n_meta <= T && bm > 0 && bn > 0, HM_ERR_INVALID,
             "need T > 0, 0 <= n_meta <= T, bm > 0, bn > 0");
  const long long nq = (T + bm - 1) / bm, nk = (T + bn - 1) / bn;
  HM_REQUIRE(cap >= nq * nk, HM_ERR_INVALID, "out_dev holds fewer than ceil(T/bm)*ceil(T/bn) ints");
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
