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
constexpr int kStages = 3;   // K/V tiles per workgroup LDS ring (48 KB: 3 workgroups per CU)
constexpr double kInv2Pi = 0.15915494309189533576888376337251;
// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] in bits 15:14): wait until at most N vector-memory ops are
// outstanding, leave the other counters unconstrained.
constexpr int kVmcnt8 = vmcnt_imm(8);
constexpr int kVmcnt4 = vmcnt_imm(4);
constexpr int kVmcnt0 = vmcnt_imm(0);

// Swap bits 2 and 3 of a row index inside a 32-row block.  K rows are stored in
// LDS in this order so that the 32x32 MFMA output gives each lane half 8
// consecutive keys per 16-key step (the order V^T is read in for O += P V).
HM_DEV int swap_b23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// ---------------------------------------------------------------- bf16 pre-pass
// sin/cos of pos * theta with the angle in double, reduced to [-1/2, 1/2]
// revolutions; hardware v_sin/v_cos (plenty for bf16 operands).
// `theta_rev` is the angular frequency in revolutions per position (theta / 2 pi).
HM_DEV void rot_rev(long long pos, double theta_rev, float* s, float* c) {
  double r = (double)pos * theta_rev;
  r -= rint(r);
  *s = __builtin_amdgcn_sinf((float)r);
  *c = __builtin_amdgcn_cosf((float)r);
}

__global__ __launch_bounds__(256) void attn_prep_bf16(
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, bf16_t* __restrict__ Kr,
    bf16_t* __restrict__ Vt, int T, int Tpad, int Hkv, long long pos0, double rstep) {
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
      // theta_d / 2 pi = rstep^d / 2 pi for d = 8c..8c+7 (rstep = base^(-1/32)),
      // by double-precision products
      const double s2 = rstep * rstep, s4 = s2 * s2, s8 = s4 * s4;
      double th = kInv2Pi;
      for (int q = 0; q < c; ++q) th *= s8;
      const double step = rstep;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float sn, cs;
        rot_rev(pos0 + j, th, &sn, &cs);
        th *= step;
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
// LDS tiles (K and V^T alike): 64 rows of 128 bytes; the 16-byte chunk c of
// row r lives in slot c ^ ((r >> 1) & 7).  A 16-lane group of an MFMA operand
// read takes chunk c of 16 consecutive rows; the slot swizzle together with
// the row parity (which 128-byte half of a 256-byte bank line the row falls
// in) puts those 16 chunks on 16 different 16-byte bank groups of the 64-bank
// LDS.  LDS row r of the K tile holds key swap_b23(r).  Tiles go HBM -> LDS
// with global_load_lds_dwordx4 (no register staging).
HM_DEV int lds_slot(int row, int c) { return c ^ ((row >> 1) & 7); }
HM_DEV int lds_off(int row, int c) { return row * 128 + (lds_slot(row, c) << 4); }

typedef __attribute__((address_space(3))) void lds_void;

// A workgroup of 4 waves owns 128 query rows of one head (32 per wave) and
// walks the key tiles visible from them: the meta tiles, then the window.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void attn_fwd_bf16(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ Kr, const bf16_t* __restrict__ Vt,
    bf16_t* __restrict__ o, int T, int Tpad, int Hq, int Hkv, int M, int W, long long pos0,
    float qscale, double rstep, int n_qt, int n_groups) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages][2][8192];

  // Work item.  A group is (query tile, b, kv head) and its items are the
  // Hq/Hkv query heads that read the same K/V.  Groups are ranked heaviest
  // first (the visible key count never decreases with the query tile), rank r
  // goes to XCD r % 8 (blockIdx % 8 selects the XCD), and an XCD runs its
  // groups in rank order with the heads of a group side by side, so that
  // every XCD gets the same mix of long and short items, the longest first,
  // and the heads of a group share K/V tiles in one L2.
  const int grp = Hq / Hkv;
  const int xcd = blockIdx.x & 7, kk = blockIdx.x >> 3;
  const int r = 8 * (kk / grp) + xcd;
  if (r >= n_groups) return;
  const int hh = kk % grp;
  const int n_pairs = n_groups / n_qt;
  const int qt = n_qt - 1 - r / n_pairs;
  const int pair = r % n_pairs;                 // b * Hkv + g
  const int g = pair % Hkv, b = pair / Hkv;
  const int h = g * grp + hh;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, gq = lane >> 5;
  const int i0 = qt * kBM, i1 = min(i0 + kBM, T);
  const int wi0 = i0 + wave * kWR, wi1 = min(wi0 + kWR, T);
  const int qrow = min(wi0 + n, T - 1);

  // Q fragment (B operand of S^T = K Q^T): lane holds query qrow, dims
  // 16 s + 8 gq + e.  Rotated in float32, scaled by scale*log2(e), rounded to
  // bf16.  theta_d / 2 pi = rstep^d / 2 pi by double-precision products.
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
    const double s2 = rstep * rstep, s4 = s2 * s2, s8 = s4 * s4, s16 = s8 * s8;
    double th_s = gq ? kInv2Pi * s8 : kInv2Pi;    // d = 8 gq
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      double th = th_s;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float sn, cs;
        rot_rev(pos0 + qrow, th, &sn, &cs);
        th *= rstep;
        const float x1 = xs[s][e], x2 = xs[s + 2][e];
        xs[s][e] = (x1 * cs - x2 * sn) * qscale;
        xs[s + 2][e] = (x2 * cs + x1 * sn) * qscale;
      }
      th_s *= s16;                                // d = 16 + 8 gq
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s][e] = (__bf16)xs[s][e];
  }

  const KvRanges rg = hm_kv_ranges(i0, i1, M, W, kBN);
  const int nt0 = rg.e0;
  const int ntiles = nt0 + (rg.e1 - rg.b1);

  const unsigned char* Kbase = (const unsigned char*)(Kr + (size_t)pair * Tpad * 64);
  const unsigned char* Vbase = (const unsigned char*)(Vt + (size_t)pair * (Tpad / 64) * 4096);
  // This thread's two 16-byte chunks of each tile: LDS rows 16*wave + 8*i + lane/8,
  // slot lane & 7 (global_load_lds writes lane L of a wave at base + 16 L).
  int koff[2], voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rr = 16 * wave + 8 * i + (lane >> 3);
    const int c = lds_slot(rr, lane & 7);   // the slot map is an involution in c
    koff[i] = swap_b23(rr) * 128 + c * 16;
    voff[i] = rr * 128 + c * 16;
  }
  auto tile_at = [&](int it) { return it < nt0 ? it : rg.b1 + (it - nt0); };
  auto issue = [&](int it) {
    const int tile = tile_at(it);
    const unsigned char* kp = Kbase + (size_t)tile * 8192;
    const unsigned char* vp = Vbase + (size_t)tile * 8192;
    unsigned char* st = smem[it % kStages][0];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      __builtin_amdgcn_global_load_lds((const void*)(kp + koff[i]),
                                       (lds_void*)(st + (16 * wave + 8 * i) * 128), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vp + voff[i]),
                                       (lds_void*)(st + 8192 + (16 * wave + 8 * i) * 128), 16, 0,
                                       0);
    }
  };

  // Online softmax in log2 units with a lazily moved reference m_ref: the
  // MFMA accumulates onto -m_ref, so it yields S - m_ref directly; m_ref moves
  // (and O, l are rescaled) only when a tile's maximum exceeds it by > 8.
  f32x16_v acc[2], cinit;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    acc[0][i] = 0.f;
    acc[1][i] = 0.f;
    cinit[i] = 0.f;
  }
  float m_ref = 0.f, l_run = 0.f;
  bool fresh = true;
  const float NEG_INF = -__builtin_huge_valf();
  const int qi = wi0 + n;

  // LDS ring of kStages = 3 tiles: tile t is issued two iterations before it
  // is used, into the stage that tile t-3 released.  At the top of iteration
  // `it` a thread waits until its own loads of tile `it` have landed (4 loads
  // per thread per tile; tile it+1 may stay in flight), and the barrier
  // publishes the tile to every wave and frees the stage of tile it-1.
  static_assert(kStages == 3, "the wait counts below assume a 3-stage ring");
#pragma unroll
  for (int p = 0; p < kStages - 1; ++p)
    if (p < ntiles) issue(p);

  for (int it = 0; it < ntiles; ++it) {
    if (it + 1 < ntiles) __builtin_amdgcn_s_waitcnt(kVmcnt4);
    else __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    if (it + 2 < ntiles) issue(it + 2);
    const int j0 = tile_at(it) * kBN;
    const int cls = hm_tile_class(wi0, wi1, j0, min(j0 + kBN, T), M, W);
    if (cls == 0) continue;
    // S^T - m_ref (accumulated onto -m_ref); the two 32-key blocks are
    // independent accumulation chains, alternated
    const unsigned char* sk = smem[it % kStages][0];
    f32x16_v S[2];
    S[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_v*)(sk + lds_off(n, gq)),
                                                   qf[0], cinit, 0, 0, 0);
    S[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_v*)(sk + lds_off(32 + n, gq)),
                                                   qf[0], cinit, 0, 0, 0);
#pragma unroll
    for (int k4 = 1; k4 < 4; ++k4)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *(const bf16x8_v*)(sk + lds_off(kb * 32 + n, 2 * k4 + gq)), qf[k4], S[kb], 0, 0, 0);
    if (cls == 1 || j0 + kBN > T) {
      // element (kb, i) is key kbase + off with off = 32 kb + 16 (i / 8) + i % 8;
      // visible iff off <= a and (off < mm or off >= w)  (hm_visible, shifted)
      const int kbase = j0 + 8 * gq;
      const int a = qi - kbase;
      const int mm = M - kbase;
      const int w = W > 0 ? qi - W + 1 - kbase : -1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = 32 * kb + 16 * (i >> 3) + (i & 7);
          const bool vis = (off <= a) & ((off < mm) | (off >= w));
          S[kb][i] = vis ? S[kb][i] : NEG_INF;
        }
    }
    float mx = fmaxf(S[0][0], S[0][1]);
#pragma unroll
    for (int i = 2; i < 16; ++i) mx = fmaxf(mx, S[0][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[1][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool need = fresh ? (mx > NEG_INF) : (mx > 8.f);
    if (__ballot(need) != 0) {
      // move the reference: rescale O and l and shift this tile's scores
      const float delta = need ? mx : 0.f;
      const float alpha = fresh ? 0.f : fast_exp2(-delta);
      if (need) fresh = false;
      m_ref += delta;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        acc[0][i] *= alpha;
        acc[1][i] *= alpha;
        S[0][i] -= delta;
        S[1][i] -= delta;
        cinit[i] = -m_ref;
      }
    }
    bf16x8_v pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) pf[2 * kb + (i >> 3)][i & 7] = (__bf16)fast_exp2(S[kb][i]);
    // row sums of the bf16 probabilities actually used by the PV product
    typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
    const bf16x2_v ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2_v pr = {pf[k4][2 * e], pf[k4][2 * e + 1]};
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run, false);
      }
    const unsigned char* sv = smem[it % kStages][1];
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int row = db * 32 + n;
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *(const bf16x8_v*)(sv + lds_off(row, 2 * k4 + gq)), pf[k4], acc[db], 0, 0, 0);
    }
  }

  const float l = l_run + __shfl_xor(l_run, 32);
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
    hipLaunchKernelGGL(attn_prep_bf16, dim3(Tpad / 64, Hkv, B), dim3(256), 0, st,
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
