// Device bodies of the bf16 attention path (Dh = 64): the K/V pre-pass and the
// flash kernel, shared by the standalone kernels and the fused prefill kernels.
// See attn.hip for the method.
#pragma once

#include <math.h>

#include "hm_common.h"

namespace {


constexpr int kBM = 128;     // query rows per workgroup
constexpr int kWR = 32;      // query rows per wave
constexpr int kBN = 64;      // keys per tile
constexpr int kStages = 2;   // K/V tiles per workgroup (32 KB of LDS: 4 workgroups per CU)
constexpr double kInv2Pi = 0.15915494309189533576888376337251;
// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] in bits 15:14): wait until at most N vector-memory ops are
// outstanding, leave the other counters unconstrained.
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

// One 64-thread workgroup per (quarter of a 64-key tile, KV head, batch): it
// rotates 16 K rows and writes 16 rows (dims) of the transposed V tile.  Key
// row j < Mk comes from the cached meta rows meta_k / meta_v [Mk, Hkv, 64]
// (shared by the batch), key row Mk + i from row i of k / v [B, T, Hkv, 64].
HM_DEV void attn_prep_bf16_body(int bx, int g, int b, const bf16_t* __restrict__ k,
                                const bf16_t* __restrict__ v,
                                const bf16_t* __restrict__ meta_k,
                                const bf16_t* __restrict__ meta_v, int Mk,
                                bf16_t* __restrict__ Kr, bf16_t* __restrict__ Vt, int T,
                                int Tpad, int Hkv, long long pos0, double rstep) {
  __shared__ __attribute__((aligned(16))) bf16_t sv[64][16 + 2];
  const int part = bx & 3, tile = bx >> 2;
  const int t = threadIdx.x;
  const int j0 = tile * 64;
  {  // K row 16 part + t/4: dims 8c..8c+7 and their rotation partners +32
    const int r = 16 * part + (t >> 2), c = t & 3;
    const int j = j0 + r;
    uint4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (j < Mk + T) {
      const bf16_t* src = j < Mk ? meta_k + ((size_t)j * Hkv + g) * 64
                                 : k + (((size_t)b * T + (j - Mk)) * Hkv + g) * 64;
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
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float sn, cs;
        rot_rev(pos0 + j, th, &sn, &cs);
        th *= rstep;
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
  {  // V: dims 16 part .. +15 of the 64 keys (zero past T), written out transposed
    const int j = j0 + t;
    uint4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
    if (j < Mk + T) {
      const bf16_t* src = (j < Mk ? meta_v + ((size_t)j * Hkv + g) * 64
                                  : v + (((size_t)b * T + (j - Mk)) * Hkv + g) * 64) +
                          16 * part;
      v0 = *(const uint4*)src;
      v1 = *(const uint4*)(src + 8);
    }
    const bf16_t* p0 = (const bf16_t*)&v0;
    const bf16_t* p1 = (const bf16_t*)&v1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sv[t][e] = p0[e];
      sv[t][8 + e] = p1[e];
    }
  }
  __syncthreads();
  {  // thread -> V^T row d = 16 part + t/4, keys 16 (t & 3) .. +15
    const int dl = t >> 2, kq = t & 3;
    bf16_t tmp[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) tmp[e] = sv[16 * kq + e][dl];
    bf16_t* vt = Vt + ((((size_t)b * Hkv + g) * (Tpad / 64) + tile) * 64 + 16 * part + dl) * 64 +
                 16 * kq;
    *(uint4*)vt = *(const uint4*)tmp;
    *(uint4*)(vt + 8) = *(const uint4*)(tmp + 8);
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
// smem: the workgroup's kStages x 2 x 8 KB of LDS (K and V^T tile per stage).
// Tk key rows (prepared K/V); the Tq query rows of q and o are rows
// qoff .. qoff + Tq - 1 of X~ (qoff = 0 unless the meta rows are cached).
HM_DEV void attn_fwd_bf16_body(
    unsigned char (*smem)[2][8192], int bid, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ Kr, const bf16_t* __restrict__ Vt, bf16_t* __restrict__ o, int Tk,
    int Tpad, int Hq, int Hkv, int M, int W, long long pos0, float qscale, double rstep, int n_qt,
    int n_groups, int Tq, int qoff) {
  // Work item.  A group is (query tile, b, kv head) and its items are the
  // Hq/Hkv query heads that read the same K/V.  Groups are ranked heaviest
  // first (the visible key count never decreases with the query tile), rank r
  // goes to XCD r % 8 (workgroup id % 8 selects the XCD), and an XCD runs its
  // groups in rank order with the heads of a group side by side, so that
  // every XCD gets the same mix of long and short items, the longest first,
  // and the heads of a group share K/V tiles in one L2.
  const int grp = Hq / Hkv;
  const int xcd = bid & 7, kk = bid >> 3;
  const int r = 8 * (kk / grp) + xcd;
  if (r >= n_groups) return;
  const int hh = kk % grp;
  const int n_pairs = n_groups / n_qt;
  const int qt = n_qt - 1 - r / n_pairs;
  const int pair = r % n_pairs;                 // b * Hkv + g
  const int g = pair % Hkv, b = pair / Hkv;
  const int h = g * grp + hh;

  // Attention waves issue at priority 2, 3 while their QK product is issued:
  // in the fused prefill launch they share CUs with final-scan waves (priority
  // 0), whose VALU work then fills the attention waves' idle issue slots
  // instead of delaying their softmax (measured: the swa-prefill fused launch
  // 48.7 -> 46.7 us).
  __builtin_amdgcn_s_setprio(2);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, gq = lane >> 5;
  const int qend = qoff + Tq;                   // one past the last query row of X~
  const int i0 = qoff + qt * kBM, i1 = min(i0 + kBM, qend);
  const int wi0 = i0 + wave * kWR, wi1 = min(wi0 + kWR, qend);
  const int qrow = min(wi0 + n, qend - 1);

  // Q fragment (B operand of S^T = K Q^T): lane holds query qrow, dims
  // 16 s + 8 gq + e.  Rotated in float32, scaled by scale*log2(e), rounded to
  // bf16.  theta_d / 2 pi = rstep^d / 2 pi by double-precision products.
  bf16x8_v qf[4];
  {
    const bf16_t* src = q + (((size_t)b * Tq + (qrow - qoff)) * Hq + h) * 64;
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

  // Double-buffered K/V tiles: tile it+1 is issued right after the barrier of
  // iteration it (which frees the buffer of tile it-1) and is loading while
  // tile it is computed.  At the top of iteration it a thread waits for its own
  // loads of tile it, and the barrier publishes the tile to every wave.  With
  // 32 KB of LDS and at most 128 VGPRs per wave, four workgroups share a CU, so
  // four waves per SIMD hide each other's latencies.
  if (ntiles > 0) issue(0);
  for (int it = 0; it < ntiles; ++it) {
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    if (it + 1 < ntiles) issue(it + 1);
    const int j0 = tile_at(it) * kBN;
    const int cls = hm_tile_class(wi0, wi1, j0, min(j0 + kBN, Tk), M, W);
    if (cls == 0) continue;
    // S^T - m_ref (accumulated onto -m_ref); the two 32-key blocks are
    // independent accumulation chains, alternated
    const unsigned char* sk = smem[it % kStages][0];
    __builtin_amdgcn_s_setprio(3);
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
    __builtin_amdgcn_s_setprio(2);
    if (cls == 1 || j0 + kBN > Tk) {
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
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(mx), __float_as_int(mx),
                                                       false, false);
      mx = fmaxf(__int_as_float(sw[0]), __int_as_float(sw[1]));
    }
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
    // row sums of the bf16 probabilities actually used by the PV product, one
    // dot2 chain (the compiler interleaves it with the PV MFMAs; four
    // independent chains measured no faster)
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
  if (qi < qend) {
    const float inv = 1.f / l;
    bf16_t* dst = o + (((size_t)b * Tq + (qi - qoff)) * Hq + h) * 64;
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

}  // namespace
