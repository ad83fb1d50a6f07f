// One decode token through one layer of an adjacent pair sharing a KV cache.
//
// Sources: adjacent sliding-window blocks share one KV cache (Hymba blog,
// juejin.cn "NVIDIA提出Hymba网络", "Hymba 的整体架构"); generation with the
// cache enabled (Hymba-1.5B-Base model card, "模型使用"); attention Eq. (1),
// SSM Eq. (2) and the norm-and-average fusion ("数学表示" §3-§5).
//
// Cache rows per sequence: meta tokens 0..M-1, then a ring of window slots
// (token s -> slot M + s mod W; global layers append).  K is stored rotated.
// With one n_prev for the batch the visible rows are exactly the contiguous
// range [0, M + min(n_prev+1, W)).
//
// bf16 path: step_fused_bf16, one workgroup per (sequence, kv group, key split)
// that streams its K/V tiles through LDS, plus workgroups that run the SSM
// step, then step_combine (one workgroup per sequence) merges the key splits
// into Y_attn and applies the branch RMS norm, rescale and average: two
// launches per layer.
// float32 path (Dh in {16, 32, 64}): SSM step + KV write, one thread per
// (b, head) over all visible rows, then the same combine kernel.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>

#include "hm_common.h"

namespace {

constexpr int kNS = 16;

template <typename Tact>
HM_DEV float ldx(const Tact* p) { return ActIO<Tact>::ld(p); }

// ---------------------------------------------------------------- per-sequence combine
// One workgroup of kCombThreads per sequence b.  Part layout per sequence:
// [Hkv][n_split][grp][Dh + 2] = (max in log2 units, sum, unnormalised O[Dh]).
// Every load is issued up front (one round trip to memory): the (max, sum) of
// every (head, split) go to LDS, and each thread holds the split partials of
// its outputs.  Then per output Y_attn[h, d] = sum_s w_s O_s[h, d] with
// w_s = exp2(m_s - M) / sum_s' exp2(m_s' - M) l_s', and
// out = 0.5 (beta_a Y_attn / rms(Y_attn) + beta_s Y_ssm / rms(Y_ssm)).
// 1024 threads of 4 outputs each (measured per cold decode pair: 57.4 us,
// against 59.2 us with 512 x 8 and 64.2 us with 256 x 16): the merge is a
// chain of memory round trips, shorter with more loads in flight.
constexpr int kCombThreads = 1024;
constexpr int kCombMaxW = 2048;      // Hq * n_split entries held in LDS
constexpr int kCombPer = 4;          // outputs per thread (Di <= 4096)
constexpr int kCombMaxSplit = 8;     // split partials held in registers per output (more: re-read)

template <typename Tact>
__global__ __launch_bounds__(kCombThreads) void step_combine(
    const float* __restrict__ part, size_t part_b_stride, const float* __restrict__ ys_ws,
    size_t ys_stride, const float* __restrict__ ba, const float* __restrict__ bs, float eps,
    Tact* __restrict__ out, float* __restrict__ ya_out, float* __restrict__ ys_out, int Hq,
    int Hkv, int Dh, int n_split, int Di) {
  __shared__ float sm[kCombMaxW], sl[kCombMaxW];
  __shared__ float red[2][kCombThreads / 64];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int grp = Hq / Hkv, stride = Dh + 2;
  const float* pb = part + (size_t)b * part_b_stride;
  const float* yb = ys_ws + (size_t)b * ys_stride;
  // (max, sum) of entry e = h * n_split + s
  for (int e = tid; e < Hq * n_split; e += kCombThreads) {
    const int h = e / n_split, sp = e % n_split;
    const int g = h / grp, hh = h % grp;
    const float* ph = pb + (((size_t)g * n_split + sp) * grp + hh) * stride;
    sm[e] = ph[0];
    sl[e] = ph[1];
  }
  // this thread's outputs: split partials, SSM branch, betas
  float o[kCombPer][kCombMaxSplit], yv[kCombPer], wa[kCombPer], wsv[kCombPer];
#pragma unroll
  for (int k = 0; k < kCombPer; ++k) {
    const int idx = tid + k * kCombThreads;
    if (idx < Di) {
      const int h = idx / Dh, d = idx % Dh;
      const int g = h / grp, hh = h % grp;
      const float* base = pb + ((size_t)g * n_split * grp + hh) * stride + 2 + d;
#pragma unroll
      for (int sp = 0; sp < kCombMaxSplit; ++sp)
        o[k][sp] = sp < n_split ? base[(size_t)sp * grp * stride] : 0.f;
      yv[k] = yb[idx];
      wa[k] = ba[idx];
      wsv[k] = bs[idx];
    }
  }
  __syncthreads();
  float ya[kCombPer];
  float sa = 0.f, ss = 0.f;
#pragma unroll
  for (int k = 0; k < kCombPer; ++k) {
    const int idx = tid + k * kCombThreads;
    ya[k] = 0.f;
    if (idx < Di) {
      const int h = idx / Dh, d = idx % Dh;
      const float* mh = sm + h * n_split;
      const float* lh = sl + h * n_split;
      float M = mh[0];
      for (int sp = 1; sp < n_split; ++sp) M = fmaxf(M, mh[sp]);
      float L = 0.f, acc = 0.f;
#pragma unroll
      for (int sp = 0; sp < kCombMaxSplit; ++sp)
        if (sp < n_split) {
          const float w = fast_exp2(mh[sp] - M);
          L += w * lh[sp];
          acc += w * o[k][sp];
        }
      // splits beyond those held in registers (long global caches)
      const int g = h / grp, hh = h % grp;
      const float* base = pb + ((size_t)g * n_split * grp + hh) * stride + 2 + d;
      for (int sp = kCombMaxSplit; sp < n_split; ++sp) {
        const float w = fast_exp2(mh[sp] - M);
        L += w * lh[sp];
        acc += w * base[(size_t)sp * grp * stride];
      }
      ya[k] = acc / L;
      sa += ya[k] * ya[k];
      ss += yv[k] * yv[k];
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    sa += __shfl_xor(sa, off);
    ss += __shfl_xor(ss, off);
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = sa;
    red[1][tid >> 6] = ss;
  }
  __syncthreads();
  sa = 0.f;
  ss = 0.f;
#pragma unroll
  for (int w = 0; w < kCombThreads / 64; ++w) {
    sa += red[0][w];
    ss += red[1][w];
  }
  const float ra = 0.5f / sqrtf(sa / (float)Di + eps);
  const float rs = 0.5f / sqrtf(ss / (float)Di + eps);
#pragma unroll
  for (int k = 0; k < kCombPer; ++k) {
    const int idx = tid + k * kCombThreads;
    if (idx < Di) {
      ActIO<Tact>::st(out + (size_t)b * Di + idx, wa[k] * ya[k] * ra + wsv[k] * yv[k] * rs);
      if (ya_out) ya_out[(size_t)b * Di + idx] = ya[k];
      if (ys_out) ys_out[(size_t)b * Di + idx] = yv[k];
    }
  }
}

// ---------------------------------------------------------------- one SSM-branch step
template <typename Tact>
HM_DEV float ssm_step_one(int b, int c, int Di, const Tact* __restrict__ x,
                          const Tact* __restrict__ dl, const Tact* __restrict__ Bm,
                          const Tact* __restrict__ Cm, const Tact* __restrict__ z,
                          const float* __restrict__ A, const float* __restrict__ D,
                          const float* __restrict__ cw, const float* __restrict__ cb,
                          float* __restrict__ conv_state, float* __restrict__ ssm_state) {
  const size_t idx = (size_t)b * Di + c;
  float* cs = conv_state + idx * 3;
  const float s0 = cs[0], s1 = cs[1], s2 = cs[2];
  const float xv = ldx(x + idx);
  const float u = cb[c] + cw[c * 4 + 0] * s0 + cw[c * 4 + 1] * s1 + cw[c * 4 + 2] * s2 +
                  cw[c * 4 + 3] * xv;
  cs[0] = s1;
  cs[1] = s2;
  cs[2] = xv;
  const float xc = siluf_(u);
  const float dv = ldx(dl + idx);
  const float du = dv * xc;
  float* hs = ssm_state + idx * kNS;
  float h[kNS];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 t = ((const float4*)hs)[i];
    h[4 * i] = t.x; h[4 * i + 1] = t.y; h[4 * i + 2] = t.z; h[4 * i + 3] = t.w;
  }
  const Tact* Bb = Bm + (size_t)b * kNS;
  const Tact* Cb = Cm + (size_t)b * kNS;
  float y4[4] = {D[c] * xc, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nn = 0; nn < kNS; ++nn) {
    h[nn] = fast_exp2(dv * (A[c * kNS + nn] * kLog2e)) * h[nn] + du * ldx(Bb + nn);
    y4[nn & 3] += ldx(Cb + nn) * h[nn];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    ((float4*)hs)[i] = make_float4(h[4 * i], h[4 * i + 1], h[4 * i + 2], h[4 * i + 3]);
  return ((y4[0] + y4[1]) + (y4[2] + y4[3])) * siluf_(ldx(z + idx));
}

// ---------------------------------------------------------------- bf16 attention + SSM step
// LDS tiles of 64 cache rows x 128 bytes (K or V); the 16-byte chunk c of row r
// sits in slot c ^ ((r >> 1) & 7), so that 16 lanes reading one chunk of 16
// consecutive rows hit 16 different bank groups of the 64-bank LDS.
HM_DEV int dec_slot(int row, int c) { return c ^ ((row >> 1) & 7); }
HM_DEV int dec_off(int row, int c) { return row * 128 + (dec_slot(row, c) << 4); }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short s16x4_v __attribute__((ext_vector_type(4)));

constexpr int kDecStages = 3;   // 64-row K/V tiles in flight per workgroup (48 KB)

// One workgroup of 4 waves per (sequence b, kv head g, key split).  The split's
// 64-row tiles of K and V stream HBM -> LDS with global_load_lds through a
// 3-stage ring; wave w takes rows 16w..16w+15 of every tile: S^T = K Q^T with
// v_mfma_f32_16x16x32_bf16 (the group's query heads on the 16 columns), an
// online softmax per head, and O^T += V^T P^T with v_mfma_f32_16x16x16_bf16
// (V^T read from the row-major tile).  The 4 waves merge in LDS and write one
// partial (max, sum, unnormalised O) per head; step_combine merges the splits.
// The workgroups past the attention ones run the SSM step, one (b, channel)
// item per thread (conv step + one scan step, in place on the states).  The
// workgroup whose rows hold the new token's slot (producer layer) first
// rotates k_new and writes k_new / v_new there.
__global__ __launch_bounds__(256) void step_fused_bf16(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_new,
    const bf16_t* __restrict__ v_new, bf16_t* __restrict__ kc, bf16_t* __restrict__ vc,
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ dl, const bf16_t* __restrict__ Bm,
    const bf16_t* __restrict__ Cm, const bf16_t* __restrict__ z, const float* __restrict__ A,
    const float* __restrict__ D, const float* __restrict__ cw, const float* __restrict__ cb,
    float* __restrict__ conv_state, float* __restrict__ ssm_state, float* __restrict__ ys_ws,
    size_t ys_stride, float* __restrict__ part, size_t part_b_stride, int Hq, int Hkv, int Di,
    int S, SeqPos sp, float qscale, double log2_base, double rstep,
    int n_split, int tiles_per_split, int n_ssm, int n_attn) {
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kDecStages][2][8192];
  // per-wave (max, sum) of each head for the merge after the stream: carved
  // from the ring (free by then), so that the workgroup's LDS is exactly the
  // 48 KB ring (measured: 59.3 against 61.5 us per cold decode pair with them
  // as separate arrays)
  float (*sm)[16] = (float (*)[16])&ring[1][0][0];
  float (*sl)[16] = (float (*)[16])&ring[1][0][256];
  const int tid = threadIdx.x;
  if ((int)blockIdx.x >= n_attn) {
    // workgroups past the attention ones: SSM-step items
    const int nb = (int)gridDim.x - n_attn;
    for (int j = ((int)blockIdx.x - n_attn) * 256 + tid; j < n_ssm; j += nb * 256) {
      const int bs = j / Di, c = j % Di;
      ys_ws[(size_t)bs * ys_stride + c] =
          ssm_step_one<bf16_t>(bs, c, Di, x, dl, Bm, Cm, z, A, D, cw, cb, conv_state, ssm_state);
    }
    return;
  }
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, G = lane >> 4;
  const int grp = Hq / Hkv;
  const int split = blockIdx.x % n_split, pair = blockIdx.x / n_split;
  const int b = pair / Hkv, g = pair % Hkv;
  int L, slot;
  long long pos;
  seq_pos(sp, b, &L, &slot, &pos);
  const size_t rs = (size_t)Hkv * 64;                       // cache row stride (elements)
  const int kt0 = split * tiles_per_split;                  // first tile of the split
  const int ntile = max(0, min(tiles_per_split, (L + 63) / 64 - kt0));

  // 1) producer: the new token's row first, if it lies in this split
  if (k_new != nullptr && slot >= kt0 * 64 && slot < (kt0 + ntile) * 64) {
    if (tid < 32) {
      const bf16_t* ks = k_new + ((size_t)b * Hkv + g) * 64;
      const bf16_t* vs = v_new + ((size_t)b * Hkv + g) * 64;
      float sn, cs;
      rope_sincos(pos, tid, 64, log2_base, &sn, &cs);
      const float x1 = bf2f(ks[tid]), x2 = bf2f(ks[tid + 32]);
      const size_t off = ((size_t)b * S + slot) * rs + (size_t)g * 64;
      kc[off + tid] = f2bf(x1 * cs - x2 * sn);
      kc[off + tid + 32] = f2bf(x2 * cs + x1 * sn);
      vc[off + tid] = vs[tid];
      vc[off + tid + 32] = vs[tid + 32];
    }
    __threadfence_block();
    __syncthreads();
  }

  // 2) the first two tiles: thread -> LDS rows 16 wave + 8 i + lane / 8, slot
  // lane & 7 (global_load_lds writes lane L of a wave at base + 16 L)
  const bf16_t* kb0 = kc + (size_t)b * S * rs + (size_t)g * 64;
  const bf16_t* vb0 = vc + (size_t)b * S * rs + (size_t)g * 64;
  int roff[2], coff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    roff[i] = 16 * wave + 8 * i + (lane >> 3);
    coff[i] = dec_slot(roff[i], lane & 7) * 8;   // the slot map is an involution
  }
  auto issue = [&](int t) {
    unsigned char* st = ring[t % kDecStages][0];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = min((kt0 + t) * 64 + roff[i], S - 1);   // rows past the cache: unused
      __builtin_amdgcn_global_load_lds((const void*)(kb0 + (size_t)key * rs + coff[i]),
                                       (lds_void_t*)(st + (16 * wave + 8 * i) * 128), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vb0 + (size_t)key * rs + coff[i]),
                                       (lds_void_t*)(st + 8192 + (16 * wave + 8 * i) * 128), 16,
                                       0, 0);
    }
  };
  if (ntile > 0) issue(0);
  if (ntile > 1) issue(1);

  // 3) Q^T fragment (B operand): lane holds head n of the group, dims 8G+e and 32+8G+e
  bf16x8_v qf[2];
  {
    const bf16_t* src = q + ((size_t)b * Hq + g * grp + min(n, grp - 1)) * 64;
    const uint4 r0 = *(const uint4*)(src + 8 * G);
    const uint4 r1 = *(const uint4*)(src + 32 + 8 * G);
    const bf16_t* p0 = (const bf16_t*)&r0;
    const bf16_t* p1 = (const bf16_t*)&r1;
    const float qs = n < grp ? qscale : 0.f;
    // theta_d / 2 pi = rstep^d / 2 pi for d = 8G..8G+7 by double-precision products
    const double s2 = rstep * rstep, s4 = s2 * s2, s8 = s4 * s4;
    double th = 0.15915494309189533576888376337251;
    for (int gg = 0; gg < G; ++gg) th *= s8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      double r = (double)pos * th;
      r -= rint(r);
      const float sn = __builtin_amdgcn_sinf((float)r), cs = __builtin_amdgcn_cosf((float)r);
      th *= rstep;
      const float x1 = bf2f(p0[e]), x2 = bf2f(p1[e]);
      qf[0][e] = (__bf16)((x1 * cs - x2 * sn) * qs);
      qf[1][e] = (__bf16)((x2 * cs + x1 * sn) * qs);
    }
  }

  // 4) stream the tiles; per lane: head n, keys 16 wave + 4G + i of each tile
  const float NEG_INF = -__builtin_huge_valf();
  float m_run = -1e30f, l_run = 0.f;
  f32x4_v acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[db][i] = 0.f;
  const int krow = 16 * wave + n;            // A-operand row of this lane (K)
  // V^T operand offsets in a tile: dim 16 db + n, rows 16 wave + 4G + e
  int voff[4][4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d = 16 * db + n, row = 16 * wave + 4 * G + e;
      voff[db][e] = dec_off(row, d >> 3) + (d & 7) * 2;
    }
  // The loop is unrolled by the ring depth so that every LDS address is a
  // register plus an immediate.
  for (int t0 = 0; t0 < ntile; t0 += kDecStages) {
#pragma unroll
    for (int u = 0; u < kDecStages; ++u) {
      const int t = t0 + u;
      if (t >= ntile) break;
      // A wave reads only the 16 rows of each tile it loaded itself (K rows
      // 16 wave.., V^T keys 16 wave..), so waiting for its own loads suffices:
      // no workgroup barrier per tile (measured: cold pair 57.1 -> 56.5 us).
      // Slot (t+2) % 3 held tile t-1, whose reads this wave finished last step.
      if (t == 0 || t + 1 >= ntile) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(4));   // tile t+1 may stay in flight
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (t + 2 < ntile) issue(t + 2);
      const unsigned char* sk = ring[u][0];
      const unsigned char* sv = ring[u][1];
      f32x4_v sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 2; ++s)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            *(const bf16x8_v*)(sk + dec_off(krow, G + 4 * s)), qf[s], sc, 0, 0, 0);
      const int kbase = (kt0 + t) * 64 + 16 * wave + 4 * G;
      float mx = NEG_INF;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (kbase + i >= L) sc[i] = NEG_INF;
        mx = fmaxf(mx, sc[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // lazily moved reference: O and l are rescaled only when a tile's maximum
      // exceeds the running reference by more than 8 (log2 units)
      if (__ballot(mx > m_run + 8.f) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[db][i] *= alpha;
      }
      s16x4_v pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(sc[i] - m_run);
        l_run += p;
        pb[i] = (short)f2bf(p);
      }
      // V^T operand: lane holds dim 16 db + n, keys 16 wave + 4G + e (e = 0..3)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        s16x4_v va;
#pragma unroll
        for (int e = 0; e < 4; ++e) va[e] = *(const short*)(sv + voff[db][e]);
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[db], 0, 0, 0);
      }
    }
  }
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  // 5) merge the 4 waves: (max, sum) per head and O^T (dims 16 db + 4G + i, head n)
  __syncthreads();                                  // every wave is done with the ring
  float* sO = (float*)&ring[0][0][0];               // [wave][head 16][dim 64]
  if (G == 0) {
    sm[wave][n] = m_run;
    sl[wave][n] = l_run;
  }
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) sO[(wave * 16 + n) * 64 + 16 * db + 4 * G + i] = acc[db][i];
  __syncthreads();
  float* dst = part + (size_t)b * part_b_stride + ((size_t)g * n_split + split) * grp * 66;
  for (int idx = tid; idx < grp * 64; idx += 256) {
    const int hh = idx >> 6, d = idx & 63;
    float M = sm[0][hh];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sm[w][hh]);
    float Ls = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = fast_exp2(sm[w][hh] - M);
      Ls += sl[w][hh] * f;
      O += sO[(w * 16 + hh) * 64 + d] * f;
    }
    float* ph = dst + hh * 66;
    if (d == 0) {
      ph[0] = M;
      ph[1] = Ls;
    }
    ph[2 + d] = O;
  }
}

// ---------------------------------------------------------------- float32 attention
template <int DH>
__global__ __launch_bounds__(64) void step_attn_f32(const float* __restrict__ q,
                                                    const float* __restrict__ kc,
                                                    const float* __restrict__ vc,
                                                    float* __restrict__ part,
                                                    size_t part_b_stride, int B, int Hq,
                                                    int Hkv, int S, SeqPos sp,
                                                    float qscale, double log2_base) {
  const int idx = blockIdx.x * 64 + threadIdx.x;
  if (idx >= B * Hq) return;
  const int h = idx % Hq, b = idx / Hq;
  int L, slot;
  long long pos;
  seq_pos(sp, b, &L, &slot, &pos);
  const int grp = Hq / Hkv, g = h / grp;
  float qr[DH];
  const float* src = q + ((size_t)b * Hq + h) * DH;
#pragma unroll
  for (int d = 0; d < DH / 2; ++d) {
    float sn, cs;
    rope_sincos(pos, d, DH, log2_base, &sn, &cs);
    const float x1 = src[d], x2 = src[d + DH / 2];
    qr[d] = (x1 * cs - x2 * sn) * qscale;
    qr[d + DH / 2] = (x2 * cs + x1 * sn) * qscale;
  }
  float acc[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) acc[d] = 0.f;
  float m = -1e30f, l = 0.f;
  for (int j = 0; j < L; ++j) {
    const float* kr = kc + (((size_t)b * S + j) * Hkv + g) * DH;
    const float* vr = vc + (((size_t)b * S + j) * Hkv + g) * DH;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < DH; ++d) s += qr[d] * kr[d];
    const float mn = fmaxf(m, s);
    const float alpha = exp2f(m - mn), p = exp2f(s - mn);
    l = l * alpha + p;
#pragma unroll
    for (int d = 0; d < DH; ++d) acc[d] = acc[d] * alpha + p * vr[d];
    m = mn;
  }
  float* ph = part + (size_t)b * part_b_stride + ((size_t)g * grp + (h % grp)) * (DH + 2);
  ph[0] = m;
  ph[1] = l;
#pragma unroll
  for (int d = 0; d < DH; ++d) ph[2 + d] = acc[d];
}

// SSM step + producer KV write (f32 path)
template <typename Tact>
__global__ __launch_bounds__(256) void step_ssm_kv(
    const Tact* __restrict__ x, const Tact* __restrict__ dl, const Tact* __restrict__ Bm,
    const Tact* __restrict__ Cm, const Tact* __restrict__ z, const float* __restrict__ A,
    const float* __restrict__ D, const float* __restrict__ cw, const float* __restrict__ cb,
    float* __restrict__ conv_state, float* __restrict__ ssm_state, float* __restrict__ ys_ws,
    size_t ys_stride, int B, int Di, int n_ssm_blocks, const Tact* __restrict__ k_new,
    const Tact* __restrict__ v_new, Tact* __restrict__ k_cache, Tact* __restrict__ v_cache,
    int Hkv, int Dh, int S, SeqPos sp, double log2_base) {
  if ((int)blockIdx.x < n_ssm_blocks) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)B * Di) return;
    const int c = idx % Di, b = idx / Di;
    ys_ws[(size_t)b * ys_stride + c] =
        ssm_step_one<Tact>(b, c, Di, x, dl, Bm, Cm, z, A, D, cw, cb, conv_state, ssm_state);
    return;
  }
  const long long idx = (long long)(blockIdx.x - n_ssm_blocks) * 256 + threadIdx.x;
  const int half = Dh / 2;
  if (idx >= (long long)B * Hkv * half) return;
  const int d = idx % half;
  const int g = (idx / half) % Hkv;
  const int b = idx / ((long long)half * Hkv);
  int L, slot;
  long long pos;
  seq_pos(sp, b, &L, &slot, &pos);
  (void)L;
  const Tact* ks = k_new + ((size_t)b * Hkv + g) * Dh;
  const Tact* vs = v_new + ((size_t)b * Hkv + g) * Dh;
  float sn, cs;
  rope_sincos(pos, d, Dh, log2_base, &sn, &cs);
  const float x1 = ldx(ks + d), x2 = ldx(ks + d + half);
  const size_t off = (((size_t)b * S + slot) * Hkv + g) * Dh;
  ActIO<Tact>::st(k_cache + off + d, x1 * cs - x2 * sn);
  ActIO<Tact>::st(k_cache + off + d + half, x2 * cs + x1 * sn);
  v_cache[off + d] = vs[d];
  v_cache[off + d + half] = vs[d + half];
}

// One thread per sequence: the positions the decode kernels use (slot,
// visible rows, position), for the bit-exact index tests.
__global__ __launch_bounds__(64) void debug_step_pos_kernel(SeqPos sp, int B, long long* out) {
  const int b = blockIdx.x * 64 + threadIdx.x;
  if (b >= B) return;
  int L, slot;
  long long pos;
  seq_pos(sp, b, &L, &slot, &pos);
  out[3 * (size_t)b + 0] = slot;
  out[3 * (size_t)b + 1] = L;
  out[3 * (size_t)b + 2] = pos;
}

struct StepGeom {
  int L, n_split, tiles_per_split, grp;
  size_t ys_stride, part_b_stride;            // floats per sequence
  size_t ys_bytes, part_bytes;
};

// bf16 decode: key splits of whole 64-row tiles, about kDecBlocks workgroups
// in all (two to three per CU stream at once with 48 KB of LDS each).
constexpr int kDecBlocks = 640;
// The SSM step runs in workgroups of its own, one item per thread (measured:
// faster than a share of every attention workgroup, which kept the stream's
// tail waiting on the exponentials, and than 4 items per thread).

StepGeom step_geom(const hm_step_args* a) {
  StepGeom s{};
  const long long nv = a->window > 0 ? (a->n_prev + 1 < a->window ? a->n_prev + 1 : a->window)
                                     : a->n_prev + 1;
  s.L = (int)(a->n_meta + nv);
  s.grp = a->Hkv > 0 ? a->Hq / a->Hkv : 0;
  s.n_split = 1;
  s.tiles_per_split = 1;
  if (a->dtype == HM_BF16) {
    const int nt = (s.L + 63) / 64;
    const long long pairs = (long long)a->B * a->Hkv;
    // the combine holds (max, sum) of every (query head, split) in LDS: at
    // most kCombMaxW of them, so long caches get longer splits
    const long long cap = std::max(1, kCombMaxW / std::max(1, a->Hq));
    const int want = (int)std::max(
        1LL, std::min<long long>(std::min<long long>(nt, cap), (kDecBlocks + pairs - 1) / pairs));
    s.tiles_per_split = (nt + want - 1) / want;
    s.n_split = (nt + s.tiles_per_split - 1) / s.tiles_per_split;
  }
  s.ys_stride = hm::align_up((size_t)a->Di, 64);
  s.part_b_stride = hm::align_up((size_t)a->Hkv * s.n_split * s.grp * (a->Dh + 2), 64);
  s.ys_bytes = (size_t)a->B * s.ys_stride * sizeof(float);
  s.part_bytes = (size_t)a->B * s.part_b_stride * sizeof(float);
  return s;
}

}  // namespace

extern "C" {

size_t hm_mixer_step_workspace(const hm_step_args* a) {
  if (!a || a->B <= 0 || a->Hkv <= 0 || a->Hq <= 0 || a->Di <= 0 || a->Dh <= 0 || a->n_prev < 0)
    return 0;
  const StepGeom s = step_geom(a);
  return s.ys_bytes + s.part_bytes;
}

long long hm_debug_cache_slot(long long n_prev, int n_meta, int window) {
  if (n_prev < 0) return -1;
  int L, slot;
  long long pos;
  seq_pos(SeqPos{nullptr, n_meta, window, n_prev}, 0, &L, &slot, &pos);
  return slot;
}

hm_status hm_debug_step_positions(int B, long long n_prev, const int* n_prev_seq, int n_meta,
                                  int window, long long* out_dev, void* stream) {
  HM_REQUIRE(out_dev != nullptr, HM_ERR_INVALID, "out_dev is NULL");
  HM_REQUIRE(B > 0 && n_prev >= 0 && n_meta >= 0, HM_ERR_INVALID,
             "need B > 0, n_prev >= 0 and n_meta >= 0");
  HM_REQUIRE(n_meta + n_prev < (1LL << 31) - 1, HM_ERR_UNSUPPORTED, "positions must fit int32");
  hipLaunchKernelGGL(debug_step_pos_kernel, dim3((B + 63) / 64), dim3(64), 0,
                     (hipStream_t)stream, SeqPos{n_prev_seq, n_meta, window, n_prev}, B, out_dev);
  return hm::check_launch("debug_step_pos_kernel");
}

}  // extern "C"

namespace {

hm_status step_scratch_ptr(void* stream, void** out);
constexpr size_t kStepScratchBytes = (size_t)8 << 20;

// The decode step with its scratch memory given explicitly (ws, ws_bytes): the
// caller's workspace (hm_mixer_step), or, with use_scratch, the library's
// static scratch array (hm_mixer_step_noalloc), looked up only once every
// argument has been validated.  a->workspace is not read here.
hm_status mixer_step_impl(const hm_step_args* a, void* ws, size_t ws_bytes, void* stream,
                          bool use_scratch) {
  HM_REQUIRE(a != nullptr, HM_ERR_INVALID, "args is NULL");
  HM_REQUIRE(a->B > 0 && a->Hq > 0 && a->Hkv > 0 && a->Dh > 0 && a->Di > 0, HM_ERR_INVALID,
             "B, Hq, Hkv, Dh and Di must be positive");
  HM_REQUIRE(a->Hq % a->Hkv == 0, HM_ERR_INVALID, "Hq must be a multiple of Hkv");
  HM_REQUIRE(a->Di == a->Hq * a->Dh, HM_ERR_INVALID, "Di must equal Hq * Dh");
  HM_REQUIRE(a->n_prev >= 0, HM_ERR_INVALID, "n_prev must be >= 0");
  HM_REQUIRE(a->n_meta >= 0 && a->cache_slots > 0, HM_ERR_INVALID,
             "n_meta >= 0 and cache_slots > 0 required");
  if (a->window > 0)
    HM_REQUIRE(a->cache_slots >= a->window, HM_ERR_INVALID, "cache_slots must be >= window");
  else
    HM_REQUIRE(a->n_prev < a->cache_slots, HM_ERR_INVALID,
               "global layer: n_prev must be < cache_slots");
  HM_REQUIRE(a->N == kNS, HM_ERR_UNSUPPORTED, "only N = 16 states are supported");
  HM_REQUIRE(a->K == 4, HM_ERR_UNSUPPORTED, "only conv width K = 4 is supported");
  HM_REQUIRE(a->dtype == HM_BF16 || a->dtype == HM_F32, HM_ERR_UNSUPPORTED,
             "dtype must be f32 or bf16");
  if (a->dtype == HM_BF16)
    HM_REQUIRE(a->Dh == 64 && a->Hq / a->Hkv <= 16, HM_ERR_UNSUPPORTED,
               "bf16 decode supports Dh = 64 and at most 16 query heads per KV head");
  else
    HM_REQUIRE(a->Dh == 16 || a->Dh == 32 || a->Dh == 64, HM_ERR_UNSUPPORTED,
               "f32 decode supports Dh in {16, 32, 64}");
  HM_REQUIRE(a->Di <= 4096, HM_ERR_UNSUPPORTED, "Di must be <= 4096");
  HM_REQUIRE(a->rope_base > 1.0f && std::isfinite(a->rope_base) && std::isfinite(a->scale) &&
                 a->eps >= 0.f && std::isfinite(a->eps),
             HM_ERR_INVALID, "rope_base > 1, finite scale and eps >= 0 required");
  HM_PTR(a->q);
  HM_PTR(a->k_cache);
  HM_PTR(a->v_cache);
  HM_PTR(a->x);
  HM_PTR(a->delta);
  HM_PTR(a->Bm);
  HM_PTR(a->Cm);
  HM_PTR(a->z);
  HM_PTR(a->A);
  HM_PTR(a->D);
  HM_PTR(a->conv_w);
  HM_PTR(a->conv_b);
  HM_PTR(a->conv_state);
  HM_PTR(a->ssm_state);
  HM_PTR(a->beta_a);
  HM_PTR(a->beta_s);
  HM_PTR(a->out);
  HM_OPT_PTR(a->ya_out);
  HM_OPT_PTR(a->ys_out);
  const bool producer = a->k_new != nullptr;
  HM_REQUIRE(producer == (a->v_new != nullptr), HM_ERR_INVALID,
             "k_new and v_new must both be set (producer) or both NULL (consumer)");
  if (producer) {
    HM_PTR(a->k_new);
    HM_PTR(a->v_new);
  }
  HM_REQUIRE((double)a->B * (a->n_meta + a->cache_slots) * a->Hkv * a->Dh < 4.0e9 &&
                 (double)a->B * a->Hkv * (a->n_meta + a->cache_slots) / 64 < 1.0e9,
             HM_ERR_UNSUPPORTED, "cache too large");
  const StepGeom g = step_geom(a);
  const size_t need = g.ys_bytes + g.part_bytes;
  HM_REQUIRE((size_t)a->Hq * g.n_split <= (size_t)kCombMaxW, HM_ERR_UNSUPPORTED,
             "too many query heads x key splits for the combine");
  if (use_scratch) {
    HM_REQUIRE(need <= kStepScratchBytes, HM_ERR_UNSUPPORTED,
               "step needs " + std::to_string(need) + " bytes of scratch, more than the " +
                   std::to_string(kStepScratchBytes) +
                   " of the allocation-free entry point; use hm_mixer_step with a workspace");
    hm_status s = step_scratch_ptr(stream, &ws);
    if (s != HM_OK) return s;
    ws_bytes = kStepScratchBytes;
  }
  HM_REQUIRE(ws != nullptr && ws_bytes >= need && hm::aligned16(ws), HM_ERR_WORKSPACE,
             "workspace smaller than hm_mixer_step_workspace()");

  hipStream_t st = (hipStream_t)stream;
  float* ys_ws = (float*)ws;
  float* part = (float*)((char*)ws + g.ys_bytes);
  const int S = a->n_meta + a->cache_slots;
  const SeqPos sp{a->n_prev_seq, a->n_meta, a->window, a->n_prev};
  const double l2b = log2((double)a->rope_base);
  const float sc = (a->scale > 0.f ? a->scale : 1.0f / sqrtf((float)a->Dh)) * kLog2e;

  if (a->dtype == HM_BF16) {
    const int n_attn = a->B * a->Hkv * g.n_split;
    const int n_ssm = a->B * a->Di;
    const int n_ssm_blocks = (n_ssm + 255) / 256;   // one SSM-step item per thread
    hipLaunchKernelGGL(step_fused_bf16, dim3(n_attn + n_ssm_blocks), dim3(256), 0, st,
                       (const bf16_t*)a->q, (const bf16_t*)a->k_new, (const bf16_t*)a->v_new,
                       (bf16_t*)a->k_cache, (bf16_t*)a->v_cache, (const bf16_t*)a->x,
                       (const bf16_t*)a->delta, (const bf16_t*)a->Bm, (const bf16_t*)a->Cm,
                       (const bf16_t*)a->z, a->A, a->D, a->conv_w, a->conv_b, a->conv_state,
                       a->ssm_state, ys_ws, g.ys_stride, part, g.part_b_stride, a->Hq, a->Hkv,
                       a->Di, S, sp, sc, l2b, exp2(-l2b / 32.0), g.n_split,
                       g.tiles_per_split, n_ssm, n_attn);
    hm_status s = hm::check_launch("step_fused_bf16");
    if (s != HM_OK) return s;
    hipLaunchKernelGGL(step_combine<bf16_t>, dim3(a->B), dim3(kCombThreads), 0, st,
                       (const float*)part, g.part_b_stride, (const float*)ys_ws, g.ys_stride,
                       a->beta_a, a->beta_s, a->eps, (bf16_t*)a->out, a->ya_out, a->ys_out, a->Hq,
                       a->Hkv, a->Dh, g.n_split, a->Di);
    return hm::check_launch("step_combine");
  }
  const int n_ssm_blocks = (int)(((long long)a->B * a->Di + 255) / 256);
  const int n_kv_blocks =
      producer ? (int)(((long long)a->B * a->Hkv * (a->Dh / 2) + 255) / 256) : 0;
  hipLaunchKernelGGL(step_ssm_kv<float>, dim3(n_ssm_blocks + n_kv_blocks), dim3(256), 0, st,
                     (const float*)a->x, (const float*)a->delta, (const float*)a->Bm,
                     (const float*)a->Cm, (const float*)a->z, a->A, a->D, a->conv_w, a->conv_b,
                     a->conv_state, a->ssm_state, ys_ws, g.ys_stride, a->B, a->Di, n_ssm_blocks,
                     (const float*)a->k_new, (const float*)a->v_new, (float*)a->k_cache,
                     (float*)a->v_cache, a->Hkv, a->Dh, S, sp, l2b);
  hm_status s = hm::check_launch("step_ssm_kv");
  if (s != HM_OK) return s;
  const int nbh = (a->B * a->Hq + 63) / 64;
#define HM_STEP_F32(DHV)                                                                      \
  case DHV:                                                                                   \
    hipLaunchKernelGGL(step_attn_f32<DHV>, dim3(nbh), dim3(64), 0, st, (const float*)a->q,   \
                       (const float*)a->k_cache, (const float*)a->v_cache, part,               \
                       g.part_b_stride, a->B, a->Hq, a->Hkv, S, sp, sc, l2b);                  \
    break;
  switch (a->Dh) {
    HM_STEP_F32(16)
    HM_STEP_F32(32)
    HM_STEP_F32(64)
  }
#undef HM_STEP_F32
  s = hm::check_launch("step_attn_f32");
  if (s != HM_OK) return s;
  hipLaunchKernelGGL(step_combine<float>, dim3(a->B), dim3(kCombThreads), 0, st, (const float*)part,
                     g.part_b_stride, (const float*)ys_ws, g.ys_stride, a->beta_a, a->beta_s,
                     a->eps, (float*)a->out, a->ya_out, a->ys_out, a->Hq, a->Hkv, a->Dh, 1, a->Di);
  return hm::check_launch("step_combine");
}

// ---------------------------------------------------------------- allocation-free variant
// Scratch of hm_mixer_step_noalloc: a file-scope device array, one copy per
// GPU, alive until the process ends.  Host code never passes `step_scratch`
// itself (on the host it is only a stand-in for the symbol): its device
// address is looked up once per device with hipGetSymbolAddress and that
// address is what the kernels receive.
static __device__ __align__(256) unsigned char step_scratch[kStepScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchAddr {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
static ScratchAddr g_scratch[kMaxDevices];

hm_status step_scratch_ptr(void* stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return hm::fail(HM_ERR_HIP, "hipGetDevice failed or device index >= 64");
  // the array is the current device's, so the kernels must run there
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess || sdev != dev)
      return hm::fail(HM_ERR_INVALID,
                      "stream does not belong to the calling thread's current device");
  }
  ScratchAddr& s = g_scratch[dev];
  // once per device, with that device current (the calling thread's device)
  std::call_once(s.once, [&s]() {
    void* p = nullptr;
    s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(step_scratch));
    s.ptr = p;
  });
  if (s.err != hipSuccess || s.ptr == nullptr)
    return hm::fail(HM_ERR_HIP, std::string("hipGetSymbolAddress(step_scratch): ") +
                                    hipGetErrorString(s.err));
  *out = s.ptr;
  return HM_OK;
}

}  // namespace

extern "C" {

hm_status hm_mixer_step(const hm_step_args* a, void* stream) {
  HM_REQUIRE(a != nullptr, HM_ERR_INVALID, "args is NULL");
  return mixer_step_impl(a, a->workspace, a->workspace_bytes, stream, false);
}

size_t hm_mixer_step_noalloc_max_bytes(void) { return kStepScratchBytes; }

hm_status hm_mixer_step_noalloc(const hm_step_args* a, void* stream) {
  return mixer_step_impl(a, nullptr, 0, stream, true);
}

}  // extern "C"
