// Device bodies of the chunked selective scan (with the causal conv fused), shared by
// the standalone scan kernels and the fused prefill kernels.  See ssm.hip for the
// method and the three-pass structure.
#pragma once

#include "hm_common.h"

namespace {


constexpr int kNS = 16;
constexpr int kConvK = 4;
constexpr int kSubRows = 16;     // chunk lengths are whole numbers of 16-step sub-blocks
constexpr int kMinChunk = 32;    // shorter chunks cost more carry traffic than they save
constexpr int kTargetWaves = 4096;

HM_HD int scan_chunk_len(int B, int T, int Di) {
  const int groups = B * ((Di + 63) / 64);
  int nc = (kTargetWaves + groups - 1) / groups;
  const int maxc = (T + kMinChunk - 1) / kMinChunk;
  if (nc > maxc) nc = maxc;
  if (nc < 1) nc = 1;
  int L = (T + nc - 1) / nc;
  L = (L + kSubRows / 2) / kSubRows * kSubRows;   // nearest whole number of sub-blocks
  return L < kMinChunk ? kMinChunk : L;
}

template <typename Tact>
HM_DEV float ldx(const Tact* p) { return ActIO<Tact>::ld(p); }

// Conv input at time t (t may be negative: then the state or zero).
template <typename Tact>
HM_DEV float conv_in(const Tact* xrow0, long long t, int Di, const float* st_in_c) {
  if (t >= 0) return ldx(xrow0 + t * Di);
  return st_in_c ? st_in_c[kConvK - 1 + t] : 0.f;
}

// ---------------------------------------------------------------- chunk kernels
// One wave per (64-channel group, chunk, batch).  The chunk is processed in
// sub-blocks of R steps: x, delta (and z) for the wave's 64 channels and B_t
// (and C_t) are copied to LDS (B, C widened to float32), then the time loop
// reads LDS only (B, C as broadcast reads).
// FINAL = false: end state from a zero start and the chunk's sum of delta
//                (chunks 0 .. nC-2);
// FINAL = true : recurrence from the carried-in state, y written, and the last
//                chunk writes the final SSM / conv states.
template <typename Tact>
struct Stage;
template <>
struct Stage<bf16_t> { static constexpr int kPerChunk = 8; };   // 8 bf16 per 16 bytes
template <>
struct Stage<float> { static constexpr int kPerChunk = 4; };

// B_t / C_t chunk (16 bytes) to float32 LDS.
HM_DEV void store_bc(float* dst, const uint4& v, bf16_t) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dst[2 * i] = __uint_as_float(w[i] << 16);
    dst[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
HM_DEV void store_bc(float* dst, const uint4& v, float) { *(uint4*)dst = v; }

// Scalar staging for widths whose rows are not 16-byte aligned.
template <typename Tact, int R>
HM_DEV void stage_scalar(Tact (*sx)[64], Tact (*sd)[64], Tact (*sz)[64], float (*sB)[kNS],
                         float (*sC)[kNS], const Tact* x, const Tact* dl, const Tact* z,
                         const Tact* Bm, const Tact* Cm, bool has_z, bool has_c, long long t,
                         int nt, int c0, int Di, int lane) {
  const int c = min(c0 + lane, Di - 1);
  for (int r = 0; r < R; ++r) {
    const size_t off = (size_t)(t + min(r, nt - 1)) * Di + c;
    sx[r][lane] = x[off];
    sd[r][lane] = dl[off];
    if (has_z) sz[r][lane] = z[off];
  }
  for (int i = lane; i < R * kNS; i += 64) {
    const size_t off = (size_t)(t + min(i / kNS, nt - 1)) * kNS + i % kNS;
    sB[i / kNS][i % kNS] = ldx(Bm + off);
    if (has_c) sC[i / kNS][i % kNS] = ldx(Cm + off);
  }
}

// Sub-block rows staged at once: 16 for bf16, 8 for float32, so one 64-channel
// sub-block of a tensor is 2 KB = two 16-byte chunks per lane.
template <typename Tact> struct SubRows;
template <> struct SubRows<bf16_t> { static constexpr int value = 16; };
template <> struct SubRows<float> { static constexpr int value = 8; };

// LDS of one chunk wave: the staged sub-block.  The y of a step is written
// over the x of that step (each lane its own element, already consumed).
template <typename Tact, bool FINAL>
struct ScanLds {
  static constexpr int R = SubRows<Tact>::value;
  __attribute__((aligned(16))) Tact sx[R][64];
  __attribute__((aligned(16))) Tact sd[R][64];
  __attribute__((aligned(16))) Tact sz[FINAL ? R : 1][64];
  __attribute__((aligned(16))) float sB[R][kNS];
  __attribute__((aligned(16))) float sC[FINAL ? R : 1][kNS];
};

// Orders a wave's LDS writes before its later LDS reads.  The sub-block
// staging is wave-local (every lane reads what lanes of its own wave wrote, and
// LDS executes a wave's operations in order), so a workgroup that runs
// independent chunk waves needs no workgroup barrier; a one-wave workgroup
// uses the plain barrier.
template <bool WAVE_LOCAL>
HM_DEV void chunk_sync() {
  if constexpr (WAVE_LOCAL) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    __syncthreads();
  }
}

// sm: this wave's LDS.  h_init (FINAL only): the state entering the chunk, in
// the caller's registers, or nullptr to read it from E (written there by the
// carry pass).
template <typename Tact, bool CONV, bool FINAL, bool VEC, bool WAVE_LOCAL = false>
HM_DEV void scan_chunk_body(
    ScanLds<Tact, FINAL>* sm, const float* h_init,
    int gxi, int k, int b, const Tact* __restrict__ x, const Tact* __restrict__ dl, const float* __restrict__ A,
    const Tact* __restrict__ Bm, const Tact* __restrict__ Cm, const float* __restrict__ D,
    const Tact* __restrict__ z, const float* __restrict__ cw, const float* __restrict__ cb,
    const float* __restrict__ cst_in, float* __restrict__ cst_out, float* __restrict__ E,
    float* __restrict__ S, Tact* __restrict__ y, float* __restrict__ h_out, int T, int Di, int L,
    int nC) {
  constexpr int R = SubRows<Tact>::value;        // rows per sub-block
  constexpr int PC = Stage<Tact>::kPerChunk;     // elements per 16 bytes
  constexpr int CPR = 64 / PC;                   // chunks per 64-channel row
  static_assert(R * CPR == 128, "two 16-byte chunks per lane per tensor");
  static_assert(R * kNS / PC <= 64, "one B (or C) chunk per lane");
  auto& sx = sm->sx;
  auto& sd = sm->sd;
  auto& sz = sm->sz;
  auto& sB = sm->sB;
  auto& sC = sm->sC;
  auto& sy = sm->sx;
  const int lane = threadIdx.x & 63;
  const int c0 = gxi * 64;
  const bool active = c0 + lane < Di;
  const int c = active ? c0 + lane : Di - 1;
  const int t0 = k * L, t1 = min(T, t0 + L);
  const size_t boff = (size_t)b * T * Di;
  const Tact* xb = x + boff;
  const Tact* db = dl + boff;
  const Tact* zb = z ? z + boff : nullptr;
  const Tact* Bb = Bm + (size_t)b * T * kNS;
  const Tact* Cb = Cm + (size_t)b * T * kNS;
  const bool has_z = FINAL && z != nullptr;

  // Vector staging (rows 16-byte aligned): every lane loads two 16-byte chunks
  // of x, delta (and z) and one chunk of B_t (lanes < BCH) or C_t (the others)
  // into registers, writes them to LDS, and the sub-block is computed from
  // LDS.  The loads of the next sub-block are issued before the current one is
  // computed.  Every load is unconditional (rows past the sub-block and chunks
  // past Di are clamped to valid addresses, a missing z reads x, a B-only pass
  // reads B twice) so the compiler can count them exactly and wait for them
  // without also waiting for the y stores issued after them.
  constexpr int BCH = R * kNS / PC;              // chunks of B (or C) per sub-block
  const int last_ch = ((Di - 1) / PC) * PC;
  const int ra = lane / CPR, rb = (lane + 64) / CPR;
  const int col = (lane % CPR) * PC;
  const int ca = min(c0 + col, last_ch);
  const bool takes_c = FINAL && lane >= BCH;
  const int bci = lane % BCH;
  const int bc_row = bci / (kNS / PC), bc_col = (bci % (kNS / PC)) * PC;
  const Tact* zsrc = has_z ? zb : xb;
  const Tact* bcsrc = takes_c ? Cb : Bb;
  float* bcdst = takes_c ? &sC[bc_row][bc_col] : &sB[bc_row][bc_col];
  uint4 x0, x1, d0, d1, z0, z1, vbc;
  auto load = [&](long long t, int nt) {
    const size_t oa = (size_t)(t + min(ra, nt - 1)) * Di + ca;
    const size_t ob = (size_t)(t + min(rb, nt - 1)) * Di + ca;
    x0 = *(const uint4*)(xb + oa);
    x1 = *(const uint4*)(xb + ob);
    d0 = *(const uint4*)(db + oa);
    d1 = *(const uint4*)(db + ob);
    if constexpr (FINAL) {
      z0 = *(const uint4*)(zsrc + oa);
      z1 = *(const uint4*)(zsrc + ob);
    }
    vbc = *(const uint4*)(bcsrc + (size_t)(t + min(bc_row, nt - 1)) * kNS + bc_col);
  };
  auto store = [&]() {
    *(uint4*)(&sx[ra][col]) = x0;
    *(uint4*)(&sx[rb][col]) = x1;
    *(uint4*)(&sd[ra][col]) = d0;
    *(uint4*)(&sd[rb][col]) = d1;
    if constexpr (FINAL) {
      *(uint4*)(&sz[ra][col]) = z0;
      *(uint4*)(&sz[rb][col]) = z1;
    }
    store_bc(bcdst, vbc, Tact());
  };
  if constexpr (VEC) load(t0, min(R, t1 - t0));

  float a2[kNS], h[kNS];
  const float* hin = E + ((size_t)b * nC + k) * kNS * Di + c;
#pragma unroll
  for (int nn = 0; nn < kNS; ++nn) {
    a2[nn] = A[c * kNS + nn] * kLog2e;
    h[nn] = FINAL ? (h_init ? h_init[nn] : hin[(size_t)nn * Di]) : 0.f;
  }
  const float Dc = (FINAL && D) ? D[c] : 0.f;
  const Tact* xc = xb + c;
  const float* sc = (CONV && cst_in) ? cst_in + ((size_t)b * Di + c) * 3 : nullptr;
  float w0 = 0, w1 = 0, w2 = 0, w3 = 0, bb = 0, p0 = 0, p1 = 0, p2 = 0;
  if (CONV) {
    w0 = cw[c * 4 + 0]; w1 = cw[c * 4 + 1]; w2 = cw[c * 4 + 2]; w3 = cw[c * 4 + 3];
    bb = cb[c];
    // the 3 inputs before t0: from x (unconditional, clamped loads) or, for
    // the first chunk, from the conv state
    const float q0 = ldx(xc + (size_t)max(t0 - 3, 0) * Di);
    const float q1 = ldx(xc + (size_t)max(t0 - 2, 0) * Di);
    const float q2 = ldx(xc + (size_t)max(t0 - 1, 0) * Di);
    if (t0 >= 3) {
      p0 = q0; p1 = q1; p2 = q2;
    } else if (sc) {
      p0 = sc[0]; p1 = sc[1]; p2 = sc[2];   // t0 == 0: chunks are >= 16 steps
    }
  }
  float ssum = 0.f;
  // Everything the time loop reads from registers has landed: without this the
  // compiler flushes the memory counter before every sub-block's time loop,
  // which also waits for the prefetch of the next sub-block.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // One sub-block of nt steps from LDS (staged by the caller), then y out.
  auto run = [&](int ts, int nt) {
    for (int tt = 0; tt < nt; ++tt) {
      float xv = ActIO<Tact>::ld(&sx[tt][lane]);
      const float dv = ActIO<Tact>::ld(&sd[tt][lane]);
      if (CONV) {
        const float u = bb + w0 * p0 + w1 * p1 + w2 * p2 + w3 * xv;
        p0 = p1; p1 = p2; p2 = xv;
        xv = siluf_(u);
      }
      const float du = dv * xv;
      const float4* b4 = (const float4*)sB[tt];
      float Bv[kNS];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 t4 = b4[i];
        Bv[4 * i] = t4.x; Bv[4 * i + 1] = t4.y; Bv[4 * i + 2] = t4.z; Bv[4 * i + 3] = t4.w;
      }
      if (FINAL) {
        const float4* c4 = (const float4*)sC[tt];
        float Cv[kNS];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 t4 = c4[i];
          Cv[4 * i] = t4.x; Cv[4 * i + 1] = t4.y; Cv[4 * i + 2] = t4.z; Cv[4 * i + 3] = t4.w;
        }
        float ys4[4] = {Dc * xv, 0.f, 0.f, 0.f};
        // decay product first, then the input term accumulated onto it: both
        // steps update h in place (no register copies in the loop)
#pragma unroll
        for (int nn = 0; nn < kNS; ++nn) {
          h[nn] = fmaf(du, Bv[nn], fast_exp2(dv * a2[nn]) * h[nn]);
          ys4[nn & 3] += Cv[nn] * h[nn];
        }
        float yv = (ys4[0] + ys4[1]) + (ys4[2] + ys4[3]);
        if (has_z) yv *= siluf_(ActIO<Tact>::ld(&sz[tt][lane]));
        if constexpr (VEC) {
          ActIO<Tact>::st(&sy[tt][lane], yv);
        } else if (active) {
          ActIO<Tact>::st(y + boff + (size_t)(ts + tt) * Di + c, yv);
        }
      } else {
#pragma unroll
        for (int nn = 0; nn < kNS; ++nn) h[nn] = fmaf(du, Bv[nn], fast_exp2(dv * a2[nn]) * h[nn]);
        ssum += dv;
      }
    }
    chunk_sync<WAVE_LOCAL>();
    if constexpr (FINAL && VEC) {
      // y sub-block out as two 16-byte stores per lane.  Rows past nt and
      // chunks past Di are clamped onto a valid row / chunk, so such a lane
      // repeats another lane's store (same address, same bytes).
      const int cy = min(c0 + col, last_ch) - c0;
      const int ya = min(ra, nt - 1), yb2 = min(rb, nt - 1);
      Tact* yrow = y + boff + (size_t)ts * Di + c0 + cy;
      *(uint4*)(yrow + (size_t)ya * Di) = *(const uint4*)(&sy[ya][cy]);
      *(uint4*)(yrow + (size_t)yb2 * Di) = *(const uint4*)(&sy[yb2][cy]);
    }
  };
  // Sub-blocks before the last prefetch their successor (unconditionally);
  // the last one is peeled off.
  int ts = t0;
  for (; ts + R < t1; ts += R) {
    if constexpr (VEC) {
      store();
      chunk_sync<WAVE_LOCAL>();
      load(ts + R, min(R, t1 - ts - R));
    } else {
      stage_scalar<Tact, R>(sx, sd, sz, sB, sC, xb, db, zb, Bb, Cb, has_z, FINAL, ts, R, c0, Di,
                            lane);
      chunk_sync<WAVE_LOCAL>();
    }
    run(ts, R);
  }
  if constexpr (VEC) {
    store();
  } else {
    stage_scalar<Tact, R>(sx, sd, sz, sB, sC, xb, db, zb, Bb, Cb, has_z, FINAL, ts, t1 - ts, c0,
                          Di, lane);
  }
  chunk_sync<WAVE_LOCAL>();
  run(ts, t1 - ts);

  if (!FINAL) {
    if (active) {
      float* e = E + ((size_t)b * nC + k) * kNS * Di + c;
#pragma unroll
      for (int nn = 0; nn < kNS; ++nn) e[(size_t)nn * Di] = h[nn];
      S[((size_t)b * nC + k) * Di + c] = ssum;
    }
  } else if (k == nC - 1 && active) {
    if (h_out) {
      float* ho = h_out + ((size_t)b * Di + c) * kNS;
#pragma unroll
      for (int nn = 0; nn < kNS; ++nn) ho[nn] = h[nn];
    }
    if (CONV && cst_out) {
      float* so = cst_out + ((size_t)b * Di + c) * 3;
      for (int e = 0; e < 3; ++e) so[e] = conv_in(xc, (long long)T - 3 + e, Di, sc);
    }
  }
}

// ---------------------------------------------------------------- carry across chunks
// The chunk aggregates are affine maps h -> exp2(a2 * sum_delta) h + E.  A
// workgroup handles 64 (b, state, channel) lanes; its kRanges waves split the
// chunk sequence into contiguous ranges.  Each wave composes its range (loads
// issued in batches, all in flight together), the range maps are chained in
// LDS, and each wave walks its range again writing the state that enters every
// chunk over the aggregate (in place).  The state entering chunk nC-1 closes
// the sequence.
constexpr int kCarryBatch = 24;

// kRanges waves per workgroup, one contiguous chunk range each.
template <int kRanges>
HM_DEV void scan_carry_body(int bx, int nn, int b, const float* __restrict__ A,
                            const float* __restrict__ h0, float* __restrict__ E,
                            const float* __restrict__ S, int Di, int nC) {
  __shared__ float sSum[kRanges][64], sAgg[kRanges][64];
  const int lane = threadIdx.x & 63, r = threadIdx.x >> 6;
  const int c0 = bx * 64 + lane;
  const bool active = c0 < Di;
  const int c = active ? c0 : Di - 1;
  const float a2 = A[c * kNS + nn] * kLog2e;
  const int nA = nC - 1;                         // chunks with an aggregate
  const int per = (nA + kRanges - 1) / kRanges;
  const int k0 = min(nA, r * per), k1 = min(nA, k0 + per);
  float* e = E + ((size_t)b * nC * kNS + nn) * Di + c;
  const float* sp = S + (size_t)b * nC * Di + c;
  const size_t es = (size_t)kNS * Di;

  // 1) compose this range: map = (sum of delta, aggregate from a zero start).
  // A range of up to kCarryBatch chunks stays in registers for step 3.
  float ssum = 0.f, agg = 0.f;
  float ge[kCarryBatch], gs[kCarryBatch];
  const bool resident = k1 - k0 <= kCarryBatch;
  for (int kb = k0; kb < k1; kb += kCarryBatch) {
#pragma unroll
    for (int i = 0; i < kCarryBatch; ++i)
      if (kb + i < k1) {
        ge[i] = e[(size_t)(kb + i) * es];
        gs[i] = sp[(size_t)(kb + i) * Di];
      }
#pragma unroll
    for (int i = 0; i < kCarryBatch; ++i)
      if (kb + i < k1) {
        agg = fast_exp2(a2 * gs[i]) * agg + ge[i];
        ssum += gs[i];
      }
  }
  sSum[r][lane] = ssum;
  sAgg[r][lane] = agg;
  __syncthreads();
  // 2) state entering this range, and the state after all ranges (empty
  // ranges are the identity map)
  const float hstart = h0 ? h0[((size_t)b * Di + c) * kNS + nn] : 0.f;
  float H = hstart, Hend = hstart;
  for (int q = 0; q < kRanges; ++q) {
    if (q == r) H = Hend;
    Hend = fast_exp2(a2 * sSum[q][lane]) * Hend + sAgg[q][lane];
  }
  // 3) walk the range again, writing each chunk's incoming state
  if (resident) {
#pragma unroll
    for (int i = 0; i < kCarryBatch; ++i)
      if (k0 + i < k1) {
        if (active) e[(size_t)(k0 + i) * es] = H;
        H = fast_exp2(a2 * gs[i]) * H + ge[i];
      }
  } else {
    for (int kb = k0; kb < k1; kb += kCarryBatch) {
#pragma unroll
      for (int i = 0; i < kCarryBatch; ++i)
        if (kb + i < k1) {
          ge[i] = e[(size_t)(kb + i) * es];
          gs[i] = sp[(size_t)(kb + i) * Di];
        }
#pragma unroll
      for (int i = 0; i < kCarryBatch; ++i)
        if (kb + i < k1) {
          if (active) e[(size_t)(kb + i) * es] = H;
          H = fast_exp2(a2 * gs[i]) * H + ge[i];
        }
    }
  }
  if (r == 0 && active) e[(size_t)nA * es] = Hend;   // enters the last chunk
}

}  // namespace
