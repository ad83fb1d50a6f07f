// Fused launch sequence of one bf16 prefill layer of the hybrid-head mixer
// (Hymba blog, juejin.cn "NVIDIA提出Hymba网络": the attention heads and the SSM
// heads read the same input in parallel, "深入理解混合头模块"; their outputs are
// normalised and averaged, "数学表示" §5).
//
// Every kernel boundary costs a few microseconds on its own (dispatch plus the
// cache write-back that makes a kernel's results visible to the next one), so
// work items that do not depend on each other share one launch, taking
// disjoint ranges of the grid:
//   1. K/V pre-pass (rotate K, lay out V)   | chunk aggregates of the scan
//   2. flash attention                      | final scan pass: each chunk wave
//                                             composes its own incoming state
//                                             from the aggregates, then runs
//                                             the chunk (y, final states)
//   3. branch norm and average
// When both parts of a launch are resident at once (a single layer of a few
// thousand rows) the latency-bound attention and the VALU-bound scan fill each
// other's idle issue slots; when the scan waves alone fill the chip (long
// inputs) the launch runs them first and the attention after them, which
// measured faster than mixing the two on the same CUs.
// The same device code as the standalone entry points runs in each range.
#include "attn_dev.h"
#include "ssm_dev.h"

namespace {

struct PrepGeom {
  int n;       // workgroups (0: K/V already prepared)
  int tiles4;  // Tpad / 16
  int Hkv;
  int Mk;      // cached meta rows in front of the T token rows (0: none)
  const bf16_t *meta_k, *meta_v;
};
struct AggGeom {
  int n;       // workgroups = gx * (nC - 1) * B
  int gx, nA;  // channel groups, chunks with an aggregate
  int first;   // the aggregate waves take the low ids (dispatched before the K/V pre-pass)
};
// Aggregate waves that fill at least half of the chip's wave slots (4 per
// SIMD) are dispatched first: the memory-bound K/V pre-pass then runs in the
// remaining slots beside them instead of delaying their start (measured on
// the 32-layer stack: 174 -> 155 us per launch of a layer that prepares K/V,
// 165 -> 156 us for one that reuses it).  Below that both fit at once and the
// pre-pass goes first.
constexpr int kAggFirstWaves = 2048;

__global__ __launch_bounds__(64) void prefill_prep_agg(
    PrepGeom pg, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    bf16_t* __restrict__ Kr, bf16_t* __restrict__ Vt, int Tpad, long long pos0, double rstep,
    AggGeom ag, const bf16_t* __restrict__ x, const bf16_t* __restrict__ dl,
    const float* __restrict__ A, const bf16_t* __restrict__ Bm, const float* __restrict__ cw,
    const float* __restrict__ cb, const float* __restrict__ cst_in, float* __restrict__ E,
    float* __restrict__ S, int T, int Di, int L, int nC) {
  int bid = blockIdx.x;
  const int prep0 = ag.first ? ag.n : 0;       // first id of the pre-pass range
  if (bid >= prep0 && bid < prep0 + pg.n) {
    bid -= prep0;
    const int bx = bid % pg.tiles4, g = (bid / pg.tiles4) % pg.Hkv;
    const int b = bid / (pg.tiles4 * pg.Hkv);
    attn_prep_bf16_body(bx, g, b, k, v, pg.meta_k, pg.meta_v, pg.Mk, Kr, Vt, T, Tpad, pg.Hkv,
                        pos0, rstep);
    return;
  }
  if (!ag.first) bid -= pg.n;
  const int gxi = bid % ag.gx, kc = (bid / ag.gx) % ag.nA, b = bid / (ag.gx * ag.nA);
  // (the aggregate pass reads neither C, D, z nor writes y: B stands in for C)
  __shared__ ScanLds<bf16_t, false> sm;
  scan_chunk_body<bf16_t, true, false, true>(&sm, nullptr, gxi, kc, b, x, dl, A, Bm, Bm, nullptr,
                                              nullptr, cw, cb, cst_in, nullptr, E, S, nullptr,
                                              nullptr, T, Di, L, nC);
}

constexpr int kChunkWaves = 4;        // consecutive chunks per 256-thread workgroup
constexpr int kAttnLds = kStages * 2 * 8192;
constexpr int kOwnCarryBatch = 16;    // chunk maps loaded at once per wave
static_assert(sizeof(ScanLds<bf16_t, true>) <= 8192, "a chunk wave's LDS is 8 KB");
static_assert(kChunkWaves * 8192 <= kAttnLds, "chunk waves reuse the attention ring");
static_assert(kChunkWaves * kNS * 64 * 4 <= kAttnLds, "incoming states fit the ring");

struct FinalGeom {
  int gx, nJ;   // 64-channel groups; workgroups per group and batch (kChunkWaves chunks each)
  int n;        // final-pass workgroups (gx * nJ * B); the grid rounds them up to a
                // multiple of 8 so that the attention ids keep their XCD (id % 8)
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void
prefill_attn_final(int n_attn, const bf16_t* __restrict__ q, const bf16_t* __restrict__ Kr,
                   const bf16_t* __restrict__ Vt, bf16_t* __restrict__ o, int Tpad, int Hq,
                   int Hkv, int M, int W, long long pos0, float qscale, double rstep, int n_qt,
                   int n_groups, FinalGeom fg, const bf16_t* __restrict__ x,
                   const bf16_t* __restrict__ dl, const float* __restrict__ A,
                   const bf16_t* __restrict__ Bm, const bf16_t* __restrict__ Cm,
                   const float* __restrict__ D, const bf16_t* __restrict__ z,
                   const float* __restrict__ cw, const float* __restrict__ cb,
                   const float* __restrict__ cst_in, float* __restrict__ cst_out,
                   const float* __restrict__ h0, float* __restrict__ E, float* __restrict__ S,
                   bf16_t* __restrict__ y, float* __restrict__ h_out, int T, int Di, int L,
                   int nC, int Mk) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kAttnLds];
  // The final-pass workgroups take the low ids (dispatched first), the latest
  // chunks (longest own carry) first; the attention workgroups follow.
  const int n_fin = (int)gridDim.x - n_attn;
  int bid = blockIdx.x;
  if (bid >= n_fin) {
    attn_fwd_bf16_body((unsigned char(*)[2][8192])smem, bid - n_fin, q, Kr, Vt, o, Mk + T, Tpad,
                       Hq, Hkv, M, W, pos0, qscale, rstep, n_qt, n_groups, T, Mk);
    return;
  }
  bid = n_fin - 1 - bid;
  if (bid >= fg.n) return;                      // padding to a multiple of 8
  const int gxi = bid % fg.gx, jw = (bid / fg.gx) % fg.nJ, b = bid / (fg.gx * fg.nJ);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int k0 = jw * kChunkWaves, k = k0 + wave;
  const int c = min(gxi * 64 + lane, Di - 1);
  // states entering chunks k0 .. k0+3: [chunk - k0][state][lane]
  float(*sH)[kNS][64] = (float(*)[kNS][64])smem;

  // 1. Chunk kk < nC-1 maps the state h to exp2(a2 * S_kk) h + E_kk (sum of
  //    delta, end state from a zero start).  Composing the maps of chunks
  //    0 .. kk-1 from the initial state h0 (or zero) gives the state entering
  //    chunk kk.  Wave w composes states 4w .. 4w+3 of the 64 channels up to
  //    the workgroup's last chunk and keeps the states entering each of its
  //    chunks.
  {
    float a2[4], H[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a2[e] = A[c * kNS + 4 * wave + e] * kLog2e;
      H[e] = h0 ? h0[((size_t)b * Di + c) * kNS + 4 * wave + e] : 0.f;
    }
    const int kend = min(k0 + kChunkWaves, nC) - 1;   // compose chunks 0 .. kend-1
    const float* ep = E + ((size_t)b * nC * kNS + 4 * wave) * Di + c;
    const float* sp = S + (size_t)b * nC * Di + c;
    auto stash = [&](int j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sH[j][4 * wave + e][lane] = H[e];
    };
    if (k0 == 0) stash(0);
    for (int kb = 0; kb < kend; kb += kOwnCarryBatch) {
      float gs[kOwnCarryBatch], ge[kOwnCarryBatch][4];
#pragma unroll
      for (int i = 0; i < kOwnCarryBatch; ++i) {
        const int kk = min(kb + i, kend - 1);   // clamped, unconditional loads
        gs[i] = sp[(size_t)kk * Di];
#pragma unroll
        for (int e = 0; e < 4; ++e) ge[i][e] = ep[((size_t)kk * kNS + e) * Di];
      }
#pragma unroll
      for (int i = 0; i < kOwnCarryBatch; ++i)
        if (kb + i < kend) {
#pragma unroll
          for (int e = 0; e < 4; ++e) H[e] = fast_exp2(a2[e] * gs[i]) * H[e] + ge[i][e];
          if (kb + i + 1 >= k0) stash(kb + i + 1 - k0);
        }
    }
  }
  __syncthreads();
  float h[kNS];
#pragma unroll
  for (int nn = 0; nn < kNS; ++nn) h[nn] = sH[wave][nn][lane];
  __syncthreads();   // the states lie where the chunk waves stage their data
  if (k >= nC) return;
  // 3. The chunk itself, in this wave's 8 KB of the (idle) attention ring.
  scan_chunk_body<bf16_t, true, true, true, true>(
      (ScanLds<bf16_t, true>*)(smem + wave * 8192), h, gxi, k, b, x, dl, A, Bm, Cm, D, z, cw, cb,
      cst_in, cst_out, E, S, y, h_out, T, Di, L, nC);
}

}  // namespace

namespace hm {

bool prefill_fusable(const hm_prefill_args* a) {
  return a->dtype == HM_BF16 && a->stream2 == nullptr && a->Dh == 64 && a->N == kNS &&
         a->K == kConvK && a->Di % 8 == 0 && aligned16(a->x) && aligned16(a->delta) &&
         aligned16(a->Bm) && aligned16(a->Cm) && (a->z == nullptr || aligned16(a->z)) &&
         (a->meta_k == nullptr || (aligned16(a->meta_k) && aligned16(a->meta_v)));
}

// Arguments were validated by the caller (the unfused parts in dry-run mode).
hm_status prefill_fused_bf16(const hm_prefill_args* a, void* kv, void* scan_ws, hipStream_t st) {
  const int B = a->B, T = a->T, Di = a->Di, Hq = a->Hq, Hkv = a->Hkv;
  const int Mk = a->meta_k ? a->n_meta : 0;     // cached meta rows in front of the tokens
  const int Tpad = (Mk + T + 63) / 64 * 64;     // prepared key rows
  bf16_t* Kr = (bf16_t*)kv;
  bf16_t* Vt = Kr + (size_t)B * Hkv * Tpad * 64;
  const double l2b = log2((double)a->rope_base);
  const double rstep = exp2(-l2b / 32.0);   // theta_{d+1} / theta_d for Dh = 64
  const float scale = a->scale > 0.f ? a->scale : 0.125f;   // 1/sqrt(64)
  // scan geometry (as the standalone scan)
  const int L = scan_chunk_len(B, T, Di);
  const int nC = (T + L - 1) / L;
  float* E = (float*)scan_ws;
  float* S = E + (size_t)B * nC * kNS * Di;
  const int gx = (Di + 63) / 64;

  // caller's timing events around the three launches (optional)
  auto mark = [&](int i) -> hm_status {
    if (a->events == nullptr || a->events[i] == nullptr) return HM_OK;
    if (hipEventRecord((hipEvent_t)a->events[i], st) != hipSuccess)
      return fail(HM_ERR_HIP, "hipEventRecord of a timing event failed");
    return HM_OK;
  };
  hm_status s = mark(0);
  if (s != HM_OK) return s;
  // 1. K/V pre-pass | chunk aggregates (chunks 0 .. nC-2)
  PrepGeom pg{a->kv_reuse ? 0 : (Tpad / 16) * Hkv * B, Tpad / 16, Hkv, Mk,
              (const bf16_t*)a->meta_k, (const bf16_t*)a->meta_v};
  AggGeom ag{gx * (nC - 1) * B, gx, nC > 1 ? nC - 1 : 1, 0};
  ag.first = ag.n >= kAggFirstWaves;
  if (pg.n + ag.n > 0) {
    hipLaunchKernelGGL(prefill_prep_agg, dim3(pg.n + ag.n), dim3(64), 0, st, pg,
                       (const bf16_t*)a->k, (const bf16_t*)a->v, Kr, Vt, Tpad, a->pos0, rstep,
                       ag, (const bf16_t*)a->x, (const bf16_t*)a->delta, a->A,
                       (const bf16_t*)a->Bm, a->conv_w, a->conv_b, a->conv_state_in, E, S, T,
                       Di, L, nC);
    s = check_launch("prefill_prep_agg");
    if (s != HM_OK) return s;
  }
  s = mark(1);
  if (s != HM_OK) return s;
  // 2. attention | final scan pass
  const int n_qt = (T + kBM - 1) / kBM;          // query tiles over the token rows
  const int n_groups = B * Hkv * n_qt;
  const int n_attn = 8 * ((n_groups + 7) / 8) * (Hq / Hkv);
  const int nJ = (nC + kChunkWaves - 1) / kChunkWaves;
  const FinalGeom fg{gx, nJ, gx * nJ * B};
  const int n_final = 8 * ((fg.n + 7) / 8);
  hipLaunchKernelGGL(prefill_attn_final, dim3(n_attn + n_final), dim3(256), 0, st, n_attn,
                     (const bf16_t*)a->q, (const bf16_t*)Kr, (const bf16_t*)Vt, (bf16_t*)a->ya,
                     Tpad, Hq, Hkv, a->n_meta, a->window, a->pos0, scale * kLog2e, rstep, n_qt,
                     n_groups, fg, (const bf16_t*)a->x, (const bf16_t*)a->delta, a->A,
                     (const bf16_t*)a->Bm, (const bf16_t*)a->Cm, a->D, (const bf16_t*)a->z,
                     a->conv_w, a->conv_b, a->conv_state_in, a->conv_state_out, a->h0, E, S,
                     (bf16_t*)a->ys, a->h_out, T, Di, L, nC, Mk);
  s = check_launch("prefill_attn_final");
  if (s != HM_OK) return s;
  s = mark(2);
  if (s != HM_OK) return s;
  // 3. branch norm and average
  s = norm_mean_impl(a->ya, a->ys, a->beta_a, a->beta_s, a->eps, a->out, (long long)B * T, Di,
                     a->dtype, st, /*dry=*/false);
  if (s != HM_OK) return s;
  return mark(3);
}

// Scans whose aggregate waves fill half the chip: there the final pass
// composing its own incoming states beats a separate carry launch (459 -> 430
// us at 2 x 16512 rows); on a short scan it saves nothing (45 us either way
// at 2176 rows) and reads the chunk maps once per final workgroup (105
// against 79 MB), so the carry launch stays.
bool conv_scan_two_launch_pays(int B, int T, int Di) {
  const int L = scan_chunk_len(B, T, Di);
  const int nC = (T + L - 1) / L;
  return (long long)((Di + 63) / 64) * (nC - 1) * B >= kAggFirstWaves;
}

// The two scan launches of the layer above with no attention work in them:
// no K/V pre-pass range in the first, no attention range in the second (so
// the attention arguments are never read).
hm_status conv_scan_two_launch_bf16(const void* x, const float* cw, const float* cb,
                                    const float* cst_in, float* cst_out, const void* delta,
                                    const float* A, const void* Bm, const void* Cm,
                                    const float* D, const void* z, const float* h0, void* y,
                                    float* h_out, int B, int T, int Di, void* workspace,
                                    hipStream_t st) {
  const int L = scan_chunk_len(B, T, Di);
  const int nC = (T + L - 1) / L;
  float* E = (float*)workspace;
  float* S = E + (size_t)B * nC * kNS * Di;
  const int gx = (Di + 63) / 64;
  const PrepGeom pg{0, 1, 1, 0, nullptr, nullptr};
  const AggGeom ag{gx * (nC - 1) * B, gx, nC > 1 ? nC - 1 : 1, 1};
  if (ag.n > 0) {
    hipLaunchKernelGGL(prefill_prep_agg, dim3(ag.n), dim3(64), 0, st, pg, nullptr, nullptr,
                       nullptr, nullptr, 64, 0LL, 1.0, ag, (const bf16_t*)x,
                       (const bf16_t*)delta, A, (const bf16_t*)Bm, cw, cb, cst_in, E, S, T, Di,
                       L, nC);
    hm_status s = check_launch("prefill_prep_agg (scan aggregates)");
    if (s != HM_OK) return s;
  }
  const int nJ = (nC + kChunkWaves - 1) / kChunkWaves;
  const FinalGeom fg{gx, nJ, gx * nJ * B};
  const int n_final = 8 * ((fg.n + 7) / 8);
  hipLaunchKernelGGL(prefill_attn_final, dim3(n_final), dim3(256), 0, st, /*n_attn=*/0, nullptr,
                     nullptr, nullptr, nullptr, 64, 1, 1, 0, 0, 0LL, 0.f, 1.0, 1, 0, fg,
                     (const bf16_t*)x, (const bf16_t*)delta, A, (const bf16_t*)Bm,
                     (const bf16_t*)Cm, D, (const bf16_t*)z, cw, cb, cst_in, cst_out, h0, E, S,
                     (bf16_t*)y, h_out, T, Di, L, nC, 0);
  return check_launch("prefill_attn_final (scan final pass)");
}

}  // namespace hm
