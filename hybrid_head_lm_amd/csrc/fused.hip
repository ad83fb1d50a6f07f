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
//   2. flash attention                      | carry across scan chunks
//   3. final scan pass (y and the final states)
//   4. branch norm and average
// The same device code as the standalone entry points runs in each range.
#include "attn_dev.h"
#include "ssm_dev.h"

namespace {

struct PrepGeom {
  int n;       // workgroups (0: K/V already prepared)
  int tiles4;  // Tpad / 16
  int Hkv;
};
struct AggGeom {
  int n;       // workgroups = gx * (nC - 1) * B
  int gx, nA;  // channel groups, chunks with an aggregate
};

__global__ __launch_bounds__(64) void prefill_prep_agg(
    PrepGeom pg, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    bf16_t* __restrict__ Kr, bf16_t* __restrict__ Vt, int Tpad, long long pos0, double rstep,
    AggGeom ag, const bf16_t* __restrict__ x, const bf16_t* __restrict__ dl,
    const float* __restrict__ A, const bf16_t* __restrict__ Bm, const float* __restrict__ cw,
    const float* __restrict__ cb, float* __restrict__ E, float* __restrict__ S, int T, int Di,
    int L, int nC) {
  int bid = blockIdx.x;
  if (bid < pg.n) {
    const int bx = bid % pg.tiles4, g = (bid / pg.tiles4) % pg.Hkv;
    const int b = bid / (pg.tiles4 * pg.Hkv);
    attn_prep_bf16_body(bx, g, b, k, v, Kr, Vt, T, Tpad, pg.Hkv, pos0, rstep);
    return;
  }
  bid -= pg.n;
  const int gxi = bid % ag.gx, kc = (bid / ag.gx) % ag.nA, b = bid / (ag.gx * ag.nA);
  // (the aggregate pass reads neither C, D, z nor writes y: B stands in for C)
  scan_chunk_body<bf16_t, true, false, true>(gxi, kc, b, x, dl, A, Bm, Bm, nullptr, nullptr, cw,
                                              cb, nullptr, nullptr, E, S, nullptr, nullptr, T, Di,
                                              L, nC);
}

constexpr int kFusedRanges = 4;   // carry waves per 256-thread workgroup

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) void
prefill_attn_carry(int n_attn, const bf16_t* __restrict__ q, const bf16_t* __restrict__ Kr,
                   const bf16_t* __restrict__ Vt, bf16_t* __restrict__ o, int T, int Tpad, int Hq,
                   int Hkv, int M, int W, long long pos0, float qscale, double rstep, int n_qt,
                   int n_groups, int gx, const float* __restrict__ A, float* __restrict__ E,
                   const float* __restrict__ S, int Di, int nC) {
  int bid = blockIdx.x;
  if (bid < n_attn) {
    attn_fwd_bf16_body(bid, q, Kr, Vt, o, T, Tpad, Hq, Hkv, M, W, pos0, qscale, rstep, n_qt,
                       n_groups);
    return;
  }
  bid -= n_attn;
  const int gxi = bid % gx, nn = (bid / gx) % kNS, b = bid / (gx * kNS);
  scan_carry_body<kFusedRanges>(gxi, nn, b, A, nullptr, E, S, Di, nC);
}

__global__ __launch_bounds__(64) void prefill_scan_final(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ dl, const float* __restrict__ A,
    const bf16_t* __restrict__ Bm, const bf16_t* __restrict__ Cm, const float* __restrict__ D,
    const bf16_t* __restrict__ z, const float* __restrict__ cw, const float* __restrict__ cb,
    float* __restrict__ cst_out, float* __restrict__ E, float* __restrict__ S,
    bf16_t* __restrict__ y, float* __restrict__ h_out, int T, int Di, int L, int nC) {
  scan_chunk_body<bf16_t, true, true, true>(blockIdx.x, blockIdx.y, blockIdx.z, x, dl, A, Bm, Cm,
                                             D, z, cw, cb, nullptr, cst_out, E, S, y, h_out, T,
                                             Di, L, nC);
}

}  // namespace

namespace hm {

bool prefill_fusable(const hm_prefill_args* a) {
  return a->dtype == HM_BF16 && a->stream2 == nullptr && a->Dh == 64 && a->N == kNS &&
         a->K == kConvK && a->Di % 8 == 0 && aligned16(a->x) && aligned16(a->delta) &&
         aligned16(a->Bm) && aligned16(a->Cm) && (a->z == nullptr || aligned16(a->z));
}

// Arguments were validated by the caller (the unfused parts in dry-run mode).
hm_status prefill_fused_bf16(const hm_prefill_args* a, void* kv, void* scan_ws, hipStream_t st) {
  const int B = a->B, T = a->T, Di = a->Di, Hq = a->Hq, Hkv = a->Hkv;
  const int Tpad = (T + 63) / 64 * 64;
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

  // 1. K/V pre-pass | chunk aggregates
  PrepGeom pg{a->kv_reuse ? 0 : (Tpad / 16) * Hkv * B, Tpad / 16, Hkv};
  AggGeom ag{gx * (nC - 1) * B, gx, nC > 1 ? nC - 1 : 1};
  if (pg.n + ag.n > 0) {
    hipLaunchKernelGGL(prefill_prep_agg, dim3(pg.n + ag.n), dim3(64), 0, st, pg,
                       (const bf16_t*)a->k, (const bf16_t*)a->v, Kr, Vt, Tpad, a->pos0, rstep,
                       ag, (const bf16_t*)a->x, (const bf16_t*)a->delta, a->A,
                       (const bf16_t*)a->Bm, a->conv_w, a->conv_b, E, S, T, Di, L, nC);
    hm_status s = check_launch("prefill_prep_agg");
    if (s != HM_OK) return s;
  }
  // 2. attention | carry
  const int n_qt = (T + 128 - 1) / 128;
  const int n_groups = B * Hkv * n_qt;
  const int n_attn = 8 * ((n_groups + 7) / 8) * (Hq / Hkv);
  const int n_carry = gx * kNS * B;
  hipLaunchKernelGGL(prefill_attn_carry, dim3(n_attn + n_carry), dim3(256), 0, st, n_attn,
                     (const bf16_t*)a->q, (const bf16_t*)Kr, (const bf16_t*)Vt, (bf16_t*)a->ya, T,
                     Tpad, Hq, Hkv, a->n_meta, a->window, a->pos0, scale * kLog2e, rstep, n_qt,
                     n_groups, gx, a->A, E, (const float*)S, Di, nC);
  hm_status s = check_launch("prefill_attn_carry");
  if (s != HM_OK) return s;
  // 3. final scan pass
  hipLaunchKernelGGL(prefill_scan_final, dim3(gx, nC, B), dim3(64), 0, st, (const bf16_t*)a->x,
                     (const bf16_t*)a->delta, a->A, (const bf16_t*)a->Bm, (const bf16_t*)a->Cm,
                     a->D, (const bf16_t*)a->z, a->conv_w, a->conv_b, a->conv_state_out, E, S,
                     (bf16_t*)a->ys, a->h_out, T, Di, L, nC);
  s = check_launch("prefill_scan_final");
  if (s != HM_OK) return s;
  // 4. branch norm and average
  return norm_mean_impl(a->ya, a->ys, a->beta_a, a->beta_s, a->eps, a->out, (long long)B * T, Di,
                        a->dtype, st, /*dry=*/false);
}

}  // namespace hm
