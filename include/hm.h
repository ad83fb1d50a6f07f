/*
 * hm.h — C ABI of the Hymba hybrid-head mixer core on AMD MI355X (gfx950).
 *
 * The mixer is the hybrid-head module of Hymba: attention heads and SSM heads
 * read the same projected input X~ = [meta tokens; tokens] in parallel, each
 * branch output is normalised and rescaled by a learnable vector, and the two
 * are averaged.  Sources (web pages on Hymba):
 *   - juejin.cn blog "NVIDIA提出Hymba网络，Mamba+Attenation解决transformer的长序列
 *     低效难题" (below: Hymba blog): sections "深入理解混合头模块" (module),
 *     "数学表示" §1 (X~ = [R, X]), §2 (input projection), §3 Eq. (1) (attention),
 *     §4 Eq. (2) (SSM heads), §5 (norm, rescale, fuse), "Hymba 的整体架构"
 *     (global first/middle/last layers, sliding window elsewhere, adjacent
 *     layers share the KV cache);
 *   - Hymba-1.5B-Base model card, "模型架构" (GQA, RoPE, 16 SSM states).
 * The mixer entry points take already-projected tensors; hm_linear_bf16 and
 * hm_linear_bf16_ex are the projections around them, and hm_block_prefill
 * runs a whole block (norm, projections, mixer, norm, feed-forward network).
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless stated otherwise; tensors are
 *     row-major and contiguous (last index fastest) and 16-byte aligned.
 *   - Activations (q, k, v, o, x, delta, B, C, z, y, caches, out) have the
 *     dtype given by `dtype`; parameters (A, D, conv weights and bias, beta)
 *     and recurrent states are float32.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the null stream).  The library never synchronises, never
 *     allocates device memory and keeps no pointer after a call returns.  The
 *     caller owns every buffer; outputs must not alias inputs except the
 *     documented in/out states and caches.  Scratch memory is passed in as
 *     `workspace`, sized by the matching *_workspace() query.
 *   - Every argument is validated before anything is launched, so on failure
 *     no output is touched.  Errors are returned as hm_status; nothing aborts
 *     or throws across the ABI.  hm_last_error() gives a message for the last
 *     failing call on the calling thread.
 *   - Extents (batch, rows, token counts, widths, heads) must be positive: an
 *     empty call returns HM_ERR_INVALID and launches nothing.
 */
#ifndef HM_H_
#define HM_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HM_ABI_VERSION 1

typedef enum {
  HM_OK = 0,
  HM_ERR_INVALID = 1,      /* NULL required pointer, bad size or alignment      */
  HM_ERR_UNSUPPORTED = 2,  /* valid but not implemented (head dim, states, ...) */
  HM_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required        */
  HM_ERR_HIP = 4           /* a HIP launch failed; see hm_last_error()          */
} hm_status;

typedef enum { HM_F32 = 0, HM_BF16 = 1 } hm_dtype;

int hm_abi_version(void);                       /* == HM_ABI_VERSION */
const char* hm_status_string(hm_status s);      /* static string, never NULL */
const char* hm_last_error(void);                /* thread-local, "" if none */

/* ------------------------------------------------------------------------
 * Attention heads over X~ (Hymba blog, 数学表示 §3 Eq. (1); sliding window and
 * always-visible meta tokens: Hymba简介 and Hymba 的整体架构; GQA and RoPE:
 * model card 模型架构).
 *
 *   O[b,i,h,:] = sum_j softmax_j( scale * <rope(q[b,i,h]), rope(k[b,j,g])> ) v[b,j,g]
 *   over the keys j visible from row i:  j <= i  and  (j < n_meta or
 *   window <= 0 or i - j < window);  g = h / (Hq / Hkv).
 *
 * q, o: [B, T, Hq, Dh];  k, v: [B, T, Hkv, Dh] (k before RoPE).  Rows of X~
 * are meta tokens 0..n_meta-1 followed by tokens; row i has position pos0+i.
 * RoPE is the rotate-half form on pairs (d, d + Dh/2) with angle
 * pos * rope_base^(-2d/Dh) (angles evaluated in double precision).
 * scale <= 0 selects 1/sqrt(Dh).  window <= 0 selects global causal attention.
 * Supported: bf16 with Dh = 64 (MFMA path, float32 accumulation and softmax);
 * float32 with Dh in {16, 32, 64} (float32 path).
 * Workspace: hm_swa_meta_attn_workspace() bytes (rotated K and transposed V).
 * ---------------------------------------------------------------------- */
hm_status hm_swa_meta_attn(const void* q, const void* k, const void* v, void* o,
                           int B, int T, int Hq, int Hkv, int Dh, int n_meta,
                           int window, float rope_base, long long pos0, float scale,
                           hm_dtype dtype, void* workspace, size_t workspace_bytes,
                           void* stream);
size_t hm_swa_meta_attn_workspace(int B, int T, int Hkv, int Dh, hm_dtype dtype);

/* The two halves of hm_swa_meta_attn, so that the prepared K/V of one layer
 * can serve the next layer (adjacent layers share their KV: Hymba blog,
 * Hymba 的整体架构) and so that the attention kernel can run on its own.
 *   hm_attn_kv_prepare: rotate k (RoPE at positions pos0 + i) and lay out k and
 *     v for the attention kernel in `kv` (hm_attn_kv_bytes() bytes, caller-owned).
 *   hm_attn_with_kv: attention of q over a prepared `kv`.  rope_base and pos0
 *     must be the values the buffer was prepared with; k and v are not needed.
 * The layout of `kv` is private to the library (bf16: rotated K as
 * [B, Hkv, ceil(T/64)*64, 64] followed by V as 64x64 tiles transposed per
 * head; f32: rotated K [B, Hkv, T, Dh] followed by a copy of V). */
size_t hm_attn_kv_bytes(int B, int T, int Hkv, int Dh, hm_dtype dtype);
hm_status hm_attn_kv_prepare(const void* k, const void* v, void* kv, size_t kv_bytes, int B,
                             int T, int Hkv, int Dh, float rope_base, long long pos0,
                             hm_dtype dtype, void* stream);
hm_status hm_attn_with_kv(const void* q, const void* kv, size_t kv_bytes, void* o, int B, int T,
                          int Hq, int Hkv, int Dh, int n_meta, int window, float rope_base,
                          long long pos0, float scale, hm_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * Causal depthwise conv1d in front of the scan (the short convolution of a
 * Mamba head; not printed on the pages):
 *   y[b,t,c] = act( bias[c] + sum_{k<K} w[c,k] * x[b, t-K+1+k, c] )
 * act = SiLU if apply_silu else identity.  Inputs before t = 0 come from
 * state_in[b, c, 0..K-2] (oldest first) or are zero when state_in is NULL.
 * state_out (may be NULL) receives the last K-1 inputs (oldest first).
 * x, y: [B, T, Di]; w: [Di, K] f32; bias: [Di] f32 or NULL;
 * state_in/state_out: [B, Di, K-1] f32.  Supported: K = 4.
 * ---------------------------------------------------------------------- */
hm_status hm_causal_conv1d(const void* x, const float* w, const float* bias,
                           const float* state_in, void* y, float* state_out,
                           int B, int T, int Di, int K, int apply_silu,
                           hm_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * Selective scan of the SSM heads (Hymba blog, 数学表示 §4 Eq. (2), recurrent
 * form), N states per channel:
 *   h_t = exp(delta_t * A) * h_{t-1} + (delta_t * x_t) * B_t
 *   y_t = (C_t . h_t + D * x_t) * SiLU(z_t)
 * x, delta, z, y: [B, T, Di] (delta >= 0, already passed through softplus);
 * Bm, Cm: [B, T, N]; A: [Di, N] f32; D: [Di] f32 or NULL (no skip);
 * z NULL: no gate; h0: [B, Di, N] f32 or NULL (zero start);
 * h_out: [B, Di, N] f32 or NULL.  Supported: N = 16.
 * Workspace: hm_selective_scan_workspace() bytes (per-chunk carries).
 * ---------------------------------------------------------------------- */
hm_status hm_selective_scan(const void* x, const void* delta, const float* A,
                            const void* Bm, const void* Cm, const float* D,
                            const void* z, const float* h0, void* y, float* h_out,
                            int B, int T, int Di, int N, hm_dtype dtype,
                            void* workspace, size_t workspace_bytes, void* stream);
size_t hm_selective_scan_workspace(int B, int T, int Di, int N);

/* Same as hm_causal_conv1d (SiLU) followed by hm_selective_scan on its output,
 * in one pass over x (the conv output never goes to memory).  conv_state_in /
 * conv_state_out as state_in / state_out above.  Same workspace as the scan. */
hm_status hm_conv_selective_scan(const void* x, const float* conv_w,
                                 const float* conv_b, const float* conv_state_in,
                                 float* conv_state_out, const void* delta,
                                 const float* A, const void* Bm, const void* Cm,
                                 const float* D, const void* z, const float* h0,
                                 void* y, float* h_out, int B, int T, int Di, int K,
                                 int N, hm_dtype dtype, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Branch normalisation and average (Hymba blog, 深入理解混合头模块 and
 * 数学表示 §5):  per row r,
 *   out[r,:] = 0.5 * ( beta_a * ya[r,:] / rms(ya[r,:]) + beta_s * ys[r,:] / rms(ys[r,:]) )
 *   rms(y) = sqrt(mean(y^2) + eps)
 * ya, ys, out: [rows, width]; beta_a, beta_s: [width] f32.
 * ---------------------------------------------------------------------- */
hm_status hm_branch_norm_mean(const void* ya, const void* ys, const float* beta_a,
                              const float* beta_s, float eps, void* out,
                              long long rows, int width, hm_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * Projections around the mixer (Hymba blog, 数学表示 §2: X~ times W_in_proj
 * gives Q, K, V, the SSM input and the gate G; §5: W_out_proj maps the fused
 * output back to the model width).
 *   y = x W^T: x [M, K] bf16, w [N, K] bf16 (nn.Linear layout), float32
 *   accumulation, results rounded to bf16.
 * The N output columns are split into n_seg consecutive segments: segment s
 * has seg_cols[s] columns (a positive multiple of 16) and is written to
 * outs[s] as [M, seg_cols[s]], so an in-projection writes Q, K, V, x and z
 * into their own tensors.  outs and seg_cols are HOST arrays of n_seg
 * entries (1 <= n_seg <= 8; widths summing to N).  K must be a multiple of 64.
 * ---------------------------------------------------------------------- */
hm_status hm_linear_bf16(const void* x, const void* w, int M, int N, int K, int n_seg,
                         void* const* outs, const int* seg_cols, void* stream);

/* ------------------------------------------------------------------------
 * hm_linear_bf16 with an epilogue per output segment, applied in float32
 * before the bf16 rounding:
 *   y = act(x W^T + bias) + residual
 * act: HM_ACT_NONE; HM_ACT_SILU, v / (1 + e^-v) (the feed-forward network's
 * hidden layer); HM_ACT_SOFTPLUS, log(1 + e^v) (non-negative SSM step sizes).
 * bias: [width] f32 (16-byte aligned) or NULL.  residual: [M, width] bf16
 * (16-byte aligned) or NULL; it may be the
 * segment's own output (an in-place skip connection, y += ...), but no other
 * segment's output, x or w.  epilogues: HOST array of n_seg entries, or NULL
 * (then identical to hm_linear_bf16).  Other arguments and errors as for
 * hm_linear_bf16.
 * ---------------------------------------------------------------------- */
typedef enum { HM_ACT_NONE = 0, HM_ACT_SILU = 1, HM_ACT_SOFTPLUS = 2 } hm_act;
typedef struct {
  const float* bias;     /* [width] f32 or NULL */
  const void* residual;  /* [M, width] bf16 or NULL */
  int act;               /* hm_act */
} hm_linear_epilogue;
hm_status hm_linear_bf16_ex(const void* x, const void* w, int M, int N, int K, int n_seg,
                            void* const* outs, const int* seg_cols,
                            const hm_linear_epilogue* epilogues, void* stream);

/* ------------------------------------------------------------------------
 * RMS norm with a learned weight: the two normalisation layers of a Hymba
 * block (Hymba blog, "Hymba 的整体架构": a block normalises its input before
 * the hybrid-head module and again before the feed-forward network).
 *   out[r, :] = x[r, :] / sqrt(mean(x[r, :]^2) + eps) * w
 * x, out: [rows, width] (act dtype, out must not alias x); w: [width] f32.
 * ---------------------------------------------------------------------- */
hm_status hm_rms_norm(const void* x, const float* w, float eps, void* out, long long rows,
                      int width, hm_dtype dtype, void* stream);

/* ------------------------------------------------------------------------
 * One whole mixer layer in prefill: attention and the SSM branch
 * (hm_conv_selective_scan from zero states) on the same X~, then
 * hm_branch_norm_mean.  Width Di must equal Hq * Dh.
 * ya, ys: [B, T, Di] branch outputs (written; caller-owned, act dtype);
 * out: [B, T, Di].  conv_state_out [B, Di, K-1] and h_out [B, Di, N] (f32,
 * may be NULL) receive the final SSM-branch states for a following decode.
 * Prepared K/V: `kv` (hm_attn_kv_bytes() bytes, optional).  kv_reuse == 0:
 * k and v are prepared into kv (or into the workspace when kv is NULL);
 * kv_reuse != 0: kv already holds the K/V prepared by an earlier layer with
 * the same B, T, Hkv, Dh, rope_base and pos0 (the adjacent-layer KV sharing)
 * and k, v are not read.
 * stream2 (optional, a hipStream_t as void*): when set, the SSM branch runs on
 * it, concurrently with attention on `stream` (the two head types are
 * independent until the fusion); `stream` waits for it before the fusion.
 * Without stream2 a bf16 layer runs as three launches on `stream` in which
 * independent parts share a launch.
 * Workspace: hm_mixer_prefill_workspace() bytes, queried with the same
 * shapes, dtype and kv as the call.  Layers that run one after the other on
 * one stream may share one workspace, and a layer with kv_reuse may take its
 * kv from the workspace of the layer that prepared it.
 * SSM-branch initial states (optional, f32): conv_state_in [B, Di, K-1] (the
 * K-1 inputs x before the first row, oldest first) and h0 [B, Di, N]; NULL
 * means zeros.
 * Cached meta tokens (optional; Hymba blog, "Hymba 的整体架构": the meta tokens
 * are learned constants prepended to every input, so in a given layer their K
 * and V and the SSM-branch states after them do not depend on the prompt):
 * meta_k, meta_v [n_meta, Hkv, Dh] (act dtype, pre-RoPE, shared by the batch)
 * are the meta rows' K and V.  q, k, v, x, delta, Bm, Cm, z then hold only the
 * T real tokens, which are rows n_meta + i of X~ (positions pos0 + n_meta + i)
 * and attend to the meta rows and to each other under the usual visibility;
 * ya, ys, out are [B, T, Di]; conv_state_in and h0 should then hold the
 * states after the meta rows (as conv_state_out and h_out of a call over the
 * meta rows alone return them).  The prepared K/V (kv, or the workspace)
 * covers n_meta + T rows: hm_attn_kv_bytes(B, n_meta + T, Hkv, Dh, dtype).
 * Supported for bf16 with Dh = 64 on one stream (no stream2); otherwise
 * HM_ERR_UNSUPPORTED.
 * Timing (optional): events points to 4 caller-created hipEvent_t (as void*)
 * that the bf16 one-stream sequence records on `stream` before its first
 * launch, between the launches and after the last, so that the caller can
 * time each of the three kernels with hipEventElapsedTime; NULL entries are
 * skipped.  Other layer modes (stream2, float32) return HM_ERR_UNSUPPORTED
 * when events is set.
 * ---------------------------------------------------------------------- */
typedef struct {
  int B, T, Hq, Hkv, Dh, Di, N, K, n_meta, window;
  long long pos0;
  float rope_base, scale, eps;
  hm_dtype dtype;
  const void *q, *k, *v;                      /* [B,T,Hq,Dh], [B,T,Hkv,Dh] x2 */
  const void *x, *delta, *Bm, *Cm, *z;        /* [B,T,Di] x2, [B,T,N] x2, [B,T,Di] */
  const float *A, *D, *conv_w, *conv_b;       /* [Di,N], [Di], [Di,K], [Di] */
  const float *beta_a, *beta_s;               /* [Di] */
  void *ya, *ys, *out;                        /* [B,T,Di] each */
  float *conv_state_out, *h_out;              /* optional */
  void* kv;                                   /* optional prepared K/V */
  size_t kv_bytes;
  int kv_reuse;
  void* stream2;                              /* optional second stream */
  void* workspace;
  size_t workspace_bytes;
  const void *meta_k, *meta_v;                /* optional [n_meta, Hkv, Dh], see below */
  const float *conv_state_in, *h0;            /* optional [B, Di, K-1], [B, Di, N] */
  void* const* events;                        /* optional HOST array of 4 hipEvent_t */
} hm_prefill_args;
hm_status hm_mixer_prefill(const hm_prefill_args* a, void* stream);
size_t hm_mixer_prefill_workspace(const hm_prefill_args* a);

/* ------------------------------------------------------------------------
 * One whole Hymba block in prefill, over the hidden states of X~ (Hymba blog,
 * "Hymba 的整体架构": normalisation, hybrid-head module, normalisation,
 * feed-forward network; "数学表示" §2 and §5: in- and out-projection; model
 * card, "模型架构": FFN width 5504).  With pre-norm skip connections:
 *   u = rms_norm(h, ln1)
 *   [q, k, v, x, z] = u W_in^T        (consumer: [q, x, z]; K, V reused)
 *   [dt, B, C] = x W_dbc^T;  delta = softplus(dt + dt_bias)
 *   m = mixer(q, k, v, x, delta, B, C, z)      (as hm_mixer_prefill)
 *   h1 = h + m W_out^T
 *   h2 = h1 + W_down SiLU(W_up rms_norm(h1, ln2))
 * hidden [B, T, d_model] holds h on entry and h2 on return (in place).
 * Weights (bf16, nn.Linear layout [out, in]): w_in [Hq*Dh + 2*Hkv*Dh + 2*Di,
 * d_model] (rows Q, K, V, x, z), or [Hq*Dh + 2*Di, d_model] (rows Q, x, z)
 * when kv_reuse != 0; w_dbc [Di + 2*N, Di] (rows dt, B, C); w_out [d_model,
 * Di]; w_up [d_ffn, d_model]; w_down [d_model, d_ffn].  f32 vectors: ln1, ln2
 * [d_model]; dt_bias [Di]; A, D, conv_w, conv_b, beta_a, beta_s as for
 * hm_mixer_prefill.  eps is used by all four RMS norms.
 * Prepared K/V (the adjacent-layer sharing): kv_reuse == 0 prepares this
 * block's K, V into kv (hm_attn_kv_bytes(B, T, Hkv, Dh, dtype) bytes; NULL:
 * into the workspace); kv_reuse != 0 attends over kv as an earlier block
 * with the same B, T, Hkv, Dh, rope_base and pos0 left it.
 * Supported: bf16, Dh = 64, N = 16, K = 4, d_model and d_ffn multiples of 64
 * (else HM_ERR_UNSUPPORTED).  Workspace: hm_block_prefill_workspace() bytes
 * (the block's intermediate activations and the mixer's workspace); blocks
 * that run one after the other on one stream may share it.  Launches: two
 * norms, five matrix products and the mixer's three, all on `stream`.
 * ---------------------------------------------------------------------- */
typedef struct {
  int B, T, d_model, d_ffn, Hq, Hkv, Dh, Di, N, K, n_meta, window;
  long long pos0;
  float rope_base, scale, eps;
  hm_dtype dtype;
  void* hidden;                               /* [B, T, d_model] in/out */
  const float *ln1, *ln2;                     /* [d_model] */
  const void *w_in, *w_dbc;                   /* see above */
  const float* dt_bias;                       /* [Di] */
  const float *A, *D, *conv_w, *conv_b;       /* [Di,N], [Di], [Di,K], [Di] */
  const float *beta_a, *beta_s;               /* [Di] */
  const void *w_out, *w_up, *w_down;          /* see above */
  void* kv;                                   /* prepared K/V, see above */
  size_t kv_bytes;
  int kv_reuse;
  void* workspace;
  size_t workspace_bytes;
} hm_block_args;
hm_status hm_block_prefill(const hm_block_args* a, void* stream);
size_t hm_block_prefill_workspace(const hm_block_args* a);

/* ------------------------------------------------------------------------
 * One decode token per sequence through ONE layer of an adjacent pair that
 * shares k_cache / v_cache (Hymba blog, Hymba 的整体架构: adjacent blocks share
 * one KV cache; model card 模型使用: generation with use_cache).
 *
 * The token sits at position p = n_meta + n_prev (same n_prev for the whole
 * batch).  Cache rows per sequence: 0..n_meta-1 meta tokens, then cache_slots
 * ring slots (window > 0: the token after n_prev earlier ones lives in slot
 * n_meta + n_prev mod window; window <= 0: slot n_meta + n_prev).  K in the
 * cache is already rotated.
 *   producer (k_new, v_new != NULL): rotate k_new at p and write k_new/v_new
 *     to the token's slot, then attend;
 *   consumer (k_new == v_new == NULL): attend only.
 * Visible rows: the meta rows and the slots of the last min(n_prev+1, window)
 * tokens (all n_prev+1 for window <= 0).  conv_state and ssm_state advance by
 * one token in place; out = branch norm-and-average of the two branches.
 * Optional ya_out / ys_out ([B, Di] f32) receive the branch outputs.
 * Ragged batches: n_prev_seq (device int32 [B], optional) gives each sequence
 * its own n_prev, hence its own position, slot and visible rows; n_prev must
 * then be at least every entry (it sizes the key splits), and entries outside
 * [0, n_prev] are clamped into it.  NULL: every sequence is at n_prev.
 * Supported: bf16 with Dh = 64 (MFMA), f32 with Dh in {16, 32, 64}; N = 16; K = 4.
 * Workspace: hm_mixer_step_workspace() bytes (per-split partials and the SSM
 * branch output).  Calls that share a workspace must not overlap (stream-
 * ordered calls are fine).
 * ---------------------------------------------------------------------- */
typedef struct {
  int B, Hq, Hkv, Dh, Di, N, K, n_meta, window, cache_slots;
  long long n_prev;
  float rope_base, scale, eps;
  hm_dtype dtype;
  const void *q, *k_new, *v_new;           /* [B,Hq,Dh], [B,Hkv,Dh], [B,Hkv,Dh] */
  void *k_cache, *v_cache;                 /* [B, n_meta+cache_slots, Hkv, Dh] */
  const void *x, *delta, *Bm, *Cm, *z;     /* [B,Di], [B,Di], [B,N], [B,N], [B,Di] */
  const float *A, *D, *conv_w, *conv_b;    /* [Di,N], [Di], [Di,K], [Di] */
  float *conv_state, *ssm_state;           /* [B,Di,K-1], [B,Di,N]   in/out */
  const float *beta_a, *beta_s;            /* [Di] */
  void* out;                               /* [B, Di] (Di == Hq * Dh) */
  void* workspace;
  size_t workspace_bytes;
  /* optional fields after the contract's prefix (NULL: unused) */
  float *ya_out, *ys_out;                  /* [B, Di] f32 branch outputs */
  const int* n_prev_seq;                   /* [B] device int32, see above */
} hm_step_args;
hm_status hm_mixer_step(const hm_step_args* a, void* stream);
size_t hm_mixer_step_workspace(const hm_step_args* a);

/* ------------------------------------------------------------------------
 * hm_mixer_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and results as hm_mixer_step, with the scratch memory
 * taken from a static device array inside the library (one per GPU, held
 * until the process ends) instead of a->workspace, which is not read.  The
 * caller still passes every input and output.  The call allocates nothing.
 * Limit: hm_mixer_step_workspace(a) must not exceed
 * hm_mixer_step_noalloc_max_bytes() (8 MiB; the 64-sequence decode pair with
 * a 1152-row cache needs 1.3 MB), else HM_ERR_UNSUPPORTED and nothing runs.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that may overlap on one GPU (different streams without
 * ordering, several host threads) race and must not be used; calls ordered
 * on one stream are fine.  No part of the array needs clearing between calls.
 * The array is that of the calling thread's current device: a non-NULL
 * `stream` of another device is rejected (HM_ERR_INVALID, nothing runs).
 * ---------------------------------------------------------------------- */
hm_status hm_mixer_step_noalloc(const hm_step_args* a, void* stream);
size_t hm_mixer_step_noalloc_max_bytes(void);

/* ------------------------------------------------------------------------
 * Index exports, computed by the same device predicates the kernels use.
 *   hm_debug_attn_mask: out_dev[i*T + j] = 1 if row i may attend row j (u8 [T,T]).
 *   hm_debug_tile_plan: out_dev[a*nk + c] (int32 [ceil(T/bm), ceil(T/bn)]) =
 *     0 tile skipped, 1 visited with the element mask, 2 visited unmasked,
 *     for query tiles of bm rows and key tiles of bn rows (any bm, bn > 0); the
 *     key-tile walk and classification are the attention kernel's own, and
 *     hm_debug_attn_tiles() reports the tile sizes the bf16 kernel runs with
 *     (query rows per workgroup, per wave, and keys per tile).
 *     cap = number of int32 elements available at out_dev.
 *   hm_debug_cache_slot: the decode ring slot of a token after n_prev earlier
 *     ones (-1 if n_prev < 0), evaluated on the host by the same
 *     host-and-device function the decode kernels call.
 *   hm_debug_step_positions: the decode kernels' per-sequence positions,
 *     computed on the device by their own function: out_dev (int64 [B, 3],
 *     device) receives for sequence b its cache slot, its number of visible
 *     cache rows and its position, exactly as hm_mixer_step uses them for
 *     the same n_prev, n_prev_seq (device int32 [B] or NULL), n_meta and
 *     window (window <= 0: global).  HM_ERR_INVALID for B <= 0, n_prev < 0,
 *     n_meta < 0 or out_dev NULL.
 * ---------------------------------------------------------------------- */
hm_status hm_debug_attn_mask(int T, int n_meta, int window, unsigned char* out_dev,
                             void* stream);
hm_status hm_debug_tile_plan(int T, int n_meta, int window, int bm, int bn,
                             int* out_dev, int cap, void* stream);
void hm_debug_attn_tiles(int* bm_workgroup, int* bm_wave, int* bn);
long long hm_debug_cache_slot(long long n_prev, int n_meta, int window);
hm_status hm_debug_step_positions(int B, long long n_prev, const int* n_prev_seq,
                                  int n_meta, int window, long long* out_dev, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* HM_H_ */
