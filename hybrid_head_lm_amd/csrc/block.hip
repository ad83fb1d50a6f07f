// One whole Hymba block in prefill (Hymba blog, juejin.cn "NVIDIA提出Hymba网络",
// "Hymba 的整体架构": a normalisation layer, the hybrid-head module, a second
// normalisation layer and a feed-forward network; "数学表示" §2 and §5: the in-
// and out-projections around the heads; Hymba-1.5B-Base model card, "模型架构":
// FFN width 5504).  Pre-norm skip connections:
//   h1 = h + W_out mixer(rms_norm(h, ln1)),  h2 = h1 + W_down SiLU(W_up rms_norm(h1, ln2)).
// The SSM step sizes and B, C come from the SSM input x by one more projection
// (Delta = softplus(x W_dt^T + dt_bias)), because Eq. (2) indexes them by time.
//
// Host code only: the block is a fixed sequence of launches on one stream,
// every one of them a kernel of this library (the RMS norm, the bf16 MFMA
// projection with its epilogues, and the mixer's fused launches).  Both skip
// connections are the epilogues of the out- and down-projections, which add
// their product to the hidden state in place.
#include <algorithm>

#include "hm_common.h"

namespace {

// Byte offsets of the block's intermediate tensors in the workspace (each
// 256-byte aligned).  The FFN's hidden layer reuses q .. ys, which are dead
// once the mixer has run, when it fits there.
struct BlockLayout {
  size_t hn, q, k, v, x, z, dt, bm, cm, ya, ys, mo, u, mix, total;
};

size_t rows_bytes(long long rows, int width) {
  return hm::align_up((size_t)rows * (size_t)width * 2, 256);
}

// The mixer's arguments inside the block; with ws == nullptr only the fields
// that size its workspace (shapes, dtype, kv) are set.
hm_prefill_args mixer_args(const hm_block_args* a, const BlockLayout& L, char* ws) {
  hm_prefill_args p{};
  p.B = a->B;
  p.T = a->T;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.Dh = a->Dh;
  p.Di = a->Di;
  p.N = a->N;
  p.K = a->K;
  p.n_meta = a->n_meta;
  p.window = a->window;
  p.pos0 = a->pos0;
  p.rope_base = a->rope_base;
  p.scale = a->scale;
  p.eps = a->eps;
  p.dtype = a->dtype;
  p.kv = a->kv;
  p.kv_bytes = a->kv_bytes;
  p.kv_reuse = a->kv_reuse;
  if (ws == nullptr) return p;
  p.q = ws + L.q;
  p.k = ws + L.k;
  p.v = ws + L.v;
  p.x = ws + L.x;
  p.delta = ws + L.dt;
  p.Bm = ws + L.bm;
  p.Cm = ws + L.cm;
  p.z = ws + L.z;
  p.A = a->A;
  p.D = a->D;
  p.conv_w = a->conv_w;
  p.conv_b = a->conv_b;
  p.beta_a = a->beta_a;
  p.beta_s = a->beta_s;
  p.ya = ws + L.ya;
  p.ys = ws + L.ys;
  p.out = ws + L.mo;
  p.workspace = ws + L.mix;
  p.workspace_bytes = L.total > L.mix ? L.total - L.mix : 0;
  return p;
}

BlockLayout block_layout(const hm_block_args* a) {
  const long long R = (long long)a->B * a->T;
  BlockLayout L{};
  size_t o = 0;
  auto take = [&](int width) {
    const size_t at = o;
    o += rows_bytes(R, width);
    return at;
  };
  L.hn = take(a->d_model);
  L.q = take(a->Hq * a->Dh);
  L.k = take(a->Hkv * a->Dh);
  L.v = take(a->Hkv * a->Dh);
  L.x = take(a->Di);
  L.z = take(a->Di);
  L.dt = take(a->Di);
  L.bm = take(a->N);
  L.cm = take(a->N);
  L.ya = take(a->Di);
  L.ys = take(a->Di);
  L.mo = take(a->Di);
  L.u = (L.mo - L.q >= rows_bytes(R, a->d_ffn)) ? L.q : take(a->d_ffn);
  L.mix = o;
  L.total = o;
  const hm_prefill_args p = mixer_args(a, L, nullptr);
  L.total = o + hm::align_up(hm_mixer_prefill_workspace(&p), 256);
  return L;
}

bool block_extents_ok(const hm_block_args* a) {
  return a->B > 0 && a->T > 0 && a->d_model > 0 && a->d_ffn > 0 && a->Hq > 0 && a->Hkv > 0 &&
         a->Dh > 0 && a->Di > 0 && a->N > 0 && a->K > 0;
}

}  // namespace

extern "C" {

size_t hm_block_prefill_workspace(const hm_block_args* a) {
  if (!a || !block_extents_ok(a)) return 0;
  return block_layout(a).total;
}

hm_status hm_block_prefill(const hm_block_args* a, void* stream) {
  HM_REQUIRE(a != nullptr, HM_ERR_INVALID, "args is NULL");
  HM_REQUIRE(block_extents_ok(a), HM_ERR_INVALID, "every extent must be positive");
  HM_REQUIRE(a->Di == a->Hq * a->Dh, HM_ERR_INVALID, "Di must equal Hq * Dh");
  HM_REQUIRE(a->Hq % a->Hkv == 0, HM_ERR_INVALID, "Hq must be a multiple of Hkv");
  HM_REQUIRE(a->dtype == HM_BF16 && a->Dh == 64 && a->N == 16 && a->K == 4, HM_ERR_UNSUPPORTED,
             "blocks need bf16, Dh = 64, N = 16 and K = 4");
  HM_REQUIRE(a->d_model % 64 == 0 && a->d_ffn % 64 == 0, HM_ERR_UNSUPPORTED,
             "d_model and d_ffn must be multiples of 64");
  HM_PTR(a->hidden);
  HM_PTR(a->ln1);
  HM_PTR(a->ln2);
  HM_PTR(a->w_in);
  HM_PTR(a->w_dbc);
  HM_PTR(a->dt_bias);
  HM_PTR(a->w_out);
  HM_PTR(a->w_up);
  HM_PTR(a->w_down);
  HM_REQUIRE(!a->kv_reuse || a->kv != nullptr, HM_ERR_INVALID, "kv_reuse needs a kv buffer");
  HM_REQUIRE((double)a->B * a->T * (double)std::max(a->d_ffn, a->d_model) < 2.0e9,
             HM_ERR_UNSUPPORTED, "B * T * max(d_model, d_ffn) must stay below 2e9");
  const BlockLayout L = block_layout(a);
  HM_REQUIRE(a->workspace != nullptr && hm::aligned16(a->workspace) &&
                 a->workspace_bytes >= L.total,
             HM_ERR_WORKSPACE, "workspace smaller than hm_block_prefill_workspace()");
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)a->workspace;
  const int R = a->B * a->T;
  const int Qw = a->Hq * a->Dh, KVw = a->Hkv * a->Dh, Di = a->Di;
  void* hn = ws + L.hn;
  void* u = ws + L.u;
  void* mo = ws + L.mo;
  const hm_prefill_args pa = mixer_args(a, L, ws);

  // in-projection: rows Q, K, V, x, z (a block reusing K, V: Q, x, z)
  void* in_outs[5];
  int in_cols[5];
  int n_in = 0;
  auto seg = [&](void* p, int w) {
    in_outs[n_in] = p;
    in_cols[n_in++] = w;
  };
  seg(ws + L.q, Qw);
  if (!a->kv_reuse) {
    seg(ws + L.k, KVw);
    seg(ws + L.v, KVw);
  }
  seg(ws + L.x, Di);
  seg(ws + L.z, Di);
  const int n_in_rows = Qw + (a->kv_reuse ? 0 : 2 * KVw) + 2 * Di;
  // step sizes and B, C from x
  void* dbc_outs[3] = {ws + L.dt, ws + L.bm, ws + L.cm};
  const int dbc_cols[3] = {Di, a->N, a->N};
  const hm_linear_epilogue dbc_ep[3] = {{a->dt_bias, nullptr, HM_ACT_SOFTPLUS},
                                        {nullptr, nullptr, HM_ACT_NONE},
                                        {nullptr, nullptr, HM_ACT_NONE}};
  // skip connections and the FFN's hidden layer
  void* h_out[1] = {a->hidden};
  const int h_cols[1] = {a->d_model};
  const hm_linear_epilogue add_h[1] = {{nullptr, a->hidden, HM_ACT_NONE}};
  void* u_out[1] = {u};
  const int u_cols[1] = {a->d_ffn};
  const hm_linear_epilogue silu[1] = {{nullptr, nullptr, HM_ACT_SILU}};

  // Validate every step (dry), then launch them in order.
  for (int pass = 0; pass < 2; ++pass) {
    const bool dry = pass == 0;
    hm_status s;
    s = hm::rms_norm_impl(a->hidden, a->ln1, a->eps, hn, R, a->d_model, a->dtype, st, dry);
    if (s != HM_OK) return s;
    s = hm::linear_launch(hn, a->w_in, R, n_in_rows, a->d_model, n_in, in_outs, in_cols, nullptr,
                          st, dry);
    if (s != HM_OK) return s;
    s = hm::linear_launch(ws + L.x, a->w_dbc, R, Di + 2 * a->N, Di, 3, dbc_outs, dbc_cols,
                          dbc_ep, st, dry);
    if (s != HM_OK) return s;
    s = hm::mixer_prefill_impl(&pa, st, dry);
    if (s != HM_OK) return s;
    s = hm::linear_launch(mo, a->w_out, R, a->d_model, Di, 1, h_out, h_cols, add_h, st, dry);
    if (s != HM_OK) return s;
    s = hm::rms_norm_impl(a->hidden, a->ln2, a->eps, hn, R, a->d_model, a->dtype, st, dry);
    if (s != HM_OK) return s;
    s = hm::linear_launch(hn, a->w_up, R, a->d_ffn, a->d_model, 1, u_out, u_cols, silu, st, dry);
    if (s != HM_OK) return s;
    s = hm::linear_launch(u, a->w_down, R, a->d_model, a->d_ffn, 1, h_out, h_cols, add_h, st,
                          dry);
    if (s != HM_OK) return s;
  }
  return HM_OK;
}

}  // extern "C"
