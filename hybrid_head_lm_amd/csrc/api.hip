// libhm host layer: status strings, thread-local error text, and the one-call
// mixer-layer prefill that chains attention, the SSM branch and the fusion
// (Hymba blog, "数学表示" §6: both head types run on the same X~, then their
// normalised outputs are averaged).
#include <string>

#include "hm_common.h"

namespace hm {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

hm_status fail(hm_status s, const std::string& msg) {
  g_last_error = std::string(hm_status_string(s)) + ": " + msg;
  return s;
}

// Order a second stream after the first (fork) or the first after the second
// (join) with one cached event per device and direction.  No host
// synchronisation; the events are created once per thread and device.
hm_status fork_join(hipStream_t main, hipStream_t side, bool fork) {
  struct Ev { int dev = -1; hipEvent_t e[2] = {nullptr, nullptr}; };
  static thread_local Ev cache[16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16)
    return fail(HM_ERR_HIP, "hipGetDevice failed or device index >= 16");
  Ev& c = cache[dev];
  if (c.dev != dev) {
    for (int i = 0; i < 2; ++i)
      if (hipEventCreateWithFlags(&c.e[i], hipEventDisableTiming) != hipSuccess)
        return fail(HM_ERR_HIP, "hipEventCreateWithFlags failed");
    c.dev = dev;
  }
  hipEvent_t e = c.e[fork ? 0 : 1];
  hipStream_t from = fork ? main : side, to = fork ? side : main;
  if (hipEventRecord(e, from) != hipSuccess || hipStreamWaitEvent(to, e, 0) != hipSuccess)
    return fail(HM_ERR_HIP, "event record / stream wait failed");
  return HM_OK;
}

hm_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(HM_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return HM_OK;
}

}  // namespace hm

extern "C" {

int hm_abi_version(void) { return HM_ABI_VERSION; }

const char* hm_status_string(hm_status s) {
  switch (s) {
    case HM_OK: return "HM_OK";
    case HM_ERR_INVALID: return "HM_ERR_INVALID";
    case HM_ERR_UNSUPPORTED: return "HM_ERR_UNSUPPORTED";
    case HM_ERR_WORKSPACE: return "HM_ERR_WORKSPACE";
    case HM_ERR_HIP: return "HM_ERR_HIP";
  }
  return "HM_ERR_UNKNOWN";
}

const char* hm_last_error(void) { return hm::g_last_error.c_str(); }

// Workspace of one prefill layer: the scan scratch, then (when the caller gives
// no kv buffer) the prepared K/V, each 256-byte aligned.
// Rows of prepared K/V: the meta rows come first when they are cached.
static int prefill_key_rows(const hm_prefill_args* a) {
  return a->T + ((a->meta_k != nullptr || a->meta_v != nullptr) ? a->n_meta : 0);
}

size_t hm_mixer_prefill_workspace(const hm_prefill_args* a) {
  if (!a) return 0;
  size_t ws = hm::align_up(hm_selective_scan_workspace(a->B, a->T, a->Di, a->N), 256);
  if (a->kv == nullptr)
    ws += hm::align_up(hm_attn_kv_bytes(a->B, prefill_key_rows(a), a->Hkv, a->Dh, a->dtype), 256);
  return ws;
}

}  // extern "C"

namespace hm {

// dry_only: validate every part and launch nothing.
hm_status mixer_prefill_impl(const hm_prefill_args* a, hipStream_t stream, bool dry_only) {
  HM_REQUIRE(a != nullptr, HM_ERR_INVALID, "args is NULL");
  HM_REQUIRE(a->Di == a->Hq * a->Dh, HM_ERR_INVALID, "Di must equal Hq * Dh");
  HM_PTR(a->ya);
  HM_PTR(a->ys);
  HM_PTR(a->out);
  HM_REQUIRE(a->ya != a->ys && a->ya != a->out && a->ys != a->out, HM_ERR_INVALID,
             "ya, ys and out must be distinct buffers");
  HM_REQUIRE(!a->kv_reuse || a->kv != nullptr, HM_ERR_INVALID, "kv_reuse needs a kv buffer");
  if (a->events != nullptr) {
    HM_REQUIRE(hm::prefill_fusable(a), HM_ERR_UNSUPPORTED,
               "timing events are recorded by the bf16 one-stream launch sequence only");
  }
  const bool cached_meta = a->meta_k != nullptr || a->meta_v != nullptr;
  if (cached_meta) {
    HM_PTR(a->meta_k);
    HM_PTR(a->meta_v);
    HM_REQUIRE(a->n_meta > 0, HM_ERR_INVALID, "cached meta tokens need n_meta > 0");
    HM_REQUIRE(hm::prefill_fusable(a), HM_ERR_UNSUPPORTED,
               "cached meta tokens need bf16, Dh = 64, N = 16, K = 4, a width that is a "
               "multiple of 8, 16-byte aligned rows and no stream2");
  }
  const int Tk = prefill_key_rows(a);   // key rows (prepared K/V)
  const size_t need = hm_mixer_prefill_workspace(a);
  HM_REQUIRE(a->workspace != nullptr && a->workspace_bytes >= need && hm::aligned16(a->workspace),
             HM_ERR_WORKSPACE, "workspace smaller than hm_mixer_prefill_workspace()");
  const size_t wscan = hm::align_up(hm_selective_scan_workspace(a->B, a->T, a->Di, a->N), 256);
  char* ws = (char*)a->workspace;
  void* kv = a->kv ? a->kv : (void*)(ws + wscan);
  const size_t kvb = a->kv ? a->kv_bytes : a->workspace_bytes - wscan;
  hipStream_t st = stream;
  hipStream_t st2 = a->stream2 ? (hipStream_t)a->stream2 : st;
  HM_REQUIRE(st2 != st || a->stream2 == nullptr, HM_ERR_INVALID, "stream2 must differ from stream");
  // Validate all parts before the first launch, so that a failure leaves
  // every output untouched.  bf16 layers on one stream then run the fused
  // launch sequence; the others run the parts one by one.
  for (int pass = 0; pass < (dry_only ? 1 : 2); ++pass) {
    const bool dry = pass == 0;
    hm_status s;
    if (!dry && hm::prefill_fusable(a)) return hm::prefill_fused_bf16(a, kv, ws, st);
    if (!dry && st2 != st) {
      s = hm::fork_join(st, st2, /*fork=*/true);
      if (s != HM_OK) return s;
    }
    // (with cached meta tokens only the fused path runs; the parts are then
    // validated against the key rows, which include the meta rows)
    if (!a->kv_reuse) {
      s = hm::attn_kv_prepare_impl(a->k, a->v, kv, kvb, a->B, Tk, a->Hkv, a->Dh, a->rope_base,
                                   a->pos0, a->dtype, st, dry);
      if (s != HM_OK) return s;
    }
    s = hm::attn_with_kv_impl(a->q, kv, kvb, a->ya, a->B, Tk, a->Hq, a->Hkv, a->Dh, a->n_meta,
                              a->window, a->rope_base, a->pos0, a->scale, a->dtype, st, dry);
    if (s != HM_OK) return s;
    s = hm::conv_scan_impl(a->x, a->conv_w, a->conv_b, a->conv_state_in, a->conv_state_out,
                           a->delta, a->A, a->Bm, a->Cm, a->D, a->z, a->h0, a->ys, a->h_out,
                           a->B, a->T, a->Di, a->K, a->N, a->dtype, ws, wscan, st2,
                           /*fuse_conv=*/true, dry);
    if (s != HM_OK) return s;
    if (!dry && st2 != st) {
      s = hm::fork_join(st, st2, /*fork=*/false);
      if (s != HM_OK) return s;
    }
    s = hm::norm_mean_impl(a->ya, a->ys, a->beta_a, a->beta_s, a->eps, a->out,
                           (long long)a->B * a->T, a->Di, a->dtype, st, dry);
    if (s != HM_OK) return s;
  }
  return HM_OK;
}

}  // namespace hm

extern "C" {

hm_status hm_mixer_prefill(const hm_prefill_args* a, void* stream) {
  return hm::mixer_prefill_impl(a, (hipStream_t)stream, false);
}

}  // extern "C"
