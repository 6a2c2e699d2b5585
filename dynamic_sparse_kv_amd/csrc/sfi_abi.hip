// C ABI of libsfi: argument validation, workspace carving, launch planning.
// The contract of every entry point is documented in include/sfi.h.
#include "sfi.h"

#include <string.h>

#include <algorithm>
#include <mutex>

#include "sfi_internal.hpp"

// Library-owned scratch of sfi_fast_step_noalloc: the split partials of one
// call live here instead of in a caller workspace.  Each GPU the library runs
// on holds its own copy (module globals are per device) until the process
// ends.  Host code never passes this name to a kernel or a copy: on the host
// it is only a stand-in for the symbol; the device address comes from
// hipGetSymbolAddress (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[SFI_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace sfi;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool supported_group(int G) { return G == 1 || G == 2 || G == 4 || G == 5 || G == 8; }

// Validates the cache description; on success fills the device view.
bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool aligned16(const void *p) { return aligned(p, 16); }

sfi_status check_kv(const sfi_kv *kv, KVView *view, bool *paged) {
  if (!kv) return SFI_ERR_NULL;
  if (!kv->k || !kv->v || !kv->seq_len) return SFI_ERR_NULL;
  if (!aligned16(kv->k) || !aligned16(kv->v)) return SFI_ERR_RANGE;
  if (kv->B < 1 || kv->Hq < 1 || kv->Hkv < 1 || kv->Hq % kv->Hkv != 0) return SFI_ERR_SHAPE;
  if (kv->d != 64 && kv->d != 128) return SFI_ERR_UNSUPPORTED;
  if (!supported_group(kv->Hq / kv->Hkv)) return SFI_ERR_UNSUPPORTED;
  if (kv->max_seq_len < 1) return SFI_ERR_RANGE;
  if ((kv->k_new == nullptr) != (kv->v_new == nullptr)) return SFI_ERR_NULL;
  if (kv->k_new && (!aligned16(kv->k_new) || !aligned16(kv->v_new))) return SFI_ERR_RANGE;
  view->k = kv->k;
  view->v = kv->v;
  if (kv->norm_stats && !aligned(kv->norm_stats, 8)) return SFI_ERR_RANGE;
  view->k_new = kv->k_new;
  view->v_new = kv->v_new;
  view->nstat = kv->norm_stats;
  view->Hkv = kv->Hkv;
  view->page_table = kv->page_table;
  if (kv->page_table) {
    const int ps = kv->page_size;
    if (ps < 16 || ps > 1024 || (ps & (ps - 1)) != 0) return SFI_ERR_RANGE;
    if (kv->max_pages < 1 || kv->num_pages < 1) return SFI_ERR_SHAPE;
    if ((long long)kv->max_seq_len > (long long)kv->max_pages * ps) return SFI_ERR_RANGE;
    // a decode chunk's pages are staged in LDS: chunks of at most
    // kMaxSlowChunk rows, which the split plans guarantee up to this length
    if ((long long)kv->max_seq_len > (long long)kMaxSplits * kMaxSlowChunk) return SFI_ERR_UNSUPPORTED;
    int sh = 0;
    while ((1 << sh) < ps) ++sh;
    view->page_shift = sh;
    view->max_pages = kv->max_pages;
    view->num_pages = kv->num_pages;
    view->cap = 0;
    *paged = true;
  } else {
    if (kv->cap < 1) return SFI_ERR_SHAPE;
    if (kv->max_seq_len > kv->cap) return SFI_ERR_RANGE;
    view->page_shift = 0;
    view->max_pages = 0;
    view->num_pages = 0;
    view->cap = kv->cap;
    *paged = false;
  }
  return SFI_OK;
}

sfi_status check_batch(const sfi_kv *kv, int32_t batch_n) {
  if (batch_n < 0 || batch_n > kv->B) return SFI_ERR_RANGE;
  return SFI_OK;
}

struct SlowWs {
  size_t o, ml, logits, norms, total;
  int stride;
};

SlowWs slow_ws(const sfi_kv *kv) {
  SlowWs w{};
  w.stride = split_stride(kv->max_seq_len);
  const size_t rows = (size_t)kv->B * kv->Hq * w.stride;
  w.o = 0;
  w.ml = align_up(w.o + rows * kv->d * sizeof(float));
  w.logits = align_up(w.ml + rows * 2 * sizeof(float));
  // key norms of an evidence-mode step whose caller passes no key_norm
  w.norms = align_up(w.logits + (size_t)kv->B * kv->Hq * kv->max_seq_len * sizeof(float));
  w.total = align_up(w.norms + (size_t)kv->B * kv->Hkv * kv->max_seq_len * sizeof(float));
  return w;
}

struct FastWs {
  size_t o, ml, total;
  int stride;
};

FastWs fast_ws(const sfi_kv *kv, int sel_k, int n_sink, int window) {
  FastWs w{};
  const long long L = (long long)std::min(n_sink, kv->max_seq_len) +
                      std::min(window, kv->max_seq_len) + sel_k;
  w.stride = split_stride(L);
  const size_t rows = (size_t)kv->B * kv->Hq * w.stride;
  w.o = 0;
  w.ml = align_up(rows * kv->d * sizeof(float));
  w.total = align_up(w.ml + rows * 2 * sizeof(float));
  return w;
}

struct SelWs {
  int P, ld32;
  size_t ghist, cum, sorted, nsum, wsum, meta, ecnt, ebits, eghist, total;
};

// Prior workspace of the calls that form the selector's prior (fp64): the
// per-split key-norm sums [B*Hkv][stride][2], the per-split prior-weight
// sums [B*Hkv][stride] and the updated key-norm statistics [B*Hkv][2].
size_t prior_ws_bytes(const sfi_kv *kv, int stride) {
  return align_up((size_t)kv->B * kv->Hkv * (stride * 3 + 2) * sizeof(double));
}

SelWs select_ws(int B, int H, int max_seq_len) {
  SelWs w{};
  const size_t rows = (size_t)B * H;
  w.P = (max_seq_len + kSelChunk - 1) / kSelChunk;
  w.ghist = 0;
  w.cum = align_up(w.ghist + rows * 4096 * sizeof(uint32_t));
  w.sorted = align_up(w.cum + rows * w.P * 4096 * sizeof(uint16_t));
  w.nsum = align_up(w.sorted + rows * w.P * kSelChunk * sizeof(unsigned long long));
  w.wsum = align_up(w.nsum + rows * w.P * 2 * sizeof(double));
  w.meta = align_up(w.wsum + rows * w.P * sizeof(double));
  // cross-head exclusivity: per-key row counts and per-row membership bits
  // over whole chunks, and the second round's row histograms
  w.ld32 = w.P * (kSelChunk / 32);
  w.ecnt = align_up(w.meta + rows * sizeof(SelRowMeta));
  w.ebits = align_up(w.ecnt + (size_t)B * w.ld32 * 32 * sizeof(uint32_t));
  w.eghist = align_up(w.ebits + rows * w.ld32 * sizeof(uint32_t));
  w.total = align_up(w.eghist + rows * 4096 * sizeof(uint32_t));
  return w;
}

struct VerWs {
  size_t o, ml, agg, total;
  int stride, chunk;
};

// Observation-window slow step: the verify partials, then per-row stats.
struct WinWs {
  size_t o, ml, rstat, total;
  int stride, chunk;
};

WinWs window_ws(const sfi_kv *kv, int w) {
  WinWs x{};
  x.chunk = verify_chunk_for(kv->B, kv->Hkv, kv->max_seq_len, kv->d, kv->Hq / kv->Hkv);
  x.stride = verify_stride_for(kv->max_seq_len, x.chunk);
  const size_t rows = (size_t)kv->B * w * kv->Hq * x.stride;
  x.o = 0;
  x.ml = align_up(rows * kv->d * sizeof(float));
  x.rstat = align_up(x.ml + rows * 2 * sizeof(float));
  x.total = align_up(x.rstat + (size_t)kv->B * w * kv->Hq * 2 * sizeof(float));
  return x;
}

VerWs verify_ws(const sfi_kv *kv, int T) {
  VerWs w{};
  w.chunk = verify_chunk_for(kv->B, kv->Hkv, kv->max_seq_len, kv->d, kv->Hq / kv->Hkv);
  w.stride = verify_stride_for(kv->max_seq_len, w.chunk);
  const size_t rows = (size_t)kv->B * T * kv->Hq * w.stride;
  w.o = 0;
  w.ml = align_up(rows * kv->d * sizeof(float));
  w.agg = align_up(w.ml + rows * 2 * sizeof(float));
  w.total = align_up(w.agg + (size_t)kv->B * kv->Hkv * kv->max_seq_len * sizeof(float));
  return w;
}

template <typename T>
T *carve(void *ws, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

// Validated launch description of a selection (nothing is launched).
sfi_status select_launch(const sfi_select_params *p, const int32_t *batch_ids, int32_t batch_n,
                         const int32_t *seq_len, int32_t B, int32_t H, int32_t max_seq_len,
                         const float *score, const float *key_norm, int32_t ld, int32_t *sel_idx,
                         int32_t *sel_count, float *fused_out, void *ws, size_t ws_bytes,
                         bool prior_done, SelectLaunch *out) {
  if (!p || !seq_len || !score || !sel_idx || !sel_count) return SFI_ERR_NULL;
  if (p->mode != SFI_SCORE_FUSED && p->mode != SFI_SCORE_RAW) return SFI_ERR_RANGE;
  if (B < 1 || H < 1 || max_seq_len < 1) return SFI_ERR_SHAPE;
  if (max_seq_len > kSelMaxLen) return SFI_ERR_UNSUPPORTED;
  if (batch_n < 0 || batch_n > B) return SFI_ERR_RANGE;
  if (ld < max_seq_len) return SFI_ERR_RANGE;
  if (p->k < 1 || p->n_sink < 0 || p->window < 0) return SFI_ERR_RANGE;
  if (p->nms_radius < 0 || p->nms_radius > kNmsMaxRadius) return SFI_ERR_RANGE;
  if (!(p->nms_alpha >= 0.f && p->nms_alpha < 1.f) || !(p->excl_beta >= 0.f && p->excl_beta < 1.f))
    return SFI_ERR_RANGE;
  const bool fused = p->mode == SFI_SCORE_FUSED;
  if (fused) {
    if (!key_norm) return SFI_ERR_NULL;
    if (!(p->lambda >= 0.f && p->lambda <= 1.f)) return SFI_ERR_RANGE;
    if (!(p->pos_tau > 0.f) || !(p->norm_coef == p->norm_coef)) return SFI_ERR_RANGE;
  }
  const SelWs w = select_ws(B, H, max_seq_len);
  if (!ws) return SFI_ERR_NULL;
  if (!aligned(ws, kAlign)) return SFI_ERR_RANGE;
  if (ws_bytes < w.total) return SFI_ERR_WORKSPACE;

  SelectLaunch &a = *out;
  a = SelectLaunch{};
  a.mode = p->mode;
  a.lambda = p->lambda; a.norm_coef = p->norm_coef; a.pos_tau = p->pos_tau;
  a.n_sink = p->n_sink; a.window = p->window; a.k = p->k;
  a.k_seq = p->k_per_seq;
  a.batch_ids = batch_ids; a.batch_n = batch_n; a.seq_len = seq_len;
  a.B = B; a.H = H; a.max_seq_len = max_seq_len;
  a.score = score; a.key_norm = key_norm; a.ld = ld;
  a.sel_idx = sel_idx; a.sel_count = sel_count;
  a.fused_out = fused ? fused_out : nullptr;
  a.fo_ld = ld;
  a.prior_done = prior_done;
  a.nms_radius = (p->nms_alpha > 0.f) ? p->nms_radius : 0;
  a.nms_alpha = p->nms_alpha;
  a.excl_beta = (H > 1) ? p->excl_beta : 0.f;
  a.excl_cnt = carve<uint32_t>(ws, w.ecnt);
  a.excl_bits = carve<uint32_t>(ws, w.ebits);
  a.excl_ghist = carve<uint32_t>(ws, w.eghist);
  a.ld32 = w.ld32;
  a.ws.P = w.P;
  a.ws.ghist = carve<uint32_t>(ws, w.ghist);
  a.ws.cum = carve<uint16_t>(ws, w.cum);
  a.ws.sorted = carve<unsigned long long>(ws, w.sorted);
  a.ws.nsum = carve<double>(ws, w.nsum);
  a.ws.wsum = carve<double>(ws, w.wsum);
  a.ws.meta = carve<SelRowMeta>(ws, w.meta);
  return SFI_OK;
}

sfi_status select_impl(const sfi_select_params *p, const int32_t *batch_ids, int32_t batch_n,
                      const int32_t *seq_len, int32_t B, int32_t H, int32_t max_seq_len,
                      const float *score, const float *key_norm, int32_t ld, int32_t *sel_idx,
                      int32_t *sel_count, float *fused_out, void *ws, size_t ws_bytes,
                      void *stream, bool prior_done) {
  SelectLaunch a;
  const sfi_status s = select_launch(p, batch_ids, batch_n, seq_len, B, H, max_seq_len, score, key_norm,
                                     ld, sel_idx, sel_count, fused_out, ws, ws_bytes, prior_done, &a);
  if (s != SFI_OK || batch_n == 0) return s;
  return launch_select(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SFI_OK : SFI_ERR_HIP;
}

// Launch description of a deferred selection (its slow step formed the prior).
sfi_status deferred_launch(const sfi_deferred *d, SelectLaunch *out) {
  return select_launch(&d->params, d->batch_ids, d->batch_n, d->seq_len, d->B, d->H, d->max_seq_len,
                       d->evidence, d->key_norm, d->ld, d->sel_idx, d->sel_count, d->fused_out, d->ws,
                       d->ws_bytes, true, out);
}

AttnLaunch slow_launch(const sfi_kv *kv, const KVView &view, bool paged, const SlowWs &w, void *ws,
                       const int32_t *batch_ids, int32_t batch_n, const uint16_t *q, float *out,
                       float *evidence, float *key_norm, int32_t ld) {
  AttnLaunch a{};
  a.kv = view;
  a.seq_len = kv->seq_len;
  a.batch_ids = batch_ids;
  a.batch_n = batch_n;
  a.B = kv->B; a.Hq = kv->Hq; a.Hkv = kv->Hkv; a.d = kv->d; a.G = kv->Hq / kv->Hkv;
  a.max_len = kv->max_seq_len;
  a.paged = paged;
  a.q = q;
  a.out = out;
  a.part_o = carve<float>(ws, w.o);
  a.part_ml = carve<float>(ws, w.ml);
  a.plan.stride = w.stride;  // chunking is planned by the launcher
  a.len_host = kv->slow_len_host;
  a.logits = carve<float>(ws, w.logits);
  a.lld = kv->max_seq_len;
  a.evidence = evidence;
  a.key_norm = key_norm;
  a.ld = ld;
  a.nld = ld;
  if (evidence && !key_norm) {  // the evidence kernel always writes norms
    a.key_norm = carve<float>(ws, w.norms);
    a.nld = kv->max_seq_len;
  }
  return a;
}

AttnLaunch fast_launch(const sfi_kv *kv, const KVView &view, bool paged, const FastWs &w, void *ws,
                       const int32_t *batch_ids, int32_t batch_n, const uint16_t *q, float *out,
                       const int32_t *sel_idx, const int32_t *sel_count, int32_t sel_heads,
                       int32_t sel_k, int32_t n_sink, int32_t window) {
  AttnLaunch a{};
  a.kv = view;
  a.seq_len = kv->seq_len;
  a.batch_ids = batch_ids;
  a.batch_n = batch_n;
  a.B = kv->B; a.Hq = kv->Hq; a.Hkv = kv->Hkv; a.d = kv->d; a.G = kv->Hq / kv->Hkv;
  a.max_len = kv->max_seq_len;
  a.paged = paged;
  a.q = q;
  a.out = out;
  a.part_o = carve<float>(ws, w.o);
  a.part_ml = carve<float>(ws, w.ml);
  a.plan.stride = w.stride;  // chunking is planned by the launcher
  a.len_host = kv->fast_len_host;
  a.sel_idx = sel_idx;
  a.sel_count = sel_count;
  a.sel_heads = sel_heads;
  a.sel_k = sel_k;
  a.n_sink = n_sink;
  a.window = window;
  return a;
}

// Device address of `scratch` on the current device, resolved once per
// device with that device current and cached.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

sfi_status noalloc_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SFI_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SFI_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SFI_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SFI_OK;
}

sfi_status check_fast(const sfi_kv *kv, const int32_t *sel_idx, const int32_t *sel_count,
                      int32_t sel_heads, int32_t sel_k, int32_t n_sink, int32_t window) {
  if (!sel_count) return SFI_ERR_NULL;
  if (sel_k < 0 || n_sink < 0 || window < 0) return SFI_ERR_RANGE;
  if (sel_k > 0 && !sel_idx) return SFI_ERR_NULL;
  if (sel_heads != 1 && sel_heads != kv->Hkv) return SFI_ERR_SHAPE;
  return SFI_OK;
}

// The host row-count hints of a call's lists (sfi_kv::slow_len_host and
// fast_len_host), read for the entries the call lists.
sfi_status check_hints(const sfi_kv *kv, int32_t n_slow, int32_t n_fast, long long fast_max) {
  if (kv->slow_len_host)
    for (int32_t z = 0; z < n_slow; ++z)
      if (kv->slow_len_host[z] < 0 || kv->slow_len_host[z] > kv->max_seq_len) return SFI_ERR_RANGE;
  if (kv->fast_len_host)
    for (int32_t z = 0; z < n_fast; ++z)
      if (kv->fast_len_host[z] < 0 || kv->fast_len_host[z] > fast_max) return SFI_ERR_RANGE;
  return SFI_OK;
}

}  // namespace

extern "C" {

size_t sfi_slow_workspace_bytes(const sfi_kv *kv) {
  KVView v;
  bool pg;
  if (check_kv(kv, &v, &pg) != SFI_OK) return 0;
  return slow_ws(kv).total;
}

size_t sfi_select_workspace_bytes(int32_t B, int32_t H, int32_t max_seq_len) {
  if (B < 1 || H < 1 || max_seq_len < 1 || max_seq_len > kSelMaxLen) return 0;
  return select_ws(B, H, max_seq_len).total;
}

size_t sfi_fast_workspace_bytes(const sfi_kv *kv, int32_t sel_k, int32_t n_sink, int32_t window) {
  KVView v;
  bool pg;
  if (check_kv(kv, &v, &pg) != SFI_OK || sel_k < 0 || n_sink < 0 || window < 0) return 0;
  return fast_ws(kv, sel_k, n_sink, window).total;
}

sfi_status sfi_slow_step(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                         const uint16_t *q, float *out, float *evidence, float *key_norm,
                         int32_t ld, void *ws, size_t ws_bytes, void *stream) {
  KVView view;
  bool paged = false;
  sfi_status s = check_kv(kv, &view, &paged);
  if (s != SFI_OK) return s;
  if ((s = check_batch(kv, batch_n)) != SFI_OK) return s;
  if (!q || !out) return SFI_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16)) return SFI_ERR_RANGE;
  if ((evidence || key_norm) && ld < kv->max_seq_len) return SFI_ERR_RANGE;
  if ((s = check_hints(kv, batch_n, 0, 0)) != SFI_OK) return s;
  const SlowWs w = slow_ws(kv);
  if (!ws) return SFI_ERR_NULL;
  if (!aligned(ws, kAlign)) return SFI_ERR_RANGE;
  if (ws_bytes < w.total) return SFI_ERR_WORKSPACE;
  if (batch_n == 0) return SFI_OK;
  const AttnLaunch a = slow_launch(kv, view, paged, w, ws, batch_ids, batch_n, q, out, evidence,
                                   key_norm, ld);
  return launch_slow(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SFI_OK : SFI_ERR_HIP;
}

size_t sfi_decode_step_workspace_bytes(const sfi_kv *kv, int32_t sel_k, int32_t n_sink,
                                       int32_t window) {
  KVView view;
  bool paged = false;
  if (check_kv(kv, &view, &paged) != SFI_OK || sel_k < 0 || n_sink < 0 || window < 0) return 0;
  return slow_ws(kv).total + fast_ws(kv, sel_k, n_sink, window).total;
}

sfi_status sfi_decode_step(const sfi_kv *kv, const int32_t *slow_ids, int32_t n_slow,
                           const int32_t *fast_ids, int32_t n_fast, const uint16_t *q, float *out,
                           float *evidence, float *key_norm, int32_t ld, const int32_t *sel_idx,
                           const int32_t *sel_count, int32_t sel_heads, int32_t sel_k,
                           int32_t n_sink, int32_t window, void *ws, size_t ws_bytes,
                           void *stream) {
  KVView view;
  bool paged = false;
  sfi_status s = check_kv(kv, &view, &paged);
  if (s != SFI_OK) return s;
  if ((s = check_batch(kv, n_slow)) != SFI_OK) return s;
  if ((s = check_batch(kv, n_fast)) != SFI_OK) return s;
  if (n_slow + n_fast > kv->B) return SFI_ERR_RANGE;
  if (!q || !out) return SFI_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16)) return SFI_ERR_RANGE;
  if (n_slow > 0 && !evidence) return SFI_ERR_NULL;
  if (n_slow > 0 && ld < kv->max_seq_len) return SFI_ERR_RANGE;
  if (n_fast > 0 && (s = check_fast(kv, sel_idx, sel_count, sel_heads, sel_k, n_sink, window)) != SFI_OK)
    return s;
  if (sel_k < 0 || n_sink < 0 || window < 0) return SFI_ERR_RANGE;
  if ((s = check_hints(kv, n_slow, n_fast, (long long)n_sink + window + sel_k)) != SFI_OK) return s;
  const SlowWs sw = slow_ws(kv);
  const FastWs fw = fast_ws(kv, sel_k, n_sink, window);
  if (!ws) return SFI_ERR_NULL;
  if (!aligned(ws, kAlign)) return SFI_ERR_RANGE;
  if (ws_bytes < sw.total + fw.total) return SFI_ERR_WORKSPACE;
  if (n_slow == 0 && n_fast == 0) return SFI_OK;
  void *ws_fast = static_cast<char *>(ws) + sw.total;
  const AttnLaunch sa = slow_launch(kv, view, paged, sw, ws, slow_ids, n_slow, q, out, evidence,
                                    key_norm, ld);
  const AttnLaunch fa = fast_launch(kv, view, paged, fw, ws_fast, fast_ids, n_fast, q, out, sel_idx,
                                    sel_count, sel_heads, sel_k, n_sink, window);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (n_fast == 0) e = launch_slow(sa, st);
  else if (n_slow == 0) e = launch_fast(fa, st);
  else e = launch_step(sa, fa, st);
  return e == hipSuccess ? SFI_OK : SFI_ERR_HIP;
}

size_t sfi_decode_step_select_workspace_bytes(const sfi_kv *kv, int32_t sel_k, int32_t n_sink,
                                              int32_t window) {
  KVView view;
  bool paged = false;
  if (check_kv(kv, &view, &paged) != SFI_OK || sel_k < 1 || n_sink < 0 || window < 0) return 0;
  if (kv->max_seq_len > kSelMaxLen) return 0;
  const SlowWs sw = slow_ws(kv);
  return sw.total + fast_ws(kv, sel_k, n_sink, window).total +
         select_ws(kv->B, kv->Hkv, kv->max_seq_len).total + prior_ws_bytes(kv, sw.stride);
}

sfi_status sfi_decode_step_select(const sfi_kv *kv, const sfi_select_params *p,
                                  const int32_t *slow_ids, int32_t n_slow, const int32_t *fast_ids,
                                  int32_t n_fast, const uint16_t *q, float *out, float *evidence,
                                  float *key_norm, int32_t ld, int32_t *sel_idx, int32_t *sel_count,
                                  float *fused_out, void *ws, size_t ws_bytes, void *stream) {
  KVView view;
  bool paged = false;
  sfi_status s = check_kv(kv, &view, &paged);
  if (s != SFI_OK) return s;
  if (!p) return SFI_ERR_NULL;
  if (p->mode != SFI_SCORE_FUSED) return SFI_ERR_RANGE;
  if (!(p->lambda >= 0.f && p->lambda <= 1.f)) return SFI_ERR_RANGE;
  if (!(p->pos_tau > 0.f) || !(p->norm_coef == p->norm_coef)) return SFI_ERR_RANGE;
  if (p->k < 1 || p->n_sink < 0 || p->window < 0) return SFI_ERR_RANGE;
  if (kv->max_seq_len > kSelMaxLen) return SFI_ERR_UNSUPPORTED;
  if ((s = check_batch(kv, n_slow)) != SFI_OK) return s;
  if ((s = check_batch(kv, n_fast)) != SFI_OK) return s;
  if (n_slow + n_fast > kv->B) return SFI_ERR_RANGE;
  if (!q || !out || !sel_idx || !sel_count) return SFI_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16)) return SFI_ERR_RANGE;
  if (n_slow > 0 && (!evidence || !key_norm)) return SFI_ERR_NULL;
  if (n_slow > 0 && ld < kv->max_seq_len) return SFI_ERR_RANGE;
  if (n_fast > 0 &&
      (s = check_fast(kv, sel_idx, sel_count, kv->Hkv, p->k, p->n_sink, p->window)) != SFI_OK)
    return s;
  if ((s = check_hints(kv, n_slow, n_fast, (long long)p->n_sink + p->window + p->k)) != SFI_OK) return s;
  const SlowWs sw = slow_ws(kv);
  const FastWs fw = fast_ws(kv, p->k, p->n_sink, p->window);
  const SelWs ew = select_ws(kv->B, kv->Hkv, kv->max_seq_len);
  const size_t nsum_bytes = prior_ws_bytes(kv, sw.stride);
  if (!ws) return SFI_ERR_NULL;
  if (!aligned(ws, kAlign)) return SFI_ERR_RANGE;
  if (ws_bytes < sw.total + fw.total + ew.total + nsum_bytes) return SFI_ERR_WORKSPACE;
  if (n_slow == 0 && n_fast == 0) return SFI_OK;
  char *base = static_cast<char *>(ws);
  void *ws_fast = base + sw.total;
  void *ws_sel = base + sw.total + fw.total;
  double *nsum = reinterpret_cast<double *>(base + sw.total + fw.total + ew.total);
  AttnLaunch sa = slow_launch(kv, view, paged, sw, ws, slow_ids, n_slow, q, out, evidence, key_norm, ld);
  sa.nsum = nsum;
  sa.norm_coef = p->norm_coef;
  sa.pos_tau = p->pos_tau;
  sa.sel_wsum = carve<double>(ws_sel, ew.wsum);
  sa.sel_meta = carve<SelRowMeta>(ws_sel, ew.meta);
  sa.sel_ghist = carve<uint32_t>(ws_sel, ew.ghist);
  sa.selP = ew.P;
  // the prior from the key-norm statistics: the key pass moves into the
  // step's finalize and the selection ends with its pick pass
  SelectLaunch keysel{};
  bool stats = false;
  if (n_slow > 0 && view.nstat != nullptr && kv->norm_stats_valid == 1) {
    if ((s = select_launch(p, slow_ids, n_slow, kv->seq_len, kv->B, kv->Hkv, kv->max_seq_len, evidence,
                           key_norm, ld, sel_idx, sel_count, fused_out, ws_sel, ew.total, true, &keysel)) !=
        SFI_OK)
      return s;
    stats = keysel.nms_radius == 0 && keysel.excl_beta == 0.f;  // the plain key pass only
  }
  if (stats) {
    sa.stats = true;
    sa.nsum = nullptr;
    sa.wpart = nsum + (size_t)kv->B * kv->Hkv * sw.stride * 2;
    sa.nnext = sa.wpart + (size_t)kv->B * kv->Hkv * sw.stride;
    sa.keysel = &keysel;
  }
  const AttnLaunch fa = fast_launch(kv, view, paged, fw, ws_fast, fast_ids, n_fast, q, out, sel_idx,
                                    sel_count, kv->Hkv, p->k, p->n_sink, p->window);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (n_fast == 0) e = launch_slow(sa, st);
  else if (n_slow == 0) e = launch_fast(fa, st);
  else e = launch_step(sa, fa, st);
  if (e != hipSuccess) return SFI_ERR_HIP;
  if (n_slow == 0) return SFI_OK;
  if (stats) return launch_pick(keysel, st) == hipSuccess ? SFI_OK : SFI_ERR_HIP;
  return select_impl(p, slow_ids, n_slow, kv->seq_len, kv->B, kv->Hkv, kv->max_seq_len, evidence,
                     key_norm, ld, sel_idx, sel_count, fused_out, ws_sel, ew.total, stream, true);
}

sfi_status sfi_decode_layer_step(const sfi_kv *kv, const sfi_select_params *p, const int32_t *slow_ids,
                                 int32_t n_slow, const int32_t *fast_ids, int32_t n_fast,
                                 const uint16_t *q, float *out, float *evidence, float *key_norm,
                                 int32_t ld, int32_t *sel_idx, int32_t *sel_count, float *fused_out,
                                 void *ws, size_t ws_bytes, const sfi_deferred *pending,
                                 sfi_deferred *defer, void *stream) {
  const bool pend_on = pending && pending->active;
  if (!pend_on && !defer)  // the plain combined call
    return sfi_decode_step_select(kv, p, slow_ids, n_slow, fast_ids, n_fast, q, out, evidence, key_norm,
                                  ld, sel_idx, sel_count, fused_out, ws, ws_bytes, stream);
  KVView view;
  bool paged = false;
  sfi_status s = check_kv(kv, &view, &paged);
  if (s != SFI_OK) return s;
  if (!p) return SFI_ERR_NULL;
  if (p->mode != SFI_SCORE_FUSED) return SFI_ERR_RANGE;
  // a deferred selection runs one key and one pick pass inside the next
  // layer's grids: exclusivity's second round does not fit there
  if (p->excl_beta != 0.f) return SFI_ERR_UNSUPPORTED;
  if (!(p->lambda >= 0.f && p->lambda <= 1.f)) return SFI_ERR_RANGE;
  if (!(p->pos_tau > 0.f) || !(p->norm_coef == p->norm_coef)) return SFI_ERR_RANGE;
  if (p->k < 1 || p->n_sink < 0 || p->window < 0) return SFI_ERR_RANGE;
  if (kv->max_seq_len > kSelMaxLen) return SFI_ERR_UNSUPPORTED;
  if ((s = check_batch(kv, n_slow)) != SFI_OK) return s;
  if ((s = check_batch(kv, n_fast)) != SFI_OK) return s;
  if (n_slow + n_fast > kv->B) return SFI_ERR_RANGE;
  if (!q || !out || !sel_idx || !sel_count) return SFI_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16)) return SFI_ERR_RANGE;
  if (n_slow > 0 && (!evidence || !key_norm)) return SFI_ERR_NULL;
  if (n_slow > 0 && ld < kv->max_seq_len) return SFI_ERR_RANGE;
  if (n_fast > 0 &&
      (s = check_fast(kv, sel_idx, sel_count, kv->Hkv, p->k, p->n_sink, p->window)) != SFI_OK)
    return s;
  if ((s = check_hints(kv, n_slow, n_fast, (long long)p->n_sink + p->window + p->k)) != SFI_OK) return s;
  const SlowWs sw = slow_ws(kv);
  const FastWs fw = fast_ws(kv, p->k, p->n_sink, p->window);
  const SelWs ew = select_ws(kv->B, kv->Hkv, kv->max_seq_len);
  const size_t nsum_bytes = prior_ws_bytes(kv, sw.stride);
  if (!ws) return SFI_ERR_NULL;
  if (!aligned(ws, kAlign)) return SFI_ERR_RANGE;
  if (ws_bytes < sw.total + fw.total + ew.total + nsum_bytes) return SFI_ERR_WORKSPACE;
  char *base = static_cast<char *>(ws);
  void *ws_fast = base + sw.total;
  void *ws_sel = base + sw.total + fw.total;
  SelectLaunch pend;
  if (pend_on) {
    // the pending selection belongs to other buffers (another layer's)
    if (pending->ws == ws_sel || pending->sel_idx == sel_idx || pending->evidence == evidence)
      return SFI_ERR_RANGE;
    if ((s = deferred_launch(pending, &pend)) != SFI_OK) return s;
    if (pend.mode != SFI_SCORE_FUSED) return SFI_ERR_RANGE;
    if (pend.excl_beta != 0.f) return SFI_ERR_UNSUPPORTED;
  }
  const bool pend_run = pend_on && pending->batch_n > 0;
  // this call's own selection (validated before anything is launched)
  sfi_deferred own{};
  if (n_slow > 0) {
    own.active = 1;
    own.params = *p;
    own.batch_ids = slow_ids;
    own.batch_n = n_slow;
    own.seq_len = kv->seq_len;
    own.B = kv->B;
    own.H = kv->Hkv;
    own.max_seq_len = kv->max_seq_len;
    own.evidence = evidence;
    own.key_norm = key_norm;
    own.ld = ld;
    own.sel_idx = sel_idx;
    own.sel_count = sel_count;
    own.fused_out = fused_out;
    own.ws = ws_sel;
    own.ws_bytes = ew.total;
    SelectLaunch chk;
    if ((s = deferred_launch(&own, &chk)) != SFI_OK) return s;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (n_slow + n_fast > 0 || pend_run) {
    double *nsum = reinterpret_cast<double *>(base + sw.total + fw.total + ew.total);
    AttnLaunch sa = slow_launch(kv, view, paged, sw, ws, slow_ids, n_slow, q, out, evidence, key_norm, ld);
    sa.nsum = nsum;
    sa.norm_coef = p->norm_coef;
    sa.pos_tau = p->pos_tau;
    sa.sel_wsum = carve<double>(ws_sel, ew.wsum);
    sa.sel_meta = carve<SelRowMeta>(ws_sel, ew.meta);
    sa.sel_ghist = carve<uint32_t>(ws_sel, ew.ghist);
    sa.selP = ew.P;
    const AttnLaunch fa = fast_launch(kv, view, paged, fw, ws_fast, fast_ids, n_fast, q, out, sel_idx,
                                      sel_count, kv->Hkv, p->k, p->n_sink, p->window);
    hipError_t e;
    if (pend_run) e = launch_step(sa, fa, st, &pend);
    else if (n_fast == 0) e = launch_slow(sa, st);
    else if (n_slow == 0) e = launch_fast(fa, st);
    else e = launch_step(sa, fa, st);
    if (e != hipSuccess) return SFI_ERR_HIP;
  }
  if (defer) {
    *defer = own;
    return SFI_OK;
  }
  if (n_slow == 0) return SFI_OK;
  SelectLaunch a;
  if ((s = deferred_launch(&own, &a)) != SFI_OK) return s;
  return launch_select(a, st) == hipSuccess ? SFI_OK : SFI_ERR_HIP;
}

sfi_status sfi_run_deferred(const sfi_deferred *d, void *stream) {
  if (!d) return SFI_ERR_NULL;
  if (!d->active || d->batch_n == 0) return SFI_OK;
  SelectLaunch a;
  const sfi_status s = deferred_launch(d, &a);
  if (s != SFI_OK) return s;
  if (a.mode != SFI_SCORE_FUSED) return SFI_ERR_RANGE;
  return launch_select(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SFI_OK : SFI_ERR_HIP;
}

sfi_status sfi_select(const sfi_select_params *p, const int32_t *batch_ids, int32_t batch_n,
                      const int32_t *seq_len, int32_t B, int32_t H, int32_t max_seq_len,
                      const float *score, const float *key_norm, int32_t ld, int32_t *sel_idx,
                      int32_t *sel_count, float *fused_out, void *ws, size_t ws_bytes,
                      void *stream) {
  return select_impl(p, batch_ids, batch_n, seq_len, B, H, max_seq_len, score, key_norm, ld, sel_idx,
                     sel_count, fused_out, ws, ws_bytes, stream, false);
}

sfi_status sfi_fast_step(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                         const uint16_t *q, const int32_t *sel_idx, const int32_t *sel_count,
                         int32_t sel_heads, int32_t sel_k, int32_t n_sink, int32_t window,
                         float *out, void *ws, size_t ws_bytes, void *stream) {
  KVView view;
  bool paged = false;
  sfi_status s = check_kv(kv, &view, &paged);
  if (s != SFI_OK) return s;
  if ((s = check_batch(kv, batch_n)) != SFI_OK) return s;
  if (!q || !out) return SFI_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16)) return SFI_ERR_RANGE;
  if ((s = check_fast(kv, sel_idx, sel_count, sel_heads, sel_k, n_sink, window)) != SFI_OK) return s;
  if ((s = check_hints(kv, 0, batch_n, (long long)n_sink + window + sel_k)) != SFI_OK) return s;
  const FastWs w = fast_ws(kv, sel_k, n_sink, window);
  if (!ws) return SFI_ERR_NULL;
  if (!aligned(ws, kAlign)) return SFI_ERR_RANGE;
  if (ws_bytes < w.total) return SFI_ERR_WORKSPACE;
  if (batch_n == 0) return SFI_OK;
  const AttnLaunch a = fast_launch(kv, view, paged, w, ws, batch_ids, batch_n, q, out, sel_idx,
                                   sel_count, sel_heads, sel_k, n_sink, window);
  return launch_fast(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SFI_OK : SFI_ERR_HIP;
}

sfi_status sfi_fast_step_noalloc(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                                 const uint16_t *q, const int32_t *sel_idx, const int32_t *sel_count,
                                 int32_t sel_heads, int32_t sel_k, int32_t n_sink, int32_t window,
                                 float *out, void *stream) {
  KVView view;
  bool paged = false;
  sfi_status s = check_kv(kv, &view, &paged);
  if (s != SFI_OK) return s;
  if ((s = check_batch(kv, batch_n)) != SFI_OK) return s;
  if (!q || !out) return SFI_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16)) return SFI_ERR_RANGE;
  if ((s = check_fast(kv, sel_idx, sel_count, sel_heads, sel_k, n_sink, window)) != SFI_OK) return s;
  if (batch_n == 0) return SFI_OK;
  void *ptr = nullptr;
  if ((s = noalloc_scratch(&ptr)) != SFI_OK) return s;
  // The plan of sfi_fast_step (same chunks, same bits); the partials are
  // packed by batch entry with the plan's split count as their stride.
  const FastWs wfull = fast_ws(kv, sel_k, n_sink, window);
  AttnLaunch a = fast_launch(kv, view, paged, wfull, ptr, batch_ids, batch_n, q, out, sel_idx, sel_count,
                             sel_heads, sel_k, n_sink, window);
  a.len_host = nullptr;  // planned from the bound alone, whatever the hints say
  const SplitPlan plan = plan_fast(a);
  const size_t rows = (size_t)batch_n * kv->Hq * plan.splits;
  const size_t ml = align_up(rows * kv->d * sizeof(float));
  if (ml + rows * 2 * sizeof(float) > (size_t)SFI_NOALLOC_SCRATCH_BYTES) return SFI_ERR_WORKSPACE;
  a.part_o = carve<float>(ptr, 0);
  a.part_ml = carve<float>(ptr, ml);
  a.plan = SplitPlan{plan.chunk, plan.splits, plan.splits};
  a.planned = true;
  a.part_by_entry = true;
  return launch_fast(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SFI_OK : SFI_ERR_HIP;
}

sfi_status sfi_append_kv(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                         const uint16_t *k_new, const uint16_t *v_new, int32_t T, void *stream) {
  KVView view;
  bool paged = false;
  sfi_status s = check_kv(kv, &view, &paged);
  if (s != SFI_OK) return s;
  if ((s = check_batch(kv, batch_n)) != SFI_OK) return s;
  if (T < 1 || T > kv->max_seq_len) return SFI_ERR_RANGE;
  if (view.k_new) return SFI_ERR_RANGE;  // the rows come in k_new / v_new here
  if (!k_new || !v_new) return SFI_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new)) return SFI_ERR_RANGE;
  if (batch_n == 0) return SFI_OK;
  AttnLaunch a{};
  a.kv = view;
  a.seq_len = kv->seq_len;
  a.batch_ids = batch_ids;
  a.batch_n = batch_n;
  a.B = kv->B; a.Hq = kv->Hq; a.Hkv = kv->Hkv; a.d = kv->d; a.G = kv->Hq / kv->Hkv;
  a.max_len = kv->max_seq_len;
  a.paged = paged;
  return launch_append(a, k_new, v_new, T, static_cast<hipStream_t>(stream)) == hipSuccess ? SFI_OK
                                                                                            : SFI_ERR_HIP;
}

sfi_status sfi_compact_selected(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                                const int32_t *sel_idx, const int32_t *sel_count, int32_t sel_heads,
                                int32_t sel_k, uint16_t *ck, uint16_t *cv, void *stream) {
  KVView view;
  bool paged = false;
  sfi_status s = check_kv(kv, &view, &paged);
  if (s != SFI_OK) return s;
  if ((s = check_batch(kv, batch_n)) != SFI_OK) return s;
  if ((s = check_fast(kv, sel_idx, sel_count, sel_heads, sel_k, 0, 0)) != SFI_OK) return s;
  if (!ck || !cv) return SFI_ERR_NULL;
  if (!aligned16(ck) || !aligned16(cv)) return SFI_ERR_RANGE;
  if (batch_n == 0 || sel_k == 0) return SFI_OK;
  AttnLaunch a{};
  a.kv = view;
  a.seq_len = kv->seq_len;
  a.batch_ids = batch_ids;
  a.batch_n = batch_n;
  a.B = kv->B; a.Hq = kv->Hq; a.Hkv = kv->Hkv; a.d = kv->d; a.G = kv->Hq / kv->Hkv;
  a.max_len = kv->max_seq_len;
  a.paged = paged;
  a.sel_idx = sel_idx;
  a.sel_count = sel_count;
  a.sel_heads = sel_heads;
  a.sel_k = sel_k;
  return launch_compact(a, ck, cv, static_cast<hipStream_t>(stream)) == hipSuccess ? SFI_OK : SFI_ERR_HIP;
}

sfi_status sfi_fast_step_compact(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                                 const uint16_t *q, const int32_t *sel_idx, const int32_t *sel_count,
                                 int32_t sel_heads, int32_t sel_k, int32_t n_sink, int32_t window,
                                 const uint16_t *ck, const uint16_t *cv, float *out, void *ws,
                                 size_t ws_bytes, void *stream) {
  KVView view;
  bool paged = false;
  sfi_status s = check_kv(kv, &view, &paged);
  if (s != SFI_OK) return s;
  if ((s = check_batch(kv, batch_n)) != SFI_OK) return s;
  if (!q || !out) return SFI_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16)) return SFI_ERR_RANGE;
  if ((s = check_fast(kv, sel_idx, sel_count, sel_heads, sel_k, n_sink, window)) != SFI_OK) return s;
  if (!ck || !cv) return SFI_ERR_NULL;
  if (!aligned16(ck) || !aligned16(cv)) return SFI_ERR_RANGE;
  const FastWs w = fast_ws(kv, sel_k, n_sink, window);
  if (!ws) return SFI_ERR_NULL;
  if (!aligned(ws, kAlign)) return SFI_ERR_RANGE;
  if (ws_bytes < w.total) return SFI_ERR_WORKSPACE;
  if (batch_n == 0) return SFI_OK;
  AttnLaunch a = fast_launch(kv, view, paged, w, ws, batch_ids, batch_n, q, out, sel_idx, sel_count,
                             sel_heads, sel_k, n_sink, window);
  a.len_host = nullptr;  // the index-gather kernel's plan
  a.ck = ck;
  a.cv = cv;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // without selected rows there is nothing to read from the copy
  const hipError_t e = (sel_k > 0) ? launch_fast_compact(a, st) : launch_fast(a, st);
  return e == hipSuccess ? SFI_OK : SFI_ERR_HIP;
}

size_t sfi_verify_workspace_bytes(const sfi_kv *kv, int32_t T) {
  KVView v;
  bool pg;
  if (check_kv(kv, &v, &pg) != SFI_OK || T < 1 || T > 32) return 0;
  return verify_ws(kv, T).total;
}

}  // extern "C"

namespace {
sfi_status verify_impl(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n, const uint16_t *q,
                       int32_t T, uint32_t row_mask, float *out, float *agg, int32_t ld, float *raw,
                       int32_t raw_ld, void *ws, size_t ws_bytes, void *stream) {
  KVView view;
  bool paged = false;
  sfi_status s = check_kv(kv, &view, &paged);
  if (s != SFI_OK) return s;
  if ((s = check_batch(kv, batch_n)) != SFI_OK) return s;
  if (!q || !out || !agg) return SFI_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16)) return SFI_ERR_RANGE;
  if (view.k_new) return SFI_ERR_RANGE;  // T new rows: append them with sfi_append_kv
  const int G = kv->Hq / kv->Hkv;
  if (T < 1 || G * T > 32) return SFI_ERR_UNSUPPORTED;
  if (G == 5) return SFI_ERR_UNSUPPORTED;
  const uint32_t all = (T >= 32) ? 0xffffffffu : ((1u << T) - 1u);
  if (row_mask == 0u || (row_mask & ~all) != 0u) return SFI_ERR_RANGE;
  if (kv->max_seq_len < T) return SFI_ERR_RANGE;
  if (ld < kv->max_seq_len - T) return SFI_ERR_RANGE;
  if (raw && (raw_ld < kv->max_seq_len - T || !aligned16(raw))) return SFI_ERR_RANGE;
  const VerWs w = verify_ws(kv, T);
  if (!ws) return SFI_ERR_NULL;
  if (!aligned(ws, kAlign)) return SFI_ERR_RANGE;
  if (ws_bytes < w.total) return SFI_ERR_WORKSPACE;
  if (batch_n == 0) return SFI_OK;

  VerifyLaunch a{};
  a.kv = view;
  a.seq_len = kv->seq_len;
  a.batch_ids = batch_ids;
  a.batch_n = batch_n;
  a.B = kv->B; a.Hq = kv->Hq; a.Hkv = kv->Hkv; a.d = kv->d; a.G = G; a.T = T;
  a.max_seq_len = kv->max_seq_len;
  a.paged = paged;
  a.row_mask = row_mask;
  a.q = q;
  a.out = out;
  a.agg = agg;
  a.ld = ld;
  a.part_o = carve<float>(ws, w.o);
  a.part_ml = carve<float>(ws, w.ml);
  a.part_agg = carve<float>(ws, w.agg);
  a.lld = kv->max_seq_len;
  a.plan.chunk = w.chunk;
  a.plan.splits = w.stride;
  a.plan.stride = w.stride;
  a.raw = raw;
  a.raw_ld = raw_ld;
  return launch_verify(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SFI_OK : SFI_ERR_HIP;
}
}  // namespace

extern "C" {

sfi_status sfi_verify_aggregate(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                                const uint16_t *q, int32_t T, uint32_t row_mask, float *out,
                                float *agg, int32_t ld, void *ws, size_t ws_bytes, void *stream) {
  return verify_impl(kv, batch_ids, batch_n, q, T, row_mask, out, agg, ld, nullptr, 0, ws, ws_bytes, stream);
}

sfi_status sfi_verify_raw_logits(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                                 const uint16_t *q, int32_t T, uint32_t row_mask, float *out, float *agg,
                                 int32_t ld, float *logits, int32_t logits_ld, void *ws, size_t ws_bytes,
                                 void *stream) {
  if (!logits) return SFI_ERR_NULL;
  return verify_impl(kv, batch_ids, batch_n, q, T, row_mask, out, agg, ld, logits, logits_ld, ws, ws_bytes,
                     stream);
}

size_t sfi_slow_window_workspace_bytes(const sfi_kv *kv, int32_t w) {
  KVView v;
  bool pg;
  if (check_kv(kv, &v, &pg) != SFI_OK || w < 1 || w > 32) return 0;
  return window_ws(kv, w).total;
}

sfi_status sfi_slow_step_window(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                                const uint16_t *q_win, int32_t w, float *out, float *evidence,
                                float *key_norm, int32_t ld, void *ws, size_t ws_bytes, void *stream) {
  KVView view;
  bool paged = false;
  sfi_status s = check_kv(kv, &view, &paged);
  if (s != SFI_OK) return s;
  if ((s = check_batch(kv, batch_n)) != SFI_OK) return s;
  if (!q_win || !out || !evidence) return SFI_ERR_NULL;
  if (!aligned(q_win, 16) || !aligned(out, 16)) return SFI_ERR_RANGE;
  if (view.k_new) return SFI_ERR_RANGE;  // no fused append here
  const int G = kv->Hq / kv->Hkv;
  if (w < 1 || G * w > 32 || G == 5) return SFI_ERR_UNSUPPORTED;
  if (kv->max_seq_len < w) return SFI_ERR_RANGE;
  if (ld < kv->max_seq_len) return SFI_ERR_RANGE;
  const WinWs x = window_ws(kv, w);
  if (!ws) return SFI_ERR_NULL;
  if (!aligned(ws, kAlign)) return SFI_ERR_RANGE;
  if (ws_bytes < x.total) return SFI_ERR_WORKSPACE;
  if (batch_n == 0) return SFI_OK;

  VerifyLaunch a{};
  a.kv = view;
  a.seq_len = kv->seq_len;
  a.batch_ids = batch_ids;
  a.batch_n = batch_n;
  a.B = kv->B; a.Hq = kv->Hq; a.Hkv = kv->Hkv; a.d = kv->d; a.G = G; a.T = w;
  a.max_seq_len = kv->max_seq_len;
  a.paged = paged;
  a.row_mask = 0u;
  a.q = q_win;
  a.out = out;
  a.agg = nullptr;
  a.ld = ld;
  a.part_o = carve<float>(ws, x.o);
  a.part_ml = carve<float>(ws, x.ml);
  a.part_agg = nullptr;
  a.lld = kv->max_seq_len;
  a.plan.chunk = x.chunk;
  a.plan.splits = x.stride;
  a.plan.stride = x.stride;
  a.rstat = carve<float>(ws, x.rstat);
  a.evidence = evidence;
  a.key_norm = key_norm;
  return launch_verify(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SFI_OK : SFI_ERR_HIP;
}

sfi_status sfi_schedule(const uint8_t *events, int32_t steps, int32_t B, int32_t budget,
                        uint8_t *slow) {
  if (!events || !slow) return SFI_ERR_NULL;
  if (steps < 0 || B < 1) return SFI_ERR_SHAPE;
  for (int32_t b = 0; b < B; ++b) {
    int32_t run = 0;
    for (int32_t s = 0; s < steps; ++s) {
      const size_t i = (size_t)s * B + b;
      const bool is_slow = s == 0 || events[i] != 0 || (budget >= 0 && run >= budget);
      slow[i] = is_slow ? 1 : 0;
      run = is_slow ? 0 : run + 1;
    }
  }
  return SFI_OK;
}

const char *sfi_status_string(sfi_status s) {
  switch (s) {
    case SFI_OK: return "ok";
    case SFI_ERR_NULL: return "required pointer is NULL";
    case SFI_ERR_SHAPE: return "inconsistent or unsupported sizes";
    case SFI_ERR_RANGE: return "parameter out of range";
    case SFI_ERR_WORKSPACE: return "workspace too small";
    case SFI_ERR_UNSUPPORTED: return "no kernel for this configuration";
    case SFI_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char *sfi_version(void) { return "libsfi 0.2 gfx950"; }

}  // extern "C"
