// extern "C" entry points of libmsa: argument validation on the host, then
// kernel launches on the caller's stream.  Declared and documented in
// include/msa.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/msa.h"
#include "msa_internal.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return MSA_OK;
}

int dev_fail(hipError_t e, const char *what) {
  return fail(MSA_ERR_DEVICE, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define CHECK_PTR(p, al, name)                                                        \
  do {                                                                                \
    if (!(p)) return fail(MSA_ERR_ARG, "%s is null", name);                           \
    if (!aligned((p), (al))) return fail(MSA_ERR_ARG, "%s is not %d-byte aligned", name, (int)(al)); \
  } while (0)

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// row stride of kbar / vbar: the chunk capacity when the bank has spare rows
int64_t kv_stride(const msa_bank *b) { return b->chunk_cap ? (int64_t)b->chunk_cap : b->n_chunks; }

int check_bank(const msa_bank *b) {
  if (!b) return fail(MSA_ERR_ARG, "bank is null");
  if (b->dtype != MSA_F32 && b->dtype != MSA_BF16) return fail(MSA_ERR_UNSUPPORTED, "bank dtype %d", b->dtype);
  if (b->n_docs < 1) return fail(MSA_ERR_ARG, "n_docs = %d", b->n_docs);
  if (b->chunk < 1) return fail(MSA_ERR_ARG, "chunk = %d", b->chunk);
  if (b->h_kv < 1) return fail(MSA_ERR_ARG, "h_kv = %d", b->h_kv);
  if (b->d != 64 && b->d != 128) return fail(MSA_ERR_UNSUPPORTED, "head dim d = %d (64 or 128)", b->d);
  if (b->d_r != 64 && b->d_r != 128 && b->d_r != 256)
    return fail(MSA_ERR_UNSUPPORTED, "router dim d_r = %d (64, 128, or 256 for bf16)", b->d_r);
  if (b->d_r == 256 && b->dtype != MSA_BF16) return fail(MSA_ERR_UNSUPPORTED, "router dim 256 needs a bf16 bank");
  if (b->h_r != 1 && b->h_r != 2 && b->h_r != 4 && b->h_r != 8 && b->h_r != 16)
    return fail(MSA_ERR_UNSUPPORTED, "router heads h_r = %d (1, 2, 4, 8 or 16)", b->h_r);
  if (b->h_r * b->d_r > 1024) return fail(MSA_ERR_UNSUPPORTED, "h_r * d_r = %d > 1024", b->h_r * b->d_r);
  if (b->n_chunks < b->n_docs || b->n_chunks >= (int64_t)1 << 31)
    return fail(MSA_ERR_ARG, "n_chunks = %lld (must be >= n_docs and < 2^31)", (long long)b->n_chunks);
  if (b->max_doc_len < 1) return fail(MSA_ERR_ARG, "max_doc_len = %d", b->max_doc_len);
  if (b->max_doc_chunks != (b->max_doc_len + b->chunk - 1) / b->chunk)
    return fail(MSA_ERR_ARG, "max_doc_chunks = %d != ceil(max_doc_len / chunk)", b->max_doc_chunks);
  if (b->n_chunks > (int64_t)b->n_docs * b->max_doc_chunks)
    return fail(MSA_ERR_ARG, "n_chunks exceeds n_docs * max_doc_chunks");
  if (b->chunk_cap != 0 && b->chunk_cap < b->n_chunks)
    return fail(MSA_ERR_ARG, "chunk_cap = %d below n_chunks = %lld", b->chunk_cap, (long long)b->n_chunks);
  CHECK_PTR(b->doc_tok_off, 8, "bank.doc_tok_off");
  CHECK_PTR(b->doc_chunk_off, 8, "bank.doc_chunk_off");
  CHECK_PTR(b->chunk_doc, 4, "bank.chunk_doc");
  CHECK_PTR(b->kbar, 16, "bank.kbar");
  CHECK_PTR(b->vbar, 16, "bank.vbar");
  CHECK_PTR(b->krbar, 16, "bank.krbar");
  CHECK_PTR(b->kr_inv_norm, 16, "bank.kr_inv_norm");
  return MSA_OK;
}

int check_rope(const msa_rope *r, int d, int64_t need_pos) {
  if (!r) return fail(MSA_ERR_ARG, "rope is null");
  CHECK_PTR(r->cos, 16, "rope.cos");
  CHECK_PTR(r->sin, 16, "rope.sin");
  if (r->d != d) return fail(MSA_ERR_ARG, "rope.d = %d but head dim is %d", r->d, d);
  if ((int64_t)r->max_pos < need_pos)
    return fail(MSA_ERR_ARG, "rope.max_pos = %d < %lld positions needed", r->max_pos, (long long)need_pos);
  return MSA_OK;
}

int check_attend_args(const msa_bank *b, const void *Q, const void *K_loc, const void *V_loc, int32_t n_q, int32_t T,
                      int32_t L_loc, int32_t h_q, int32_t k, int32_t pos0, float scale, const msa_rope *rope,
                      const void *O) {
  CHECK_PTR(Q, 16, "Q");
  CHECK_PTR(K_loc, 16, "K_loc");
  CHECK_PTR(V_loc, 16, "V_loc");
  CHECK_PTR(O, 16, "O");
  if (n_q < 1) return fail(MSA_ERR_ARG, "n_q = %d", n_q);
  if (T < 1 || L_loc < T) return fail(MSA_ERR_ARG, "need 1 <= T <= L_loc (T = %d, L_loc = %d)", T, L_loc);
  if (h_q < b->h_kv || h_q % b->h_kv) return fail(MSA_ERR_ARG, "h_q = %d is not a multiple of h_kv = %d", h_q, b->h_kv);
  if (k < 1 || k > b->n_docs || k > 256) return fail(MSA_ERR_ARG, "k = %d (need 1 <= k <= min(n_docs, 256))", k);
  if (pos0 < 0) return fail(MSA_ERR_ARG, "pos0 = %d", pos0);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(MSA_ERR_ARG, "scale must be finite and > 0");
  if ((int64_t)n_q * T * h_q / h_q != (int64_t)n_q * T) return fail(MSA_ERR_ARG, "sizes overflow");
  if ((int64_t)n_q * b->h_kv * (((int64_t)T * (h_q / b->h_kv) + 15) / 16) * 64 >= ((int64_t)1 << 31))
    return fail(MSA_ERR_ARG, "too many query rows");
  return check_rope(rope, b->d, (int64_t)pos0 + L_loc);
}

msa::AttendArgs attend_args(const msa_bank *b, const void *Q, const void *K_loc, const void *V_loc, int32_t n_q,
                            int32_t T, int32_t L_loc, int32_t h_q, const int32_t *idx, int32_t k, int32_t pos0,
                            float scale, const msa_rope *rope, void *O) {
  msa::AttendArgs a;
  a.dtype = b->dtype;
  a.h_kv = b->h_kv;
  a.d = b->d;
  a.h_q = h_q;
  a.n_chunks = b->n_chunks;
  a.kv_stride = kv_stride(b);
  a.kv_host = b->kv_host != 0;
  a.n_docs = b->n_docs;
  a.doc_chunk_off = b->doc_chunk_off;
  a.kbar = b->kbar;
  a.vbar = b->vbar;
  a.Q = Q;
  a.K_loc = K_loc;
  a.V_loc = V_loc;
  a.n_q = n_q;
  a.T = T;
  a.L_loc = L_loc;
  a.k = k;
  a.pos0 = pos0;
  a.scale = scale;
  a.idx = idx;
  a.cos = rope ? rope->cos : nullptr;
  a.sin = rope ? rope->sin : nullptr;
  a.O = O;
  a.max_doc_chunks = b->max_doc_chunks;
  return a;
}

msa::RouteArgs route_args(const msa_bank *b, const void *qr, int32_t n_q, int32_t t_r, float *edges,
                          float *doc_scores, uint32_t *doc_keys, uint32_t *chunk_out) {
  msa::RouteArgs a;
  a.doc_chunk_off = b->doc_chunk_off;
  a.edges = edges;  // single-writer workspace: the records, then the interior-document scores
  a.dsc = edges && msa::route_single_writer(t_r)
              ? edges + msa::route_record_bytes(b->n_chunks, n_q, t_r) / sizeof(float)
              : nullptr;
  a.doc_scores = doc_scores;
  a.dtype = b->dtype;
  a.h_r = b->h_r;
  a.d_r = b->d_r;
  a.n_chunks = b->n_chunks;
  a.n_docs = b->n_docs;
  a.krbar = b->krbar;
  a.kr_inv_norm = b->kr_inv_norm;
  a.chunk_doc = b->chunk_doc;
  a.qr = qr;
  a.n_q = n_q;
  a.t_r = t_r;
  a.doc_keys = doc_keys;
  a.chunk_out = chunk_out;
  a.qinv = nullptr;
  return a;
}

int check_route_args(const void *qr, int32_t n_q, int32_t t_r) {
  CHECK_PTR(qr, 16, "QR");
  if (n_q < 1 || t_r < 1) return fail(MSA_ERR_ARG, "need n_q >= 1 and t_r >= 1 (n_q = %d, t_r = %d)", n_q, t_r);
  if ((int64_t)n_q * t_r > (int64_t)65535 * 16) return fail(MSA_ERR_ARG, "n_q * t_r = %lld > 1048560", (long long)n_q * t_r);
  return MSA_OK;
}

// layer workspace: [document scores or keys][route records][top-k candidates][attention partials]
struct LayerWs {
  size_t scores, route, topk, attend, total;
};
LayerWs layer_ws(const msa_bank *b, int32_t n_q, int32_t T, int32_t t_r, int32_t L_loc, int32_t h_q, int32_t k) {
  LayerWs w;
  w.scores = align_up((size_t)n_q * b->n_docs * sizeof(uint32_t));
  w.route = align_up(msa::route_ws_bytes(b->dtype, b->h_r, b->d_r, b->n_chunks, b->n_docs, n_q, t_r));
  w.topk = align_up(msa::topk_layer_ws_bytes(n_q, b->n_docs, k));
  msa::AttendArgs a = attend_args(b, nullptr, nullptr, nullptr, n_q, T, L_loc, h_q, nullptr, k, 0, 1.f, nullptr, nullptr);
  w.attend = align_up(msa::attend_ws_bytes(a));
  w.total = w.scores + w.route + w.topk + w.attend;
  return w;
}

}  // namespace

namespace msa {
int device_cu_count() {
  static std::atomic<int> cache[64];  // per device; 0 = not yet queried (calls from several threads are safe)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
}  // namespace msa

namespace {

// Validation shared by the layer entry points.  need_qr = false for the
// second half, which does not read QR; the workspace layout depends on every
// size.
int check_layer_route(const msa_bank *b, bool need_qr, const void *QR, int32_t n_q, int32_t T, int32_t t_r,
                      int32_t L_loc, int32_t h_q, int32_t k, const float *s_doc, const void *ws, size_t ws_bytes) {
  int rc = check_bank(b);
  if (rc) return rc;
  if (need_qr) {
    rc = check_route_args(QR, n_q, t_r);
    if (rc) return rc;
  } else if (n_q < 1 || t_r < 1) {
    return fail(MSA_ERR_ARG, "n_q = %d, t_r = %d", n_q, t_r);
  }
  if (n_q > 65535) return fail(MSA_ERR_ARG, "n_q = %d > 65535", n_q);
  if (s_doc && !aligned(s_doc, 4)) return fail(MSA_ERR_ARG, "s_doc is not 4-byte aligned");
  if (T < 1 || L_loc < T || h_q < 1 || k < 1 || k > b->n_docs || k > 256 || h_q < b->h_kv || h_q % b->h_kv)
    return fail(MSA_ERR_ARG, "T = %d, L_loc = %d, h_q = %d, k = %d", T, L_loc, h_q, k);
  const LayerWs lw = layer_ws(b, n_q, T, t_r, L_loc, h_q, k);
  if (!ws || ws_bytes < lw.total || !aligned(ws, 256))
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes (256-byte aligned) needed, got %zu", lw.total, ws_bytes);
  return 0;
}

int check_layer_tail(const msa_bank *b, const void *Q, const void *K_loc, const void *V_loc, int32_t n_q, int32_t T,
                     int32_t L_loc, int32_t h_q, int32_t k, int32_t pos0, float scale, const msa_rope *rope,
                     const void *O, const int32_t *idx, const float *val) {
  const int rc = check_attend_args(b, Q, K_loc, V_loc, n_q, T, L_loc, h_q, k, pos0, scale, rope, O);
  if (rc) return rc;
  CHECK_PTR(idx, 4, "idx");
  CHECK_PTR(val, 4, "val");
  return 0;
}

// One layer call's sizes, workspace and stream.  Workspace layout: document
// scores (or order-preserving keys), the router scan's scratch (per-tile
// records or inverse query norms), the top-k candidates, the attention's
// split partials.
struct LayerCtx {
  const msa_bank *b;
  int32_t n_q, T, t_r, L_loc, h_q, k;
  char *w;
  LayerWs lw;
  hipStream_t s;
  void *const *ev;
  // re-routing round: the document keys start from these scores (the previous
  // round's), and the scan maxes the new router tokens into them
  const float *prev = nullptr;
  // single-writer scan (records, no atomics): one writer per (query, document)
  // score and no previous scores to fold in
  bool single() const { return !prev && msa::route_single_writer(t_r); }
  void *rt_ws() const { return w + lw.scores; }
  void *tk_ws() const { return w + lw.scores + lw.route; }
  void *at_ws() const { return w + lw.scores + lw.route + lw.topk; }
  hipError_t rec(int i) const { return ev ? hipEventRecord((hipEvent_t)ev[i], s) : hipSuccess; }
  // single-writer scan: the scores live in s_doc when given, else at the workspace's start
  float *scores(float *s_doc) const { return s_doc ? s_doc : reinterpret_cast<float *>(w); }
};

// First half: the router scan.  Single-writer scans leave per-tile edge
// records and the scores of the documents inside one tile in the route
// workspace; otherwise the document keys are zeroed and maxed atomically.
hipError_t layer_route(const LayerCtx &c, const void *QR, float *s_doc) {
  hipError_t e = hipSuccess;
  if (c.single()) {
    msa::RouteArgs ra = route_args(c.b, QR, c.n_q, c.t_r, static_cast<float *>(c.rt_ws()), c.scores(s_doc), nullptr,
                                   nullptr);
    e = c.rec(0);
    if (e == hipSuccess) e = msa::launch_route_scan(ra, c.s);
  } else {
    uint32_t *keys = reinterpret_cast<uint32_t *>(c.w);
    const size_t nd = (size_t)c.n_q * c.b->n_docs;
    msa::RouteArgs ra = route_args(c.b, QR, c.n_q, c.t_r, nullptr, nullptr, keys, nullptr);
    ra.qinv = static_cast<float *>(c.rt_ws());
    if (msa::route_use_wide(c.b->dtype, c.b->h_r, c.b->d_r, c.t_r)) {
      // the many-row scan's pre-kernel zeroes the keys (or sets them to the
      // previous round's scores)
      ra.zero = keys;
      ra.n_zero = (int64_t)nd;
      ra.init = c.prev;
      e = c.rec(0);
    } else {
      e = c.prev ? msa::launch_keys_from_scores(keys, c.prev, nd, c.s) : msa::launch_fill_u32(keys, nd, 0u, c.s);
      if (e == hipSuccess) e = c.rec(0);
    }
    if (e == hipSuccess) e = msa::launch_route_scan(ra, c.s);
  }
  if (e == hipSuccess) e = c.rec(1);
  return e;
}

// Second half: complete the document scores, select the top-k, attend.
hipError_t layer_tail(const LayerCtx &c, const void *Q, const void *K_loc, const void *V_loc, int32_t pos0,
                      float scale, const msa_rope *rope, void *O, int32_t *idx, float *val, float *s_doc) {
  const msa_bank *b = c.b;
  hipError_t e = hipSuccess;
  int n_fused = 0;  // > 0: the attention selects from this many candidates per query
  if (c.single()) {
    float *scores = c.scores(s_doc);
    msa::RouteArgs ra = route_args(b, nullptr, c.n_q, c.t_r, static_cast<float *>(c.rt_ws()), scores, nullptr,
                                   nullptr);
    // the document scores come from the scan's records and interior scores:
    // a single-pass top-k completes them as it loads; over a sliced bank with
    // small k pass 1 completes them (a few queries per workgroup, adjacent
    // lanes on adjacent queries) and the attention workgroups make each
    // query's final selection (two kernels fewer); otherwise a resolve kernel
    // (coalesced over queries), then the top-k
    msa::TopkSrc src{};
    src.scores = scores;
    src.mode = msa::TopkSrc::EDGES;
    src.edges = msa::edge_layout(ra);
    src.doc_chunk_off = b->doc_chunk_off;
    src.t_r = c.t_r;
    n_fused = msa::topk_fused_candidates(b->n_docs, c.k);  // 0 for one-slice banks or large k
    if (n_fused > 0) {
      e = msa::launch_topk_pass1_resolve(src, c.n_q, b->n_docs, c.k, c.tk_ws(), c.s);
    } else if (msa::topk_single_pass(b->n_docs)) {
      e = msa::launch_topk(src, c.n_q, b->n_docs, c.k, idx, val, c.tk_ws(), c.s);
    } else {
      src.mode = msa::TopkSrc::SCORES;
      e = msa::launch_resolve_docs(ra, c.s);
      if (e == hipSuccess) e = msa::launch_topk(src, c.n_q, b->n_docs, c.k, idx, val, c.tk_ws(), c.s);
    }
    if (e == hipSuccess) e = c.rec(2);
  } else {
    uint32_t *keys = reinterpret_cast<uint32_t *>(c.w);
    msa::TopkSrc src{};
    src.mode = msa::TopkSrc::KEYS;
    src.keys = keys;
    src.scores = s_doc;  // the top-k writes the document scores as it reads their keys
    // small k over several slices: pass 1 here, the final selection in the
    // attention workgroups; otherwise the whole top-k
    n_fused = msa::topk_fused_candidates(b->n_docs, c.k);
    e = n_fused > 0 ? msa::launch_topk_pass1_keys(src, c.n_q, b->n_docs, c.k, c.tk_ws(), c.s)
                    : msa::launch_topk(src, c.n_q, b->n_docs, c.k, idx, val, c.tk_ws(), c.s);
    if (e == hipSuccess) e = c.rec(2);
  }
  if (e == hipSuccess) {
    msa::AttendArgs aa = attend_args(b, Q, K_loc, V_loc, c.n_q, c.T, c.L_loc, c.h_q, idx, c.k, pos0, scale, rope, O);
    if (n_fused > 0) {
      aa.cand = static_cast<const uint64_t *>(c.tk_ws());
      aa.n_cand = n_fused;
      aa.idx_out = idx;
      aa.val_out = val;
    }
    e = msa::launch_attend(aa, c.at_ws(), c.s);
  }
  if (e == hipSuccess) e = c.rec(3);
  return e;
}

// Workspace of msa_layer_forward_noalloc: one array per GPU in the code
// object's device memory, alive until the process ends.  Host code never
// passes `scratch` itself to a kernel or a copy (on the host it names a
// stand-in, not the device array): it uses the device address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device on the first call there.
static __device__ __align__(256) unsigned char scratch[MSA_STATIC_WORKSPACE_BYTES];

std::mutex g_scratch_mu;
void *g_scratch_addr[64] = {};  // per device; null = not looked up yet

int scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return dev_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(MSA_ERR_UNSUPPORTED, "device %d (the static workspace serves devices 0-63)", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return dev_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return MSA_OK;
}

}  // namespace

extern "C" {

int msa_abi_version(void) { return MSA_ABI_VERSION; }

const char *msa_last_error(void) { return g_err.c_str(); }

int msa_router_project(const void *X, const void *W, int64_t rows, int32_t hidden, int32_t out, void *Y,
                       void *stream) {
  try {
    CHECK_PTR(X, 16, "X");
    CHECK_PTR(W, 16, "W");
    CHECK_PTR(Y, 16, "Y");
    if (rows < 0) return fail(MSA_ERR_ARG, "rows = %lld", (long long)rows);
    if (hidden < 64 || hidden % 64) return fail(MSA_ERR_ARG, "hidden = %d (a positive multiple of 64)", hidden);
    if (out < 128 || out % 128) return fail(MSA_ERR_ARG, "out = %d (a positive multiple of 128)", out);
    if ((rows + 127) / 128 * (int64_t)(out / 128) > ((int64_t)1 << 31) - 1024)
      return fail(MSA_ERR_ARG, "rows * out too large");
    hipError_t e = msa::launch_project(X, W, rows, hidden, out, Y, (hipStream_t)stream);
    return e == hipSuccess ? ok() : dev_fail(e, "router_project");
  } catch (...) {
    return fail(MSA_ERR_DEVICE, "internal error");
  }
}

int msa_device_pointer(const void *host, void **dev) {
  if (!host || !dev) return fail(MSA_ERR_ARG, "null pointer");
  void *d = nullptr;
  const hipError_t e = hipHostGetDevicePointer(&d, const_cast<void *>(host), 0);
  if (e != hipSuccess || !d) {
    (void)hipGetLastError();  // clear the runtime's sticky error for the caller's next call
    return fail(MSA_ERR_ARG, "not pinned device-mapped host memory (%s)", hipGetErrorString(e));
  }
  *dev = d;
  return ok();
}

int msa_bank_layout(const int64_t *doc_lens, int32_t n_docs, int32_t chunk, int64_t *doc_tok_off,
                    int64_t *doc_chunk_off, int64_t *n_chunks, int32_t *max_doc_len, int32_t *max_doc_chunks) {
  if (!doc_lens || !doc_tok_off || !doc_chunk_off || !n_chunks || !max_doc_len || !max_doc_chunks)
    return fail(MSA_ERR_ARG, "null pointer");
  if (n_docs < 1) return fail(MSA_ERR_ARG, "n_docs = %d", n_docs);
  if (chunk < 1) return fail(MSA_ERR_ARG, "chunk = %d", chunk);
  int64_t tok = 0, ch = 0, mx = 0;
  doc_tok_off[0] = 0;
  doc_chunk_off[0] = 0;
  for (int32_t i = 0; i < n_docs; ++i) {
    const int64_t L = doc_lens[i];
    if (L < 1 || L > (int64_t)1 << 30) return fail(MSA_ERR_ARG, "document %d has length %lld", i, (long long)L);
    tok += L;
    ch += (L + chunk - 1) / chunk;
    mx = L > mx ? L : mx;
    doc_tok_off[i + 1] = tok;
    doc_chunk_off[i + 1] = ch;
  }
  if (ch >= (int64_t)1 << 31) return fail(MSA_ERR_ARG, "n_chunks = %lld >= 2^31", (long long)ch);
  *n_chunks = ch;
  *max_doc_len = (int32_t)mx;
  *max_doc_chunks = (int32_t)((mx + chunk - 1) / chunk);
  return ok();
}

int msa_rope_table(float *cos, float *sin, int32_t max_pos, int32_t d, double base, void *stream) {
  try {
    CHECK_PTR(cos, 16, "cos");
    CHECK_PTR(sin, 16, "sin");
    if (max_pos < 1) return fail(MSA_ERR_ARG, "max_pos = %d", max_pos);
    if (d != 64 && d != 128) return fail(MSA_ERR_UNSUPPORTED, "d = %d (64 or 128)", d);
    if (!(base > 0.0) || !std::isfinite(base)) return fail(MSA_ERR_ARG, "base must be finite and > 0");
    hipError_t e = msa::launch_rope_table(cos, sin, max_pos, d, base, (hipStream_t)stream);
    return e == hipSuccess ? ok() : dev_fail(e, "rope_table");
  } catch (...) {
    return fail(MSA_ERR_DEVICE, "internal error");
  }
}

int msa_pool_memory(const msa_bank *b, const void *K, const void *V, const void *KR, int32_t doc_begin,
                    int32_t doc_end, const msa_rope *rope, void *stream) {
  try {
    int rc = check_bank(b);
    if (rc) return rc;
    CHECK_PTR(K, 16, "K");
    CHECK_PTR(V, 16, "V");
    CHECK_PTR(KR, 16, "KR");
    if (!b->doc_tok_off_host || !b->doc_chunk_off_host) return fail(MSA_ERR_ARG, "pool needs the host offset arrays");
    if (doc_begin < 0 || doc_end < doc_begin || doc_end > b->n_docs)
      return fail(MSA_ERR_ARG, "document range [%d, %d) outside [0, %d)", doc_begin, doc_end, b->n_docs);
    const int64_t *to = b->doc_tok_off_host, *co = b->doc_chunk_off_host;
    if (to[0] != 0 || co[0] != 0 || co[b->n_docs] != b->n_chunks)
      return fail(MSA_ERR_ARG, "host offsets do not describe a bank of n_chunks chunks");
    int64_t mx = 0;
    for (int32_t i = doc_begin; i < doc_end; ++i) {
      const int64_t L = to[i + 1] - to[i];
      if (L < 1) return fail(MSA_ERR_ARG, "document %d has length %lld", i, (long long)L);
      if (co[i + 1] - co[i] != (L + b->chunk - 1) / b->chunk)
        return fail(MSA_ERR_ARG, "document %d: chunk offsets inconsistent with its length", i);
      mx = L > mx ? L : mx;
    }
    if (mx > b->max_doc_len) return fail(MSA_ERR_ARG, "a document is longer than max_doc_len");
    rc = check_rope(rope, b->d, mx);
    if (rc) return rc;
    if (doc_end == doc_begin) return ok();
    msa::PoolArgs a;
    a.dtype = b->dtype;
    a.h_kv = b->h_kv;
    a.d = b->d;
    a.h_r = b->h_r;
    a.d_r = b->d_r;
    a.chunk = b->chunk;
    a.n_chunks = b->n_chunks;
    a.kv_stride = kv_stride(b);
    a.doc_begin = doc_begin;
    a.doc_end = doc_end;
    a.slab_tok0 = to[doc_begin];
    a.chunk_begin = co[doc_begin];
    a.chunk_end = co[doc_end];
    a.doc_tok_off = b->doc_tok_off;
    a.doc_chunk_off = b->doc_chunk_off;
    a.chunk_doc = b->chunk_doc;
    a.K = K;
    a.V = V;
    a.KR = KR;
    a.kbar = b->kbar;
    a.vbar = b->vbar;
    a.krbar = b->krbar;
    a.kr_inv_norm = b->kr_inv_norm;
    a.cos = rope->cos;
    a.sin = rope->sin;
    hipError_t e = msa::launch_pool(a, (hipStream_t)stream);
    return e == hipSuccess ? ok() : dev_fail(e, "pool");
  } catch (...) {
    return fail(MSA_ERR_DEVICE, "internal error");
  }
}

size_t msa_route_workspace_bytes(const msa_bank *b, int32_t n_q, int32_t t_r) {
  if (!b || n_q < 1 || t_r < 1 || b->n_chunks < 1) return 0;
  return msa::route_ws_bytes(b->dtype, b->h_r, b->d_r, b->n_chunks, b->n_docs, n_q, t_r);
}

int msa_route_score(const msa_bank *b, const void *qr, int32_t n_q, int32_t t_r, float *s_doc, float *s_chunk,
                    void *ws, size_t ws_bytes, int32_t max_wg_per_cu, void *stream) {
  try {
    int rc = check_bank(b);
    if (rc) return rc;
    rc = check_route_args(qr, n_q, t_r);
    if (rc) return rc;
    if (max_wg_per_cu < 0) return fail(MSA_ERR_ARG, "max_wg_per_cu must be >= 0");
    CHECK_PTR(s_doc, 4, "s_doc");
    if (s_chunk && !aligned(s_chunk, 4)) return fail(MSA_ERR_ARG, "s_chunk is not 4-byte aligned");
    const size_t need = msa::route_ws_bytes(b->dtype, b->h_r, b->d_r, b->n_chunks, b->n_docs, n_q, t_r);
    if (need && (!ws || ws_bytes < need || !aligned(ws, 16)))
      return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes (16-byte aligned) needed, got %zu", need, ws_bytes);
    hipStream_t s = (hipStream_t)stream;
    const size_t nd = (size_t)n_q * b->n_docs, nc = (size_t)n_q * b->n_chunks;
    uint32_t *ck = reinterpret_cast<uint32_t *>(s_chunk);
    hipError_t e;
    if (msa::route_single_writer(t_r)) {
      msa::RouteArgs a = route_args(b, qr, n_q, t_r, static_cast<float *>(ws), s_doc, nullptr, ck);
      a.max_wg_per_cu = max_wg_per_cu;
      e = msa::launch_route_scan(a, s);
      if (e == hipSuccess) e = msa::launch_resolve_docs(a, s);
    } else {
      uint32_t *dk = reinterpret_cast<uint32_t *>(s_doc);
      e = msa::launch_fill_u32(dk, nd, 0u, s);
      if (e == hipSuccess && ck) e = msa::launch_fill_u32(ck, nc, 0u, s);
      msa::RouteArgs a = route_args(b, qr, n_q, t_r, nullptr, nullptr, dk, ck);
      a.qinv = static_cast<float *>(ws);
      a.max_wg_per_cu = max_wg_per_cu;
      if (e == hipSuccess) e = msa::launch_route_scan(a, s);
      if (e == hipSuccess) e = msa::launch_keys_to_scores(dk, nd, s);
      if (e == hipSuccess && ck) e = msa::launch_keys_to_scores(ck, nc, s);
    }
    return e == hipSuccess ? ok() : dev_fail(e, "route_score");
  } catch (...) {
    return fail(MSA_ERR_DEVICE, "internal error");
  }
}

int msa_scan_read_probe(const msa_bank *b, void *ws, size_t ws_bytes, void *stream) {
  try {
    const int rc = check_bank(b);
    if (rc) return rc;
    if (b->dtype != MSA_BF16 || b->h_r != 8 || b->d_r != 128)
      return fail(MSA_ERR_UNSUPPORTED, "the probe mirrors the bf16 scan with 8 router heads of 128");
    const size_t need = msa::route_ws_bytes(b->dtype, b->h_r, b->d_r, b->n_chunks, b->n_docs, 1, 1);
    if (!ws || ws_bytes < need || !aligned(ws, 16))
      return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes (16-byte aligned) needed, got %zu", need, ws_bytes);
    const msa::RouteArgs a = route_args(b, nullptr, 1, 1, static_cast<float *>(ws), nullptr, nullptr, nullptr);
    const hipError_t e = msa::launch_scan_read_probe(a, (hipStream_t)stream);
    return e == hipSuccess ? ok() : dev_fail(e, "scan_read_probe");
  } catch (...) {
    return fail(MSA_ERR_DEVICE, "internal error");
  }
}

size_t msa_topk_workspace_bytes(int32_t n_q, int32_t n_docs, int32_t k) {
  if (n_q < 1 || n_docs < 1 || k < 1 || k > 256 || k > n_docs) return 0;
  return msa::topk_ws_bytes(n_q, n_docs, k);
}

int msa_topk(const float *s_doc, int32_t n_q, int32_t n_docs, int32_t k, int32_t *idx, float *val, void *ws,
             size_t ws_bytes, void *stream) {
  try {
    CHECK_PTR(s_doc, 4, "s_doc");
    CHECK_PTR(idx, 4, "idx");
    CHECK_PTR(val, 4, "val");
    if (n_q < 1 || n_q > 65535) return fail(MSA_ERR_ARG, "n_q = %d (1..65535)", n_q);
    if (n_docs < 1) return fail(MSA_ERR_ARG, "n_docs = %d", n_docs);
    if (k < 1 || k > n_docs || k > 256) return fail(MSA_ERR_ARG, "k = %d (need 1 <= k <= min(n_docs, 256))", k);
    const size_t need = msa::topk_ws_bytes(n_q, n_docs, k);
    if (!ws || ws_bytes < need || !aligned(ws, 16))
      return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes (16-byte aligned) needed, got %zu", need, ws_bytes);
    msa::TopkSrc src{};
    src.mode = msa::TopkSrc::SCORES;
    src.scores = const_cast<float *>(s_doc);  // read only in this mode
    hipError_t e = msa::launch_topk(src, n_q, n_docs, k, idx, val, ws, (hipStream_t)stream);
    return e == hipSuccess ? ok() : dev_fail(e, "topk");
  } catch (...) {
    return fail(MSA_ERR_DEVICE, "internal error");
  }
}

size_t msa_attend_workspace_bytes(const msa_bank *b, int32_t n_q, int32_t T, int32_t L_loc, int32_t h_q, int32_t k) {
  if (!b || n_q < 1 || T < 1 || L_loc < T || b->h_kv < 1 || h_q < b->h_kv || h_q % b->h_kv || k < 1 ||
      (b->d != 64 && b->d != 128))
    return 0;
  msa::AttendArgs a = attend_args(b, nullptr, nullptr, nullptr, n_q, T, L_loc, h_q, nullptr, k, 0, 1.f, nullptr, nullptr);
  return msa::attend_ws_bytes(a);
}

int msa_sparse_attend(const msa_bank *b, const void *Q, const void *K_loc, const void *V_loc, int32_t n_q, int32_t T,
                      int32_t L_loc, int32_t h_q, const int32_t *idx, int32_t k, int32_t pos0, float scale,
                      const msa_rope *rope, void *O, void *ws, size_t ws_bytes, void *stream) {
  try {
    int rc = check_bank(b);
    if (rc) return rc;
    rc = check_attend_args(b, Q, K_loc, V_loc, n_q, T, L_loc, h_q, k, pos0, scale, rope, O);
    if (rc) return rc;
    CHECK_PTR(idx, 4, "idx");
    msa::AttendArgs a = attend_args(b, Q, K_loc, V_loc, n_q, T, L_loc, h_q, idx, k, pos0, scale, rope, O);
    const size_t need = msa::attend_ws_bytes(a);
    if (need && (!ws || ws_bytes < need || !aligned(ws, 16)))
      return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes (16-byte aligned) needed, got %zu", need, ws_bytes);
    hipError_t e = msa::launch_attend(a, ws, (hipStream_t)stream);
    return e == hipSuccess ? ok() : dev_fail(e, "sparse_attend");
  } catch (...) {
    return fail(MSA_ERR_DEVICE, "internal error");
  }
}

size_t msa_layer_workspace_bytes(const msa_bank *b, int32_t n_q, int32_t T, int32_t t_r, int32_t L_loc, int32_t h_q,
                                 int32_t k) {
  if (!b || n_q < 1 || T < 1 || t_r < 1 || L_loc < T || b->n_docs < 1 || b->h_kv < 1 || h_q < b->h_kv ||
      h_q % b->h_kv || k < 1 || k > b->n_docs || k > 256 || (b->d != 64 && b->d != 128))
    return 0;
  return layer_ws(b, n_q, T, t_r, L_loc, h_q, k).total;
}

// The whole layer (validated except for the workspace, whose pointer and size
// the caller has checked) on `stream`.
int layer_forward_checked(const msa_bank *b, const void *Q, const void *K_loc, const void *V_loc, const void *QR,
                          int32_t n_q, int32_t T, int32_t t_r, int32_t L_loc, int32_t h_q, int32_t k, int32_t pos0,
                          float scale, const msa_rope *rope, void *O, int32_t *idx, float *val, float *s_doc, void *ws,
                          void *const *stage_events, void *stream, const float *s_doc_prev = nullptr) {
  const LayerCtx c{b, n_q, T, t_r, L_loc, h_q, k, static_cast<char *>(ws), layer_ws(b, n_q, T, t_r, L_loc, h_q, k),
                   (hipStream_t)stream, stage_events, s_doc_prev};
  hipError_t e = layer_route(c, QR, s_doc);
  if (e == hipSuccess) e = layer_tail(c, Q, K_loc, V_loc, pos0, scale, rope, O, idx, val, s_doc);
  return e == hipSuccess ? ok() : dev_fail(e, "layer_forward");
}

// Validation of a whole layer call; check_ws = false leaves out the workspace
// (the caller checks its own).
int check_layer(const msa_bank *b, const void *Q, const void *K_loc, const void *V_loc, const void *QR, int32_t n_q,
                int32_t T, int32_t t_r, int32_t L_loc, int32_t h_q, int32_t k, int32_t pos0, float scale,
                const msa_rope *rope, const void *O, const int32_t *idx, const float *val, const float *s_doc,
                bool check_ws, const void *ws, size_t ws_bytes, void *const *stage_events) {
  // without the workspace check an aligned stand-in of unbounded size passes it
  int rc = check_layer_route(b, true, QR, n_q, T, t_r, L_loc, h_q, k, s_doc,
                             check_ws ? ws : reinterpret_cast<const void *>(256), check_ws ? ws_bytes : ~(size_t)0);
  if (rc) return rc;
  rc = check_layer_tail(b, Q, K_loc, V_loc, n_q, T, L_loc, h_q, k, pos0, scale, rope, O, idx, val);
  if (rc) return rc;
  if (stage_events)
    for (int i = 0; i < 4; ++i)
      if (!stage_events[i]) return fail(MSA_ERR_ARG, "stage_events[%d] is null", i);
  return MSA_OK;
}

int msa_layer_forward(const msa_bank *b, const void *Q, const void *K_loc, const void *V_loc, const void *QR,
                      int32_t n_q, int32_t T, int32_t t_r, int32_t L_loc, int32_t h_q, int32_t k, int32_t pos0,
                      float scale, const msa_rope *rope, void *O, int32_t *idx, float *val, float *s_doc, void *ws,
                      size_t ws_bytes, void *const *stage_events, void *stream) {
  try {
    const int rc = check_layer(b, Q, K_loc, V_loc, QR, n_q, T, t_r, L_loc, h_q, k, pos0, scale, rope, O, idx, val,
                               s_doc, true, ws, ws_bytes, stage_events);
    if (rc) return rc;
    return layer_forward_checked(b, Q, K_loc, V_loc, QR, n_q, T, t_r, L_loc, h_q, k, pos0, scale, rope, O, idx, val,
                                 s_doc, ws, stage_events, stream);
  } catch (...) {
    return fail(MSA_ERR_DEVICE, "internal error");
  }
}

int msa_layer_forward_noalloc(const msa_bank *b, const void *Q, const void *K_loc, const void *V_loc, const void *QR,
                              int32_t n_q, int32_t T, int32_t t_r, int32_t L_loc, int32_t h_q, int32_t k, int32_t pos0,
                              float scale, const msa_rope *rope, void *O, int32_t *idx, float *val, float *s_doc,
                              void *const *stage_events, void *stream) {
  try {
    // every argument and the size are checked before any device call: a layer
    // whose workspace exceeds the static array is refused
    int rc = check_layer(b, Q, K_loc, V_loc, QR, n_q, T, t_r, L_loc, h_q, k, pos0, scale, rope, O, idx, val, s_doc,
                         false, nullptr, 0, stage_events);
    if (rc) return rc;
    const size_t need = layer_ws(b, n_q, T, t_r, L_loc, h_q, k).total;
    if (need > (size_t)MSA_STATIC_WORKSPACE_BYTES)
      return fail(MSA_ERR_WORKSPACE, "this layer needs a %zu-byte workspace; the static workspace holds %zu bytes",
                  need, (size_t)MSA_STATIC_WORKSPACE_BYTES);
    void *ws = nullptr;
    rc = scratch_address(&ws);
    if (rc) return rc;
    return layer_forward_checked(b, Q, K_loc, V_loc, QR, n_q, T, t_r, L_loc, h_q, k, pos0, scale, rope, O, idx, val,
                                 s_doc, ws, stage_events, stream);
  } catch (...) {
    return fail(MSA_ERR_DEVICE, "internal error");
  }
}

int msa_layer_forward_reroute(const msa_bank *b, const void *Q, const void *K_loc, const void *V_loc,
                              const void *QR_new, int32_t n_q, int32_t T, int32_t t_new, int32_t L_loc, int32_t h_q,
                              int32_t k, int32_t pos0, float scale, const msa_rope *rope, const float *s_doc_prev,
                              void *O, int32_t *idx, float *val, float *s_doc, void *ws, size_t ws_bytes,
                              void *const *stage_events, void *stream) {
  try {
    const int rc = check_layer(b, Q, K_loc, V_loc, QR_new, n_q, T, t_new, L_loc, h_q, k, pos0, scale, rope, O, idx, val,
                               s_doc, true, ws, ws_bytes, stage_events);
    if (rc) return rc;
    CHECK_PTR(s_doc_prev, 4, "s_doc_prev");
    return layer_forward_checked(b, Q, K_loc, V_loc, QR_new, n_q, T, t_new, L_loc, h_q, k, pos0, scale, rope, O, idx,
                                 val, s_doc, ws, stage_events, stream, s_doc_prev);
  } catch (...) {
    return fail(MSA_ERR_DEVICE, "internal error");
  }
}

int msa_layer_route(const msa_bank *b, const void *QR, int32_t n_q, int32_t T, int32_t t_r, int32_t L_loc,
                    int32_t h_q, int32_t k, float *s_doc, void *ws, size_t ws_bytes, void *stream) {
  try {
    const int rc = check_layer_route(b, true, QR, n_q, T, t_r, L_loc, h_q, k, s_doc, ws, ws_bytes);
    if (rc) return rc;
    const LayerCtx c{b, n_q, T, t_r, L_loc, h_q, k, static_cast<char *>(ws), layer_ws(b, n_q, T, t_r, L_loc, h_q, k),
                     (hipStream_t)stream, nullptr};
    const hipError_t e = layer_route(c, QR, s_doc);
    return e == hipSuccess ? ok() : dev_fail(e, "layer_route");
  } catch (...) {
    return fail(MSA_ERR_DEVICE, "internal error");
  }
}

int msa_layer_select_attend(const msa_bank *b, const void *Q, const void *K_loc, const void *V_loc, int32_t n_q,
                            int32_t T, int32_t t_r, int32_t L_loc, int32_t h_q, int32_t k, int32_t pos0, float scale,
                            const msa_rope *rope, void *O, int32_t *idx, float *val, float *s_doc, void *ws,
                            size_t ws_bytes, void *stream) {
  try {
    int rc = check_layer_route(b, false, nullptr, n_q, T, t_r, L_loc, h_q, k, s_doc, ws, ws_bytes);
    if (rc) return rc;
    rc = check_layer_tail(b, Q, K_loc, V_loc, n_q, T, L_loc, h_q, k, pos0, scale, rope, O, idx, val);
    if (rc) return rc;
    const LayerCtx c{b, n_q, T, t_r, L_loc, h_q, k, static_cast<char *>(ws), layer_ws(b, n_q, T, t_r, L_loc, h_q, k),
                     (hipStream_t)stream, nullptr};
    const hipError_t e = layer_tail(c, Q, K_loc, V_loc, pos0, scale, rope, O, idx, val, s_doc);
    return e == hipSuccess ? ok() : dev_fail(e, "layer_select_attend");
  } catch (...) {
    return fail(MSA_ERR_DEVICE, "internal error");
  }
}

}  // extern "C"
