// Internal launchers of the MSA library (host side, not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

int device_cu_count();  // compute units of the current device (cached per device)

// ---- RoPE table ------------------------------------------------------------
hipError_t launch_rope_table(float *cos, float *sin, int max_pos, int d, double base, hipStream_t s);

// ---- pooling ---------------------------------------------------------------
struct PoolArgs {
  int dtype;                     // 0 fp32, 1 bf16
  int h_kv, d, h_r, d_r, chunk;
  int64_t n_chunks;              // bank chunks
  int64_t kv_stride;             // row stride of kbar / vbar (chunk capacity)
  int doc_begin, doc_end;        // slab documents
  int64_t slab_tok0;             // first token of doc_begin
  int64_t chunk_begin, chunk_end;
  const int64_t *doc_tok_off;    // device
  const int64_t *doc_chunk_off;  // device
  int32_t *chunk_doc;
  const void *K, *V, *KR;        // slab tensors
  void *kbar, *vbar, *krbar;
  float *kr_inv_norm;
  const float *cos, *sin;        // [max_pos][d/2]
};
hipError_t launch_pool(const PoolArgs &a, hipStream_t s);

// ---- router scan -----------------------------------------------------------
struct RouteArgs {
  int dtype;
  int h_r, d_r;
  int64_t n_chunks;
  int n_docs;
  const void *krbar;
  const float *kr_inv_norm;
  const int32_t *chunk_doc;
  const int64_t *doc_chunk_off;  // device [n_docs+1]
  const void *qr;                // [n_q][t_r][h_r][d_r]
  int n_q, t_r;
  // single-writer mode (edges != null): per-tile records and the scores of the
  // documents inside one tile (layout: EdgeLayout below); a resolve pass or a
  // record-reading top-k writes doc_scores
  float *edges;                  // records
  float *dsc = nullptr;          // [row blocks][n_docs][16 or 1] scores of documents inside one tile
  float *doc_scores;             // [n_q][n_docs] fp32
  // atomic mode (edges == null): order-preserving keys, zeroed before the scan
  uint32_t *doc_keys;            // [n_q][n_docs]
  // optional per-chunk scores [n_q][n_chunks]: fp32 in single-writer mode, keys otherwise
  uint32_t *chunk_out;
  // many-row (wide) scan: (1/h_r)/||Q^R|| per head and query row, [h_r][n_q * t_r] (workspace)
  float *qinv;
  // many-row scan: words its pre-kernel sets to zero before the scan (the
  // document keys, in place of a separate fill launch); null = none.  With
  // init set, they are set to score_key(init[i]) instead (a re-routing
  // round starts from the previous round's document scores).
  uint32_t *zero = nullptr;
  int64_t n_zero = 0;
  const float *init = nullptr;
  // streaming scan: at most this many workgroups per compute unit in the
  // persistent grid (0 = as many as stay resident)
  int max_wg_per_cu = 0;
};
bool route_single_writer(int t_r);                    // (query, document) scores have one writer
bool route_use_wide(int dtype, int h_r, int d_r, int t_r);     // GEMM-tiled scan for many rows per query
bool route_use_rows(int dtype, int h_r, int d_r, int n_q, int t_r);  // of those, few rows: a streaming scan
hipError_t launch_route_rows(const RouteArgs &a, hipStream_t s);
size_t route_wide_ws_bytes(int n_q, int t_r, int h_r);
size_t route_ws_bytes(int dtype, int h_r, int d_r, int64_t n_chunks, int n_docs, int n_q, int t_r);
// single-writer workspace: the records (this many bytes, a multiple of 256), then the interior-document scores
size_t route_record_bytes(int64_t n_chunks, int n_q, int t_r);
hipError_t launch_route_wide(const RouteArgs &a, hipStream_t s);
hipError_t launch_resolve_docs(const RouteArgs &a, hipStream_t s);
// read-only probe of the decode scan's traffic (bf16, 8 x 128 router heads);
// writes one record per 16-chunk tile to a.edges
hipError_t launch_scan_read_probe(const RouteArgs &a, hipStream_t s);
hipError_t launch_fill_u32(uint32_t *p, size_t n, uint32_t v, hipStream_t s);
// p[i] = score_key(init[i]): order-preserving keys of fp32 scores
hipError_t launch_keys_from_scores(uint32_t *p, const float *init, size_t n, hipStream_t s);
hipError_t launch_route_scan(const RouteArgs &a, hipStream_t s);
hipError_t launch_keys_to_scores(uint32_t *p, size_t n, hipStream_t s);  // in place

// Single-writer scan output (one writer per (query, document) score).  The
// scan takes its 16-chunk tiles in pairs, so its unit is 32 chunks: per unit
// a record rec[row block][unit][first segment 0..15 | last segment 16..31]
// holds the maxima of the unit's first and last document segments for the
// rows of the block (16 rows when t_r == 1, row 0 when t_r == 16).  A
// document strictly inside one unit has its scores for the block's rows in
// one row of the document-major array dsc[row block][doc][rw] (one 64-byte
// store instead of a scattered store per query).
struct EdgeLayout {
  const float *rec = nullptr;
  const float *dsc = nullptr;
  int64_t n_units = 0;
  int rw = 16;  // rows per document in dsc
};
EdgeLayout edge_layout(const RouteArgs &a);

// Score of document `doc` for query `q` from a single-writer scan's output:
// for a document inside one unit the stored score, otherwise the max of its
// last segment in the first unit it touches and its first segments in the
// later ones.  c0 / c1: the document's first and last chunk.
__device__ __forceinline__ float edge_range_score(const EdgeLayout &L, int n_docs, int t_r, int q, int doc, int64_t c0,
                                                  int64_t c1) {
  const int rb = t_r == 1 ? q / 16 : q;  // row block of this query
  const int r = t_r == 1 ? q % 16 : 0;   // its row within the block
  const int64_t ta = c0 / 32, tb = c1 / 32;
  if (ta == tb && (c0 % 32) != 0 && (c1 % 32) != 31) return L.dsc[((int64_t)rb * n_docs + doc) * L.rw + r];
  const float *rec = L.rec + (int64_t)rb * L.n_units * 32;
  if (ta == tb) return rec[ta * 32 + ((c0 % 32) == 0 ? 0 : 16) + r];
  float m = rec[ta * 32 + 16 + r];
  for (int64_t t = ta + 1; t <= tb; ++t) m = fmaxf(m, rec[t * 32 + r]);
  return m;
}

__device__ __forceinline__ float edge_doc_score(const EdgeLayout &L, const int64_t *doc_chunk_off, int n_docs, int t_r,
                                                int q, int doc) {
  return edge_range_score(L, n_docs, t_r, q, doc, doc_chunk_off[doc], doc_chunk_off[doc + 1] - 1);
}

// ---- top-k -----------------------------------------------------------------
size_t topk_ws_bytes(int n_q, int n_docs, int k);
size_t topk_layer_ws_bytes(int n_q, int n_docs, int k);  // the layer's top-k (pass 1 alone included)
bool topk_single_pass(int n_docs);  // one workgroup per query, no workspace
// Where the document scores [n_q][n_docs] come from
struct TopkSrc {
  enum Mode { SCORES = 0, KEYS = 1, EDGES = 2 } mode;
  float *scores;                 // SCORES: read; EDGES: written (the completed document scores);
                                 // KEYS: written when not null (the keys as scores)
  const uint32_t *keys;          // KEYS: order-preserving keys
  EdgeLayout edges;              // EDGES: the single-writer scan's output
  const int64_t *doc_chunk_off;  // EDGES
  int t_r;                       // EDGES
};
hipError_t launch_topk(const TopkSrc &src, int n_q, int n_docs, int k, int32_t *idx, float *val, void *ws,
                       hipStream_t s);
// Whether the final selection can be left to the attention kernel after
// pass 1 alone (the per-slice candidates, ws as for launch_topk): the number
// of candidates per query, or 0 when this top-k does not take that form
// (small k over more than one 512-document slice, at most ATTEND_MAX_CAND
// candidates).
int topk_fused_candidates(int n_docs, int k);
// Pass 1 straight from a single-writer scan's records (EDGES source): one
// workgroup per (slice, 4 queries) completes the slice's document scores
// into src.scores and selects each query's k (no separate resolve kernel).
hipError_t launch_topk_pass1_resolve(const TopkSrc &src, int n_q, int n_docs, int k, void *ws, hipStream_t s);
// Pass 1 alone over order-preserving keys (KEYS source; writes src.scores when set).
hipError_t launch_topk_pass1_keys(const TopkSrc &src, int n_q, int n_docs, int k, void *ws, hipStream_t s);

// ---- router projection -------------------------------------------------------
// Y[rows][out] = X[rows][hidden] W[out][hidden]^T, bf16 in and out, fp32 accumulation;
// hidden % 64 == 0, out % 128 == 0
hipError_t launch_project(const void *X, const void *W, int64_t rows, int hidden, int out, void *Y, hipStream_t s);

// ---- sparse attention ------------------------------------------------------
struct AttendArgs {
  int dtype;
  int h_kv, d, h_q;
  int64_t n_chunks;
  int64_t kv_stride;  // row stride of kbar / vbar (chunk capacity)
  int kv_host;        // kbar / vbar in host memory: gather with few workgroups
  int n_docs;
  const int64_t *doc_chunk_off;
  const void *kbar, *vbar;
  const void *Q, *K_loc, *V_loc;
  int n_q, T, L_loc, k, pos0;
  float scale;
  const int32_t *idx;
  const float *cos, *sin;
  void *O;
  int max_doc_chunks;
  // In-kernel selection (optional): when cand is set, the documents are the
  // top-k of the query's n_cand pass-1 candidates (composites, 0 = empty),
  // taken by each workgroup itself instead of read from idx; the workgroups
  // of KV head 0, split 0, row group 0 write them to idx_out / val_out.
  const uint64_t *cand = nullptr;
  int n_cand = 0;
  int32_t *idx_out = nullptr;
  float *val_out = nullptr;
};
// candidates per query an attention workgroup can select from (16 per lane)
constexpr int ATTEND_MAX_CAND = 1024;
int attend_splits(const AttendArgs &a);
size_t attend_ws_bytes(const AttendArgs &a);
hipError_t launch_attend(const AttendArgs &a, void *ws, hipStream_t s);

}  // namespace msa
