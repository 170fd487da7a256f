/*
 * msa.h -- C ABI of the Memory Sparse Attention (MSA) routed-layer hot path
 * on AMD Instinct MI355X (gfx950).
 *
 * The method (sources cited by page title and section):
 *  - [LH] Lighthouse AI-research digest, "MSA: Memory Sparse Attention for
 *    Efficient End-to-End Memory Model Scaling to 100M Tokens";
 *  - [HD] hotdry blog, "EverMind MSA router sparse attention architecture";
 *  - [WC] wiselychen blog, "MSA: 4B model beats a 235B RAG system".
 * Three inference stages ([WC] mechanism 3): offline encoding of the memory
 * (msa_pool_memory), online routing against the cached router keys
 * (msa_route_score, msa_topk), and sparse attention over the selected
 * documents (msa_sparse_attend); msa_layer_forward chains the online stages.
 *
 * Conventions (every entry point):
 *  - Pointers are DEVICE pointers owned by the caller unless marked "host".
 *    The library never allocates device memory and keeps no pointer past the
 *    call.  Device buffers must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  A
 *    call validates on the host, enqueues its kernels on `stream` and returns;
 *    buffers must stay alive until the stream has passed the work.
 *  - Return value: MSA_OK, or an MSA_ERR_* code with a message available from
 *    msa_last_error() (per thread, valid until the next call on that thread).
 *    When validation fails nothing is enqueued.  MSA_ERR_DEVICE reports a
 *    failed launch; device faults surface at the caller's next
 *    synchronisation.  No C++ exception crosses this interface.
 *  - Element types: MSA_F32 (float) or MSA_BF16 (bfloat16 storage, fp32
 *    accumulation).  All bank and activation tensors of a call share the
 *    bank's dtype; scores, norms and RoPE tables are fp32.
 *  - Calls that share a workspace, or write the same outputs, must not run
 *    concurrently on different streams.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_ABI_VERSION 3

enum {
  MSA_OK = 0,
  MSA_ERR_ARG = 1,          /* invalid argument (null/misaligned pointer, bad size) */
  MSA_ERR_UNSUPPORTED = 2,  /* valid but not supported (dtype, head dim)            */
  MSA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required          */
  MSA_ERR_DEVICE = 4        /* HIP launch or runtime error                          */
};

enum { MSA_F32 = 0, MSA_BF16 = 1 };

/* RoPE cos/sin tables, fp32 [max_pos][d/2] each, 16-byte aligned (see msa_rope_table). */
typedef struct msa_rope {
  const float *cos;
  const float *sin;
  int32_t max_pos;
  int32_t d;
} msa_rope;

/*
 * A memory bank of n_docs contiguous documents, document i holding L_i
 * tokens split into ceil(L_i / chunk) chunks ([HD] core architecture of the
 * memory routing layer: fixed-size chunks, chunk-mean pooling).
 * Layouts:
 *   doc_tok_off   [n_docs+1] int64, prefix sums of L_i           (device)
 *   doc_chunk_off [n_docs+1] int64, prefix sums of ceil(L_i/chunk) (device)
 *   doc_tok_off_host / doc_chunk_off_host: the same arrays in host memory,
 *                 read by msa_pool_memory only (may be NULL elsewhere)
 *   chunk_doc     [n_chunks] int32, owning document of each chunk (written by pool)
 *   kbar, vbar    [h_kv][S][d]          pooled keys (document-wise RoPE applied) / values,
 *                 S = chunk_cap if nonzero, else n_chunks (rows n_chunks..S-1 unused)
 *   krbar         [n_chunks][h_r][d_r]  pooled router keys
 *   kr_inv_norm   [n_chunks][h_r] fp32  1 / ||stored krbar row|| (0 for a zero row)
 * max_doc_len = max L_i and max_doc_chunks = max ceil(L_i/chunk) are host
 * values that msa_bank_layout computes; n_chunks must be below 2^31.
 *
 * Tiered bank (the pages' deployment keeps Kbar/Vbar in host memory and only
 * the router keys on the GPU; [HD] key engineering details; [WC] mechanism
 * 3): kbar and vbar may live in pinned host memory mapped into the device
 * address space (their device addresses from msa_device_pointer; set
 * kv_host).  Pooling then writes them over the host link and sparse
 * attention gathers the selected documents' rows from there, with few
 * workgroups (the host link, not the GPU, bounds the gather, and the rest of
 * the GPU stays free for a concurrent router scan); the scan reads only
 * krbar, kr_inv_norm and chunk_doc, which stay in HBM.
 *
 * Incremental append (the pages' corpus updates without re-encoding the
 * whole memory; [LH] overall architecture, offline encoding once): a bank
 * allocated with spare capacity -- offset arrays for more documents, chunk
 * arrays for chunk_cap >= n_chunks chunks -- takes new documents at its end
 * by extending the offset arrays (device and host), raising n_docs,
 * n_chunks, max_doc_len and max_doc_chunks, and pooling only the new
 * document range with msa_pool_memory; pooled rows already in place do not
 * move.  Re-pooling an existing range replaces it in place (its lengths
 * must not change).  chunk_cap = 0 means no spare rows.
 */
typedef struct msa_bank {
  int32_t dtype;
  int32_t n_docs;
  int32_t chunk;
  int32_t h_kv;
  int32_t d;
  int32_t h_r;
  int32_t d_r;         /* 64, 128, or 256 (bf16); h_r * d_r <= 1024 */
  int32_t max_doc_len;
  int32_t max_doc_chunks;
  int32_t chunk_cap;   /* row capacity of kbar/vbar, >= n_chunks; 0 = n_chunks */
  int32_t kv_host;     /* nonzero: kbar/vbar in pinned host memory (tiered bank) */
  int32_t reserved;    /* 0 */
  int64_t n_chunks;
  const int64_t *doc_tok_off;
  const int64_t *doc_chunk_off;
  const int64_t *doc_tok_off_host;
  const int64_t *doc_chunk_off_host;
  int32_t *chunk_doc;
  void *kbar;
  void *vbar;
  void *krbar;
  float *kr_inv_norm;
} msa_bank;

/* ABI version of the loaded library (MSA_ABI_VERSION it was built with). */
int msa_abi_version(void);

/* Message of the last failed call on this thread ("" after success). */
const char *msa_last_error(void);

/*
 * Device address of pinned, device-mapped host memory (as allocated by
 * hipHostMalloc), for the kbar / vbar pointers of a tiered bank.
 * host: host pointer into such an allocation; *dev receives the address
 * kernels use (host memory).  Errors: MSA_ERR_ARG on null pointers or when
 * the runtime does not know `host` as pinned device-mapped memory.
 */
int msa_device_pointer(const void *host, void **dev);

/*
 * Host helper: bank layout from document lengths (all pointers host).
 * doc_lens [n_docs] (each >= 1) -> doc_tok_off, doc_chunk_off [n_docs+1],
 * *n_chunks, *max_doc_len, *max_doc_chunks.  Errors: MSA_ERR_ARG on null
 * pointers, n_docs < 1, chunk < 1, a length < 1, or n_chunks >= 2^31.
 */
int msa_bank_layout(const int64_t *doc_lens, int32_t n_docs, int32_t chunk, int64_t *doc_tok_off,
                    int64_t *doc_chunk_off, int64_t *n_chunks, int32_t *max_doc_len, int32_t *max_doc_chunks);

/*
 * RoPE tables ([LH] Component 2; [HD] key engineering details, position
 * encoding; rotate-half pairing (i, i+d/2), theta_i = base^(-2i/d)):
 * cos[p][i] = cos(p * theta_i), sin[p][i] = sin(p * theta_i) for p < max_pos,
 * i < d/2, evaluated in fp64 on the device and rounded once to fp32.
 * cos, sin: [max_pos][d/2] fp32.  Errors: MSA_ERR_ARG (null/misaligned,
 * max_pos < 1, base <= 0), MSA_ERR_UNSUPPORTED (d not 64 or 128).
 */
int msa_rope_table(float *cos, float *sin, int32_t max_pos, int32_t d, double base, void *stream);

/*
 * Offline chunk-mean pooling of documents [doc_begin, doc_end) ([HD] core
 * architecture: average the tokens of each chunk into Kbar, Vbar, Kbar^R;
 * [LH] Component 1 steps 1-3; [LH] Component 2: document-wise RoPE, every
 * document's positions start at 0; [WC] mechanism 3, offline encoding).
 * For chunk j of document i (in-document tokens [j*C, min(L_i,(j+1)*C))):
 *   kbar  = mean of R(t) K_t   (t = in-document position)
 *   vbar  = mean of V_t,   krbar = mean of KR_t   (no RoPE on values or router keys)
 * accumulated in fp32, rounded once to the bank dtype (round to nearest
 * even); kr_inv_norm from the stored krbar; chunk_doc for these chunks.
 * K, V: [n_slab][h_kv][d], KR: [n_slab][h_r][d_r] hold the slab's tokens,
 * n_slab = doc_tok_off[doc_end] - doc_tok_off[doc_begin], token 0 being the
 * first token of doc_begin.  Needs the host offset arrays in *b.
 * Errors: MSA_ERR_ARG (null/misaligned, bad range, inconsistent layout,
 * rope too short for max_doc_len or wrong d), MSA_ERR_UNSUPPORTED (dtype,
 * d not 64/128, d_r not 64/128/256 -- 256, a router twice the head width, for
 * bf16 banks -- or h_r * d_r > 1024).
 */
int msa_pool_memory(const msa_bank *b, const void *K, const void *V, const void *KR, int32_t doc_begin,
                    int32_t doc_end, const msa_rope *rope, void *stream);

/*
 * Router projection ([HD] core architecture of the learnable memory routing
 * layer: projectors map hidden states to the router query Q^R and, at
 * encoding time, to the router key K^R of every memory token; [HD] parameter
 * advice: router width 2-4x the head dimension):
 *   Y[r][o] = sum_i X[r][i] * W[o][i]
 * X [rows][hidden], W [out][hidden] (one row per output feature, i.e.
 * h_r * d_r rows), Y [rows][out]; all bf16, accumulated in fp32 and rounded
 * once (nearest even).  rows >= 0 (0 enqueues nothing), hidden a positive
 * multiple of 64, out a positive multiple of 128.  Y reshaped as
 * [rows][h_r][d_r] is the QR argument of msa_route_score, or the KR slab of
 * msa_pool_memory.  Errors: MSA_ERR_ARG (null/misaligned pointers, sizes).
 */
int msa_router_project(const void *X, const void *W, int64_t rows, int32_t hidden, int32_t out, void *Y,
                       void *stream);

/* Workspace bytes msa_route_score needs for these sizes (0 = none; 0 on invalid sizes). */
size_t msa_route_workspace_bytes(const msa_bank *b, int32_t n_q, int32_t t_r);

/*
 * Router scan with the document reduction ([LH] Component 1, key formula:
 * S = max over query tokens of the head-mean of cos(Q^R_t,h, Kbar^R_ij,h);
 * [HD] core architecture: cosine, mean over heads, max over tokens):
 *   s_chunk[q][c] = max_{t < t_r} (1/h_r) sum_h <QR[q,t,h], krbar[c,h]> / (||QR[q,t,h]|| ||krbar[c,h]||)
 *   s_doc[q][i]   = max over the chunks c of document i of s_chunk[q][c]
 * (the document score is the max over its chunks; cosine 0 for a zero norm).
 * qr: [n_q][t_r][h_r][d_r] bank dtype; s_doc: [n_q][n_docs] fp32;
 * s_chunk: [n_q][n_chunks] fp32 or NULL; ws: msa_route_workspace_bytes bytes
 * (16-byte aligned; may be NULL when that is 0).  max_wg_per_cu: 0 sizes the
 * streaming scan's persistent grid to every workgroup that stays resident
 * (fastest when the scan runs alone); n >= 1 caps it at n workgroups per
 * compute unit, which leaves room for kernels on other streams (a decode
 * pipeline overlapping scans and the top-k/attention of earlier steps uses
 * 1).  The results do not depend on it.  Errors: MSA_ERR_ARG (also
 * max_wg_per_cu < 0), MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE.
 */
int msa_route_score(const msa_bank *b, const void *qr, int32_t n_q, int32_t t_r, float *s_doc, float *s_chunk,
                    void *ws, size_t ws_bytes, int32_t max_wg_per_cu, void *stream);

/* Workspace bytes msa_topk needs for these sizes (0 on invalid sizes). */
size_t msa_topk_workspace_bytes(int32_t n_q, int32_t n_docs, int32_t k);

/*
 * Top-k document selection ([LH] Component 1, select the Top-k documents;
 * [HD] Top-k selection mechanism): for each query, the k documents with the
 * largest s_doc, sorted by descending score, ties to the lower index.
 * s_doc: [n_q][n_docs] fp32 (finite); idx: [n_q][k] int32; val: [n_q][k] fp32.
 * Errors: MSA_ERR_ARG (k < 1, k > n_docs, k > 256, null/misaligned),
 * MSA_ERR_WORKSPACE.
 */
int msa_topk(const float *s_doc, int32_t n_q, int32_t n_docs, int32_t k, int32_t *idx, float *val, void *ws,
             size_t ws_bytes, void *stream);

/* Workspace bytes msa_sparse_attend needs for these sizes on the current
 * device (0 on invalid sizes; the amount depends on the device's compute-unit
 * count, by which the work of single-token queries is split). */
size_t msa_attend_workspace_bytes(const msa_bank *b, int32_t n_q, int32_t T, int32_t L_loc, int32_t h_q, int32_t k);

/*
 * Sparse attention ([LH] Component 1, last step: the selected documents'
 * compressed KV concatenated with the query's local KV; [HD] core
 * architecture; [LH] Component 2 and [HD] position encoding: the active
 * context uses global RoPE starting at position k):
 * for query q, query token t (local index s_t = L_loc - T + t, position
 * pos0 + s_t) and q-head h (KV head h / (h_q / h_kv)):
 *   keys   = [kbar rows of the chunks of idx[q][0..k) in rank order ; R(pos0 + s) K_loc[q][s]]
 *   values = [vbar rows ; V_loc[q][s]]
 *   O[q][t][h] = softmax(scale * <R(pos0 + s_t) Q[q][t][h], keys>) . values
 * with every memory key visible and local key s visible when s <= s_t.
 * Q: [n_q][T][h_q][d]; K_loc, V_loc: [n_q][L_loc][h_kv][d] (before RoPE);
 * idx: [n_q][k] int32 document ids in [0, n_docs) (device memory the host
 * does not read: a query whose ids include one outside that range gets NaN
 * in every element of its output instead of an error code); O:
 * [n_q][T][h_q][d], bank dtype.  Errors: MSA_ERR_ARG (T > L_loc, h_q % h_kv,
 * rope too short for pos0 + L_loc, ...), MSA_ERR_UNSUPPORTED,
 * MSA_ERR_WORKSPACE.
 */
int msa_sparse_attend(const msa_bank *b, const void *Q, const void *K_loc, const void *V_loc, int32_t n_q, int32_t T,
                      int32_t L_loc, int32_t h_q, const int32_t *idx, int32_t k, int32_t pos0, float scale,
                      const msa_rope *rope, void *O, void *ws, size_t ws_bytes, void *stream);

/*
 * Measurement aid (no part of the method): reads the bank's router keys,
 * inverse norms and chunk->document ids with exactly the access pattern,
 * grid and tile order of the decode router scan (t_r = 1), without its
 * arithmetic, and writes one 128-byte record per pair of 16-chunk tiles into ws.  Its
 * duration is the practical floor of msa_route_score's scan on this device
 * (the nominal HBM peak is not reachable by any access pattern); bench.py
 * reports the scan against both.  bf16 banks with h_r = 8, d_r = 128 only
 * (else MSA_ERR_UNSUPPORTED).  ws: at least msa_route_workspace_bytes(b, 1, 1)
 * bytes, 16-byte aligned, contents overwritten (MSA_ERR_WORKSPACE otherwise).
 */
int msa_scan_read_probe(const msa_bank *b, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes msa_layer_forward needs for these sizes (0 on invalid sizes). */
size_t msa_layer_workspace_bytes(const msa_bank *b, int32_t n_q, int32_t T, int32_t t_r, int32_t L_loc, int32_t h_q,
                                 int32_t k);

/*
 * One routed layer ([LH] overall architecture; [WC] mechanism 3, online
 * routing then sparse generation): msa_route_score over the t_r router
 * tokens QR [n_q][t_r][h_r][d_r], msa_topk, then msa_sparse_attend of the T
 * query tokens, all on `stream` with no host synchronisation.
 * idx [n_q][k] int32, val [n_q][k] fp32 and O are outputs; s_doc
 * [n_q][n_docs] fp32 is an optional output (NULL to skip).
 * stage_events: NULL, or 4 hipEvent_t (as void*) recorded on `stream` just
 * before and just after the router-scan kernel, after the top-k (which
 * includes any per-document resolve step) and after the attention.
 * Errors: as the three calls, plus MSA_ERR_WORKSPACE.
 */
int msa_layer_forward(const msa_bank *b, const void *Q, const void *K_loc, const void *V_loc, const void *QR,
                      int32_t n_q, int32_t T, int32_t t_r, int32_t L_loc, int32_t h_q, int32_t k, int32_t pos0,
                      float scale, const msa_rope *rope, void *O, int32_t *idx, float *val, float *s_doc, void *ws,
                      size_t ws_bytes, void *const *stage_events, void *stream);

/*
 * A Memory Interleave re-routing round ([HD] sparse strategy: routing
 * alternates with generation and is redone after every round; [HD] practical
 * advice: re-route after each iteration to use the updated context; [LH]
 * Component 3): the layer of msa_layer_forward for a round whose router
 * tokens are the previous round's plus t_new new ones, given the previous
 * round's document scores.  The router score is a max over router tokens, so
 *   s_doc[q][i] = max(s_doc_prev[q][i], max over the t_new new tokens' scores of document i)
 * equals the score over all of the round's router tokens (the same value
 * msa_layer_forward computes from all of them); only the new tokens are
 * scanned.  Top-k and attention then run as in msa_layer_forward.
 * QR_new: [n_q][t_new][h_r][d_r], the new router tokens only; s_doc_prev:
 * [n_q][n_docs] fp32 input (the previous round's s_doc, e.g. from
 * msa_layer_forward over the first round's tokens); s_doc: optional output of
 * this round's scores, may be s_doc_prev itself (updated in place).  Other
 * arguments as msa_layer_forward with t_r = t_new; workspace
 * msa_layer_workspace_bytes(b, n_q, T, t_new, L_loc, h_q, k).  Errors: as
 * msa_layer_forward, plus MSA_ERR_ARG for a null or misaligned s_doc_prev.
 */
int msa_layer_forward_reroute(const msa_bank *b, const void *Q, const void *K_loc, const void *V_loc,
                              const void *QR_new, int32_t n_q, int32_t T, int32_t t_new, int32_t L_loc, int32_t h_q,
                              int32_t k, int32_t pos0, float scale, const msa_rope *rope, const float *s_doc_prev,
                              void *O, int32_t *idx, float *val, float *s_doc, void *ws, size_t ws_bytes,
                              void *const *stage_events, void *stream);

/*
 * msa_layer_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and results, with the workspace taken from a static device
 * array of MSA_STATIC_WORKSPACE_BYTES that the library holds on every GPU it
 * runs on until the process ends.  The call allocates nothing.  It serves
 * every layer whose msa_layer_workspace_bytes is at most that size (the
 * 100M-token decode layer of 16 single-token queries and k = 16 needs about
 * 8 MiB); larger ones fail with MSA_ERR_WORKSPACE before anything is enqueued.
 * Every call on one GPU shares that GPU's array (the kernels reset whatever
 * must start from zero): calls that overlap on one GPU, on any streams, race
 * and must be serialised by the caller.  The first call on a device looks up
 * the array's address there (no allocation).  Arguments, outputs and errors as
 * msa_layer_forward.
 */
#define MSA_STATIC_WORKSPACE_BYTES (16u << 20)
int msa_layer_forward_noalloc(const msa_bank *b, const void *Q, const void *K_loc, const void *V_loc, const void *QR,
                              int32_t n_q, int32_t T, int32_t t_r, int32_t L_loc, int32_t h_q, int32_t k, int32_t pos0,
                              float scale, const msa_rope *rope, void *O, int32_t *idx, float *val, float *s_doc,
                              void *const *stage_events, void *stream);

/*
 * The two halves of msa_layer_forward, for callers that overlap independent
 * batches (the router scan of one batch streams the bank while the top-k and
 * attention of the previous one run on another stream -- the pages overlap
 * the loading of the selected documents with the search, [HD] key
 * engineering details).  msa_layer_route runs the router scan into the layer
 * workspace (and into s_doc, when given); msa_layer_select_attend then
 * completes the document scores, selects the top-k and attends.  Called in
 * this order on one workspace, with the same sizes and the same s_doc (or
 * NULL both times), they enqueue exactly the kernels of msa_layer_forward:
 * the outputs are identical.  The two calls may use different streams; the
 * caller orders the second after the first (e.g. with an event) and keeps the
 * workspace and s_doc untouched in between.  Workspace:
 * msa_layer_workspace_bytes.  Errors: as msa_layer_forward.
 */
int msa_layer_route(const msa_bank *b, const void *QR, int32_t n_q, int32_t T, int32_t t_r, int32_t L_loc,
                    int32_t h_q, int32_t k, float *s_doc, void *ws, size_t ws_bytes, void *stream);
int msa_layer_select_attend(const msa_bank *b, const void *Q, const void *K_loc, const void *V_loc, int32_t n_q,
                            int32_t T, int32_t t_r, int32_t L_loc, int32_t h_q, int32_t k, int32_t pos0, float scale,
                            const msa_rope *rope, void *O, int32_t *idx, float *val, float *s_doc, void *ws,
                            size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
