// Top-k document selection (Lighthouse digest, Component 1: keep the Top-k
// documents; hotdry blog, Top-k selection mechanism): the k largest scores
// per query, sorted by descending score, ties to the lower document index.
//
// Every document becomes one distinct 64-bit composite
//   (order-preserving score key << 32) | (0xFFFFFFFF - doc)
// so "larger composite" is exactly "higher score, then lower index": the
// selection is unique and independent of thread order.
//   pass 1: the top-k of each (query, slice) by an 8-bit radix select held in
//           registers (MSB first, stopping as soon as the boundary digit bin is
//           taken whole): for k <= 32 one wave per slice of 512 documents (its
//           own LDS histogram and shuffles, no workgroup barrier), else one
//           256-thread workgroup per slice of 2048 (per-wave histograms);
//   pass 2: one workgroup per query selects the top-k of the candidates
//           the same way (from registers when they fit, 2048 per query) and
//           sorts them (bitonic, in LDS).
// Up to 8K documents per query a single pass does it all: one 1024-thread
// workgroup per query holds the whole row in registers (24 composites per
// thread), selects, compacts the k winners and sorts them.
// The scores are read as fp32, as order-preserving keys, or resolved from the
// router scan's per-tile records (single-writer scan: the documents that
// touch a tile edge are resolved here, and stored, while loading).
#include <algorithm>

#include "msa_device.hpp"
#include "msa_internal.hpp"
#include "select_wave.hpp"

namespace msa {
namespace {

constexpr int TK_THREADS = 256;
constexpr int TK_SLICE = 2048;
constexpr int TK_MAX_K = 256;

struct SelShared {
  uint32_t hist[256];
  int32_t wave_tot[TK_THREADS / 64];
  uint32_t bin;      // chosen digit
  uint32_t above;    // elements with a larger digit among the matching ones
  uint32_t in_bin;   // elements in the chosen bin
};

// Single-pass limit (documents per query).
constexpr int TOPK_SINGLE_MAX = 8192;

// Exclusive prefix sum over the block; returns this thread's offset, *total.
__device__ int block_excl_scan(int v, SelShared &sh, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh.wave_tot[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < TK_THREADS / 64; ++w) {
    if (w < wave) base += sh.wave_tot[w];
    tot += sh.wave_tot[w];
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Radix select of the `need` largest of n distinct composites get(i), i < n.
// Returns (shift, prefix): the selected elements are those with
// (v >> shift) >= (prefix >> shift); exactly `need` of them.
template <typename Get>
__device__ void radix_select(Get get, int64_t n, uint32_t need, SelShared &sh, int *out_shift, uint64_t *out_prefix) {
  uint64_t prefix = 0;
  int shift = 56;
  for (;; shift -= 8) {
    for (int b = threadIdx.x; b < 256; b += TK_THREADS) sh.hist[b] = 0;
    __syncthreads();
    for (int64_t base = 0; base < n; base += TK_THREADS) {
      const int64_t i = base + threadIdx.x;
      const uint64_t v = i < n ? get(i) : 0;
      const bool match = i < n && ((shift == 56) || ((v ^ prefix) >> (shift + 8)) == 0);
      const uint32_t digit = (uint32_t)(v >> shift) & 255;
      if (shift == 56) hist_add_wave(sh.hist, digit, match);
      else if (match) atomicAdd(&sh.hist[digit], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l owns bins 255-4l .. 252-4l (descending digit order)
      const int lane = threadIdx.x;
      uint32_t c[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = sh.hist[255 - 4 * lane - j];
        s += c[j];
      }
      uint32_t incl = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      const unsigned long long m = __ballot(incl >= need);
      const int first = __ffsll((long long)m) - 1;
      if (lane == first) {
        uint32_t cum = incl - s;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (cum + c[j] >= need) {
            sh.bin = 255 - 4 * lane - j;
            sh.above = cum;
            sh.in_bin = c[j];
            break;
          }
          cum += c[j];
        }
      }
    }
    __syncthreads();
    const uint32_t bin = sh.bin, above = sh.above, in_bin = sh.in_bin;
    __syncthreads();
    prefix |= (uint64_t)bin << shift;
    need -= above;
    if (in_bin == need || shift == 0) break;
  }
  *out_shift = shift;
  *out_prefix = prefix;
}

__global__ __launch_bounds__(TK_THREADS) void topk_pass2(const uint64_t *cand, int64_t n_cand, int k, int kpad,
                                                           int32_t *idx, float *val) {
  __shared__ SelShared sh;
  __shared__ uint64_t sel[TK_MAX_K];
  const int q = blockIdx.x;
  const uint64_t *c = cand + (int64_t)q * n_cand;
  auto get = [&](int64_t i) -> uint64_t { return c[i]; };
  int shift;
  uint64_t prefix;
  radix_select(get, n_cand, (uint32_t)k, sh, &shift, &prefix);
  for (int j = threadIdx.x; j < kpad; j += TK_THREADS) sel[j] = 0;
  __syncthreads();
  int written = 0;
  for (int64_t base = 0; base < n_cand; base += TK_THREADS) {
    const int64_t i = base + threadIdx.x;
    uint64_t v = 0;
    int f = 0;
    if (i < n_cand) {
      v = c[i];
      f = v != 0 && (v >> shift) >= (prefix >> shift);
    }
    int tot;
    const int pos = block_excl_scan(f, sh, &tot);
    if (f) sel[written + pos] = v;
    written += tot;
  }
  __syncthreads();
  // bitonic sort, descending
  for (int size = 2; size <= kpad; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < kpad; i += TK_THREADS) {
        const int j = i ^ stride;
        if (j > i) {
          const uint64_t x = sel[i], y = sel[j];
          const bool desc = (i & size) == 0;
          if (desc ? (x < y) : (x > y)) {
            sel[i] = y;
            sel[j] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int r = threadIdx.x; r < k; r += TK_THREADS) {
    const uint64_t v = sel[r];
    idx[(int64_t)q * k + r] = (int32_t)(0xFFFFFFFFu - (uint32_t)v);
    val[(int64_t)q * k + r] = key_score((uint32_t)(v >> 32));
  }
}

// ---- selection over register-resident composites ------------------------------
template <int WAVES>
struct RegShared {
  uint32_t hist[WAVES][256];  // per-wave histograms
  uint32_t total[256];
  int32_t wave_tot[WAVES];
  uint32_t bin, above, in_bin;
};

// Composite of document `doc` (< n_docs) for query q from the score source.
template <int MODE>
__device__ __forceinline__ uint64_t load_composite(const TopkSrc &src, int q, int n_docs, int doc) {
  const int64_t at = (int64_t)q * n_docs + doc;
  uint32_t key;
  if constexpr (MODE == TopkSrc::KEYS) {
    key = src.keys[at];
    if (src.scores) src.scores[at] = key_score(key);  // the document scores for the caller, when asked
  } else if constexpr (MODE == TopkSrc::SCORES) {
    key = score_key(src.scores[at]);
  } else {
    const float v = edge_doc_score(src.edges, src.doc_chunk_off, n_docs, src.t_r, q, doc);
    src.scores[at] = v;  // complete the document scores for the caller
    key = score_key(v);
  }
  return composite(key, doc);
}

// Radix select of the `need` largest nonzero composites held ITEMS per thread
// by a THREADS-wide workgroup.  Returns (shift, prefix): the selected are the v
// with (v >> shift) >= (prefix >> shift), exactly `need` of them.
template <int ITEMS, int THREADS>
__device__ void select_regs(const uint64_t (&v)[ITEMS], uint32_t need, RegShared<THREADS / 64> &sh, int *out_shift,
                            uint64_t *out_prefix) {
  constexpr int WAVES = THREADS / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t prefix = 0;
  int shift = 56;
  for (;; shift -= 8) {
    for (int e = tid; e < WAVES * 256; e += THREADS) (&sh.hist[0][0])[e] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const bool match = v[j] != 0 && ((shift == 56) || ((v[j] ^ prefix) >> (shift + 8)) == 0);
      const uint32_t digit = (uint32_t)(v[j] >> shift) & 255;
      if (shift == 56) hist_add_wave(sh.hist[wave], digit, match);
      else if (match) atomicAdd(&sh.hist[wave][digit], 1u);
    }
    __syncthreads();
    for (int b = tid; b < 256; b += THREADS) {
      uint32_t t = 0;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) t += sh.hist[w][b];
      sh.total[b] = t;
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns bins 255-4l .. 252-4l (descending digit order)
      uint32_t c[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = sh.total[255 - 4 * lane - j];
        s += c[j];
      }
      uint32_t incl = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      const unsigned long long m = __ballot(incl >= need);
      const int first = __ffsll((long long)m) - 1;
      if (lane == first) {
        uint32_t cum = incl - s;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (cum + c[j] >= need) {
            sh.bin = 255 - 4 * lane - j;
            sh.above = cum;
            sh.in_bin = c[j];
            break;
          }
          cum += c[j];
        }
      }
    }
    __syncthreads();
    const uint32_t bin = sh.bin, above = sh.above, in_bin = sh.in_bin;
    prefix |= (uint64_t)bin << shift;
    need -= above;
    if (in_bin == need || shift == 0) break;
  }
  *out_shift = shift;
  *out_prefix = prefix;
}

// Writes the selected composites to out[0 ..) (in thread order); returns their number.
template <int ITEMS, int THREADS>
__device__ int compact_regs(const uint64_t (&v)[ITEMS], int shift, uint64_t prefix, RegShared<THREADS / 64> &sh,
                            uint64_t *out) {
  constexpr int WAVES = THREADS / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) cnt += (v[j] != 0 && (v[j] >> shift) >= (prefix >> shift));
  int x = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh.wave_tot[wave] = x;
  __syncthreads();
  int pos = x - cnt, total = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    if (w < wave) pos += sh.wave_tot[w];
    total += sh.wave_tot[w];
  }
#pragma unroll
  for (int j = 0; j < ITEMS; ++j)
    if (v[j] != 0 && (v[j] >> shift) >= (prefix >> shift)) out[pos++] = v[j];
  return total;
}

// ---- pass 1: the top-k of each (query, slice) ------------------------------------
constexpr int P1_ITEMS = TK_SLICE / TK_THREADS;

template <int MODE>
__global__ __launch_bounds__(TK_THREADS) void topk_pass1(TopkSrc src, int n_docs, int k, int n_slices,
                                                           uint64_t *cand) {
  __shared__ RegShared<TK_THREADS / 64> sh;
  const int q = blockIdx.y, slice = blockIdx.x, tid = threadIdx.x;
  const int lo = slice * TK_SLICE;
  const int n = std::min(TK_SLICE, n_docs - lo);
  const uint32_t kk = (uint32_t)std::min(k, n);
  uint64_t v[P1_ITEMS];
#pragma unroll
  for (int j = 0; j < P1_ITEMS; ++j) {
    const int i = j * TK_THREADS + tid;  // coalesced
    v[j] = i < n ? load_composite<MODE>(src, q, n_docs, lo + i) : 0;
  }
  int shift;
  uint64_t prefix;
  select_regs<P1_ITEMS, TK_THREADS>(v, kk, sh, &shift, &prefix);
  uint64_t *out = cand + ((int64_t)q * n_slices + slice) * k;
  compact_regs<P1_ITEMS, TK_THREADS>(v, shift, prefix, sh, out);
  for (int j = kk + tid; j < k; j += TK_THREADS) out[j] = 0;
}

// ---- pass 1 for small k: one wave per (query, slice of 512 documents) ---------
// Each wave selects on its own, with its own LDS histogram and shuffles: no
// workgroup barrier, so a radix pass costs a few LDS round trips.
constexpr int WS_SLICE = 512;
constexpr int WS_ITEMS = WS_SLICE / 64;
constexpr int WS_MAX_K = 32;  // k up to this uses the wave pass (k <= slice / 16)

// The wave's k largest of its slice's composites (v[j]: document j * 64 + lane,
// 0 past the slice) written to out[0, k) in descending order, padded with
// zeros (k <= WS_MAX_K).  sel: 128 composites of LDS scratch for the wave.
__device__ __forceinline__ void wave_slice_select(const uint64_t (&v)[WS_ITEMS], int n, int k, uint32_t *hist,
                                                  uint64_t *sel, uint64_t *out, int lane) {
  const uint32_t kk = (uint32_t)std::min(k, n);
  const uint64_t r = wave_topk_sorted_fast<WS_ITEMS>(v, kk, hist, sel);  // lane r: rank r, 0 past kk
  if (lane < k) out[lane] = r;
}

template <int MODE>
__global__ __launch_bounds__(256) void topk_pass1_wave(TopkSrc src, int n_docs, int k, int n_slices,
                                                        uint64_t *cand) {
  __shared__ __align__(16) uint32_t hist[4][256];
  __shared__ __align__(16) uint64_t sel[4][128];
  const int q = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slice = blockIdx.x * 4 + wave;
  if (slice >= n_slices) return;  // whole wave; no workgroup barrier below
  const int lo = slice * WS_SLICE;
  const int n = std::min(WS_SLICE, n_docs - lo);
  uint64_t v[WS_ITEMS];
#pragma unroll
  for (int j = 0; j < WS_ITEMS; ++j) {
    const int i = j * 64 + lane;  // coalesced
    v[j] = i < n ? load_composite<MODE>(src, q, n_docs, lo + i) : 0;
  }
  wave_slice_select(v, n, k, hist[wave], sel[wave], cand + ((int64_t)q * n_slices + slice) * k, lane);
}

// ---- pass 1 from the scan's records, RS_Q queries per workgroup -----------------
// The workgroup first completes the slice's document scores for its RS_Q
// queries with the query fastest across lanes (RS_Q lanes read adjacent words
// of one document's row of stored scores or records and share its chunk-range
// loads), keeps them in LDS and writes them to src.scores; then wave w selects
// query q0 + w's k from LDS as the wave pass does.  Measured at 16 queries x
// 23,048 documents, k = 16: resolve + pass 1 16.0 us as two kernels, 14.0 us
// fused with RS_Q = 4 (8: 14.2; 16 waves per workgroup: 18.6, four selecting
// waves per SIMD on a quarter of the CUs); without the batched loads below
// 20 us.
constexpr int RS_Q = 4;                    // queries per workgroup (one selecting wave each)
constexpr int RS_ITEMS = WS_SLICE / 64;    // documents per thread: j = u * 64 + tid / RS_Q
static_assert(RS_Q <= 16 && 16 % RS_Q == 0, "a workgroup's queries share one 16-query row block");
static_assert(RS_ITEMS == WS_ITEMS, "the resolve and the selection cover the same slice");

// edge_range_score for N documents of one query with their loads batched (a
// loop per document would wait on each one in turn): the chunk ranges, then
// in one round each document's stored score or first record together with
// the records of its next EB units, then one round per further unit (loads
// clamped to the document's last unit, masked after)
constexpr int EB = 2;  // further units read with the first record: a document of <= 65 chunks needs no more
template <int N>
__device__ __forceinline__ void edge_scores_batched(const EdgeLayout &L, const int64_t *doc_chunk_off, int n_docs,
                                                    int t_r, int q, const int (&doc)[N], float (&out)[N]) {
  const int rb = t_r == 1 ? q / 16 : q;
  const int r = t_r == 1 ? q % 16 : 0;
  const float *rec = L.rec + (int64_t)rb * L.n_units * 32;
  int64_t c0[N], c1[N];
#pragma unroll
  for (int u = 0; u < N; ++u) {
    c0[u] = doc_chunk_off[doc[u]];
    c1[u] = doc_chunk_off[doc[u] + 1] - 1;
  }
  int64_t ta[N], tb[N];
  int extra = 0;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    ta[u] = c0[u] / 32;
    tb[u] = c1[u] / 32;
    const bool one = ta[u] == tb[u];
    const bool interior = one && (c0[u] % 32) != 0 && (c1[u] % 32) != 31;
    const float *p = interior ? L.dsc + ((int64_t)rb * n_docs + doc[u]) * L.rw + r
                              : rec + ta[u] * 32 + ((one && (c0[u] % 32) == 0) ? 0 : 16) + r;
    out[u] = *p;
    extra = max(extra, (int)(tb[u] - ta[u]));
  }
  float xb[EB][N];
#pragma unroll
  for (int e = 1; e <= EB; ++e)
#pragma unroll
    for (int u = 0; u < N; ++u) xb[e - 1][u] = rec[min(ta[u] + e, tb[u]) * 32 + r];
#pragma unroll
  for (int e = 1; e <= EB; ++e)
#pragma unroll
    for (int u = 0; u < N; ++u)
      if (ta[u] + e <= tb[u]) out[u] = fmaxf(out[u], xb[e - 1][u]);
  for (int e = EB + 1; e <= extra; ++e) {
    float x[N];
#pragma unroll
    for (int u = 0; u < N; ++u) x[u] = rec[min(ta[u] + e, tb[u]) * 32 + r];
#pragma unroll
    for (int u = 0; u < N; ++u)
      if (ta[u] + e <= tb[u]) out[u] = fmaxf(out[u], x[u]);
  }
}

__global__ __launch_bounds__(64 * RS_Q) void topk_pass1_resolve(TopkSrc src, int n_q, int n_docs, int k,
                                                                 int n_slices, uint64_t *cand) {
  __shared__ float sS[RS_Q][WS_SLICE + 1];
  __shared__ __align__(16) uint32_t hist[RS_Q][256];
  __shared__ __align__(16) uint64_t sel[RS_Q][128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slice = blockIdx.x, q0 = blockIdx.y * RS_Q;
  const int lo = slice * WS_SLICE;
  const int n = std::min(WS_SLICE, n_docs - lo);
  const int nq = std::min(RS_Q, n_q - q0);
  const int qq = tid % RS_Q;  // this thread's query; its documents j = u * 64 + tid / RS_Q
  if (qq < nq) {
    int doc[RS_ITEMS];
#pragma unroll
    for (int u = 0; u < RS_ITEMS; ++u) doc[u] = lo + std::min(u * 64 + tid / RS_Q, n - 1);
    float sv[RS_ITEMS];
    edge_scores_batched<RS_ITEMS>(src.edges, src.doc_chunk_off, n_docs, src.t_r, q0 + qq, doc, sv);
#pragma unroll
    for (int u = 0; u < RS_ITEMS; ++u) {
      const int j = u * 64 + tid / RS_Q;
      if (j < n) {
        src.scores[(int64_t)(q0 + qq) * n_docs + lo + j] = sv[u];
        sS[qq][j] = sv[u];
      }
    }
  }
  __syncthreads();
  if (wave >= nq) return;  // whole wave; no barrier below
  uint64_t v[WS_ITEMS];
#pragma unroll
  for (int j = 0; j < WS_ITEMS; ++j) {
    const int i = j * 64 + lane;
    v[j] = i < n ? composite(score_key(sS[wave][i]), lo + i) : 0;
  }
  wave_slice_select(v, n, k, hist[wave], sel[wave], cand + ((int64_t)(q0 + wave) * n_slices + slice) * k, lane);
}

// ---- pass 2 over register-resident candidates (up to 8 per thread) ----------
constexpr int P2_THREADS = 256;
constexpr int P2_ITEMS = 8;

__global__ __launch_bounds__(P2_THREADS) void topk_pass2_regs(const uint64_t *cand, int n_cand, int k, int kpad,
                                                                int32_t *idx, float *val) {
  __shared__ RegShared<P2_THREADS / 64> sh;
  __shared__ uint64_t sel[TK_MAX_K];
  const int q = blockIdx.x, tid = threadIdx.x;
  const uint64_t *c = cand + (int64_t)q * n_cand;
  uint64_t v[P2_ITEMS];
#pragma unroll
  for (int j = 0; j < P2_ITEMS; ++j) {
    const int i = j * P2_THREADS + tid;
    v[j] = i < n_cand ? c[i] : 0;  // empty candidate slots are 0
  }
  int shift;
  uint64_t prefix;
  select_regs<P2_ITEMS, P2_THREADS>(v, (uint32_t)k, sh, &shift, &prefix);
  for (int e = tid; e < kpad; e += P2_THREADS) sel[e] = 0;
  __syncthreads();
  compact_regs<P2_ITEMS, P2_THREADS>(v, shift, prefix, sh, sel);
  __syncthreads();
  for (int size = 2; size <= kpad; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (tid < kpad) {
        const int j = tid ^ stride;
        if (j > tid) {
          const uint64_t a = sel[tid], b = sel[j];
          const bool desc = (tid & size) == 0;
          if (desc ? (a < b) : (a > b)) {
            sel[tid] = b;
            sel[j] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  if (tid < k) {
    const uint64_t w64 = sel[tid];
    idx[(int64_t)q * k + tid] = (int32_t)(0xFFFFFFFFu - (uint32_t)w64);
    val[(int64_t)q * k + tid] = key_score((uint32_t)(w64 >> 32));
  }
}

// ---- single pass: one 1024-thread workgroup per query ---------------------
constexpr int TS_THREADS = 1024;
constexpr int TS_ITEMS = 24;

template <int MODE>
__global__ __launch_bounds__(TS_THREADS) void topk_single(TopkSrc src, int n_docs, int k, int kpad, int32_t *idx,
                                                             float *val) {
  __shared__ RegShared<TS_THREADS / 64> sh;
  __shared__ uint64_t sel[TK_MAX_K];
  const int q = blockIdx.x, tid = threadIdx.x;
  uint64_t v[TS_ITEMS];
#pragma unroll
  for (int j = 0; j < TS_ITEMS; ++j) {
    const int i = j * TS_THREADS + tid;  // coalesced
    v[j] = i < n_docs ? load_composite<MODE>(src, q, n_docs, i) : 0;
  }
  int shift;
  uint64_t prefix;
  select_regs<TS_ITEMS, TS_THREADS>(v, (uint32_t)k, sh, &shift, &prefix);
  for (int e = tid; e < kpad; e += TS_THREADS) sel[e] = 0;
  __syncthreads();
  compact_regs<TS_ITEMS, TS_THREADS>(v, shift, prefix, sh, sel);
  __syncthreads();
  for (int size = 2; size <= kpad; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (tid < kpad) {
        const int j = tid ^ stride;
        if (j > tid) {
          const uint64_t a = sel[tid], b = sel[j];
          const bool desc = (tid & size) == 0;
          if (desc ? (a < b) : (a > b)) {
            sel[tid] = b;
            sel[j] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  if (tid < k) {
    const uint64_t w64 = sel[tid];
    idx[(int64_t)q * k + tid] = (int32_t)(0xFFFFFFFFu - (uint32_t)w64);
    val[(int64_t)q * k + tid] = key_score((uint32_t)(w64 >> 32));
  }
}

// documents per pass-1 slice: 512 (one wave) for small k, else 2048 (one workgroup)
int slice_for(int k) { return k <= WS_MAX_K ? WS_SLICE : TK_SLICE; }
int n_slices_for(int n_docs, int k) { return (n_docs + slice_for(k) - 1) / slice_for(k); }

}  // namespace

bool topk_single_pass(int n_docs) { return n_docs <= TS_THREADS * TS_ITEMS && n_docs <= TOPK_SINGLE_MAX; }

size_t topk_ws_bytes(int n_q, int n_docs, int k) {
  if (topk_single_pass(n_docs)) return 0;
  return (size_t)n_q * n_slices_for(n_docs, k) * k * sizeof(uint64_t);
}

size_t topk_layer_ws_bytes(int n_q, int n_docs, int k) {
  // pass 1's candidates also where the layer runs pass 1 alone on a bank the
  // single pass could take (the attention makes the final selection)
  const size_t fused = topk_fused_candidates(n_docs, k) > 0 ? (size_t)n_q * n_slices_for(n_docs, k) * k * sizeof(uint64_t) : 0;
  return std::max(topk_ws_bytes(n_q, n_docs, k), fused);
}

template <int MODE>
hipError_t topk_launch(const TopkSrc &src, int n_q, int n_docs, int k, int32_t *idx, float *val, void *ws,
                       hipStream_t s) {
  int kpad = 1;
  while (kpad < k) kpad <<= 1;
  if (topk_single_pass(n_docs)) {
    hipLaunchKernelGGL(topk_single<MODE>, dim3(n_q), dim3(TS_THREADS), 0, s, src, n_docs, k, kpad, idx, val);
    return hipGetLastError();
  }
  const int ns = n_slices_for(n_docs, k);
  uint64_t *cand = static_cast<uint64_t *>(ws);
  if (slice_for(k) == WS_SLICE)
    hipLaunchKernelGGL(topk_pass1_wave<MODE>, dim3((ns + 3) / 4, n_q), dim3(256), 0, s, src, n_docs, k, ns, cand);
  else
    hipLaunchKernelGGL(topk_pass1<MODE>, dim3(ns, n_q), dim3(TK_THREADS), 0, s, src, n_docs, k, ns, cand);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_cand = (int64_t)ns * k;
  if (n_cand <= (int64_t)P2_THREADS * P2_ITEMS)
    hipLaunchKernelGGL(topk_pass2_regs, dim3(n_q), dim3(P2_THREADS), 0, s, cand, (int)n_cand, k, kpad, idx, val);
  else
    hipLaunchKernelGGL(topk_pass2, dim3(n_q), dim3(TK_THREADS), 0, s, cand, n_cand, k, kpad, idx, val);
  return hipGetLastError();
}

// The layer leaves the final selection to the attention kernel where it can.
int topk_fused_candidates(int n_docs, int k) {
  // one slice: the single pass is as short as pass 1 alone
  if (n_docs <= WS_SLICE || slice_for(k) != WS_SLICE) return 0;
  const int64_t n = (int64_t)n_slices_for(n_docs, k) * k;
  return n <= ATTEND_MAX_CAND ? (int)n : 0;
}

hipError_t launch_topk_pass1_keys(const TopkSrc &src, int n_q, int n_docs, int k, void *ws, hipStream_t s) {
  if (src.mode != TopkSrc::KEYS || slice_for(k) != WS_SLICE) return hipErrorInvalidValue;
  const int ns = n_slices_for(n_docs, k);
  hipLaunchKernelGGL(topk_pass1_wave<TopkSrc::KEYS>, dim3((ns + 3) / 4, n_q), dim3(256), 0, s, src, n_docs, k, ns,
                     static_cast<uint64_t *>(ws));
  return hipGetLastError();
}

hipError_t launch_topk_pass1_resolve(const TopkSrc &src, int n_q, int n_docs, int k, void *ws, hipStream_t s) {
  if (src.mode != TopkSrc::EDGES || slice_for(k) != WS_SLICE) return hipErrorInvalidValue;
  const int ns = n_slices_for(n_docs, k);
  hipLaunchKernelGGL(topk_pass1_resolve, dim3(ns, (n_q + RS_Q - 1) / RS_Q), dim3(64 * RS_Q), 0, s, src, n_q, n_docs,
                     k, ns, static_cast<uint64_t *>(ws));
  return hipGetLastError();
}

hipError_t launch_topk(const TopkSrc &src, int n_q, int n_docs, int k, int32_t *idx, float *val, void *ws,
                       hipStream_t s) {
  switch (src.mode) {
    case TopkSrc::SCORES: return topk_launch<TopkSrc::SCORES>(src, n_q, n_docs, k, idx, val, ws, s);
    case TopkSrc::KEYS: return topk_launch<TopkSrc::KEYS>(src, n_q, n_docs, k, idx, val, ws, s);
    default: return topk_launch<TopkSrc::EDGES>(src, n_q, n_docs, k, idx, val, ws, s);
  }
}

}  // namespace msa
