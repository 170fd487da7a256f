// Router scan with the document reduction fused into the MFMA epilogue.
//
// Score (Lighthouse digest, Component 1, key formula; hotdry blog, core
// architecture of the memory routing layer): for query q and chunk c,
//   S[q,c] = max_t (1/H_r) sum_h cos(Q^R[q,t,h], Kbar^R[c,h]),
// and the document score is the max of S over the document's chunks.
//
// Design (gfx950):
//  * the bank's router keys are streamed from HBM exactly once per row block
//    of 16 query-token rows; each lane loads 16 contiguous bytes of one chunk
//    row straight into the MFMA B operand (v_mfma_f32_16x16x32_bf16);
//  * the query fragments of the row block sit in LDS in operand order (one
//    conflict-free 16-byte read per lane per MFMA), their inverse norms
//    (times 1/H_r) next to them;
//  * cosines are formed in fp32 in the epilogue from the raw dot products:
//    dot * invQ[row,h] * invK[c,h] summed over heads, so no normalised bf16
//    copy of either side is made;
//  * max over the query tokens of a query runs across the lanes of the tile,
//    then a segmented max-scan over the runs of chunks that belong to one
//    document;
//  * persistent waves take tiles in an interleaved order (wave w: tiles w,
//    w + W, ...), so the waves stream one compact window of the bank;
//  * when every (query, document) score has a single writer (one query per
//    row, or one row block per query) the waves take their tiles in pairs of
//    consecutive tiles, carry the document open at the end of the first
//    tile into the second, and emit one coalesced 128-byte record per pair
//    with the max of its first and of its last document segment per query; a
//    document lying strictly inside the pair has its scores for the block's
//    rows stored as one 64-byte row of a document-major array; a small
//    second kernel then writes every document score from these -- no
//    atomics and no zero fill.  Stores inside the 1.65 GB read stream are
//    costly: 16 scattered 4-byte stores per interior document had cost the
//    scan 2-3 %, a record per tile instead of per pair another 3 %.
//    Otherwise each segment goes out as an order-preserving atomicMax on
//    uint32 keys.
#include <algorithm>
#include <atomic>

#include "msa_device.hpp"
#include "msa_internal.hpp"

// Prefetch depth of the key stream in heads, and the waves per SIMD the scan
// kernels are compiled for (launch bounds).
#define MSA_ROUTE_PD 2
#define MSA_ROUTE_WAVES 3

namespace msa {
namespace {

template <typename T>
__device__ __forceinline__ typename Frag<T>::type load_stream(const T *p) {
  return load_frag<T>(p);
}

__global__ void fill_u32_kernel(uint32_t *p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

__global__ void keys_from_scores_kernel(uint32_t *p, const float *init, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = score_key(init[i]);
}

__global__ void keys_to_scores_kernel(uint32_t *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = __float_as_uint(key_score(p[i]));
}

// Inclusive max-scan within runs of equal document over the 16 columns of a
// lane group (columns hold consecutive chunks); match[j] says whether column
// col - 2^j holds the same document.  The last column of a run then holds
// the run's max.
__device__ __forceinline__ float seg_scan16(float v, const bool (&match)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float nv = __shfl_up(v, 1 << j, 16);
    if (match[j]) v = fmaxf(v, nv);
  }
  return v;
}

template <typename T, int HR, int DR, bool EDGE>
__global__ __launch_bounds__(256, MSA_ROUTE_WAVES) void route_scan_kernel(RouteArgs a, int64_t n_tiles, int64_t n_waves) {
  using F = Frag<T>;
  using FT = typename F::type;
  constexpr int EL = F::EL, KW = F::KW, KS = DR / KW, NF = HR * KS;
  __shared__ FT qfrag[NF][64];
  __shared__ __align__(16) float qinv[HR][16];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, G = lane >> 4;
  const int rb = blockIdx.y;
  const int n_rows = a.n_q * a.t_r;
  const T *qr = static_cast<const T *>(a.qr);

  // rows of this lane: 16 rb + 4 G + i; a row block lies in one query when t_r % 16 == 0
  const bool uniform = (a.t_r % 16) == 0;
  int rowq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = rb * 16 + 4 * G + i;
    rowq[i] = row < n_rows ? row / a.t_r : -1;
  }
  // interleaved tile order: at any moment the waves stream one compact window
  const int64_t wave_id = (int64_t)blockIdx.x * 4 + wave;
  // wave w takes the pairs of consecutive tiles w, w + W, ... (tiles 2p, 2p + 1)
  auto tile_of = [&](int64_t j) { return 2 * (wave_id + (j >> 1) * n_waves) + (j & 1); };
  const int64_t t_lo = tile_of(0), t_hi = n_tiles;
  const T *krbar = static_cast<const T *>(a.krbar);

  // Prefetch ring: the key fragments of PD (tile, head) steps are in flight
  // while the MFMAs of the current step run; it streams across tile ends.
  // Inverse norms and document ids of the next tile are fetched one tile ahead.
  constexpr int PD = HR < MSA_ROUTE_PD ? HR : MSA_ROUTE_PD;
  static_assert(HR % PD == 0, "ring slots are reused across tiles: the depth must divide the head count");
  FT ring[PD][KS];
  float ik_cur[HR], ik_nxt[HR];
  int doc_cur = -1, doc_nxt = -1;
  auto lane_chunk = [&](int64_t tl) -> int64_t {
    const int64_t cp = tl * 16 + col;
    return cp < a.n_chunks ? cp : a.n_chunks - 1;
  };
  auto load_meta = [&](int64_t tl, float (&ik)[HR], int &doc) {
    const int64_t cp = lane_chunk(tl);
    const float *ip = a.kr_inv_norm + cp * HR;
    if constexpr (HR % 4 == 0) {
#pragma unroll
      for (int j = 0; j < HR / 4; ++j) {
        const float4 v = reinterpret_cast<const float4 *>(ip)[j];
        ik[4 * j] = v.x; ik[4 * j + 1] = v.y; ik[4 * j + 2] = v.z; ik[4 * j + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < HR; ++j) ik[j] = ip[j];
    }
    const int d = a.chunk_doc[cp];  // unconditional load (cp is clamped)
    doc = (tl * 16 + col < a.n_chunks) ? d : -1;
  };
  const T *kp_cur = krbar + lane_chunk(t_lo) * (HR * DR) + G * EL;
  const T *kp_nxt = kp_cur;
  // the key stream starts before the query staging below (unconditionally:
  // a wave without tiles reads a clamped, valid chunk and never uses it)
#pragma unroll
  for (int p = 0; p < PD; ++p)
#pragma unroll
    for (int s = 0; s < KS; ++s) ring[p][s] = load_stream<T>(kp_cur + p * DR + s * KW);
  load_meta(t_lo, ik_cur, doc_cur);

  // query fragments of rows [16 rb, 16 rb + 16) in MFMA A-operand order: all
  // loads in flight together, then written to LDS
  {
    constexpr int QPT = (NF * 64 + 255) / 256;
    FT qt[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int e = threadIdx.x + 256 * i;
      const int f = e >> 6, l = e & 63, h = f / KS, s = f % KS;
      const int row = rb * 16 + (l & 15);
      if constexpr (EL == 1) qt[i] = 0.f; else qt[i] = FT{};
      if (e < NF * 64 && row < n_rows) qt[i] = load_frag<T>(qr + ((int64_t)row * HR + h) * DR + s * KW + (l >> 4) * EL);
    }
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int e = threadIdx.x + 256 * i;
      if (e < NF * 64) qfrag[e >> 6][e & 63] = qt[i];
    }
  }
  __syncthreads();
  // (1/H_r) / ||Q^R[row, h]|| from the staged fragments (0 for a zero or absent row)
  if (threadIdx.x < 16 * HR) {
    const int r = threadIdx.x & 15, h = threadIdx.x >> 4;
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const FT v = qfrag[h * KS + s][16 * g + r];
        if constexpr (EL == 1) {
          ss += v * v;
        } else {
#pragma unroll
          for (int j = 0; j < EL; ++j) {
            const float x = (float)v[j];
            ss += x * x;
          }
        }
      }
    qinv[h][r] = ss > 0.f ? (1.0f / sqrtf(ss)) * (1.0f / HR) : 0.f;
  }
  __syncthreads();

#define MSA_QOP(f) qfrag[(f) + zoff][lane]

  // single writer: a record per pair of tiles (a 32-chunk unit); the open
  // document of the pair's first tile is carried into its second
  float carry[4] = {0.f, 0.f, 0.f, 0.f};  // running max of that document (per row)
  float rfirst[4] = {0.f, 0.f, 0.f, 0.f};  // the pair's first-segment maxima, once closed
  int cdoc = -2;                          // the carried document (-2: none)
  bool first_open = false;                // the pair's first document runs on into the second tile
  for (int64_t j = 0;; ++j) {
    const int64_t tile = tile_of(j);
    if (tile >= t_hi) break;
    const int kk = (int)(j & 1);  // first / second tile of the pair
    const int64_t tile_next = tile_of(j + 1);
    const int64_t c = tile * 16 + col;
    const bool cv = c < a.n_chunks;
    // The loads for the next tile are issued unconditionally (after the
    // wave's last tile they re-read this tile and are never used): loads
    // under a branch make the compiler's wait counts at the join assume the
    // branch was not taken, which drains every load in flight once per tile.
    const bool has_next = tile_next < t_hi;
    const int64_t tile_pf = has_next ? tile_next : tile;
    // (the last tile's stand-in loads read its own final PD heads, fetched
    // moments earlier, so they are served by L2 rather than HBM)
    kp_nxt = krbar + lane_chunk(tile_pf) * (HR * DR) + G * EL + (has_next ? 0 : (HR - PD) * DR);
    load_meta(tile_pf, ik_nxt, doc_nxt);
    // opaque zero: keeps the query-fragment LDS reads inside the loop rather
    // than hoisting all of Q into VGPRs (registers go to the prefetch ring)
    int zoff;
    asm volatile("s_mov_b32 %0, 0" : "=s"(zoff));
    f32x4 S = zero4();
#pragma unroll
    for (int h = 0; h < HR; ++h) {
      const int slot = h % PD;
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = mfma16(MSA_QOP(h * KS + s), ring[slot][s], acc);
      const float ik = ik_cur[h];
      const float4 iq = *reinterpret_cast<const float4 *>(&qinv[h][4 * G]);
      S[0] += acc[0] * (iq.x * ik);
      S[1] += acc[1] * (iq.y * ik);
      S[2] += acc[2] * (iq.z * ik);
      S[3] += acc[3] * (iq.w * ik);
      if (h + PD < HR) {
#pragma unroll
        for (int s = 0; s < KS; ++s) ring[slot][s] = load_stream<T>(kp_cur + (h + PD) * DR + s * KW);
      } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) ring[slot][s] = load_stream<T>(kp_nxt + (h + PD - HR) * DR + s * KW);
      }
      // keep the head steps in order: later heads' loads are not hoisted above this one
      __builtin_amdgcn_sched_barrier(0);
    }
#undef MSA_QOP
    const int doc = doc_cur;
    kp_cur = kp_nxt;
#pragma unroll
    for (int j = 0; j < HR; ++j) ik_cur[j] = ik_nxt[j];
    doc_cur = doc_nxt;
    // ---- epilogue: token max, then per-document max over runs of columns ----
    // (cross-lane reads are made by every lane: a lane that skips a shuffle
    // leaves its value undefined for the lanes that read it)
    const int d0 = __shfl(doc, 0, 16), d15 = __shfl(doc, 15, 16);
    const int doc_right = __shfl_down(doc, 1, 16);
    const bool tail = (col == 15) || (doc_right != doc);
    bool match[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int doc_left = __shfl_up(doc, 1 << j, 16);
      match[j] = col >= (1 << j) && doc_left == doc;
    }
    // last column holding the tile's first document (documents are contiguous)
    const unsigned long long same0 = __ballot(doc == d0);
    const int tail0 = __popcll((same0 >> (16 * G)) & 0xFFFFull) - 1;
    // the pair's tiles: a second tile follows this one in the same pair
    const bool pair2 = kk == 0 && has_next;
    const int dn0 = __shfl(doc_cur, 0, 16);  // (doc_cur now holds the next tile's documents)
    const bool cont = pair2 && d15 >= 0 && dn0 == d15;  // this tile's last document runs on into the next
    const int64_t n_units = (n_tiles + 1) / 2;
    float *erec = EDGE ? a.edges + (rb * n_units + (tile >> 1)) * 32 : nullptr;  // [2][16] floats
    // the pair ends with this tile; a pair of one tile (the bank's last tile
    // alone) holds no chunk 31 of its unit, so only its first segment is read
    const bool rec_now = kk == 1 || !pair2;
    if (uniform) {
      // every row of the block belongs to one query: max over the 16 rows first
      float v = fmaxf(fmaxf(S[0], S[1]), fmaxf(S[2], S[3]));
      v = fmaxf(v, __shfl_xor(v, 16, 64));
      v = fmaxf(v, __shfl_xor(v, 32, 64));
      const int q = rb * 16 / a.t_r;
      if (a.chunk_out && G == 0 && cv) {
        if constexpr (EDGE) reinterpret_cast<float *>(a.chunk_out)[(int64_t)q * a.n_chunks + c] = v;
        else atomicMax(a.chunk_out + (int64_t)q * a.n_chunks + c, score_key(v));
      }
      v = seg_scan16(cv ? v : -INFINITY, match);
      if constexpr (EDGE) {
        // (single writer with t_r % 16 == 0: the row block is query q, one row per document)
        if (kk == 1 && doc == cdoc) v = fmaxf(v, carry[0]);
        const float at_tail0 = __shfl(v, tail0, 16), at15 = __shfl(v, 15, 16);
        const int dfirst_open = kk == 1 && first_open ? cdoc : -2;
        const bool pair_first = kk == 0 ? doc == d0 : doc == dfirst_open;
        const bool pair_last = kk == 1 && doc == d15;  // (a pair of one tile has no last segment)
        const bool carried = kk == 0 && cont && doc == d15;
        if (G == 0 && tail && doc >= 0 && !pair_first && !pair_last && !carried)
          a.dsc[(int64_t)rb * a.n_docs + doc] = v;
        if (kk == 0) {
          first_open = cont && d0 == d15;
          rfirst[0] = at_tail0;
          carry[0] = at15;
          cdoc = cont ? d15 : -2;
        }
        if (rec_now) {
          const float first = (kk == 1 && first_open) ? at_tail0 : rfirst[0];
          if (G == 0 && col < 2) erec[col * 16] = col == 0 ? first : at15;
        }
      } else {
        if (G == 0 && tail && doc >= 0) atomicMax(a.doc_keys + (int64_t)q * a.n_docs + doc, score_key(v));
      }
    } else {
      float at_tail0[4], at15[4], sv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = rowq[i];
        float v = S[i];
        if (a.chunk_out && cv && q >= 0) {
          if constexpr (EDGE) reinterpret_cast<float *>(a.chunk_out)[(int64_t)q * a.n_chunks + c] = v;
          else atomicMax(a.chunk_out + (int64_t)q * a.n_chunks + c, score_key(v));
        }
        v = seg_scan16(cv ? v : -INFINITY, match);
        if constexpr (EDGE) {
          if (kk == 1 && doc == cdoc) v = fmaxf(v, carry[i]);
          at_tail0[i] = __shfl(v, tail0, 16);
          at15[i] = __shfl(v, 15, 16);
          sv[i] = v;
        } else {
          if (tail && doc >= 0 && q >= 0) atomicMax(a.doc_keys + (int64_t)q * a.n_docs + doc, score_key(v));
        }
      }
      if constexpr (EDGE) {
        // a document strictly inside the pair: its 16 rows as one 64-byte row
        // (rows past n_rows hold unused values)
        const int dfirst_open = kk == 1 && first_open ? cdoc : -2;
        const bool pair_first = kk == 0 ? doc == d0 : doc == dfirst_open;
        const bool pair_last = kk == 1 && doc == d15;  // (a pair of one tile has no last segment)
        const bool carried = kk == 0 && cont && doc == d15;
        if (tail && doc >= 0 && !pair_first && !pair_last && !carried)
          reinterpret_cast<float4 *>(a.dsc + ((int64_t)rb * a.n_docs + doc) * 16)[G] = float4{sv[0], sv[1], sv[2], sv[3]};
        float first[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) first[i] = (kk == 1 && first_open) ? at_tail0[i] : rfirst[i];
        if (kk == 0) {
          first_open = cont && d0 == d15;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            rfirst[i] = at_tail0[i];
            carry[i] = at15[i];
          }
          cdoc = cont ? d15 : -2;
        }
        // one 128-byte record per pair: lanes (G, col 0) hold the first-segment maxima
        // of rows 4G..4G+3, lanes (G, col 1) the last-segment maxima
        if (rec_now && col < 2) {
          const float *src = col == 0 ? (kk == 0 ? at_tail0 : first) : at15;
          *reinterpret_cast<float4 *>(erec + col * 16 + 4 * G) = float4{src[0], src[1], src[2], src[3]};
        }
      }
    }
  }
}

// Every document score (single-writer mode): a document spanning 32-chunk
// units ua..ub is the max of the last segment of ua and the first segment of
// every later unit it reaches (the records); a document strictly inside one
// unit is copied from the scan's document-major scores.
__global__ void resolve_docs_kernel(EdgeLayout L, const int64_t *doc_chunk_off, int n_q, int n_docs, int t_r,
                                    float *doc_scores) {
  // query fastest: the lanes of a wave read consecutive rows of the same records
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)n_q * n_docs) return;
  const int q = (int)(i % n_q), doc = (int)(i / n_q);
  doc_scores[(int64_t)q * n_docs + doc] = edge_doc_score(L, doc_chunk_off, n_docs, t_r, q, doc);
}

// Bandwidth probe: the decode scan's memory traffic without its arithmetic.
// Same persistent grid and tile order (pairs of tiles), the same 16-byte
// loads of each tile's key rows (8 in flight per wave), the same inverse-norm
// and document-id loads and one 128-byte record written per pair; the loaded
// words are only XOR-folded.  Its time is the practical floor of the scan on
// this device.
template <int HR, int DR>
__global__ __launch_bounds__(256, MSA_ROUTE_WAVES) void scan_read_probe_kernel(RouteArgs a, int64_t n_tiles,
                                                                                 int64_t n_waves) {
  constexpr int SEG = DR * 2 / 64;  // 64-byte segments per head row
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, G = lane >> 4;
  const bf16_t *krbar = static_cast<const bf16_t *>(a.krbar);
  uint32_t acc = 0;
  for (int64_t pr = (int64_t)blockIdx.x * 4 + wave; 2 * pr < n_tiles; pr += n_waves) {
   for (int kk = 0; kk < 2; ++kk) {
    const int64_t tile = 2 * pr + kk;
    if (tile >= n_tiles) break;
    int64_t cp = tile * 16 + col;
    cp = cp < a.n_chunks ? cp : a.n_chunks - 1;
    const uint4 *row = reinterpret_cast<const uint4 *>(krbar + cp * (HR * DR)) + G;
    const float *ip = a.kr_inv_norm + cp * HR;
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < HR; ++j) m += ip[j];
    const int d = a.chunk_doc[cp];
#pragma unroll 8
    for (int i = 0; i < HR * SEG; ++i) {
      const uint4 v = row[4 * i];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    acc ^= __float_as_uint(m) ^ (uint32_t)d;
   }
    if (lane < 32) a.edges[pr * 32 + lane] = __uint_as_float(acc & 0x3FFFFFFFu);
  }
}

struct ScanGrid {
  int64_t wgs = 1, n_waves = 4;
};

// Persistent grid of the streaming scan: as many workgroups as stay resident
// together (occupancy of this kernel x compute units, at most max_wg_per_cu
// per CU when the caller caps it), so no second, partial round.
template <typename T, int HR, int DR, bool EDGE>
ScanGrid grid_of(const RouteArgs &a) {
  static std::atomic<int> resident{0};  // workgroups per CU for this instantiation
  int res = resident.load(std::memory_order_relaxed);
  if (res == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, route_scan_kernel<T, HR, DR, EDGE>, 256, 0) != hipSuccess ||
        n < 1)
      n = 1;
    res = n;
    resident.store(res, std::memory_order_relaxed);
  }
  // a caller that runs other kernels beside the scan (a pipelined decode step)
  // caps the workgroups per compute unit: while every compute unit holds more
  // than one of the scan's persistent workgroups, kernels on other streams
  // wait for the scan's waves to retire
  const int per_cu = a.max_wg_per_cu > 0 && a.max_wg_per_cu < res ? a.max_wg_per_cu : res;
  const int64_t n_tiles = (a.n_chunks + 15) / 16;
  const int rbs = (a.n_q * a.t_r + 15) / 16;
  const int64_t slots = (int64_t)device_cu_count() * per_cu;  // resident workgroups
  int64_t wgs = std::max<int64_t>(1, slots / rbs);
  wgs = std::max<int64_t>(1, std::min<int64_t>(wgs, (n_tiles + 3) / 4));
  // Balance: as few waves as still need the same number of rounds of tiles,
  // so that no small set of waves finishes a last, partial round alone at a
  // fraction of the bandwidth.  (Counted in tiles although the waves take
  // pairs of tiles: at the 100M-token decode workload this grid -- 729
  // workgroups, 8 or 9 pairs per wave -- streams at 277 us, the one balanced
  // in pairs -- 689 workgroups, 9 pairs each -- at 294 us, the full 768 at 291 us.)
  if (n_tiles > 0) {
    const int64_t rounds = (n_tiles + 4 * wgs - 1) / (4 * wgs);
    wgs = (n_tiles + 4 * rounds - 1) / (4 * rounds);
  }
  ScanGrid g;
  g.wgs = wgs;
  g.n_waves = wgs * 4;  // wave w starts at tile w
  return g;
}

template <typename T, int HR, int DR, bool EDGE>
hipError_t route_launch(const RouteArgs &a, hipStream_t s) {
  const ScanGrid g = grid_of<T, HR, DR, EDGE>(a);
  const int64_t n_tiles = (a.n_chunks + 15) / 16;
  const int rbs = (a.n_q * a.t_r + 15) / 16;
  dim3 grid((unsigned)g.wgs, (unsigned)rbs), block(256);
  hipLaunchKernelGGL((route_scan_kernel<T, HR, DR, EDGE>), grid, block, 0, s, a, n_tiles, g.n_waves);
  return hipGetLastError();
}

template <typename T, int HR, int DR>
hipError_t route_mode(const RouteArgs &a, hipStream_t s) {
  return a.edges ? route_launch<T, HR, DR, true>(a, s) : route_launch<T, HR, DR, false>(a, s);
}

template <typename T, int DR>
hipError_t route_by_hr(const RouteArgs &a, hipStream_t s) {
  // the API admits h_r * d_r <= 1024
  switch (a.h_r) {
    case 1: return route_mode<T, 1, DR>(a, s);
    case 2: return route_mode<T, 2, DR>(a, s);
    case 4: return route_mode<T, 4, DR>(a, s);
    case 8:
      if constexpr (DR <= 128) return route_mode<T, 8, DR>(a, s);
      return hipErrorInvalidValue;
    default:
      if constexpr (DR == 64) return route_mode<T, 16, DR>(a, s);
      return hipErrorInvalidValue;
  }
}

}  // namespace

EdgeLayout edge_layout(const RouteArgs &a) {
  EdgeLayout L;
  L.rec = a.edges;
  L.dsc = a.dsc;
  L.n_units = (a.n_chunks + 31) / 32;
  L.rw = a.t_r == 1 ? 16 : 1;
  return L;
}

hipError_t launch_fill_u32(uint32_t *p, size_t n, uint32_t v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t g = std::min<size_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)g), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_keys_from_scores(uint32_t *p, const float *init, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t g = std::min<size_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(keys_from_scores_kernel, dim3((unsigned)g), dim3(256), 0, s, p, init, n);
  return hipGetLastError();
}

hipError_t launch_keys_to_scores(uint32_t *p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t g = std::min<size_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(keys_to_scores_kernel, dim3((unsigned)g), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

bool route_single_writer(int t_r) { return t_r == 1 || t_r == 16; }

hipError_t launch_scan_read_probe(const RouteArgs &a, hipStream_t s) {
  if (a.n_chunks == 0) return hipSuccess;
  if (a.dtype != 1 || a.h_r != 8 || a.d_r != 128) return hipErrorInvalidValue;
  // the decode scan's grid (one row block, full occupancy)
  RouteArgs d = a;
  d.n_q = 1;
  d.t_r = 1;
  d.max_wg_per_cu = 0;
  const ScanGrid g = grid_of<bf16_t, 8, 128, true>(d);
  const int64_t n_tiles = (a.n_chunks + 15) / 16;
  hipLaunchKernelGGL((scan_read_probe_kernel<8, 128>), dim3((unsigned)g.wgs), dim3(256), 0, s, a, n_tiles, g.n_waves);
  return hipGetLastError();
}

size_t route_record_bytes(int64_t n_chunks, int n_q, int t_r) {
  const int64_t rbs = ((int64_t)n_q * t_r + 15) / 16;
  return ((size_t)rbs * ((n_chunks + 31) / 32) * 32 * sizeof(float) + 255) & ~(size_t)255;
}

size_t route_ws_bytes(int dtype, int h_r, int d_r, int64_t n_chunks, int n_docs, int n_q, int t_r) {
  if (route_single_writer(t_r)) {
    // records, then the scores of the documents inside one tile [row block][doc][16 or 1]
    const int64_t rbs = ((int64_t)n_q * t_r + 15) / 16;
    return route_record_bytes(n_chunks, n_q, t_r) + (size_t)rbs * n_docs * (t_r == 1 ? 16 : 1) * sizeof(float);
  }
  if (route_use_wide(dtype, h_r, d_r, t_r)) return route_wide_ws_bytes(n_q, t_r, h_r);
  return 0;
}

hipError_t launch_resolve_docs(const RouteArgs &a, hipStream_t s) {
  const int64_t n = (int64_t)a.n_q * a.n_docs;
  hipLaunchKernelGGL(resolve_docs_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, edge_layout(a),
                     a.doc_chunk_off, a.n_q, a.n_docs, a.t_r, a.doc_scores);
  return hipGetLastError();
}

hipError_t launch_route_scan(const RouteArgs &a, hipStream_t s) {
  if (a.n_chunks == 0) {
    if (!a.zero) return hipSuccess;
    return a.init ? launch_keys_from_scores(a.zero, a.init, (size_t)a.n_zero, s)
                  : launch_fill_u32(a.zero, (size_t)a.n_zero, 0u, s);
  }
  if (!a.edges && a.qinv && route_use_wide(a.dtype, a.h_r, a.d_r, a.t_r)) return launch_route_wide(a, s);
  if (a.dtype == 0) return a.d_r == 64 ? route_by_hr<float, 64>(a, s) : route_by_hr<float, 128>(a, s);
  if (a.d_r == 256) return route_by_hr<bf16_t, 256>(a, s);  // a router twice the head width
  return a.d_r == 64 ? route_by_hr<bf16_t, 64>(a, s) : route_by_hr<bf16_t, 128>(a, s);
}

}  // namespace msa
