// Router scan for many query-token rows (prefill, Memory Interleave rounds):
// a bf16 GEMM per router head, the cosine normalisation applied to each
// head's fp32 accumulator, then max over each query's rows and over each
// document's chunks.
//
// Score (Lighthouse digest, Component 1, key formula; hotdry blog, core
// architecture of the memory routing layer): S[q,c] = max_t (1/H_r) sum_h
// cos(Q^R[q,t,h], Kbar^R[c,h]); document score = max over its chunks.
//
// With hundreds of rows per query the scan is MFMA-bound (about 600 FLOP per
// byte of router keys), so it is tiled like a GEMM:
//  * a workgroup owns 128 rows x 128 chunks; four waves of 64 x 64;
//  * the head loop is the K loop: per head the accumulator <q_h, k_h>
//    (v_mfma_f32_16x16x32_bf16 on the stored bf16 values, copied into LDS as
//    they are) is scaled by the fp32 inverse norms of its row, (1/H_r) /
//    ||Q^R_t,h|| from a small pre-kernel, and of its chunk, 1/||Kbar^R_c,h||,
//    and added to the score: no operand is re-rounded;
//  * each chunk tile walks the heads in a rotated order (start = tile mod H_r):
//    a head's slices sit at one offset inside every 2 KB key row, and
//    concurrent tiles on different heads spread the reads over the L2
//    channels;
//  * the K loop runs in stages of half a head, filled by direct-to-LDS loads
//    into XOR-swizzled 128-byte rows, double-buffered: the next stage fills
//    while the current one is multiplied;
//  * all row tiles of one chunk tile are scheduled on the same XCD
//    (blockIdx % 8), so the chunk tile is read from HBM once and re-read from
//    that XCD's L2;
//  * epilogue: max over the rows of each query inside the tile, then per run
//    of chunks of one document one atomicMax on order-preserving keys.
#include <algorithm>

#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int MW = 128;  // rows per workgroup
constexpr int WIDE_NW = 128;  // chunks per workgroup (4 waves of 64 x 64)

// qinv[h][row] = (1/H_r) / ||Q^R[row][h]|| (0 for a zero row); 16 lanes per
// (row, head).  Also sets zero[0, n_zero) (the document keys the scan maxes
// into) to 0, or to the keys of init[] (the previous round's scores when
// re-routing), so the scan needs no separate launch for them.
template <int DR>
__global__ void q_inv_norm_kernel(const bf16_t *qr, int n_rows, int h_r, float *qinv, uint32_t *zero, int64_t n_zero,
                                  const float *init) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_zero; i += (int64_t)gridDim.x * blockDim.x)
    zero[i] = init ? score_key(init[i]) : 0u;
  const int n_pairs = n_rows * h_r;
  constexpr int SEGS = DR / 8;  // 16-byte segments per row slice
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t pair = t / SEGS;
  const int seg = (int)(t % SEGS);
  float ss = 0.f;
  if (pair < n_pairs) {
    const uint4 v = *reinterpret_cast<const uint4 *>(qr + pair * DR + seg * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = __uint_as_float(w[e] << 16), hi = __uint_as_float(w[e] & 0xFFFF0000u);
      ss = fmaf(lo, lo, fmaf(hi, hi, ss));
    }
  }
#pragma unroll
  for (int o = SEGS / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if (pair < n_pairs && seg == 0)
    qinv[(pair % h_r) * n_rows + pair / h_r] = ss > 0.f ? (1.0f / sqrtf(ss)) * (1.0f / h_r) : 0.f;
}

// XOR swizzle of the eight 16-byte slots of a 128-byte chunk row in LDS: rows
// r..r+7 (and the even / odd rows of r..r+15) put a given logical slot in
// eight different bank groups, so fragment reads of 16 rows are conflict-free.
__device__ __forceinline__ int slot_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// 16-byte direct-to-LDS load: this lane's 16 bytes at g land at lds_base +
// 16 * lane (lds_base is wave-uniform)
__device__ __forceinline__ void lds_fill16(const bf16_t *g, bf16_t *lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void *)lds_base, 16, 0, 0);
}

// s_waitcnt immediates (gfx9 encoding): wait until at most N vector-memory
// operations of this wave are outstanding, leaving the other counters alone
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int LGKM0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);  // lgkmcnt(0) only

// Workgroup barrier for the stage pipeline, without the memory fence of
// __syncthreads (whose full vmcnt(0) wait would also wait for the fills in
// flight): this wave's LDS reads have returned (lgkmcnt 0) and its fills of
// the next stage have landed (explicit vmcnt wait before the call).
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(LGKM0);
  __builtin_amdgcn_s_barrier();
}

template <int HR, int DR, int NW>
__global__ __launch_bounds__(2 * NW, 2) void route_wide_kernel(RouteArgs a, int n_mtiles, int64_t n_ntiles) {
  static_assert(DR == 128, "stage layout assumes 128-dim router heads");
  constexpr int SD = DR / 2;       // one stage = half of a head's dimensions (128 bytes per row)
  constexpr int NT = 2 * NW;       // threads: 2 x (NW / 64) waves of 64 rows x 64 chunks
  constexpr int WAVES = NT / 64;
  constexpr int FA = MW / WAVES / 8;  // direct-to-LDS loads per wave per stage: query rows
  constexpr int FB = NW / WAVES / 8;  //                                          chunk rows
  // Stage buffers (rows of 128 bytes, slots swizzled, filled by direct-to-LDS
  // loads), double-buffered: buffers 0 hold the first half of a head, buffers
  // 1 the second.  Each buffer is its own variable so that the compiler can
  // tell the buffer being filled from the one being read and does not wait
  // for the fill in flight.
  __shared__ __align__(16) bf16_t sA0[MW * SD], sA1[MW * SD];  // query rows
  __shared__ __align__(16) bf16_t sB0[NW * SD], sB1[NW * SD];  // chunk rows
  __shared__ __align__(16) float sqi[HR][MW];  // (1/H_r)/||Q^R|| of the tile's rows
  __shared__ float sik[HR][NW];                // 1/||Kbar^R|| of the tile's chunks

  // tile order: row tiles of one chunk tile share blockIdx % 8 (one XCD)
  const int b = blockIdx.x;
  const int64_t r8 = b / 8;
  const int m_tile = (int)(r8 % n_mtiles);
  const int64_t n_tile = (r8 / n_mtiles) * 8 + (b % 8);
  if (n_tile >= n_ntiles) return;  // padding workgroup: exits as a whole before any barrier

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, G = lane >> 4;
  const int wr = wave & 1, wc = wave >> 1;  // waves of 64 rows x 64 chunks
  const int n_rows = a.n_q * a.t_r;
  const int64_t row0 = (int64_t)m_tile * MW, c0 = n_tile * NW;
  const int rows_here = (int)std::min<int64_t>(MW, n_rows - row0);
  const int chunks_here = (int)std::min<int64_t>(NW, a.n_chunks - c0);
  const bf16_t *qt = static_cast<const bf16_t *>(a.qr) + row0 * HR * DR;    // this tile's rows
  const bf16_t *kt = static_cast<const bf16_t *>(a.krbar) + c0 * HR * DR;   // this tile's chunks
  const int rot = (int)(n_tile % HR);

  // Fill of a stage: wave w writes its share of the rows (MW / WAVES query rows,
  // NW / WAVES chunk rows) with 16-byte direct-to-LDS loads; in load p, lane L
  // writes row base + 8p + L/8 at physical slot L%8, which holds the logical
  // slot (L%8) ^ slot_swz(row).  Rows and chunks past the end read the last
  // valid one (clamped, no branch); the epilogue discards them.
  uint32_t aoff[FA], boff[FB];
#pragma unroll
  for (int p = 0; p < FA; ++p) {
    const int row = (MW / WAVES) * wave + 8 * p + lane / 8;
    aoff[p] = (uint32_t)(std::min(row, rows_here - 1) * HR * DR + ((lane % 8) ^ slot_swz(row)) * 8);
  }
#pragma unroll
  for (int p = 0; p < FB; ++p) {
    const int row = (NW / WAVES) * wave + 8 * p + lane / 8;
    boff[p] = (uint32_t)(std::min(row, chunks_here - 1) * HR * DR + ((lane % 8) ^ slot_swz(row)) * 8);
  }
  auto fill = [&](bf16_t *dA, bf16_t *dB, int h, int half) {
    const int o = h * DR + half * SD;
#pragma unroll
    for (int p = 0; p < FA; ++p)
      lds_fill16(qt + aoff[p] + o, dA + ((MW / WAVES) * wave + 8 * p) * SD);
#pragma unroll
    for (int p = 0; p < FB; ++p)
      lds_fill16(kt + boff[p] + o, dB + ((NW / WAVES) * wave + 8 * p) * SD);
  };
  // k-step ks of a stage pairs logical slot 2G + ks of a query row and of a
  // chunk row: lane group G covers the stage's dimensions 16G .. 16G+15
  auto multiply = [&](const bf16_t *sA, const bf16_t *sB, f32x4 (&acc)[4][4]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = 64 * wr + 16 * i + col, rb = 64 * wc + 16 * i + col;
        fa[i] = *reinterpret_cast<const bf16x8 *>(sA + ra * SD + ((2 * G + ks) ^ slot_swz(ra)) * 8);
        fb[i] = *reinterpret_cast<const bf16x8 *>(sB + rb * SD + ((2 * G + ks) ^ slot_swz(rb)) * 8);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(fa[i], fb[j], acc[i][j]);
    }
  };

  f32x4 score[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) score[i][j] = zero4();

  // scales of the tile's rows and chunks (qinv is [h][n_rows], kr_inv_norm
  // [chunk][h]), every load in flight before the first LDS write
  {
    constexpr int SQ = (MW * HR + NT - 1) / NT, SC = (NW * HR + NT - 1) / NT;
    float vq[SQ], vc[SC];
#pragma unroll
    for (int i = 0; i < SQ; ++i) {
      const int k = tid + i * NT, h = k / MW, row = k % MW;
      const bool ok = k < MW * HR && row < rows_here;
      vq[i] = a.qinv[ok ? (int64_t)h * n_rows + row0 + row : 0];
      if (!ok) vq[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < SC; ++i) {
      const int k = tid + i * NT, c = k / HR, h = k % HR;
      const bool ok = k < NW * HR && c < chunks_here;
      vc[i] = a.kr_inv_norm[ok ? (c0 + c) * HR + h : 0];
      if (!ok) vc[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < SQ; ++i) {
      const int k = tid + i * NT;
      if (k < MW * HR) sqi[k / MW][k % MW] = vq[i];
    }
#pragma unroll
    for (int i = 0; i < SC; ++i) {
      const int k = tid + i * NT;
      if (k < NW * HR) sik[k % HR][k / HR] = vc[i];
    }
  }
  const int mydoc = tid < chunks_here ? a.chunk_doc[c0 + tid] : -1;  // document of chunk tid (tid < NW)
  fill(sA0, sB0, rot, 0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();  // the scales and the first stage are in LDS
#pragma unroll 1
  for (int hs = 0; hs < HR; ++hs) {
    const int h = (hs + rot) % HR, hn = (hs + 1 + rot) % HR;
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = zero4();
    // first half from buffers 0 while the second half fills buffers 1
    fill(sA1, sB1, h, 1);
    multiply(sA0, sB0, acc);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    stage_barrier();
    // second half from buffers 1 while the next head's first half fills buffers 0
    if (hs + 1 < HR) fill(sA0, sB0, hn, 0);
    multiply(sA1, sB1, acc);
    // this head's cosines: acc * (1/H_r)/||q|| (per row) * 1/||k|| (per chunk)
    float ik[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ik[j] = sik[h][64 * wc + 16 * j + col];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 iq = *reinterpret_cast<const float4 *>(&sqi[h][64 * wr + 16 * i + 4 * G]);
      const float iqe[4] = {iq.x, iq.y, iq.z, iq.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) score[i][j][e] = fmaf(acc[i][j][e] * iqe[e], ik[j], score[i][j][e]);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    stage_barrier();
  }

  float (*red)[NW] = reinterpret_cast<float (*)[NW]>(sA0);  // per row block: max over its 16 rows

  // ---- max over the 16 rows of each row block (rows of one query), per chunk ----
  // score[i][j]: rows 64 wr + 16 i + 4 G + e, chunk 64 wc + 16 j + col
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rblk = 4 * wr + i;
    const bool rows_ok = row0 + 16 * rblk < n_rows;  // row blocks are all-valid or all-invalid (t_r % 16 == 0)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = fmaxf(fmaxf(score[i][j][0], score[i][j][1]), fmaxf(score[i][j][2], score[i][j][3]));
      v = fmaxf(v, __shfl_xor(v, 16, 64));
      v = fmaxf(v, __shfl_xor(v, 32, 64));
      if (G == 0) red[rblk][64 * wc + 16 * j + col] = rows_ok ? v : -INFINITY;
    }
  }
  __syncthreads();

  // ---- per query in the tile: chunk max, then one atomicMax per document run ----
  const int q_first = (int)(row0 / a.t_r);
  const int q_last = (int)(std::min<int64_t>(row0 + MW, n_rows) - 1) / a.t_r;
  for (int q = q_first; q <= q_last; ++q) {
    const int rb_lo = (int)std::max<int64_t>(0, ((int64_t)q * a.t_r - row0) / 16);
    const int rb_hi = (int)std::min<int64_t>(MW / 16, ((int64_t)(q + 1) * a.t_r - row0 + 15) / 16);
    if (tid < NW) {  // the first NW / 64 waves, one chunk per lane
      float v = -INFINITY;
      for (int i = rb_lo; i < rb_hi; ++i) v = fmaxf(v, red[i][tid]);
      if (a.chunk_out && mydoc >= 0) atomicMax(a.chunk_out + (int64_t)q * a.n_chunks + c0 + tid, score_key(v));
      // segmented suffix max over the runs of one document within the wave
      // (chunks of a document are consecutive); every lane takes part in
      // every shuffle
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float w = __shfl_down(v, o, 64);
        const int d = __shfl_down(mydoc, o, 64);
        if (lane + o < 64 && d == mydoc) v = fmaxf(v, w);
      }
      // the first lane of each run in the wave publishes it (a run crossing
      // waves is published by each part)
      const int prev = __shfl_up(mydoc, 1, 64);
      if (mydoc >= 0 && (lane == 0 || prev != mydoc))
        atomicMax(a.doc_keys + (int64_t)q * a.n_docs + mydoc, score_key(v));
    }
  }
}

// Inclusive max-scan within runs of equal document over the 16 columns of a
// lane group (consecutive chunks); match[j]: column col - 2^j holds the same
// document.  The last column of a run then holds the run's max.
__device__ __forceinline__ float run_max16(float v, const bool (&match)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float nv = __shfl_up(v, 1 << j, 16);
    if (match[j]) v = fmaxf(v, nv);
  }
  return v;
}

// ---- streaming scan for a few row blocks (17-64 router rows) ------------------
// The tiled many-row scan walks each 128-chunk tile through 16 dependent
// stage fills, which caps it near 55 us over a 10M-token bank whatever its
// row count up to 128; with at most four 16-row blocks the scan is bound by
// the bank's bytes (about 63 FLOP per byte at 64 rows), so it streams the bank
// once like the decode scan: persistent waves, a two-head prefetch ring of
// 16-chunk tiles, and every loaded key fragment multiplied by the RB row
// blocks' query fragments (held in LDS for the whole scan).  Rows are whole
// 16-row blocks of one query each (t_r % 16 == 0); the document scores are
// maxed atomically into order-preserving keys (zeroed or initialised before).
constexpr int RW_WAVES = 8;  // waves per workgroup (one workgroup per compute unit: the queries fill LDS)

template <int HR, int RB>
__global__ __launch_bounds__(64 * RW_WAVES, 1) void route_rows_kernel(RouteArgs a, int64_t n_tiles, int64_t n_waves) {
  constexpr int DR = 128, KW = 32, EL = 8, KS = DR / KW, NF = HR * KS;
  constexpr int PD = HR < 2 ? HR : 2;  // heads in flight
  static_assert(HR % PD == 0, "ring depth divides the head count");
  __shared__ bf16x8 qfrag[RB][NF][64];
  __shared__ __align__(16) float qinv[RB][HR][16];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, G = lane >> 4;
  const int n_rows = a.n_q * a.t_r;
  const int nrb = (n_rows + 15) / 16;  // row blocks in use (<= RB)
  const bf16_t *qr = static_cast<const bf16_t *>(a.qr);
  const bf16_t *krbar = static_cast<const bf16_t *>(a.krbar);
  const int64_t wave_id = (int64_t)blockIdx.x * RW_WAVES + wave;

  auto lane_chunk = [&](int64_t tl) -> int64_t {
    const int64_t cp = tl * 16 + col;
    return cp < a.n_chunks ? cp : a.n_chunks - 1;
  };
  float ik_cur[HR], ik_nxt[HR];
  int doc_cur = -1, doc_nxt = -1;
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
    const int d = a.chunk_doc[cp];
    doc = (tl * 16 + col < a.n_chunks) ? d : -1;
  };
  // the key stream starts before the query staging (a wave without tiles
  // reads a clamped, valid chunk and never uses it)
  const int64_t t0 = wave_id;
  bf16x8 ring[PD][KS];
  const bf16_t *kp_cur = krbar + lane_chunk(t0) * (HR * DR) + G * EL;
  const bf16_t *kp_nxt = kp_cur;
#pragma unroll
  for (int p = 0; p < PD; ++p)
#pragma unroll
    for (int st = 0; st < KS; ++st) ring[p][st] = load_frag<bf16_t>(kp_cur + p * DR + st * KW);
  load_meta(t0, ik_cur, doc_cur);

  // query fragments of the row blocks in MFMA A-operand order, and their
  // norms: every load in flight before the first is written to LDS (one
  // round trip at a time had cost ~9 us per call)
  {
    constexpr int QPT = (RB * NF * 64 + 64 * RW_WAVES - 1) / (64 * RW_WAVES);
    bf16x8 qt[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int e = threadIdx.x + i * 64 * RW_WAVES;
      const int r = e / (NF * 64), f = (e / 64) % NF, l = e % 64, h = f / KS, st = f % KS;
      const int row = r * 16 + (l & 15);
      const bool ok = e < RB * NF * 64 && row < n_rows;
      const int64_t src = ok ? ((int64_t)row * HR + h) * DR + st * KW + (l >> 4) * EL : 0;  // row 0: a valid address
      qt[i] = load_frag<bf16_t>(qr + src);
      if (!ok) qt[i] = bf16x8{};
    }
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int e = threadIdx.x + i * 64 * RW_WAVES;
      if (e < RB * NF * 64) qfrag[e / (NF * 64)][(e / 64) % NF][e % 64] = qt[i];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < RB * HR * 16; e += 64 * RW_WAVES) {
    const int r = e / (HR * 16), h = (e / 16) % HR, rr = e % 16;
    float ss = 0.f;
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x8 v = qfrag[r][h * KS + st][16 * g + rr];
#pragma unroll
        for (int j = 0; j < EL; ++j) {
          const float x = (float)v[j];
          ss += x * x;
        }
      }
    qinv[r][h][rr] = ss > 0.f ? (1.0f / sqrtf(ss)) * (1.0f / HR) : 0.f;
  }
  __syncthreads();

  for (int64_t tile = t0; tile < n_tiles; tile += n_waves) {
    const int64_t tile_next = tile + n_waves;
    const bool has_next = tile_next < n_tiles;
    const int64_t tile_pf = has_next ? tile_next : tile;
    // next tile's loads issued unconditionally (a last tile re-reads its own final heads)
    kp_nxt = krbar + lane_chunk(tile_pf) * (HR * DR) + G * EL + (has_next ? 0 : (HR - PD) * DR);
    load_meta(tile_pf, ik_nxt, doc_nxt);
    int zoff;  // opaque zero: the query fragments are read from LDS inside the loop
    asm volatile("s_mov_b32 %0, 0" : "=s"(zoff));
    f32x4 S[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) S[r] = zero4();
#pragma unroll
    for (int h = 0; h < HR; ++h) {
      const int slot = h % PD;
      const float ik = ik_cur[h];
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (r >= nrb) break;  // wave-uniform
        f32x4 acc = zero4();
#pragma unroll
        for (int st = 0; st < KS; ++st) acc = mfma16(qfrag[r][h * KS + st + zoff][lane], ring[slot][st], acc);
        const float4 iq = *reinterpret_cast<const float4 *>(&qinv[r][h][4 * G]);
        S[r][0] += acc[0] * (iq.x * ik);
        S[r][1] += acc[1] * (iq.y * ik);
        S[r][2] += acc[2] * (iq.z * ik);
        S[r][3] += acc[3] * (iq.w * ik);
      }
      if (h + PD < HR) {
#pragma unroll
        for (int st = 0; st < KS; ++st) ring[slot][st] = load_frag<bf16_t>(kp_cur + (h + PD) * DR + st * KW);
      } else {
#pragma unroll
        for (int st = 0; st < KS; ++st) ring[slot][st] = load_frag<bf16_t>(kp_nxt + (h + PD - HR) * DR + st * KW);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const int doc = doc_cur;
    const int64_t c = tile * 16 + col;
    const bool cv = c < a.n_chunks;
    kp_cur = kp_nxt;
#pragma unroll
    for (int j = 0; j < HR; ++j) ik_cur[j] = ik_nxt[j];
    doc_cur = doc_nxt;
    // epilogue: per query, the max over its rows of each chunk, then the
    // max over each run of chunks of one document, one atomic per run
    const int doc_right = __shfl_down(doc, 1, 16);
    const bool tail = (col == 15) || (doc_right != doc);
    bool match[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int doc_left = __shfl_up(doc, 1 << j, 16);
      match[j] = col >= (1 << j) && doc_left == doc;
    }
    float v = -INFINITY;
    int q_cur = -1;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      if (r >= nrb) break;  // wave-uniform
      float m = fmaxf(fmaxf(S[r][0], S[r][1]), fmaxf(S[r][2], S[r][3]));
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      const int q = r * 16 / a.t_r;  // the block's query
      if (q != q_cur && q_cur >= 0) {  // a new query: publish the previous one's chunk maxima
        if (a.chunk_out && G == 0 && cv) atomicMax(a.chunk_out + (int64_t)q_cur * a.n_chunks + c, score_key(v));
        const float w = run_max16(cv ? v : -INFINITY, match);
        if (G == 0 && tail && doc >= 0) atomicMax(a.doc_keys + (int64_t)q_cur * a.n_docs + doc, score_key(w));
        v = -INFINITY;
      }
      q_cur = q;
      v = fmaxf(v, m);
    }
    if (a.chunk_out && G == 0 && cv) atomicMax(a.chunk_out + (int64_t)q_cur * a.n_chunks + c, score_key(v));
    const float w = run_max16(cv ? v : -INFINITY, match);
    if (G == 0 && tail && doc >= 0) atomicMax(a.doc_keys + (int64_t)q_cur * a.n_docs + doc, score_key(w));
  }
}

}  // namespace

bool route_use_wide(int dtype, int h_r, int d_r, int t_r) {
  return dtype == 1 && (h_r == 1 || h_r == 2 || h_r == 4 || h_r == 8) && t_r % 16 == 0 && t_r >= 32 && d_r == 128;
}

bool route_use_rows(int dtype, int h_r, int d_r, int n_q, int t_r) {
  return route_use_wide(dtype, h_r, d_r, t_r) && (int64_t)n_q * t_r <= 64;
}

namespace {
template <int HR>
hipError_t route_rows_launch(const RouteArgs &a, hipStream_t s) {
  const int64_t n_tiles = (a.n_chunks + 15) / 16;
  // one workgroup per compute unit; as many waves as still need the same
  // number of rounds of tiles (no small set of waves on a last, partial round)
  const int64_t slots = (int64_t)device_cu_count() * RW_WAVES;
  const int64_t rounds = (n_tiles + slots - 1) / slots;
  const int64_t waves = (n_tiles + rounds - 1) / rounds;
  const int64_t wgs = (waves + RW_WAVES - 1) / RW_WAVES;
  hipLaunchKernelGGL((route_rows_kernel<HR, 4>), dim3((unsigned)wgs), dim3(64 * RW_WAVES), 0, s, a, n_tiles,
                     wgs * RW_WAVES);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_rows(const RouteArgs &a, hipStream_t s) {
  if (a.zero) {  // the document keys start at zero, or at the previous round's scores
    const hipError_t e = a.init ? launch_keys_from_scores(a.zero, a.init, (size_t)a.n_zero, s)
                                : launch_fill_u32(a.zero, (size_t)a.n_zero, 0u, s);
    if (e != hipSuccess) return e;
  }
  switch (a.h_r) {
    case 1: return route_rows_launch<1>(a, s);
    case 2: return route_rows_launch<2>(a, s);
    case 4: return route_rows_launch<4>(a, s);
    case 8: return route_rows_launch<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

size_t route_wide_ws_bytes(int n_q, int t_r, int h_r) { return (size_t)n_q * t_r * h_r * sizeof(float); }

hipError_t launch_route_wide(const RouteArgs &a, hipStream_t s) {
  if (route_use_rows(a.dtype, a.h_r, a.d_r, a.n_q, a.t_r)) return launch_route_rows(a, s);
  const int n_rows = a.n_q * a.t_r;
  const int n_pairs = n_rows * a.h_r;
  const int64_t threads = (int64_t)n_pairs * (128 / 8);
  hipLaunchKernelGGL(q_inv_norm_kernel<128>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     static_cast<const bf16_t *>(a.qr), n_rows, a.h_r, a.qinv, a.zero, a.zero ? a.n_zero : 0, a.init);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_mtiles = (n_rows + MW - 1) / MW;
  const int64_t n_ntiles = (a.n_chunks + WIDE_NW - 1) / WIDE_NW;
  const int64_t grid = 8 * n_mtiles * ((n_ntiles + 7) / 8);
  const dim3 block(2 * WIDE_NW);
  switch (a.h_r) {
    case 1: hipLaunchKernelGGL((route_wide_kernel<1, 128, WIDE_NW>), dim3((unsigned)grid), block, 0, s, a, n_mtiles, n_ntiles); break;
    case 2: hipLaunchKernelGGL((route_wide_kernel<2, 128, WIDE_NW>), dim3((unsigned)grid), block, 0, s, a, n_mtiles, n_ntiles); break;
    case 4: hipLaunchKernelGGL((route_wide_kernel<4, 128, WIDE_NW>), dim3((unsigned)grid), block, 0, s, a, n_mtiles, n_ntiles); break;
    case 8: hipLaunchKernelGGL((route_wide_kernel<8, 128, WIDE_NW>), dim3((unsigned)grid), block, 0, s, a, n_mtiles, n_ntiles); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace msa
