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
//  * the K loop runs in stages of half a head; the next stage's slices are
//    loaded into registers while the current one is multiplied;
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

constexpr int MW = 128;  // rows per workgroup
constexpr int NW = 128;  // chunks per workgroup

// qinv[row][h] = (1/H_r) / ||Q^R[row][h]|| (0 for a zero row); 16 lanes per (row, head)
template <int DR>
__global__ void q_inv_norm_kernel(const bf16_t *qr, int n_pairs, int h_r, float *qinv) {
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
  if (pair < n_pairs && seg == 0) qinv[pair] = ss > 0.f ? (1.0f / sqrtf(ss)) * (1.0f / h_r) : 0.f;
}

template <int HR, int DR>
__global__ __launch_bounds__(256, 2) void route_wide_kernel(RouteArgs a, int n_mtiles,
                                                                 int64_t n_ntiles) {
  constexpr int SD = DR / 2;             // one stage = half of a head's dimensions
  constexpr int PITCH = SD + 8;          // LDS row pitch (elements): conflict-free fragment reads
  constexpr int KS = SD / 32;            // MFMA k-steps per stage
  constexpr int SEGS = SD / 8;           // 16-byte segments per row per stage
  constexpr int SPT = MW * SEGS / 256;   // segments per thread per operand
  __shared__ __align__(16) bf16_t sA[MW * PITCH];
  __shared__ __align__(16) bf16_t sB[NW * PITCH];
  __shared__ float red[MW / 16][NW];     // per row block: max over its 16 rows
  __shared__ __align__(16) float sqi[HR][MW];  // (1/H_r)/||Q^R|| of the tile's rows
  __shared__ int sdoc[NW];

  // tile order: row tiles of one chunk tile share blockIdx % 8 (one XCD)
  const int b = blockIdx.x;
  const int64_t r8 = b / 8;
  const int m_tile = (int)(r8 % n_mtiles);
  const int64_t n_tile = (r8 / n_mtiles) * 8 + (b % 8);
  if (n_tile >= n_ntiles) return;  // padding workgroup: exits as a whole before any barrier

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, G = lane >> 4;
  const int wr = wave >> 1, wc = wave & 1;  // 2 x 2 waves of 64 rows x 64 chunks
  const int n_rows = a.n_q * a.t_r;
  const int64_t row0 = (int64_t)m_tile * MW, c0 = n_tile * NW;
  const bf16_t *qr = static_cast<const bf16_t *>(a.qr);
  const bf16_t *kr = static_cast<const bf16_t *>(a.krbar);
  const int rot = (int)(n_tile % HR);

  // staging of one stage's slices: global -> registers (issued a stage ahead) -> LDS
  u32x4 ra[SPT], rb[SPT];
  float ikn[4];  // 1/||Kbar^R|| of this lane's four chunk columns for the next head
  // rows and chunks past the end read the last valid one (clamped, no branch):
  // their results are discarded by the epilogue (row blocks past n_rows, chunks
  // without a document).  Per stage a thread moves SPT 16-byte segments of each
  // operand: rows tid / SEGS + i * (256 / SEGS), segment tid % SEGS.
  const int seg = tid % SEGS;
  const bf16_t *pa[SPT];
  const bf16_t *pb[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    const int row = tid / SEGS + i * (256 / SEGS);
    const int64_t m = std::min<int64_t>(row0 + row, n_rows - 1), c = std::min<int64_t>(c0 + row, a.n_chunks - 1);
    pa[i] = qr + m * HR * DR + seg * 8;
    pb[i] = kr + c * HR * DR + seg * 8;
  }
  const float *pik[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pik[j] = a.kr_inv_norm + std::min<int64_t>(c0 + 64 * wc + 16 * j + col, a.n_chunks - 1) * HR;
  auto load = [&](int h, int half) {
    const int off = h * DR + half * SD;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      ra[i] = *reinterpret_cast<const u32x4 *>(pa[i] + off);
      rb[i] = *reinterpret_cast<const u32x4 *>(pb[i] + off);
    }
    if (half == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) ikn[j] = pik[j][h];
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
      const int row = tid / SEGS + i * (256 / SEGS);
      *reinterpret_cast<u32x4 *>(sA + row * PITCH + seg * 8) = ra[i];
      *reinterpret_cast<u32x4 *>(sB + row * PITCH + seg * 8) = rb[i];
    }
  };
  auto multiply = [&](f32x4 (&acc)[4][4]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[i] = load_frag<bf16_t>(sA + (64 * wr + 16 * i + col) * PITCH + ks * 32 + G * 8);
        fb[i] = load_frag<bf16_t>(sB + (64 * wc + 16 * i + col) * PITCH + ks * 32 + G * 8);
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

  if (tid < NW) sdoc[tid] = (c0 + tid < a.n_chunks) ? a.chunk_doc[c0 + tid] : -1;
  for (int k = tid; k < MW * HR; k += 256) {
    const int row = k / HR, h = k % HR;
    sqi[h][row] = row0 + row < n_rows ? a.qinv[(row0 + row) * HR + h] : 0.f;
  }
  load(rot, 0);
  store();
  __syncthreads();
#pragma unroll 1
  for (int hs = 0; hs < HR; ++hs) {
    const int h = (hs + rot) % HR, hn = (hs + 1 + rot) % HR;
    float ik[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ik[j] = ikn[j];
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = zero4();
    load(h, 1);  // second half of this head in flight during the first half's MFMAs
    multiply(acc);
    __syncthreads();
    store();
    __syncthreads();
    if (hs + 1 < HR) load(hn, 0);
    multiply(acc);
    // this head's cosines: acc * (1/H_r)/||q|| (per row) * 1/||k|| (per chunk)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 iq = *reinterpret_cast<const float4 *>(&sqi[h][64 * wr + 16 * i + 4 * G]);
      const float iqe[4] = {iq.x, iq.y, iq.z, iq.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) score[i][j][e] = fmaf(acc[i][j][e] * iqe[e], ik[j], score[i][j][e]);
    }
    __syncthreads();
    if (hs + 1 < HR) {
      store();
      __syncthreads();
    }
  }

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
    if (tid < NW) {
      float v = -INFINITY;
      for (int i = rb_lo; i < rb_hi; ++i) v = fmaxf(v, red[i][tid]);
      const int doc = sdoc[tid];
      if (a.chunk_out && doc >= 0) atomicMax(a.chunk_out + (int64_t)q * a.n_chunks + c0 + tid, score_key(v));
      // the first chunk of each run of one document reduces the run
      if (doc >= 0 && (tid == 0 || sdoc[tid - 1] != doc)) {
        float m = v;
        for (int j = tid + 1; j < NW && sdoc[j] == doc; ++j) {
          float w = -INFINITY;
          for (int i = rb_lo; i < rb_hi; ++i) w = fmaxf(w, red[i][j]);
          m = fmaxf(m, w);
        }
        atomicMax(a.doc_keys + (int64_t)q * a.n_docs + doc, score_key(m));
      }
    }
  }
}

}  // namespace

bool route_use_wide(int dtype, int h_r, int d_r, int t_r) {
  return dtype == 1 && (h_r == 1 || h_r == 2 || h_r == 4 || h_r == 8) && t_r % 16 == 0 && t_r >= 32 && d_r == 128;
}

size_t route_wide_ws_bytes(int n_q, int t_r, int h_r) { return (size_t)n_q * t_r * h_r * sizeof(float); }

hipError_t launch_route_wide(const RouteArgs &a, hipStream_t s) {
  const int n_rows = a.n_q * a.t_r;
  const int n_pairs = n_rows * a.h_r;
  const int64_t threads = (int64_t)n_pairs * (128 / 8);
  hipLaunchKernelGGL(q_inv_norm_kernel<128>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     static_cast<const bf16_t *>(a.qr), n_pairs, a.h_r, a.qinv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_mtiles = (n_rows + MW - 1) / MW;
  const int64_t n_ntiles = (a.n_chunks + NW - 1) / NW;
  const int64_t grid = 8 * n_mtiles * ((n_ntiles + 7) / 8);
  switch (a.h_r) {
    case 1: hipLaunchKernelGGL((route_wide_kernel<1, 128>), dim3((unsigned)grid), dim3(256), 0, s, a, n_mtiles, n_ntiles); break;
    case 2: hipLaunchKernelGGL((route_wide_kernel<2, 128>), dim3((unsigned)grid), dim3(256), 0, s, a, n_mtiles, n_ntiles); break;
    case 4: hipLaunchKernelGGL((route_wide_kernel<4, 128>), dim3((unsigned)grid), dim3(256), 0, s, a, n_mtiles, n_ntiles); break;
    case 8: hipLaunchKernelGGL((route_wide_kernel<8, 128>), dim3((unsigned)grid), dim3(256), 0, s, a, n_mtiles, n_ntiles); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace msa
