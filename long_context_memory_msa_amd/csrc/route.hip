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
//    then a segmented max over each run of chunks of one document, and one
//    order-preserving atomicMax per (query, document run) into the scores;
//  * persistent waves each own a contiguous range of chunk tiles.
#include <algorithm>

#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {
namespace {

__global__ void fill_u32_kernel(uint32_t *p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

__global__ void keys_to_scores_kernel(uint32_t *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = __float_as_uint(key_score(p[i]));
}

// Segmented max over the 16 columns of a lane group: columns hold chunks in
// bank order, `doc` their documents (-1 = no chunk).  Returns, in the first
// lane of each run of equal doc, the max over the run.
__device__ __forceinline__ float seg_max16(float v, int doc, int col) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    float nv = __shfl_down(v, o, 16);
    int nd = __shfl_down(doc, o, 16);
    if (col + o < 16 && nd == doc) v = fmaxf(v, nv);
  }
  return v;
}

template <typename T, int HR, int DR>
__global__ __launch_bounds__(256, 3) void route_scan_kernel(RouteArgs a, int64_t n_tiles, int tiles_per_wave) {
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

  // query fragments of rows [16 rb, 16 rb + 16) in MFMA A-operand order
  for (int e = threadIdx.x; e < NF * 64; e += 256) {
    const int f = e >> 6, l = e & 63, h = f / KS, s = f % KS;
    const int row = rb * 16 + (l & 15);
    if (row < n_rows) {
      qfrag[f][l] = load_frag<T>(qr + ((int64_t)row * HR + h) * DR + s * KW + (l >> 4) * EL);
    } else {
      FT z;
      if constexpr (EL == 1) z = 0.f; else z = FT{};
      qfrag[f][l] = z;
    }
  }
  if (threadIdx.x < 16 * HR) {
    const int r = threadIdx.x & 15, h = threadIdx.x >> 4;
    const int row = rb * 16 + r;
    float ss = 0.f;
    if (row < n_rows) {
      const T *p = qr + ((int64_t)row * HR + h) * DR;
      for (int i = 0; i < DR; ++i) {
        float x = Elem<T>::to_f32(p[i]);
        ss += x * x;
      }
    }
    qinv[h][r] = ss > 0.f ? (1.0f / sqrtf(ss)) * (1.0f / HR) : 0.f;
  }
  __syncthreads();

  // rows of this lane: 16 rb + 4 G + i; a row block lies in one query when t_r % 16 == 0
  const bool uniform = (a.t_r % 16) == 0;
  int rowq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = rb * 16 + 4 * G + i;
    rowq[i] = row < n_rows ? row / a.t_r : -1;
  }
  const int64_t wave_id = (int64_t)blockIdx.x * 4 + wave;
  const int64_t t_lo = wave_id * tiles_per_wave;
  const int64_t t_hi = t_lo + tiles_per_wave < n_tiles ? t_lo + tiles_per_wave : n_tiles;
  const T *krbar = static_cast<const T *>(a.krbar);

  // Prefetch ring: the key fragments of PD (tile, head) steps are in flight
  // while the MFMAs of the current step run; it streams across tile ends.
  constexpr int PD = HR < 4 ? HR : 4;
  FT ring[PD][KS];
  float ring_ik[PD];
  auto lane_chunk = [&](int64_t tl) -> int64_t {
    const int64_t cp = tl * 16 + col;
    return cp < a.n_chunks ? cp : a.n_chunks - 1;
  };
  int64_t c_nxt = lane_chunk(t_lo);
  const T *kp_nxt = krbar + c_nxt * (HR * DR) + G * EL;
  const float *ik_nxt = a.kr_inv_norm + c_nxt * HR;
  const T *kp_cur = kp_nxt;
  const float *ik_cur = ik_nxt;
  if (t_lo < t_hi) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
#pragma unroll
      for (int s = 0; s < KS; ++s) ring[p][s] = load_frag<T>(kp_cur + p * DR + s * KW);
      ring_ik[p] = ik_cur[p];
    }
  }

  for (int64_t tile = t_lo; tile < t_hi; ++tile) {
    const int64_t c = tile * 16 + col;
    const bool cv = c < a.n_chunks;
    const int64_t cc = cv ? c : a.n_chunks - 1;
    kp_cur = kp_nxt;
    ik_cur = ik_nxt;
    const bool more = tile + 1 < t_hi;
    if (more) {
      c_nxt = lane_chunk(tile + 1);
      kp_nxt = krbar + c_nxt * (HR * DR) + G * EL;
      ik_nxt = a.kr_inv_norm + c_nxt * HR;
    }
    const int doc = cv ? a.chunk_doc[cc] : -1;
    // opaque zero: keeps the query-fragment LDS reads inside the loop rather
    // than hoisting all of Q into VGPRs (registers go to the prefetch ring)
    int zoff;
    asm volatile("s_mov_b32 %0, 0" : "=s"(zoff));
    f32x4 S = zero4();
    // heads in groups of PD; slot p of the ring holds head hg + p
#pragma unroll 1
    for (int hg = 0; hg < HR; hg += PD) {
#pragma unroll
      for (int p = 0; p < PD; ++p) {
        const int h = hg + p;
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = mfma16(qfrag[h * KS + s + zoff][lane], ring[p][s], acc);
        const float ik = ring_ik[p];
        const float4 iq = *reinterpret_cast<const float4 *>(&qinv[h][4 * G]);
        S[0] += acc[0] * (iq.x * ik);
        S[1] += acc[1] * (iq.y * ik);
        S[2] += acc[2] * (iq.z * ik);
        S[3] += acc[3] * (iq.w * ik);
        if (hg + PD < HR) {
#pragma unroll
          for (int s = 0; s < KS; ++s) ring[p][s] = load_frag<T>(kp_cur + (h + PD) * DR + s * KW);
          ring_ik[p] = ik_cur[h + PD];
        } else if (more) {
#pragma unroll
          for (int s = 0; s < KS; ++s) ring[p][s] = load_frag<T>(kp_nxt + (h + PD - HR) * DR + s * KW);
          ring_ik[p] = ik_nxt[h + PD - HR];
        }
      }
    }
    const int prev_doc = __shfl_up(doc, 1, 16);
    const bool head = (col == 0) || (prev_doc != doc);
    if (uniform) {
      // every row of the block belongs to query rowq[0]: max over the 16 rows
      float v = fmaxf(fmaxf(S[0], S[1]), fmaxf(S[2], S[3]));
      v = fmaxf(v, __shfl_xor(v, 16, 64));
      v = fmaxf(v, __shfl_xor(v, 32, 64));
      const int q = rb * 16 / a.t_r;
      if (a.chunk_keys && G == 0 && cv) atomicMax(a.chunk_keys + (int64_t)q * a.n_chunks + c, score_key(v));
      v = seg_max16(v, doc, col);
      if (G == 0 && head && doc >= 0) atomicMax(a.doc_keys + (int64_t)q * a.n_docs + doc, score_key(v));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = S[i];
        if (a.chunk_keys && cv && rowq[i] >= 0)
          atomicMax(a.chunk_keys + (int64_t)rowq[i] * a.n_chunks + c, score_key(v));
        v = seg_max16(v, doc, col);
        if (head && doc >= 0 && rowq[i] >= 0) atomicMax(a.doc_keys + (int64_t)rowq[i] * a.n_docs + doc, score_key(v));
      }
    }
  }
}

template <typename T, int HR, int DR>
hipError_t route_launch(const RouteArgs &a, hipStream_t s) {
  const int64_t n_tiles = (a.n_chunks + 15) / 16;
  const int n_rows = a.n_q * a.t_r;
  const int rbs = (n_rows + 15) / 16;
  const int64_t target_waves = (int64_t)device_cu_count() * 16;
  int64_t waves = std::max<int64_t>(4, target_waves / rbs);
  if (waves > n_tiles) waves = n_tiles;
  int tiles_per_wave = (int)((n_tiles + waves - 1) / waves);
  waves = (n_tiles + tiles_per_wave - 1) / tiles_per_wave;
  int64_t wgs = (waves + 3) / 4;
  dim3 grid((unsigned)wgs, (unsigned)rbs), block(256);
  hipLaunchKernelGGL((route_scan_kernel<T, HR, DR>), grid, block, 0, s, a, n_tiles, tiles_per_wave);
  return hipGetLastError();
}

template <typename T, int DR>
hipError_t route_by_hr(const RouteArgs &a, hipStream_t s) {
  // the API admits h_r * d_r <= 1024
  switch (a.h_r) {
    case 1: return route_launch<T, 1, DR>(a, s);
    case 2: return route_launch<T, 2, DR>(a, s);
    case 4: return route_launch<T, 4, DR>(a, s);
    case 8: return route_launch<T, 8, DR>(a, s);
    default:
      if constexpr (DR == 64) return route_launch<T, 16, DR>(a, s);
      return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fill_u32(uint32_t *p, size_t n, uint32_t v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t g = std::min<size_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)g), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_keys_to_scores(uint32_t *p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t g = std::min<size_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(keys_to_scores_kernel, dim3((unsigned)g), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_route_scan(const RouteArgs &a, hipStream_t s) {
  if (a.n_chunks == 0) return hipSuccess;
  if (a.dtype == 0) return a.d_r == 64 ? route_by_hr<float, 64>(a, s) : route_by_hr<float, 128>(a, s);
  return a.d_r == 64 ? route_by_hr<bf16_t, 64>(a, s) : route_by_hr<bf16_t, 128>(a, s);
}

}  // namespace msa
