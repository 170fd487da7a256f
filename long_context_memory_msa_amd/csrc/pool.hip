// RoPE tables and offline chunk-mean pooling of the memory bank.
//
// Chunk-mean pooling: hotdry blog, core architecture of the memory routing
// layer (split each document into fixed-size chunks, average each chunk's
// tokens into Kbar, Vbar, Kbar^R); Lighthouse digest, Component 1 steps 1-3.
// Document-wise RoPE: Lighthouse digest, Component 2 (every memory document's
// positions start at 0) -- applied per token before the mean.
//
// Memory-bound: each chunk reads C * (2 h_kv d + h_r d_r) elements once and
// writes (2 h_kv d + h_r d_r) elements plus h_r norms.  One workgroup per
// chunk.  bf16 banks whose token rows are whole 1 KB pieces (h_kv d and h_r d_r
// multiples of 512): one wave per piece of the K, V and K^R rows, lane l owning
// elements 8l..8l+7 of the piece for every token of the chunk -- each load
// instruction reads 1 KB of one token row, and no cross-lane sum is needed.
// Other shapes: each wave reduces whole head rows of one tensor, 16-byte
// loads, the tokens of a chunk spread over the wave's token groups.
#include "msa_device.hpp"
#include "msa_internal.hpp"


namespace msa {
namespace {

__global__ void rope_table_kernel(float *cosv, float *sinv, int max_pos, int half, double base, int d) {
  int64_t n = (int64_t)max_pos * half;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    int p = (int)(e / half), i = (int)(e % half);
    double theta = pow(base, -2.0 * (double)i / (double)d);
    double a = (double)p * theta;
    cosv[e] = (float)cos(a);
    sinv[e] = (float)sin(a);
  }
}

__global__ void chunk_doc_kernel(const int64_t *doc_chunk_off, int32_t *chunk_doc, int doc_begin, int doc_end) {
  int doc = doc_begin + blockIdx.x * blockDim.x + threadIdx.x;
  if (doc >= doc_end) return;
  int64_t a = doc_chunk_off[doc], b = doc_chunk_off[doc + 1];
  for (int64_t c = a; c < b; ++c) chunk_doc[c] = doc;
}

// Sum over n_tok token rows of one head row of RD elements (optionally rotated
// at positions pos0 + t), spread over the wave: lane = token group * LPR + slot.
// Returns the full sum of this lane's EPL elements in every lane.
template <typename T, int RD, bool ROPE>
__device__ __forceinline__ void row_sum(const T *src, int64_t stride, int n_tok, int pos0, const float *cosv,
                                        const float *sinv, float (&acc)[16 / sizeof(T)], int lane) {
  constexpr int EPL = 16 / sizeof(T);
  constexpr int LPR = RD / EPL;
  constexpr int TPI = 64 / LPR;
  constexpr int HALF = RD / 2;
  const int tg = lane / LPR, li = lane % LPR, e0 = li * EPL;
#pragma unroll
  for (int j = 0; j < EPL; ++j) acc[j] = 0.f;
#pragma unroll 4
  for (int t = tg; t < n_tok; t += TPI) {
    uint4 raw = *reinterpret_cast<const uint4 *>(src + (int64_t)t * stride + e0);
    float x[EPL];
    if constexpr (sizeof(T) == 4) {
      x[0] = __uint_as_float(raw.x); x[1] = __uint_as_float(raw.y);
      x[2] = __uint_as_float(raw.z); x[3] = __uint_as_float(raw.w);
    } else {
      uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = __uint_as_float(w[j] << 16);
        x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
    if constexpr (ROPE) {
      // partner lane holds element e +- RD/2 of the same token
      const int64_t row = (int64_t)(pos0 + t) * HALF + (e0 % HALF);
      const bool lo = e0 < HALF;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        float p = __shfl_xor(x[j], LPR / 2, 64);
        float c = cosv[row + j], s = sinv[row + j];
        acc[j] += lo ? (x[j] * c - p * s) : (p * s + x[j] * c);
      }
    } else {
#pragma unroll
      for (int j = 0; j < EPL; ++j) acc[j] += x[j];
    }
  }
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
    for (int j = 0; j < EPL; ++j) acc[j] += __shfl_xor(acc[j], o, 64);
}

template <typename T, int RD>
__device__ __forceinline__ void store_row(T *dst, const float (&acc)[16 / sizeof(T)], int n_tok, int lane,
                                          float *inv_norm) {
  constexpr int EPL = 16 / sizeof(T);
  constexpr int LPR = RD / EPL;
  const int tg = lane / LPR, li = lane % LPR;
  const float cnt = (float)n_tok;
  float r[EPL];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    r[j] = Elem<T>::round(acc[j] / cnt);
    ss += r[j] * r[j];
  }
  if (tg == 0) {
    uint4 o;
    if constexpr (sizeof(T) == 4) {
      o = uint4{__float_as_uint(r[0]), __float_as_uint(r[1]), __float_as_uint(r[2]), __float_as_uint(r[3])};
    } else {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = (__float_as_uint(r[2 * j]) >> 16) | (__float_as_uint(r[2 * j + 1]) & 0xFFFF0000u);
      o = uint4{w[0], w[1], w[2], w[3]};
    }
    *reinterpret_cast<uint4 *>(dst + li * EPL) = o;
  }
  if (inv_norm) {
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) ss += __shfl_xor(ss, o, 64);
    if (lane == 0) *inv_norm = ss > 0.f ? 1.0f / sqrtf(ss) : 0.0f;
  }
}

template <typename T, int D, int DR>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
  const int64_t c = a.chunk_begin + blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int doc = a.chunk_doc[c];
  const int64_t dtok = a.doc_tok_off[doc];
  const int64_t L = a.doc_tok_off[doc + 1] - dtok;
  const int64_t j0 = (c - a.doc_chunk_off[doc]) * a.chunk;  // in-document start
  const int n_tok = (int)min((int64_t)a.chunk, L - j0);
  const int64_t row0 = dtok + j0 - a.slab_tok0;               // slab row of the first token
  const int units = 2 * a.h_kv + a.h_r;
  constexpr int EPL = 16 / sizeof(T);
  float acc[EPL];
  for (int u = wave; u < units; u += 4) {
    if (u < a.h_kv) {  // K head u: document-wise RoPE at in-document positions
      const T *src = static_cast<const T *>(a.K) + row0 * (a.h_kv * D) + u * D;
      row_sum<T, D, true>(src, a.h_kv * D, n_tok, (int)j0, a.cos, a.sin, acc, lane);
      store_row<T, D>(static_cast<T *>(a.kbar) + ((int64_t)u * a.kv_stride + c) * D, acc, n_tok, lane, nullptr);
    } else if (u < 2 * a.h_kv) {
      const int h = u - a.h_kv;
      const T *src = static_cast<const T *>(a.V) + row0 * (a.h_kv * D) + h * D;
      row_sum<T, D, false>(src, a.h_kv * D, n_tok, 0, nullptr, nullptr, acc, lane);
      store_row<T, D>(static_cast<T *>(a.vbar) + ((int64_t)h * a.kv_stride + c) * D, acc, n_tok, lane, nullptr);
    } else {
      const int h = u - 2 * a.h_kv;
      const T *src = static_cast<const T *>(a.KR) + row0 * (a.h_r * DR) + h * DR;
      row_sum<T, DR, false>(src, a.h_r * DR, n_tok, 0, nullptr, nullptr, acc, lane);
      store_row<T, DR>(static_cast<T *>(a.krbar) + (c * a.h_r + h) * DR, acc, n_tok, lane,
                       a.kr_inv_norm + c * a.h_r + h);
    }
  }
}

// 16 bytes of the raw token stream, read once: a non-temporal load (the
// slab is far larger than the caches; keeping it out of them measured 74-75 %
// of HBM peak against 68-69 % with ordinary loads, both with 16 tokens per
// lane in flight)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const bf16_t *p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)));
}

// bf16, one wave per 1 KB piece of a token row (512 elements): pieces
// [0, PK) of K, [PK, 2 PK) of V, [2 PK, 2 PK + PR) of K^R.
template <int D, int DR>
__global__ __launch_bounds__(1024) void pool_pieces_kernel(PoolArgs a) {
  constexpr int XL = D / 16;  // lanes between RoPE partners (elements e and e + D/2)
  const int64_t c = a.chunk_begin + blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int piece = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int doc = a.chunk_doc[c];
  const int64_t dtok = a.doc_tok_off[doc];
  const int64_t L = a.doc_tok_off[doc + 1] - dtok;
  const int64_t j0 = (c - a.doc_chunk_off[doc]) * a.chunk;  // in-document start
  const int n_tok = (int)min((int64_t)a.chunk, L - j0);
  const int64_t row0 = dtok + j0 - a.slab_tok0;
  const int PK = a.h_kv * D / 512;
  const int kind = piece < PK ? 0 : (piece < 2 * PK ? 1 : 2);  // K, V, K^R
  const int pi = kind == 2 ? piece - 2 * PK : piece - kind * PK;
  const int rowlen = kind == 2 ? a.h_r * DR : a.h_kv * D;     // elements per token row
  const int e = pi * 512 + lane * 8;                          // this lane's first element in the row
  const bf16_t *src = static_cast<const bf16_t *>(kind == 0 ? a.K : (kind == 1 ? a.V : a.KR)) + row0 * rowlen + e;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  if (kind == 0) {
    // document-wise RoPE at in-document positions j0 + t (rotate-half pairs)
    const int ei = e % D;
    const bool lo = ei < D / 2;
    const float *cp = a.cos + j0 * (D / 2) + ei % (D / 2);
    const float *sp = a.sin + j0 * (D / 2) + ei % (D / 2);
#pragma unroll 16
    for (int t = 0; t < n_tok; ++t) {
      const uint4 raw = load_stream16(src + (int64_t)t * rowlen);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
      const float4 c0 = *reinterpret_cast<const float4 *>(cp + t * (D / 2));
      const float4 c1 = *reinterpret_cast<const float4 *>(cp + t * (D / 2) + 4);
      const float4 s0 = *reinterpret_cast<const float4 *>(sp + t * (D / 2));
      const float4 s1 = *reinterpret_cast<const float4 *>(sp + t * (D / 2) + 4);
      const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = __uint_as_float(w[j] << 16), x1 = __uint_as_float(w[j] & 0xFFFF0000u);
        const float p0 = __shfl_xor(x0, XL, 64), p1 = __shfl_xor(x1, XL, 64);
        acc[2 * j] += lo ? (x0 * cs[2 * j] - p0 * sn[2 * j]) : (p0 * sn[2 * j] + x0 * cs[2 * j]);
        acc[2 * j + 1] += lo ? (x1 * cs[2 * j + 1] - p1 * sn[2 * j + 1]) : (p1 * sn[2 * j + 1] + x1 * cs[2 * j + 1]);
      }
    }
  } else {
#pragma unroll 16
    for (int t = 0; t < n_tok; ++t) {
      const uint4 raw = load_stream16(src + (int64_t)t * rowlen);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += __uint_as_float(w[j] << 16);
        acc[2 * j + 1] += __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
  }
  // chunk mean, rounded once to bf16 (RNE); 16 bytes per lane
  const float cnt = (float)n_tok;
  float r[8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    r[j] = Elem<bf16_t>::round(acc[j] / cnt);
    ss += r[j] * r[j];
  }
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = (__float_as_uint(r[2 * j]) >> 16) | (__float_as_uint(r[2 * j + 1]) & 0xFFFF0000u);
  const uint4 ov{o[0], o[1], o[2], o[3]};
  if (kind == 2) {
    const int h = e / DR, eh = e % DR;
    *reinterpret_cast<uint4 *>(static_cast<bf16_t *>(a.krbar) + (c * a.h_r + h) * DR + eh) = ov;
    // 1/||stored row|| over the DR / 8 lanes of head h
#pragma unroll
    for (int m = 1; m < DR / 8; m <<= 1) ss += __shfl_xor(ss, m, 64);
    if (eh == 0) a.kr_inv_norm[c * a.h_r + h] = ss > 0.f ? 1.0f / sqrtf(ss) : 0.0f;
  } else {
    const int h = e / D, eh = e % D;
    bf16_t *dst = static_cast<bf16_t *>(kind == 0 ? a.kbar : a.vbar);
    *reinterpret_cast<uint4 *>(dst + ((int64_t)h * a.kv_stride + c) * D + eh) = ov;
  }
}

bool pool_pieces_ok(const PoolArgs &a) {
  return a.dtype == 1 && (a.h_kv * a.d) % 512 == 0 && (a.h_r * a.d_r) % 512 == 0 &&
         2 * (a.h_kv * a.d / 512) + a.h_r * a.d_r / 512 <= 16;
}

template <int D, int DR>
hipError_t pool_pieces_launch(const PoolArgs &a, hipStream_t s) {
  const int pieces = 2 * (a.h_kv * D / 512) + a.h_r * DR / 512;
  hipLaunchKernelGGL((pool_pieces_kernel<D, DR>), dim3((unsigned)(a.chunk_end - a.chunk_begin)), dim3(64 * pieces), 0,
                     s, a);
  return hipGetLastError();
}

hipError_t pool_pieces_dispatch(const PoolArgs &a, hipStream_t s) {
  if (a.d == 64) {
    if (a.d_r == 64) return pool_pieces_launch<64, 64>(a, s);
    if (a.d_r == 128) return pool_pieces_launch<64, 128>(a, s);
    return pool_pieces_launch<64, 256>(a, s);
  }
  if (a.d_r == 64) return pool_pieces_launch<128, 64>(a, s);
  if (a.d_r == 128) return pool_pieces_launch<128, 128>(a, s);
  return pool_pieces_launch<128, 256>(a, s);
}

template <typename T>
hipError_t pool_dispatch(const PoolArgs &a, hipStream_t s) {
  dim3 grid((unsigned)(a.chunk_end - a.chunk_begin)), block(256);
  if (a.d == 64 && a.d_r == 64) hipLaunchKernelGGL((pool_kernel<T, 64, 64>), grid, block, 0, s, a);
  else if (a.d == 64 && a.d_r == 128) hipLaunchKernelGGL((pool_kernel<T, 64, 128>), grid, block, 0, s, a);
  else if (a.d == 128 && a.d_r == 64) hipLaunchKernelGGL((pool_kernel<T, 128, 64>), grid, block, 0, s, a);
  else if (a.d == 128 && a.d_r == 128) hipLaunchKernelGGL((pool_kernel<T, 128, 128>), grid, block, 0, s, a);
  else if constexpr (sizeof(T) == 2) {  // router width 256: bf16 banks
    if (a.d == 64) hipLaunchKernelGGL((pool_kernel<T, 64, 256>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((pool_kernel<T, 128, 256>), grid, block, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_table(float *cosv, float *sinv, int max_pos, int d, double base, hipStream_t s) {
  int64_t n = (int64_t)max_pos * (d / 2);
  int64_t g = (n + 255) / 256;
  if (g > 16384) g = 16384;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)g), dim3(256), 0, s, cosv, sinv, max_pos, d / 2, base, d);
  return hipGetLastError();
}

hipError_t launch_pool(const PoolArgs &a, hipStream_t s) {
  int nd = a.doc_end - a.doc_begin;
  hipLaunchKernelGGL(chunk_doc_kernel, dim3((nd + 255) / 256), dim3(256), 0, s, a.doc_chunk_off, a.chunk_doc,
                     a.doc_begin, a.doc_end);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.chunk_end <= a.chunk_begin) return hipSuccess;
  if (pool_pieces_ok(a)) return pool_pieces_dispatch(a, s);
  return a.dtype == 0 ? pool_dispatch<float>(a, s) : pool_dispatch<bf16_t>(a, s);
}

}  // namespace msa
