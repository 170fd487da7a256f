// Device helpers shared by the MSA kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bfloat16 storage type (bit pattern).
struct bf16_t {
  uint16_t u;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// fp32 -> bf16, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t b = __float_as_uint(f);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// Element traits: T is float or bf16_t.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float *p) { return *p; }
  static __device__ __forceinline__ float to_f32(float v) { return v; }
  static __device__ __forceinline__ float from_f32(float v) { return v; }
  static __device__ __forceinline__ float round(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v.u); }
  static __device__ __forceinline__ bf16_t from_f32(float v) { return bf16_t{f32_to_bf16(v)}; }
  static __device__ __forceinline__ float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};

// Order-preserving map of fp32 scores to uint32 keys: a < b  <=>  key(a) < key(b)
// (finite values; -0 is folded into +0 so equal scores get equal keys).
// Key 0 lies below every finite score and marks "no score yet".
__device__ __forceinline__ uint32_t score_key(float f) {
  f = (f == 0.0f) ? 0.0f : f;
  uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(b);
}

// ---- MFMA ----------------------------------------------------------------
// 16x16 output tiles.  For both instructions the A operand of lane l is row
// (l % 16), the B operand of lane l is column (l % 16), and the k-slots of a
// lane are the same for A and B; lane l of the result holds column (l % 16),
// rows 4 * (l / 16) + i, i < 4.
//   bf16: v_mfma_f32_16x16x32_bf16, 8 consecutive k per lane (k-step 32)
//   fp32: v_mfma_f32_16x16x4_f32,   1 k per lane           (k-step 4)
__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(float a, float b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Operand fragment of one lane for one k-step.
template <typename T> struct Frag;
template <> struct Frag<float> {
  using type = float;
  static constexpr int EL = 1;  // elements per lane per k-step
  static constexpr int KW = 4;  // k-step width
};
template <> struct Frag<bf16_t> {
  using type = bf16x8;
  static constexpr int EL = 8;
  static constexpr int KW = 32;
};

template <typename T>
__device__ __forceinline__ typename Frag<T>::type load_frag(const T *p);
template <>
__device__ __forceinline__ float load_frag<float>(const float *p) {
  return *p;
}
template <>
__device__ __forceinline__ bf16x8 load_frag<bf16_t>(const bf16_t *p) {
  uint4 v = *reinterpret_cast<const uint4 *>(p);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace msa
