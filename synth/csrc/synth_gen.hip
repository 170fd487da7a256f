// Device (gfx950) implementation of the counter-based input generator.
//
// Same definition as synth/rng.py and synth/csrc/synth_host.c:
//   element n of stream `key` = mix64(key + (n + 1) * 0x9E3779B97F4A7C15),
//   mix64 = SplitMix64 output finaliser (Steele, Lea & Flood, OOPSLA 2014);
//   normal value = float(2 * (sum of the four 16-bit fields) - 262140) * C,
//   C = 0x1.bb67aep-17 (fp32); optional bf16 round-to-nearest-even.
// The fp32 multiply and add use explicitly rounded intrinsics so that no
// multiply-add is fused: results are bit-identical to the host generator.
// Input generation only (raw per-token tensors of the synthetic bank); nothing
// of the method's arithmetic is here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ULL;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float normal_at(uint64_t key, uint64_t n) {
  uint64_t z = mix64(key + (n + 1) * kGolden);
  int32_t s = (int32_t)(z & 0xFFFF) + (int32_t)((z >> 16) & 0xFFFF) +
              (int32_t)((z >> 32) & 0xFFFF) + (int32_t)(z >> 48);
  return __fmul_rn((float)(2 * s - 262140), 0x1.bb67aep-17f);
}

__device__ __forceinline__ uint32_t bf16_bits(float x) {
  uint32_t b = __float_as_uint(x);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// out has n elements: fp32 (bf16 == 0) or bf16 bit patterns (bf16 != 0).
__global__ void fill_normal_kernel(uint64_t key, uint64_t c0, int64_t n, int bf16, void *out) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    float v = normal_at(key, c0 + (uint64_t)i);
    if (bf16)
      static_cast<uint16_t *>(out)[i] = (uint16_t)bf16_bits(v);
    else
      static_cast<float *>(out)[i] = v;
  }
}

__global__ void plant_kernel(void *x, int64_t n_tok, int32_t row, const float *uhat, float cg, int bf16) {
  int64_t n = n_tok * row;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    int32_t e = (int32_t)(i % row);
    float v = bf16 ? __uint_as_float((uint32_t)static_cast<uint16_t *>(x)[i] << 16)
                   : static_cast<float *>(x)[i];
    float r = __fadd_rn(__fmul_rn(0.5f, v), __fmul_rn(cg, uhat[e]));
    if (bf16)
      static_cast<uint16_t *>(x)[i] = (uint16_t)bf16_bits(r);
    else
      static_cast<float *>(x)[i] = r;
  }
}

int grid_for(int64_t n) {
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

extern "C" {

// Fill n elements of `out` (device) with stream `key` from counter c0.
int synth_dev_fill_normal(void *out, uint64_t key, uint64_t c0, int64_t n, int bf16, hipStream_t s) {
  if (n <= 0) return 0;
  if (!out) return 1;
  hipLaunchKernelGGL(fill_normal_kernel, dim3(grid_for(n)), dim3(256), 0, s, key, c0, n, bf16, out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// Gold planting on n_tok rows of H*d stored router keys; uhat is device [H*d] fp32.
int synth_dev_plant(void *x, int64_t n_tok, int32_t H, int32_t d, const float *uhat, float cg, int bf16,
                    hipStream_t s) {
  if (n_tok <= 0) return 0;
  if (!x || !uhat || H <= 0 || d <= 0) return 1;
  int64_t n = n_tok * (int64_t)H * d;
  hipLaunchKernelGGL(plant_kernel, dim3(grid_for(n)), dim3(256), 0, s, x, n_tok, H * d, uhat, cg, bf16);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
