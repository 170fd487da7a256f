/* Host (CPU) implementation of the counter-based input generator.
 *
 * Same definition as synth/rng.py and synth/csrc/synth_gen.hip:
 *   element n of stream `key` = mix64(key + (n + 1) * 0x9E3779B97F4A7C15),
 *   mix64 = SplitMix64 output finaliser (Steele, Lea & Flood, OOPSLA 2014);
 *   normal value = float(2 * (sum of the four 16-bit fields) - 262140) * C,
 *   C = 0x1.bb67aep-17 (fp32); optional bf16 round-to-nearest-even.
 * Built with -ffp-contract=off so that no multiply-add is fused.
 * Input generation only: nothing of the method's arithmetic is here.
 */
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline float to_f32(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static inline uint32_t to_u32(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

static inline float round_bf16(float x) {
  uint32_t b = to_u32(x);
  b = (b + 0x7FFFu + ((b >> 16) & 1u)) & 0xFFFF0000u;
  return to_f32(b);
}

static inline float normal_at(uint64_t key, uint64_t n) {
  uint64_t z = mix64(key + (n + 1) * GOLDEN);
  int32_t s = (int32_t)(z & 0xFFFF) + (int32_t)((z >> 16) & 0xFFFF) +
              (int32_t)((z >> 32) & 0xFFFF) + (int32_t)(z >> 48);
  const float c = 0x1.bb67aep-17f;
  return (float)(2 * s - 262140) * c;
}

/* out[i] = store(normal(key, c0 + i)), i < n; bf16 != 0 rounds to bf16. */
void synth_normal(uint64_t key, uint64_t c0, int64_t n, int bf16, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    float v = normal_at(key, c0 + (uint64_t)i);
    out[i] = bf16 ? round_bf16(v) : v;
  }
}

/* Same values as bf16 bit patterns (uint16), for direct upload. */
void synth_normal_bf16_bits(uint64_t key, uint64_t c0, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = (uint16_t)(to_u32(round_bf16(normal_at(key, c0 + (uint64_t)i))) >> 16);
}

/* Gold planting on stored router keys x[n_tok][H][d]:
 * x = store(0.5 * x + cg * uhat[h][i]) with separate fp32 roundings. */
void synth_plant(float *x, int64_t n_tok, int32_t H, int32_t d, const float *uhat, float cg, int bf16) {
  const int64_t row = (int64_t)H * d;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n_tok; ++t) {
    for (int64_t e = 0; e < row; ++e) {
      float half = 0.5f * x[t * row + e];
      float prod = cg * uhat[e];
      float v = half + prod;
      x[t * row + e] = bf16 ? round_bf16(v) : v;
    }
  }
}
