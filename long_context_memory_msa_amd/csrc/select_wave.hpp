// Wave-level top-k selection over 64-bit composites, shared by the top-k
// kernels and by the attention kernel that selects its documents itself
// (Lighthouse digest, Component 1: keep the Top-k documents; hotdry blog,
// Top-k selection mechanism).
//
// A composite is (order-preserving score key << 32) | (0xFFFFFFFF - doc):
// larger means a higher score, then a lower document index, so every
// selection and every order is unique; 0 marks an empty slot.
#pragma once
#include "msa_device.hpp"

namespace msa {

// Histogram add for a digit that most lanes share (the first, sign/exponent
// digit of cosine scores): the two digits met first in the wave are added with
// one LDS atomic each, the remaining lanes add one by one.  (An exhaustive
// loop over distinct digits costs one shuffle round trip per digit; scores
// spread over several binades made it slower than plain atomics.)  Every lane
// of the wave must call it.
__device__ __forceinline__ void hist_add_wave(uint32_t *hist, uint32_t digit, bool active) {
  unsigned long long pending = __ballot(active);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    if (!pending) break;
    const int leader = __ffsll((long long)pending) - 1;
    const uint32_t d = __shfl(digit, leader, 64);
    const unsigned long long same = __ballot(active && digit == d);
    if ((int)(threadIdx.x & 63) == leader) atomicAdd(&hist[d], (uint32_t)__popcll(same));
    pending &= ~same;
  }
  if ((pending >> (threadIdx.x & 63)) & 1ull) atomicAdd(&hist[digit], 1u);
}

__device__ __forceinline__ uint64_t composite(uint32_t key, int64_t i) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
}

// orders this wave's LDS accesses before and after it (LDS executes a wave's
// operations in order; this keeps the compiler from moving them across)
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int ITEMS>
__device__ void select_wave(const uint64_t (&v)[ITEMS], uint32_t need, uint32_t *hist, int *out_shift,
                            uint64_t *out_prefix) {
  const int lane = threadIdx.x & 63;
  uint64_t prefix = 0;
  int shift = 56;
  for (;; shift -= 8) {
    reinterpret_cast<uint4 *>(hist)[lane] = uint4{0u, 0u, 0u, 0u};
    wave_sync();
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const bool match = v[j] != 0 && ((shift == 56) || ((v[j] ^ prefix) >> (shift + 8)) == 0);
      const uint32_t digit = (uint32_t)(v[j] >> shift) & 255;
      if (shift == 56) hist_add_wave(hist, digit, match);
      else if (match) atomicAdd(&hist[digit], 1u);
    }
    wave_sync();
    // lane l owns bins 255-4l .. 252-4l (descending digit order)
    uint32_t c[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = hist[255 - 4 * lane - j];
      sum += c[j];
    }
    uint32_t incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    const unsigned long long m = __ballot(incl >= need);
    const int first = __ffsll((long long)m) - 1;
    uint32_t bin = 0, above = 0, in_bin = 0;
    {
      uint32_t cum = incl - sum;
      bool found = false;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!found && cum + c[j] >= need) {
          bin = 255 - 4 * lane - j;
          above = cum;
          in_bin = c[j];
          found = true;
        }
        cum += c[j];
      }
    }
    bin = __shfl(bin, first, 64);
    above = __shfl(above, first, 64);
    in_bin = __shfl(in_bin, first, 64);
    wave_sync();  // the histogram is read before the next pass clears it
    prefix |= (uint64_t)bin << shift;
    need -= above;
    if (in_bin == need || shift == 0) break;
  }
  *out_shift = shift;
  *out_prefix = prefix;
}

// The `need` largest composites of this wave, sorted in descending order:
// select (radix, as above), compact into sel[0, 64), then each winner finds
// its rank by counting the larger winners (independent LDS reads, no chain
// of cross-lane steps) and lands in sel[64 + rank].  Returns lane r's rank-r
// composite (0 past the selected ones).  need <= 64; sel holds 128 slots;
// every lane of the wave calls it.
template <int ITEMS>
__device__ uint64_t wave_topk_sorted(const uint64_t (&v)[ITEMS], uint32_t need, uint32_t *hist, uint64_t *sel) {
  const int lane = threadIdx.x & 63;
  int shift;
  uint64_t prefix;
  select_wave<ITEMS>(v, need, hist, &shift, &prefix);
  sel[lane] = 0;
  sel[64 + lane] = 0;
  wave_sync();
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) cnt += (v[j] != 0 && (v[j] >> shift) >= (prefix >> shift));
  int x = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  int pos = x - cnt;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j)
    if (v[j] != 0 && (v[j] >> shift) >= (prefix >> shift)) sel[pos++] = v[j];
  wave_sync();
  if ((uint32_t)lane < need) {
    const uint64_t e = sel[lane];
    int rank = 0;
    for (uint32_t j = 0; j < need; ++j) rank += sel[j] > e;
    sel[64 + rank] = e;
  }
  wave_sync();
  const uint64_t r = sel[64 + lane];
  wave_sync();  // sel is read before any later reuse
  return r;
}

// Bitonic sort of one 64-bit value per lane across the wave, descending
// (lane 0 ends with the largest).
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t y = __shfl_xor(x, j, 64);
      // in a block with (lane & k) == 0 the lower lane keeps the larger value
      const bool keep_max = ((lane & j) == 0) == ((lane & k) == 0);
      x = keep_max ? (x > y ? x : y) : (x < y ? x : y);
    }
  return x;
}

// wave_topk_sorted, first trying a threshold: the need-th largest of the lane
// maxima is at most the need-th largest composite overall, so every winner is
// at least that large; when at most 64 composites reach it (the usual case
// for top-k candidates spread over many lanes) one sort of those gives the
// result, otherwise the radix selection runs.  Same contract and result as
// wave_topk_sorted (lane r: rank-r composite, 0 past the selected ones).
template <int ITEMS>
__device__ uint64_t wave_topk_sorted_fast(const uint64_t (&v)[ITEMS], uint32_t need, uint32_t *hist, uint64_t *sel) {
  const int lane = threadIdx.x & 63;
  uint64_t mx = 0;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) mx = v[j] > mx ? v[j] : mx;
  const uint64_t sorted_max = wave_sort_desc(mx);
  const uint64_t tau = __shfl(sorted_max, (int)need - 1, 64);  // 0 when fewer lanes hold a composite
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) cnt += v[j] != 0 && v[j] >= tau;
  int x = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  const int total = __shfl(x, 63, 64);
  if (total > 64) return wave_topk_sorted<ITEMS>(v, need, hist, sel);  // wave-uniform
  sel[lane] = 0;
  wave_sync();
  int pos = x - cnt;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j)
    if (v[j] != 0 && v[j] >= tau) sel[pos++] = v[j];
  wave_sync();
  const uint64_t mine = sel[lane];
  wave_sync();  // sel is read before any later reuse
  const uint64_t r = wave_sort_desc(mine);
  return (uint32_t)lane < need ? r : 0;
}

}  // namespace msa
