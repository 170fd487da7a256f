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

// Rank of this lane's value among the first n entries of an LDS array of
// distinct 64-bit values (how many are larger).  Broadcast reads, 16 entries
// per step with all eight 16-byte reads in flight before any compare.  arr
// holds n rounded up to a multiple of 16 slots, those past n zero.
__device__ __forceinline__ int lds_rank16(const uint64_t *arr, int n, uint64_t x) {
  int r = 0;
  for (int m = 0; m < n; m += 16) {  // (n is wave-uniform)
    uint4 w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = reinterpret_cast<const uint4 *>(arr + m)[i];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      r += ((((uint64_t)w[i].y << 32) | w[i].x) > x) + ((((uint64_t)w[i].w << 32) | w[i].z) > x);
  }
  return r;
}

// wave_topk_sorted, first trying a threshold: the need-th largest of the lane
// maxima's score keys is at most that of the need-th largest composite
// overall, so every winner's key reaches it; when at most 64 composites do
// (the usual case when each lane's composites are spread over the score
// range, or are whole sorted lists) they are ranked among themselves,
// otherwise the radix selection runs.  The threshold comes from a 32-step
// binary search on ballot counts, the survivors are compacted by ballots and
// ranked by counting larger survivors in LDS, so no step waits on a chain of
// cross-lane shuffles.  Same contract and result as wave_topk_sorted (lane r:
// rank-r composite, 0 past the selected ones; need <= 64; sel holds 128
// slots, 16-byte aligned).
template <int ITEMS>
__device__ uint64_t wave_topk_sorted_fast(const uint64_t (&v)[ITEMS], uint32_t need, uint32_t *hist, uint64_t *sel) {
  const int lane = threadIdx.x & 63;
  uint64_t mx = 0;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) mx = v[j] > mx ? v[j] : mx;
  const uint32_t key = (uint32_t)(mx >> 32);  // (an empty lane: 0)
  // tau = the largest t with at least `need` lane keys >= t
  uint32_t tau = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t t = tau | (1u << b);
    if ((uint32_t)__popcll(__ballot(key >= t)) >= need) tau = t;
  }
  // survivors (key >= tau) compacted into sel[0, 64) in item-major order
  int total = 0;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const bool keep = v[j] != 0 && (uint32_t)(v[j] >> 32) >= tau;
    const unsigned long long b = __ballot(keep);
    const int pos = total + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
    if (keep && pos < 64) sel[pos] = v[j];
    total += __popcll(b);
  }
  if (total > 64) {  // wave-uniform
    wave_sync();
    return wave_topk_sorted<ITEMS>(v, need, hist, sel);
  }
  if (lane >= total) sel[lane] = 0;  // lds_rank16 reads whole groups of 16
  sel[64 + lane] = 0;
  wave_sync();
  const uint64_t e = lane < total ? sel[lane] : 0;
  const int r = lds_rank16(sel, total, e);
  if (lane < total) sel[64 + r] = e;  // survivors are distinct: ranks are unique
  wave_sync();
  const uint64_t out = (uint32_t)lane < need ? sel[64 + lane] : 0;
  wave_sync();  // sel is read before any later reuse
  return out;
}

}  // namespace msa
