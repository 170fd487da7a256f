// Router projection Y = X W^T: hidden states to router queries or keys.
//
// The router's projectors map the backbone's hidden states to the router
// query Q^R (for the current tokens) and the router key K^R (for every memory
// token, at encoding time) -- hotdry blog, core architecture of the learnable
// memory routing layer; its parameter advice puts the router width at 2-4x
// the head dimension.  X [rows][hidden] bf16, W [out][hidden] bf16 (one row
// per output feature), Y [rows][out] bf16 rounded once from an fp32
// accumulation.
//
// A bf16 GEMM with both operands contiguous along K:
//  * a workgroup owns 256 rows x 256 outputs (sixteen waves of 64 x 64 on
//    v_mfma_f32_16x16x32_bf16, four per SIMD: a 256K x 2560 x 1024 slab at
//    40 % of the bf16 MFMA peak against 33 % for 128 x 128 tiles of four waves
//    at two workgroups per CU, and 28-30 % for 256 x 128 or 128 x 256 tiles of
//    eight waves), or 128 x 128 where the outputs are not a multiple of 256 or
//    the rows few;
//  * the K loop runs in stages of 64 elements (128 bytes per row) filled by
//    direct-to-LDS loads into swizzled rows, double-buffered (separate LDS
//    variables per buffer, so the compiler does not wait for the fill in
//    flight), one barrier per stage;
//  * output tiles of one row tile share an XCD (blockIdx % 8), so the row
//    tile is re-read from that XCD's L2;
//  * the product is taken as W X^T, so that a lane's accumulator holds four
//    consecutive outputs of one row: 8-byte stores.
//
// A few rows (a decode step's queries) leave that tiling with out/128
// workgroups walking the whole K loop one after another; there the product is
// a stream of W (out x hidden) with X held in L2, and it runs skinny instead:
// one workgroup per 16 outputs, its eight waves splitting K into contiguous
// ranges (16-byte loads straight into MFMA operands, no LDS staging), the
// eight partial 16 x 16 tiles summed through LDS.
#include <algorithm>

#include "msa_device.hpp"
#include "msa_internal.hpp"

namespace msa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int SK = 64;   // K elements per stage
// row counts up to this take the skinny kernel (at most 4 row tiles of 16)
constexpr int SKINNY_ROWS = 64;
static_assert(SKINNY_ROWS <= 64, "skinny projection holds at most 4 row tiles");

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ void fill16(const bf16_t *g, bf16_t *lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void *)lds_base, 16, 0, 0);
}

constexpr int VM0 = 0 | (7 << 4) | (15 << 8);            // vmcnt(0)
constexpr int LGKM0 = 15 | (7 << 4) | (0 << 8) | (3 << 14);  // lgkmcnt(0)

__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(VM0);
  __builtin_amdgcn_s_waitcnt(LGKM0);
  __builtin_amdgcn_s_barrier();
}

// PM rows x PN outputs per workgroup, waves of 64 x 64
template <int PM, int PN, int PW = (PM / 64) * (PN / 64)>
__global__ __launch_bounds__(64 * PW) void project_kernel(const bf16_t *X, const bf16_t *W, int64_t rows, int hidden,
                                                         int out, bf16_t *Y, int n_rtiles, int n_otiles) {
  __shared__ __align__(16) bf16_t sA0[PM * SK], sA1[PM * SK];
  __shared__ __align__(16) bf16_t sB0[PN * SK], sB1[PN * SK];
  constexpr int FA = PM / PW / 8, FB = PN / PW / 8;  // 1 KB direct-to-LDS loads per wave per stage

  // tile order: output tiles of one row tile share blockIdx % 8 (one XCD)
  const int b = blockIdx.x;
  const int r8 = b / 8;
  const int o_tile = r8 % n_otiles;
  const int r_tile = (r8 / n_otiles) * 8 + (b % 8);
  if (r_tile >= n_rtiles) return;  // padding workgroup: exits as a whole before any barrier

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, G = lane >> 4;
  const int wr = wave % (PM / 64), wc = wave / (PM / 64);
  const int64_t row0 = (int64_t)r_tile * PM;
  const int o0 = o_tile * PN;
  const int rows_here = (int)std::min<int64_t>(PM, rows - row0);
  const bf16_t *xt = X + row0 * hidden;
  const bf16_t *wt = W + (int64_t)o0 * hidden;

  // fill of a stage: wave w writes rows 32w .. 32w+31 of each operand; in load
  // p, lane L writes row 32w + 8p + L/8 at physical slot L%8 = logical slot
  // (L%8) ^ swz(row); rows past the end read the last valid row (discarded)
  uint32_t aoff[FA], boff[FB];
#pragma unroll
  for (int p = 0; p < FA; ++p) {
    const int row = 8 * FA * wave + 8 * p + lane / 8;
    const int slot = (lane % 8) ^ swz(row);
    aoff[p] = (uint32_t)(std::min(row, rows_here - 1) * hidden + slot * 8);
  }
#pragma unroll
  for (int p = 0; p < FB; ++p) {
    const int row = 8 * FB * wave + 8 * p + lane / 8;
    const int slot = (lane % 8) ^ swz(row);
    boff[p] = (uint32_t)(row * hidden + slot * 8);
  }
  auto fill = [&](bf16_t *dA, bf16_t *dB, int k0) {
#pragma unroll
    for (int p = 0; p < FA; ++p) fill16(xt + aoff[p] + k0, dA + (8 * FA * wave + 8 * p) * SK);
#pragma unroll
    for (int p = 0; p < FB; ++p) fill16(wt + boff[p] + k0, dB + (8 * FB * wave + 8 * p) * SK);
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = zero4();
  // k-step ks pairs logical slot 2G + ks of a row of X and of W
  auto multiply = [&](const bf16_t *sA, const bf16_t *sB) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra = 64 * wr + 16 * i + col, rb = 64 * wc + 16 * i + col;
        fa[i] = *reinterpret_cast<const bf16x8 *>(sA + ra * SK + ((2 * G + ks) ^ swz(ra)) * 8);
        fb[i] = *reinterpret_cast<const bf16x8 *>(sB + rb * SK + ((2 * G + ks) ^ swz(rb)) * 8);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(fb[j], fa[i], acc[i][j]);
    }
  };

  const int n_stages = hidden / SK;
  fill(sA0, sB0, 0);
  stage_barrier();
#pragma unroll 1
  for (int st = 0; st < n_stages; st += 2) {
    if (st + 1 < n_stages) fill(sA1, sB1, (st + 1) * SK);
    multiply(sA0, sB0);
    stage_barrier();
    if (st + 1 < n_stages) {
      if (st + 2 < n_stages) fill(sA0, sB0, (st + 2) * SK);
      multiply(sA1, sB1);
      stage_barrier();
    }
  }

  // acc[i][j]: outputs 64 wc + 16 j + 4 G + e of row 64 wr + 16 i + col (8 bytes per lane)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 64 * wr + 16 * i + col;
    if (r < rows_here) {
      bf16_t *yrow = Y + (row0 + r) * out + o0 + 64 * wc + 4 * G;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w0 = (uint32_t)f32_to_bf16(acc[i][j][0]) | ((uint32_t)f32_to_bf16(acc[i][j][1]) << 16);
        const uint32_t w1 = (uint32_t)f32_to_bf16(acc[i][j][2]) | ((uint32_t)f32_to_bf16(acc[i][j][3]) << 16);
        *reinterpret_cast<uint2 *>(yrow + 16 * j) = uint2{w0, w1};
      }
    }
  }
}

// rows <= 16 * MT; grid = out / 16 workgroups of 8 waves
template <int MT>
__global__ __launch_bounds__(512) void project_skinny_kernel(const bf16_t *X, const bf16_t *W, int rows, int hidden,
                                                             int out, bf16_t *Y) {
  __shared__ f32x4 red[8][MT][64];
  // The wave index goes through a scalar register so the k-range and batch
  // bounds below are scalar and every branch around an MFMA is a scalar
  // branch: MFMA ignores EXEC, so an MFMA left under an all-false lane mask
  // would still accumulate stale operands.
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, G = lane >> 4;
  const int o0 = blockIdx.x * 16;
  // k-step s covers elements 32 s .. 32 s + 31; lane group G takes 8 of them
  const int n_steps = hidden / 32;
  const int s0 = n_steps * wave / 8, s1 = n_steps * (wave + 1) / 8;
  const bf16_t *wrow = W + (int64_t)(o0 + col) * hidden + 8 * G;
  const bf16_t *xrow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) xrow[m] = X + (int64_t)std::min(16 * m + col, rows - 1) * hidden + 8 * G;
  f32x4 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = zero4();
  // batches of U k-steps: every load of a batch is issued before its first MFMA
  constexpr int U = MT <= 2 ? 8 : 4;
  auto batch = [&](int st, int n) {
    bf16x8 b[U], a[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (u < n) {
        b[u] = *reinterpret_cast<const bf16x8 *>(wrow + 32 * (st + u));
#pragma unroll
        for (int m = 0; m < MT; ++m) a[u][m] = *reinterpret_cast<const bf16x8 *>(xrow[m] + 32 * (st + u));
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (u < n)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = mfma16(a[u][m], b[u], acc[m]);
  };
  int st = s0;
#pragma unroll 1
  for (; st + U <= s1; st += U) batch(st, U);
  if (st < s1) batch(st, s1 - st);
#pragma unroll
  for (int m = 0; m < MT; ++m) red[wave][m][lane] = acc[m];
  __syncthreads();
  // acc[m] of lane l, element e: row 16 m + 4 (l / 16) + e, output o0 + l % 16;
  // thread t takes (m, l / 16, e) = t / 16 and output t % 16
  for (int t = threadIdx.x; t < MT * 256; t += 512) {
    const int c = t & 15, e = (t >> 4) & 3, g = (t >> 6) & 3, m = t >> 8;
    const int row = 16 * m + 4 * g + e;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) sum += red[w][m][16 * g + c][e];
    if (row < rows) Y[(int64_t)row * out + o0 + c] = bf16_t{f32_to_bf16(sum)};
  }
}

template <int MT>
void launch_skinny(const void *X, const void *W, int rows, int hidden, int out, void *Y, hipStream_t s) {
  hipLaunchKernelGGL((project_skinny_kernel<MT>), dim3(out / 16), dim3(512), 0, s, static_cast<const bf16_t *>(X),
                     static_cast<const bf16_t *>(W), rows, hidden, out, static_cast<bf16_t *>(Y));
}

template <int PM, int PN>
hipError_t launch_tiled(const void *X, const void *W, int64_t rows, int hidden, int out, void *Y, hipStream_t s) {
  const int n_rtiles = (int)((rows + PM - 1) / PM), n_otiles = out / PN;
  const int64_t grid = 8 * (int64_t)n_otiles * ((n_rtiles + 7) / 8);
  hipLaunchKernelGGL((project_kernel<PM, PN>), dim3((unsigned)grid), dim3(64 * (PM / 64) * (PN / 64)), 0, s,
                     static_cast<const bf16_t *>(X), static_cast<const bf16_t *>(W), rows, hidden, out,
                     static_cast<bf16_t *>(Y), n_rtiles, n_otiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_project(const void *X, const void *W, int64_t rows, int hidden, int out, void *Y, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (rows <= SKINNY_ROWS) {
    const int r = (int)rows;
    if (r <= 16) launch_skinny<1>(X, W, r, hidden, out, Y, s);
    else if (r <= 32) launch_skinny<2>(X, W, r, hidden, out, Y, s);
    else if (r <= 48) launch_skinny<3>(X, W, r, hidden, out, Y, s);
    else launch_skinny<4>(X, W, r, hidden, out, Y, s);
    return hipGetLastError();
  }
  // 256 x 256 tiles (sixteen waves, four per SIMD, one workgroup per CU)
  // where the outputs and rows fill them; 128 x 128 (four waves, two
  // workgroups per CU) otherwise
  if (out % 256 == 0 && rows >= 1024) return launch_tiled<256, 256>(X, W, rows, hidden, out, Y, s);
  return launch_tiled<128, 128>(X, W, rows, hidden, out, Y, s);
}

}  // namespace msa
