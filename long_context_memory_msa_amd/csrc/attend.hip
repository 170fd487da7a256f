// Sparse GQA attention over the selected documents' pooled keys/values plus
// the query's causal local context.
//
// Lighthouse digest, Component 1 (last step: concatenate the selected
// documents' compressed KV with the query's local KV and attend) and
// Component 2 (the active context uses global RoPE from position k); hotdry
// blog, core architecture (Top-k paragraph) and key engineering details
// (position encoding); gitcode/CSDN article, Document-wise RoPE paragraph
// (background -> query -> generation causal order).
//
// Design (gfx950, flash-attention style, fp32 softmax and accumulation):
//  * one wave owns 16 query rows of one (query, KV head): rows are
//    (token, head-in-group) pairs, so GQA heads share every K/V tile;
//  * scores are computed transposed, S^T = K Q^T (keys as MFMA rows), so that
//    each lane's probabilities are already the B operand of O^T = V^T P^T;
//  * K/V tiles of 32 keys are gathered into LDS by the workgroup: pooled rows
//    of the selected documents' chunks in rank order, then local keys rotated
//    at pos0 + s on the fly; bf16 V rows are stored as they are and read
//    transposed by ds_read_b64_tr_b16 (gfx950) into the V^T operand, fp32 V
//    is stored transposed;
//  * the key list is split across workgroups when there are few rows
//    (decode); partial (max, sum, O) triples are merged by a log-sum-exp pass.
#include <algorithm>

#include "msa_device.hpp"
#include "msa_internal.hpp"
#include "select_wave.hpp"

namespace msa {
namespace {

// Split heuristics (compile-time knobs): splits target SPLIT_MUL waves per
// CU in total, with at least MIN_TILES key tiles per split.  (Counting waves,
// not workgroups: prefill with 4-wave workgroups already fills the GPU and
// every further split only adds merge traffic -- 512 query tokens 56 -> 44
// us; 64 tokens 25 -> 21 us; decode unchanged.)
#ifndef MSA_ATTEND_SPLIT_MUL
#define MSA_ATTEND_SPLIT_MUL 4
#endif
#ifndef MSA_ATTEND_MIN_TILES
#define MSA_ATTEND_MIN_TILES 2
#endif

constexpr int KT = 32;          // keys per tile
constexpr int MAX_K = 256;      // selected documents per query
constexpr float LOG2E = 1.4426950408889634f;

template <typename T> struct VPack;
template <> struct VPack<float> { static constexpr int PAD = 4; };
template <> struct VPack<bf16_t> { static constexpr int PAD = 8; };

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

// ds_read_b64_tr_b16: 8 bytes per lane, 16-bit elements transposed within
// each group of 16 lanes (gfx950)
template <typename T>
__device__ __forceinline__ v4i16 lds_read_tr16(const T *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16 *)(reinterpret_cast<uintptr_t>(p)));
}

struct SplitOut {
  float *o;  // [rows][n_split][d]
  float *m;  // [rows][n_split]
  float *l;  // [rows][n_split]
};

template <typename T, int D, int WGW>
__global__ __launch_bounds__(64 * WGW) void attend_kernel(AttendArgs a, int n_split, int n_rbg, SplitOut so) {
  using F = Frag<T>;
  using FT = typename F::type;
  constexpr int EL = F::EL, KW = F::KW, KS = D / KW;  // k-steps over the head dim
  constexpr int EPS = 16 / sizeof(T);                 // elements per 16-byte segment
  constexpr int NP = D / (2 * EPS);                   // segment pairs (x, x + D/2) per key row
  constexpr int KROW = D + VPack<T>::PAD;             // LDS row pitch of K (elements)
  constexpr bool VTR = sizeof(T) == 2;                // bf16: V row-major, transposed on read
  constexpr int VROW = VTR ? KROW : KT + VPack<T>::PAD;  // pitch of V rows (bf16) / of V^T rows (fp32)
  constexpr int NT = 64 * WGW;

  __shared__ __align__(16) T sK[KT * KROW];
  __shared__ __align__(16) T sV[VTR ? KT * VROW : D * VROW];
  __shared__ int32_t sP[MAX_K + 1];   // prefix of selected documents' chunk counts
  __shared__ int64_t sCB[MAX_K];      // first chunk of each selected document
  __shared__ __align__(16) uint32_t sHist[256];  // in-kernel selection: radix histogram
  __shared__ uint64_t sSel[128];                 // and the compacted / ranked winners

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, G = lane >> 4;
  int bid = blockIdx.x;
  const int split = bid % n_split; bid /= n_split;
  const int rbg = bid % n_rbg; bid /= n_rbg;
  const int kvh = bid % a.h_kv;
  const int q = bid / a.h_kv;
  const int g = a.h_q / a.h_kv;
  const int R = a.T * g;

  // this workgroup's rows and key range
  const int rb = rbg * WGW + wave;
  const int row = rb * 16 + col;               // this lane's query row (S^T / O^T column)
  const bool row_ok = row < R;
  const int t = row_ok ? row / g : 0;
  const int h = kvh * g + (row_ok ? row % g : 0);
  const int s_t = a.L_loc - a.T + t;           // local index of this row's token
  // query fragments first: their loads overlap the document-prefix round trips
  // (B operand of S^T): dims [KW s + EL G, +EL), rotated at pos0 + s_t
  FT qf[KS];
  {
    const T *qp = static_cast<const T *>(a.Q) + (((int64_t)q * a.T + t) * a.h_q + h) * D;
    float x[KS][EL];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if constexpr (EL == 8) {  // bf16: one 16-byte load per k-step
        const uint4 w = row_ok ? *reinterpret_cast<const uint4 *>(qp + s * KW + G * EL) : uint4{0u, 0u, 0u, 0u};
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[s][2 * e] = __uint_as_float(ws[e] << 16);
          x[s][2 * e + 1] = __uint_as_float(ws[e] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < EL; ++e) x[s][e] = row_ok ? Elem<T>::to_f32(qp[s * KW + G * EL + e]) : 0.f;
      }
    }
    const int64_t crow = (int64_t)(a.pos0 + s_t) * (D / 2);
#pragma unroll
    for (int s = 0; s < KS / 2; ++s)
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        const int i = s * KW + G * EL + e;  // < D/2; partner i + D/2 is step s + KS/2
        const float c = a.cos[crow + i], sn = a.sin[crow + i];
        const float lo = x[s][e], hi = x[s + KS / 2][e];
        x[s][e] = lo * c - hi * sn;
        x[s + KS / 2][e] = lo * sn + hi * c;
      }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if constexpr (EL == 1) {
        qf[s] = x[s][0];
      } else {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = (uint32_t)f32_to_bf16(x[s][2 * j]) | ((uint32_t)f32_to_bf16(x[s][2 * j + 1]) << 16);
        qf[s] = __builtin_bit_cast(bf16x8, uint4{w[0], w[1], w[2], w[3]});
      }
    }
  }

  // selected documents -> chunk prefix
  if (threadIdx.x < 64) {
    // in-kernel selection: rank-r document of this query in lane r (k <= 64)
    int sel_doc = 0;
    if (a.cand) {
      constexpr int CI = ATTEND_MAX_CAND / 64;
      const uint64_t *cq = a.cand + (int64_t)q * a.n_cand;
      uint64_t v[CI];
#pragma unroll
      for (int j = 0; j < CI; ++j) v[j] = j * 64 + lane < a.n_cand ? cq[j * 64 + lane] : 0;
      const uint64_t e = wave_topk_sorted<CI>(v, (uint32_t)a.k, sHist, sSel);
      sel_doc = (int)(0xFFFFFFFFu - (uint32_t)e);
      if (a.idx_out && kvh == 0 && split == 0 && rbg == 0 && lane < a.k) {
        a.idx_out[(int64_t)q * a.k + lane] = sel_doc;
        a.val_out[(int64_t)q * a.k + lane] = key_score((uint32_t)(e >> 32));
      }
    }
    int carry = 0;
    for (int base = 0; base < a.k; base += 64) {
      const int r = base + lane;
      int cnt = 0;
      if (r < a.k) {
        int doc = a.cand ? sel_doc : a.idx[(int64_t)q * a.k + r];
        doc = doc < 0 ? 0 : (doc >= a.n_docs ? a.n_docs - 1 : doc);
        const int64_t c0 = a.doc_chunk_off[doc];
        cnt = (int)(a.doc_chunk_off[doc + 1] - c0);
        sCB[r] = c0;
      }
      int x = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      if (r < a.k) sP[r] = carry + x - cnt;
      carry += __shfl(x, 63, 64);
    }
    if (lane == 0) sP[a.k] = carry;
  }
  __syncthreads();
  const int n_mem = sP[a.k];
  const int n_keys = n_mem + a.L_loc;

  const int last_row = std::min(R, (rbg * WGW + WGW) * 16) - 1;
  const int s_last = a.L_loc - a.T + last_row / g;
  int kps = (n_keys + n_split - 1) / n_split;
  kps = (kps + KT - 1) / KT * KT;
  const int k_lo = split * kps;
  const int k_hi = std::min(std::min(n_keys, k_lo + kps), n_mem + s_last + 1);  // causal trim

  const float c2 = a.scale * LOG2E;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc_o[D / 16];
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) acc_o[mb] = zero4();

  const T *kbar = static_cast<const T *>(a.kbar) + (int64_t)kvh * a.kv_stride * D;
  const T *vbar = static_cast<const T *>(a.vbar) + (int64_t)kvh * a.kv_stride * D;
  const T *kloc = static_cast<const T *>(a.K_loc);
  const T *vloc = static_cast<const T *>(a.V_loc);

  // ---- tile gather, split in two phases so that the next tile's global
  // loads are in flight while the current tile is computed:
  //   load:  unit u (key, segment pair m) of the tile -> raw 16-byte words in
  //          registers, plus the RoPE position for local keys (-1: none)
  //   store: rotate local keys, convert, write K and V^T into LDS
  constexpr int UPT = (KT * NP + NT - 1) / NT;  // units per thread per tile (threads past the tile idle)
  uint4 rk[UPT][2], rv[UPT][2];
  int rpos[UPT];
  auto load_tile = [&](int kb) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = threadIdx.x + i * NT;
      const int key = u / NP, m = u % NP;
      const int j = kb + key;
      const T *ks = nullptr, *vs = nullptr;
      rpos[i] = -1;
      if (u >= KT * NP) {
        // no unit for this thread
      } else if (j < k_hi && j < n_mem) {
        int lo_r = 0, hi_r = a.k - 1;  // rank r with sP[r] <= j < sP[r+1]
        while (lo_r < hi_r) {
          const int mid = (lo_r + hi_r + 1) >> 1;
          if (sP[mid] <= j) lo_r = mid; else hi_r = mid - 1;
        }
        int64_t ch = sCB[lo_r] + (j - sP[lo_r]);
        ch = ch < a.n_chunks ? ch : a.n_chunks - 1;
        ks = kbar + ch * D;
        vs = vbar + ch * D;
      } else if (j < k_hi) {
        const int s = j - n_mem;
        const int64_t off = (((int64_t)q * a.L_loc + s) * a.h_kv + kvh) * D;
        ks = kloc + off;
        vs = vloc + off;
        rpos[i] = a.pos0 + s;
      }
      if (ks) {
        rk[i][0] = *reinterpret_cast<const uint4 *>(ks + m * EPS);
        rk[i][1] = *reinterpret_cast<const uint4 *>(ks + D / 2 + m * EPS);
        rv[i][0] = *reinterpret_cast<const uint4 *>(vs + m * EPS);
        rv[i][1] = *reinterpret_cast<const uint4 *>(vs + D / 2 + m * EPS);
      } else {
        rk[i][0] = rk[i][1] = rv[i][0] = rv[i][1] = uint4{0u, 0u, 0u, 0u};  // zeros: no NaN reaches P*V
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = threadIdx.x + i * NT;
      if (u >= KT * NP) continue;
      const int key = u / NP, m = u % NP;
      if constexpr (sizeof(T) == 2) {
        // bf16 V rows (pooled or local: no rotation) go to LDS as they are
        *reinterpret_cast<uint4 *>(sV + key * VROW + m * EPS) = rv[i][0];
        *reinterpret_cast<uint4 *>(sV + key * VROW + D / 2 + m * EPS) = rv[i][1];
        if (rpos[i] < 0) {
          // pooled (or zero) bf16 key: the words go to LDS as they are
          *reinterpret_cast<uint4 *>(sK + key * KROW + m * EPS) = rk[i][0];
          *reinterpret_cast<uint4 *>(sK + key * KROW + D / 2 + m * EPS) = rk[i][1];
          continue;
        }
      }
      float lo[EPS], hi[EPS], vlo[EPS], vhi[EPS];
      float *dk[2] = {lo, hi}, *dv[2] = {vlo, vhi};
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const uint32_t wk[4] = {rk[i][p].x, rk[i][p].y, rk[i][p].z, rk[i][p].w};
        const uint32_t wv[4] = {rv[i][p].x, rv[i][p].y, rv[i][p].z, rv[i][p].w};
        if constexpr (EPS == 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) { dk[p][e] = __uint_as_float(wk[e]); dv[p][e] = __uint_as_float(wv[e]); }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dk[p][2 * e] = __uint_as_float(wk[e] << 16); dk[p][2 * e + 1] = __uint_as_float(wk[e] & 0xFFFF0000u);
            dv[p][2 * e] = __uint_as_float(wv[e] << 16); dv[p][2 * e + 1] = __uint_as_float(wv[e] & 0xFFFF0000u);
          }
        }
      }
      if (rpos[i] >= 0) {
        const int64_t crow = (int64_t)rpos[i] * (D / 2) + m * EPS;
#pragma unroll
        for (int e = 0; e < EPS; ++e) {
          const float c = a.cos[crow + e], sn = a.sin[crow + e];
          const float x0 = lo[e], x1 = hi[e];
          lo[e] = x0 * c - x1 * sn;
          hi[e] = x0 * sn + x1 * c;
        }
      }
      T *dK = sK + key * KROW + m * EPS;
#pragma unroll
      for (int e = 0; e < EPS; ++e) {
        dK[e] = Elem<T>::from_f32(lo[e]);
        dK[D / 2 + e] = Elem<T>::from_f32(hi[e]);
        if constexpr (!VTR) {
          sV[(m * EPS + e) * VROW + key] = Elem<T>::from_f32(vlo[e]);
          sV[(D / 2 + m * EPS + e) * VROW + key] = Elem<T>::from_f32(vhi[e]);
        }
      }
    }
  };

  if (k_lo < k_hi) load_tile(k_lo);
  for (int kb = k_lo; kb < k_hi; kb += KT) {
    store_tile();
    if (kb + KT < k_hi) load_tile(kb + KT);  // next tile in flight during this one
    __syncthreads();

    if (rb * 16 < R) {
      // ---- S^T = K Q^T for the 32 keys (two 16-key blocks) -----------------
      f32x4 sc[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        sc[b] = zero4();
        const T *kr = sK + (16 * b + col) * KROW + G * EL;
#pragma unroll
        for (int s = 0; s < KS; ++s) sc[b] = mfma16(load_frag<T>(kr + s * KW), qf[s], sc[b]);
      }
      // lane holds keys 16 b + 4 G + i of column `row`
      float x[2][4];
      float mt = -INFINITY;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = kb + 16 * b + 4 * G + i;
          const bool vis = row_ok && j < k_hi && (j < n_mem || (j - n_mem) <= s_t);
          x[b][i] = vis ? sc[b][i] * c2 : -INFINITY;
          mt = fmaxf(mt, x[b][i]);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_run == -INFINITY) ? (m_new == -INFINITY ? 1.f : 0.f) : exp2f(m_run - m_new);
      float p[2][4];
      float ps = 0.f;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[b][i] = (x[b][i] == -INFINITY) ? 0.f : exp2f(x[b][i] - m_new);
          ps += p[b][i];
        }
      l_run = l_run * alpha + ps;
      m_run = m_new;
#pragma unroll
      for (int mb = 0; mb < D / 16; ++mb) acc_o[mb] *= alpha;

      // ---- O^T += V^T P^T ---------------------------------------------------
      if constexpr (EL == 1) {
#pragma unroll
        for (int mb = 0; mb < D / 16; ++mb) {
          const T *vr = sV + (16 * mb + col) * VROW;
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc_o[mb] = mfma16(Elem<T>::to_f32(vr[16 * b + 4 * G + i]), p[b][i], acc_o[mb]);
        }
      } else {
        // k-slots 0..3 <-> keys 4G..4G+3, slots 4..7 <-> keys 16+4G..16+4G+3
        uint32_t w[4];
        w[0] = (uint32_t)f32_to_bf16(p[0][0]) | ((uint32_t)f32_to_bf16(p[0][1]) << 16);
        w[1] = (uint32_t)f32_to_bf16(p[0][2]) | ((uint32_t)f32_to_bf16(p[0][3]) << 16);
        w[2] = (uint32_t)f32_to_bf16(p[1][0]) | ((uint32_t)f32_to_bf16(p[1][1]) << 16);
        w[3] = (uint32_t)f32_to_bf16(p[1][2]) | ((uint32_t)f32_to_bf16(p[1][3]) << 16);
        const bf16x8 pf = __builtin_bit_cast(bf16x8, uint4{w[0], w[1], w[2], w[3]});
        // V^T operand of lane (col, G): dims 16 mb + col, keys 4G..4G+3 and
        // 16+4G..16+4G+3.  ds_read_b64_tr_b16 hands lane i of a 16-lane group
        // element j of the 4 x 16 block that lanes 4j + i/4 address (8 bytes
        // each), so lane a of the group addresses key 4G + a/4, dims
        // 16 mb + 4 (a % 4) .. +3 of the row-major V tile.
        const T *vb = sV + (4 * G + col / 4) * VROW + 4 * (col % 4);
#pragma unroll
        for (int mb = 0; mb < D / 16; ++mb) {
          const v4i16 v0 = lds_read_tr16(vb + 16 * mb);
          const v4i16 v1 = lds_read_tr16(vb + 16 * VROW + 16 * mb);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, (v8i16){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
          acc_o[mb] = mfma16(vf, pf, acc_o[mb]);
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds dims 16 mb + 4 G + i of row `row` ----------------
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (!row_ok) return;
  const int64_t orow = ((int64_t)q * a.T + t) * a.h_q + h;
  if (n_split == 1) {
    const float inv = 1.0f / l_tot;
    T *op = static_cast<T *>(a.O) + orow * D + 4 * G;
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      if constexpr (EL == 1) {
        *reinterpret_cast<float4 *>(op + 16 * mb) =
            float4{acc_o[mb][0] * inv, acc_o[mb][1] * inv, acc_o[mb][2] * inv, acc_o[mb][3] * inv};
      } else {
        const uint32_t w0 = (uint32_t)f32_to_bf16(acc_o[mb][0] * inv) | ((uint32_t)f32_to_bf16(acc_o[mb][1] * inv) << 16);
        const uint32_t w1 = (uint32_t)f32_to_bf16(acc_o[mb][2] * inv) | ((uint32_t)f32_to_bf16(acc_o[mb][3] * inv) << 16);
        *reinterpret_cast<uint2 *>(op + 16 * mb) = uint2{w0, w1};
      }
    }
  } else {
    float *po = so.o + (orow * n_split + split) * D + 4 * G;
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb)
      *reinterpret_cast<float4 *>(po + 16 * mb) = float4{acc_o[mb][0], acc_o[mb][1], acc_o[mb][2], acc_o[mb][3]};
    if (G == 0) {
      so.m[orow * n_split + split] = m_run;
      so.l[orow * n_split + split] = l_tot;
    }
  }
}

// Log-sum-exp merge of the split partials: one thread per (row, dim).
template <typename T, int D>
__global__ void attend_combine_kernel(int64_t rows, int n_split, SplitOut so, void *O) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= rows * D) return;
  const int64_t r = e / D;
  const int dd = (int)(e % D);
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, so.m[r * n_split + s]);
  float L = 0.f, acc = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const float ms = so.m[r * n_split + s];
    const float w = ms == -INFINITY ? 0.f : exp2f(ms - M);
    L += w * so.l[r * n_split + s];
    acc += w * so.o[(r * n_split + s) * D + dd];
  }
  static_cast<T *>(O)[r * D + dd] = Elem<T>::from_f32(acc / L);
}

struct Plan {
  int wgw, n_rb, n_rbg, n_split;
};

Plan plan(const AttendArgs &a) {
  Plan p;
  const int g = a.h_q / a.h_kv;
  const int R = a.T * g;
  p.n_rb = (R + 15) / 16;
  p.wgw = p.n_rb >= 4 ? 4 : 1;
  p.n_rbg = (p.n_rb + p.wgw - 1) / p.wgw;
  const int64_t base = (int64_t)a.n_q * a.h_kv * p.n_rbg;
  const int64_t est_keys = std::min<int64_t>((int64_t)a.k * std::max(1, a.max_doc_chunks), a.n_chunks) + a.L_loc;
  const int64_t tiles = (est_keys + KT - 1) / KT;
  // keys/values in host memory: the host link bounds the gather, and a
  // workgroup per (query, KV head, row group) keeps enough rows in flight
  // while leaving the GPU to a concurrent router scan
  const int64_t waves = base * p.wgw;
  int64_t ns = a.kv_host ? 1 : ((int64_t)MSA_ATTEND_SPLIT_MUL * device_cu_count() + waves - 1) / waves;
  ns = std::min<int64_t>(ns, std::max<int64_t>(1, tiles / MSA_ATTEND_MIN_TILES));
  ns = std::max<int64_t>(1, std::min<int64_t>(ns, 64));
  p.n_split = (int)ns;
  return p;
}

template <typename T, int D, int WGW>
hipError_t launch_kernel(const AttendArgs &a, const Plan &p, const SplitOut &so, hipStream_t s) {
  const int64_t grid = (int64_t)a.n_q * a.h_kv * p.n_rbg * p.n_split;
  hipLaunchKernelGGL((attend_kernel<T, D, WGW>), dim3((unsigned)grid), dim3(64 * WGW), 0, s, a, p.n_split, p.n_rbg, so);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_split == 1) return e;
  const int64_t rows = (int64_t)a.n_q * a.T * a.h_q;
  const int64_t n = rows * D;
  hipLaunchKernelGGL((attend_combine_kernel<T, D>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, rows,
                     p.n_split, so, a.O);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t dispatch_wgw(const AttendArgs &a, const Plan &p, const SplitOut &so, hipStream_t s) {
  return p.wgw == 4 ? launch_kernel<T, D, 4>(a, p, so, s) : launch_kernel<T, D, 1>(a, p, so, s);
}

}  // namespace

int attend_splits(const AttendArgs &a) { return plan(a).n_split; }

size_t attend_ws_bytes(const AttendArgs &a) {
  const Plan p = plan(a);
  if (p.n_split == 1) return 0;
  const size_t rows = (size_t)a.n_q * a.T * a.h_q;
  return rows * p.n_split * (a.d + 2) * sizeof(float);
}

hipError_t launch_attend(const AttendArgs &a, void *ws, hipStream_t s) {
  const Plan p = plan(a);
  const size_t rows = (size_t)a.n_q * a.T * a.h_q;
  SplitOut so{nullptr, nullptr, nullptr};
  if (p.n_split > 1) {
    float *base = static_cast<float *>(ws);
    so.o = base;
    so.m = base + rows * p.n_split * a.d;
    so.l = so.m + rows * p.n_split;
  }
  if (a.dtype == 0) return a.d == 64 ? dispatch_wgw<float, 64>(a, p, so, s) : dispatch_wgw<float, 128>(a, p, so, s);
  return a.d == 64 ? dispatch_wgw<bf16_t, 64>(a, p, so, s) : dispatch_wgw<bf16_t, 128>(a, p, so, s);
}

}  // namespace msa
