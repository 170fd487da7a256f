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
//  * a pair of waves owns 16 query rows of one (query, KV head), each wave
//    one half of every tile's keys, their partial (max, sum, O) merged
//    through LDS at the end; rows are (token, head-in-group) pairs, so GQA
//    heads share every K/V tile;
//  * scores are computed transposed, S^T = K Q^T (keys as MFMA rows), so that
//    each lane's probabilities are already the B operand of O^T = V^T P^T;
//  * K/V tiles of 128 (bf16) or 64 (fp32) keys are gathered into LDS by the
//    workgroup, each row block's two waves taking one half of them: pooled rows
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

// Split heuristics: splits target SPLIT_MUL waves per CU in total, with at
// least MIN_TILES key tiles per split.  (Counting waves,
// not workgroups: prefill with 4-wave workgroups already fills the GPU and
// every further split only adds merge traffic -- 512 query tokens 56 -> 44
// us; 64 tokens 25 -> 21 us; decode unchanged.)
constexpr int SPLIT_MUL = 4;
constexpr int MIN_TILES = 2;

constexpr int KT0 = 32;         // keys per MFMA k-step of O^T = V^T P^T (a tile holds NK of them)
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

template <typename T, int D, int WGW, int NK, int KH>
__global__ __launch_bounds__(64 * WGW * KH) void attend_kernel(AttendArgs a, int n_split, int n_rbg, SplitOut so) {
  constexpr int KT = KT0 * NK;                        // keys per tile
  using F = Frag<T>;
  using FT = typename F::type;
  constexpr int EL = F::EL, KW = F::KW, KS = D / KW;  // k-steps over the head dim
  constexpr int EPS = 16 / sizeof(T);                 // elements per 16-byte segment
  constexpr int NP = D / (2 * EPS);                   // segment pairs (x, x + D/2) per key row
  constexpr int KROW = D + VPack<T>::PAD;             // LDS row pitch of K (elements)
  constexpr bool VTR = sizeof(T) == 2;                // bf16: V row-major, transposed on read
  constexpr int VROW = VTR ? KROW : KT + VPack<T>::PAD;  // pitch of V rows (bf16) / of V^T rows (fp32)
  constexpr int NT = 64 * WGW * KH;
  constexpr int BPW = 2 * NK / KH, KSW = NK / KH;    // 16-key blocks and 32-key k-steps per wave and tile
  static_assert(KH == 1 || KH == 2, "one or two key halves");

  __shared__ __align__(16) T sK[KT * KROW];
  __shared__ __align__(16) T sV[VTR ? KT * VROW : D * VROW];
  __shared__ int32_t sP[MAX_K + 1];   // prefix of selected documents' chunk counts
  __shared__ int64_t sCB[MAX_K];      // first chunk of each selected document
  __shared__ __align__(16) uint32_t sHist[256];  // in-kernel selection: radix histogram
  __shared__ __align__(16) uint64_t sSel[128];   // and the compacted / ranked winners
  __shared__ int sBadK;                          // a document id outside [0, n_docs)
  __shared__ float sMerge[KH > 1 ? WGW * 64 * (D / 4 + 2) : 1];  // second key half's (max, sum, O) per lane

  const int lane = threadIdx.x & 63;
  const int wave = (threadIdx.x >> 6) % WGW;  // row block of the group
  const int kh = (threadIdx.x >> 6) / WGW;    // key half of each tile this wave takes (KH = 2)
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
      // lane l: candidates [c l, c l + c), runs of the sorted per-slice lists
      constexpr int CI = ATTEND_MAX_CAND / 64;
      const int c = (a.n_cand + 63) / 64;
      const uint64_t *cq = a.cand + (int64_t)q * a.n_cand;
      uint64_t v[CI];
#pragma unroll
      for (int j = 0; j < CI; ++j) {
        const int i = lane * c + j;
        const bool in = j < c && i < a.n_cand;
        const uint64_t x = cq[in ? i : a.n_cand - 1];
        v[j] = in ? x : 0;
      }
      const uint64_t e = wave_topk_sorted_fast<CI>(v, (uint32_t)a.k, sHist, sSel);
      sel_doc = (int)(0xFFFFFFFFu - (uint32_t)e);
      if (a.idx_out && kvh == 0 && split == 0 && rbg == 0 && lane < a.k) {
        a.idx_out[(int64_t)q * a.k + lane] = sel_doc;
        a.val_out[(int64_t)q * a.k + lane] = key_score((uint32_t)(e >> 32));
      }
    }
    int carry = 0;
    bool any_bad = false;
    for (int base = 0; base < a.k; base += 64) {
      const int r = base + lane;
      int cnt = 0;
      if (r < a.k) {
        int doc = a.cand ? sel_doc : a.idx[(int64_t)q * a.k + r];
        const bool bad_doc = doc < 0 || doc >= a.n_docs;  // the query's output becomes NaN
        any_bad |= __ballot(bad_doc) != 0;
        doc = bad_doc ? 0 : doc;
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
    if (lane == 0) {
      sP[a.k] = carry;
      sBadK = any_bad ? 1 : 0;
    }
  }
  __syncthreads();
  const bool bad = sBadK != 0;
  const int n_mem = bad ? 0 : sP[a.k];
  const int n_keys = n_mem + a.L_loc;

  const int last_row = std::min(R, (rbg * WGW + WGW) * 16) - 1;
  const int s_last = a.L_loc - a.T + last_row / g;
  int kps = (n_keys + n_split - 1) / n_split;
  kps = (kps + KT - 1) / KT * KT;
  const int k_lo = split * kps;
  const int k_hi = bad ? k_lo : std::min(std::min(n_keys, k_lo + kps), n_mem + s_last + 1);  // causal trim

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
  float rcs[UPT][EPS], rsn[UPT][EPS];  // rotation of a local key's unit, loaded with it
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
      // the rotation's cos/sin travel with the rows (a memory key's unit
      // reads row 0 of the table and does not use it), not one round trip later
      {
        const int64_t crow = (int64_t)(rpos[i] >= 0 ? rpos[i] : 0) * (D / 2) + m * EPS;
#pragma unroll
        for (int e = 0; e < EPS; e += 4) {
          const float4 cv4 = *reinterpret_cast<const float4 *>(a.cos + crow + e);
          const float4 sv4 = *reinterpret_cast<const float4 *>(a.sin + crow + e);
          rcs[i][e] = cv4.x; rcs[i][e + 1] = cv4.y; rcs[i][e + 2] = cv4.z; rcs[i][e + 3] = cv4.w;
          rsn[i][e] = sv4.x; rsn[i][e + 1] = sv4.y; rsn[i][e + 2] = sv4.z; rsn[i][e + 3] = sv4.w;
        }
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
#pragma unroll
        for (int e = 0; e < EPS; ++e) {
          const float c = rcs[i][e], sn = rsn[i][e];
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
      // ---- S^T = K Q^T for the tile's keys (16-key blocks) --------------------
      // this wave's blocks: kh BPW .. kh BPW + BPW - 1 of the tile
      f32x4 sc[BPW];
#pragma unroll
      for (int bl = 0; bl < BPW; ++bl) {
        sc[bl] = zero4();
        const T *kr = sK + (16 * (kh * BPW + bl) + col) * KROW + G * EL;
#pragma unroll
        for (int s = 0; s < KS; ++s) sc[bl] = mfma16(load_frag<T>(kr + s * KW), qf[s], sc[bl]);
      }
      // lane holds keys 16 b + 4 G + i of column `row`
      float x[BPW][4];
      float mt = -INFINITY;
#pragma unroll
      for (int bl = 0; bl < BPW; ++bl)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int b = kh * BPW + bl;
          const int j = kb + 16 * b + 4 * G + i;
          const bool vis = row_ok && j < k_hi && (j < n_mem || (j - n_mem) <= s_t);
          x[bl][i] = vis ? sc[bl][i] * c2 : -INFINITY;
          mt = fmaxf(mt, x[bl][i]);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_run == -INFINITY) ? (m_new == -INFINITY ? 1.f : 0.f) : exp2f(m_run - m_new);
      float p[BPW][4];
      float ps = 0.f;
#pragma unroll
      for (int bl = 0; bl < BPW; ++bl)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[bl][i] = (x[bl][i] == -INFINITY) ? 0.f : exp2f(x[bl][i] - m_new);
          ps += p[bl][i];
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
          for (int bl = 0; bl < BPW; ++bl)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc_o[mb] = mfma16(Elem<T>::to_f32(vr[16 * (kh * BPW + bl) + 4 * G + i]), p[bl][i], acc_o[mb]);
        }
      } else {
        // per 32-key k-step ks: k-slots 0..3 <-> keys 32 ks + 4G..+3, slots
        // 4..7 <-> keys 32 ks + 16 + 4G..+3
#pragma unroll
        for (int ksl = 0; ksl < KSW; ++ksl) {
          const int ks = kh * KSW + ksl;
          uint32_t w[4];
          w[0] = (uint32_t)f32_to_bf16(p[2 * ksl][0]) | ((uint32_t)f32_to_bf16(p[2 * ksl][1]) << 16);
          w[1] = (uint32_t)f32_to_bf16(p[2 * ksl][2]) | ((uint32_t)f32_to_bf16(p[2 * ksl][3]) << 16);
          w[2] = (uint32_t)f32_to_bf16(p[2 * ksl + 1][0]) | ((uint32_t)f32_to_bf16(p[2 * ksl + 1][1]) << 16);
          w[3] = (uint32_t)f32_to_bf16(p[2 * ksl + 1][2]) | ((uint32_t)f32_to_bf16(p[2 * ksl + 1][3]) << 16);
          const bf16x8 pf = __builtin_bit_cast(bf16x8, uint4{w[0], w[1], w[2], w[3]});
          // V^T operand of lane (col, G): dims 16 mb + col, keys 4G..4G+3 and
          // 16+4G..16+4G+3 of the k-step.  ds_read_b64_tr_b16 hands lane i of a
          // 16-lane group element j of the 4 x 16 block that lanes 4j + i/4
          // address (8 bytes each), so lane a of the group addresses key
          // 4G + a/4, dims 16 mb + 4 (a % 4) .. +3 of the row-major V tile.
          const T *vb = sV + (32 * ks + 4 * G + col / 4) * VROW + 4 * (col % 4);
#pragma unroll
          for (int mb = 0; mb < D / 16; ++mb) {
            const v4i16 v0 = lds_read_tr16(vb + 16 * mb);
            const v4i16 v1 = lds_read_tr16(vb + 16 * VROW + 16 * mb);
            const bf16x8 vf = __builtin_bit_cast(bf16x8, (v8i16){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
            acc_o[mb] = mfma16(vf, pf, acc_o[mb]);
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- the two key halves of each row block merge (second half -> LDS -> first)
  if constexpr (KH > 1) {
    float *mg = sMerge + (wave * 64 + lane) * (D / 4 + 2);
    if (kh == 1) {
      mg[0] = m_run;
      mg[1] = l_run;
#pragma unroll
      for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mg[2 + 4 * mb + i] = acc_o[mb][i];
    }
    __syncthreads();
    if (kh == 1) return;
    const float m1 = mg[0], M = fmaxf(m_run, m1);
    const float w0 = m_run == -INFINITY ? 0.f : exp2f(m_run - M), w1 = m1 == -INFINITY ? 0.f : exp2f(m1 - M);
    l_run = l_run * w0 + mg[1] * w1;
    m_run = M;
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc_o[mb][i] = acc_o[mb][i] * w0 + mg[2 + 4 * mb + i] * w1;
  }

  // ---- epilogue: lane holds dims 16 mb + 4 G + i of row `row` ----------------
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (!row_ok) return;
  const int64_t orow = ((int64_t)q * a.T + t) * a.h_q + h;
  if (n_split == 1) {
    const float inv = bad ? __builtin_nanf("") : 1.0f / l_tot;
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
      so.l[orow * n_split + split] = bad ? __builtin_nanf("") : l_tot;
    }
  }
}

// Log-sum-exp merge of the split partials: one thread per (row, dim).
// Splits are taken CS at a time with all of a group's loads in flight (a
// loop over the splits would wait for each load in turn); groups after the
// first fold in by the same log-sum-exp rescaling.
constexpr int CS = 8;
template <typename T, int D>
__global__ void attend_combine_kernel(int64_t rows, int n_split, SplitOut so, void *O) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= rows * D) return;
  const int64_t r = e / D;
  const int dd = (int)(e % D);
  float M = -INFINITY, L = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < n_split; s0 += CS) {
    float mv[CS], lv[CS], ov[CS];
#pragma unroll
    for (int i = 0; i < CS; ++i) {
      const int64_t k = r * n_split + min(s0 + i, n_split - 1);  // past the last split: re-read it, unused
      mv[i] = so.m[k];
      lv[i] = so.l[k];
      ov[i] = so.o[k * D + dd];
    }
    float Mg = M;
#pragma unroll
    for (int i = 0; i < CS; ++i)
      if (s0 + i < n_split) Mg = fmaxf(Mg, mv[i]);
    const float sc = M == -INFINITY ? 0.f : exp2f(M - Mg);  // (L and acc are 0 while M is -inf)
    L *= sc;
    acc *= sc;
#pragma unroll
    for (int i = 0; i < CS; ++i)
      if (s0 + i < n_split) {
        const float w = mv[i] == -INFINITY ? 0.f : exp2f(mv[i] - Mg);
        L += w * lv[i];
        acc += w * ov[i];
      }
    M = Mg;
  }
  static_cast<T *>(O)[r * D + dd] = Elem<T>::from_f32(acc / L);
}

// 16 bytes of a row as fp32 values (8 bf16 or 4 fp32 elements)
template <typename T>
__device__ __forceinline__ void unpack16(const uint4 &w, float (&x)[16 / sizeof(T)]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(ws[e] << 16);
      x[2 * e + 1] = __uint_as_float(ws[e] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(ws[e]);
  }
}
template <typename T>
__device__ __forceinline__ void load_row16(const T *p, float (&x)[16 / sizeof(T)]) {
  unpack16<T>(*reinterpret_cast<const uint4 *>(p), x);
}

// fp32 values <-> an MFMA operand fragment (bf16: 8 values, rounded to nearest even)
template <typename T>
__device__ __forceinline__ typename Frag<T>::type to_frag(const float (&x)[Frag<T>::EL]) {
  if constexpr (Frag<T>::EL == 1) {
    return x[0];
  } else {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = (uint32_t)f32_to_bf16(x[2 * j]) | ((uint32_t)f32_to_bf16(x[2 * j + 1]) << 16);
    return __builtin_bit_cast(bf16x8, uint4{w[0], w[1], w[2], w[3]});
  }
}
template <typename T>
__device__ __forceinline__ void from_frag(const typename Frag<T>::type &f, float (&x)[Frag<T>::EL]) {
  if constexpr (Frag<T>::EL == 1) {
    x[0] = f;
  } else {
    const uint4 w = __builtin_bit_cast(uint4, f);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(ws[j] << 16);
      x[2 * j + 1] = __uint_as_float(ws[j] & 0xFFFF0000u);
    }
  }
}

// ---- single-token queries (decode) -------------------------------------------
// ns workgroups of DW waves per (query, KV head) (decode_splits: enough for
// one workgroup per compute unit, since a workgroup's gather is bound by its
// compute unit's memory throughput); the g query heads of the KV head are the
// token's rows.  The work is the gather of the selected documents' pooled
// rows, so no key or value tile is staged in LDS and there is no barrier per
// tile:
//  * the ns * DW waves of a (query, KV head) take 16-key blocks in turn; a
//    block's scores S^T = K Q^T come from MFMAs whose A operand is loaded
//    straight from the key rows (lane: key l % 16, 16 bytes per k-step), Q^T
//    in registers (column = query head);
//  * the running softmax is kept per column; values are read in row layout
//    (a key row spread over LPK lanes, 16 bytes each);
//  * bf16: O^T += V^T P^T on MFMA (16x16x16): the block's probabilities are
//    the B operand in the scores' own lane layout, and the block's V rows go
//    to a per-wave LDS slot as they are and come back transposed
//    (ds_read_b64_tr_b16); fp32: the probabilities go through the wave's LDS
//    slot and O[h][dims] accumulates on the vector units;
//  * loads for NB blocks are in flight before any of them is used;
//  * the waves' (max, sum, O) are merged through LDS; with ns > 1 the
//    workgroups' merged partials go to attend_combine_kernel.
// Four waves of about 200 VGPRs, two 16-key blocks in flight per wave: the
// workgroup fits on a compute unit beside two persistent router-scan
// workgroups (128 VGPRs per wave), so a decode pipeline's attention runs
// during the next steps' scans.  Measured at the 100M-token decode layer (16
// queries, k = 16, one workgroup per (query, KV head)): pipelined step 285 us
// against 304 us for eight waves of three blocks (which does not fit beside
// the scans) and 307 us for the many-row kernel with split merge.  Two
// workgroups per (query, KV head) (256 on 256 compute units): the layer's
// top-k + attention 48 -> 37 us.  Measured and not kept for the layer's call:
// four blocks in flight (39 us), the next batch's loads issued before the
// current one is computed (two batches of registers: 39-41 us).
constexpr int DW = 4;          // waves per workgroup
constexpr int DPASS = 1024;    // keys listed per pass (chunk ids in LDS)
constexpr int DNB = 2;         // 16-key blocks in flight per wave

template <typename T, int D, int GQ>
__global__ __launch_bounds__(64 * DW) void attend_decode_kernel(AttendArgs a, int ns, SplitOut so) {
  using F = Frag<T>;
  using FT = typename F::type;
  constexpr int EL = F::EL, KW = F::KW, KS = D / KW;  // MFMA k-steps over the head dim
  constexpr int EPL = 16 / sizeof(T);   // value elements per lane (one 16-byte load)
  constexpr int LPK = D / EPL;          // lanes per value row
  constexpr int KPI = 64 / LPK;         // value rows per load instruction
  constexpr int VPB = 16 / KPI;         // value loads per lane per block
  constexpr int NT = 64 * DW;
  constexpr int NB = sizeof(T) == 2 ? DNB : 1;  // blocks in flight (fp32 operands take 8x the registers)
  static_assert(GQ <= 16 && KPI >= 1 && 16 % KPI == 0, "decode layout");

  __shared__ int32_t sP[MAX_K + 1];          // prefix of the selected documents' chunk counts
  __shared__ int64_t sCB[MAX_K];             // first chunk of each selected document
  __shared__ int64_t sList[DPASS];           // chunk of each memory key of the pass (-1 - s: local key s)
  constexpr bool PV_MFMA = sizeof(T) == 2;   // bf16: O^T += V^T P^T on MFMA; fp32: on the vector units
  constexpr int VP = D + 8;                  // LDS pitch of a wave's V block (elements)
  __shared__ __align__(16) T sVb[PV_MFMA ? DW : 1][PV_MFMA ? 16 * VP : 1];  // a wave's 16 V rows
  __shared__ float sPr[PV_MFMA ? 1 : DW][16][GQ + 1];  // a wave's block probabilities [key][head]
  __shared__ float sAl[DW][GQ];              // and its rescale factors per head
  __shared__ float sM[DW][GQ], sL[DW][GQ];
  __shared__ float sAcc[DW][GQ][D];
  __shared__ __align__(16) uint32_t sHist[256];
  __shared__ __align__(16) uint64_t sSel[128];
  __shared__ int sBad;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // ns workgroups share each (query, KV head): split s takes the blocks of
  // "waves" s DW .. s DW + DW - 1 out of VW
  const int split = blockIdx.x % ns;
  const int kvh = (blockIdx.x / ns) % a.h_kv;
  const int q = blockIdx.x / ns / a.h_kv;
  const int VW = DW * ns;
  const int col = lane & 15, G = lane >> 4;  // MFMA layout: key / head column, k-slot group
  const int vr = lane / LPK, e0 = (lane % LPK) * EPL;  // value layout: key slot, dims
  const int s_q = a.L_loc - 1;               // local index of the query token

  // the layer's candidates are loaded first, so that their round trip
  // overlaps that of the query rows.  Lane l takes candidates [c l, c l + c),
  // c = ceil(n_cand / 64): runs of the sorted per-slice lists, so that the
  // lane maxima are run heads and the selection's threshold (the k-th
  // largest head) passes few values (dealt round-robin, a lane would hold
  // the same rank of many lists).
  constexpr int CI = ATTEND_MAX_CAND / 64;
  const int c_run = (a.n_cand + 63) / 64;
  uint64_t cv[CI];
  if (a.cand && wave == 0) {
    const uint64_t *cq = a.cand + (int64_t)q * a.n_cand;
#pragma unroll
    for (int j = 0; j < CI; ++j) {  // (unconditional loads: slots past the run re-read the last one,
      const int i = lane * c_run + j;  //  masked where the selection reads them)
      cv[j] = cq[j < c_run && i < a.n_cand ? i : a.n_cand - 1];
    }
  }

  // Q^T fragments (B operand): column col = query head kvh * GQ + col, dims
  // [KW s + EL G, +EL), rotated at pos0 + s_q, rounded to the operand type
  FT qf[KS];
  {
    const bool ok = col < GQ;
    const T *qp = static_cast<const T *>(a.Q) + ((int64_t)q * a.h_q + kvh * GQ + (ok ? col : 0)) * D;
    float x[KS][EL];
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      if constexpr (EL == 8) {
        float v[8];
        load_row16<T>(qp + st * KW + G * EL, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[st][e] = ok ? v[e] : 0.f;
      } else {
        x[st][0] = ok ? Elem<T>::to_f32(qp[st * KW + G * EL]) : 0.f;
      }
    }
    const int64_t crow = (int64_t)(a.pos0 + s_q) * (D / 2);
#pragma unroll
    for (int st = 0; st < KS / 2; ++st)
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        const int i = st * KW + G * EL + e;  // < D/2; partner i + D/2 is k-step st + KS/2
        const float c = a.cos[crow + i], sn = a.sin[crow + i];
        const float lo = x[st][e], hi = x[st + KS / 2][e];
        x[st][e] = lo * c - hi * sn;
        x[st + KS / 2][e] = lo * sn + hi * c;
      }
#pragma unroll
    for (int st = 0; st < KS; ++st) qf[st] = to_frag<T>(x[st]);
  }

  // selected documents: the layer's in-kernel selection, or idx; wave 0
  // then loads their chunk ranges (ranks r = lane + 64 j, all loads issued
  // before the first is used) and forms the prefix of the counts with wave
  // scans, so one barrier publishes the list (an id outside [0, n_docs)
  // makes the query's output NaN)
  if (wave == 0) {
    constexpr int RPL = MAX_K / 64;  // ranks per lane
    int doc[RPL];
    if (a.cand) {  // (k <= 64: the rank-r winner is in lane r)
#pragma unroll
      for (int j = 0; j < CI; ++j) cv[j] = j < c_run && lane * c_run + j < a.n_cand ? cv[j] : 0;
      const uint64_t e = wave_topk_sorted_fast<CI>(cv, (uint32_t)a.k, sHist, sSel);
      doc[0] = (int)(0xFFFFFFFFu - (uint32_t)e);
      if (lane < a.k && a.idx_out && kvh == 0 && split == 0) {
        a.idx_out[(int64_t)q * a.k + lane] = doc[0];
        a.val_out[(int64_t)q * a.k + lane] = key_score((uint32_t)(e >> 32));
      }
#pragma unroll
      for (int j = 1; j < RPL; ++j) doc[j] = 0;
    } else {
#pragma unroll
      for (int j = 0; j < RPL; ++j) {
        const int r = lane + 64 * j;
        doc[j] = r < a.k ? a.idx[(int64_t)q * a.k + r] : 0;
      }
    }
    bool any_bad = false;
    int64_t c0[RPL];
    int64_t c1[RPL];
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
      c0[j] = c1[j] = 0;
      if (64 * j >= a.k) break;  // (wave-uniform)
      const int r = lane + 64 * j;
      const bool bad_doc = r < a.k && (doc[j] < 0 || doc[j] >= a.n_docs);
      any_bad |= bad_doc;
      const int d = r < a.k && !bad_doc ? doc[j] : 0;
      c0[j] = a.doc_chunk_off[d];
      c1[j] = a.doc_chunk_off[d + 1];
    }
    int carry = 0;
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
      if (64 * j >= a.k) break;
      const int r = lane + 64 * j;
      const int cnt = r < a.k ? (int)(c1[j] - c0[j]) : 0;
      int x = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      if (r < a.k) {
        sCB[r] = c0[j];
        sP[r] = carry + x - cnt;
      }
      carry += __shfl(x, 63, 64);
    }
    const bool bad_any = __ballot(any_bad) != 0;
    if (lane == 0) {
      sP[a.k] = carry;
      sBad = bad_any ? 1 : 0;
    }
  }
  __syncthreads();
  const bool bad = sBad != 0;
  const int n_mem = bad ? 0 : sP[a.k];
  const int n_keys = bad ? 0 : n_mem + a.L_loc;  // the query token sees every local key

  const T *kbar = static_cast<const T *>(a.kbar) + (int64_t)kvh * a.kv_stride * D;
  const T *vbar = static_cast<const T *>(a.vbar) + (int64_t)kvh * a.kv_stride * D;
  const float c2 = a.scale * LOG2E;
  float m_run = -INFINITY, l_run = 0.f;  // column col's running max; this lane's share of its sum
  float acc[GQ][EPL];  // vector path: O[h][dims e0 ..] of this lane's key slots
#pragma unroll
  for (int h = 0; h < GQ; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  f32x4 oacc[D / 16];  // MFMA path: O^T tile mb, lane (head col, G): dims 16 mb + 4 G .. + 3
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) oacc[mb] = zero4();

  for (int pb = 0; pb < n_keys; pb += DPASS) {
    const int np = min(DPASS, n_keys - pb);
    // the pass's keys: memory key j -> its chunk (rank by binary search), local key s -> -1 - s
    // 16 threads per rank write its chunks that fall in this pass (the
    // local keys form rank k)
    for (int r = tid >> 4; r <= a.k; r += NT >> 4) {
      const int lo = r < a.k ? sP[r] : n_mem, hi = r < a.k ? sP[r + 1] : n_keys;
      const int j1 = min(hi, pb + np);
      for (int j = max(lo, pb) + (tid & 15); j < j1; j += 16)
        sList[j - pb] = r < a.k ? sCB[r] + (j - lo) : -1 - (int64_t)(j - n_mem);
    }
    __syncthreads();
    const int n_blk = (np + 15) / 16;
    // wave w of split s takes blocks s DW + w, + VW, ...; NB of them per batch
    auto load_batch = [&](int b0, FT (&kf)[NB][KS], uint4 (&vw)[NB][VPB]) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int kb = (b0 + nb * VW) * 16;
        // key rows (A operand): key kb + col, k-step st: dims KW st + EL G
        {
          const int jl = kb + col;
          const int64_t ent = jl < np ? sList[jl] : 0;
          const T *kp;
          if (ent >= 0) {
            kp = kbar + ent * D;
          } else {
            const int s = (int)(-1 - ent);
            kp = static_cast<const T *>(a.K_loc) + (((int64_t)q * a.L_loc + s) * a.h_kv + kvh) * D;
          }
#pragma unroll
          for (int st = 0; st < KS; ++st) kf[nb][st] = load_frag<T>(kp + st * KW + G * EL);
        }
        // value rows: keys kb + vr + KPI u, dims e0
#pragma unroll
        for (int u = 0; u < VPB; ++u) {
          const int jl = kb + vr + KPI * u;
          const int64_t ent = jl < np ? sList[jl] : 0;
          const T *vp = ent >= 0 ? vbar + ent * D
                                 : static_cast<const T *>(a.V_loc) +
                                       (((int64_t)q * a.L_loc + (-1 - ent)) * a.h_kv + kvh) * D;
          vw[nb][u] = *reinterpret_cast<const uint4 *>(vp + e0);
        }
      }
    };
    auto compute_batch = [&](int b0, FT (&kf)[NB][KS], uint4 (&vw)[NB][VPB]) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int kb = (b0 + nb * VW) * 16;
        if (b0 + nb * VW < n_blk) {  // wave-uniform (a predicate, not a break: the indices stay constant)
        // local keys: RoPE at pos0 + s (partner dims are k-step st + KS/2 of this lane)
        {
          const int jl = kb + col;
          const int64_t ent = jl < np ? sList[jl] : 0;
          if (ent < 0) {
            const int64_t crow = (a.pos0 + (-1 - ent)) * (int64_t)(D / 2);
#pragma unroll
            for (int st = 0; st < KS / 2; ++st) {
              float lo[EL], hi[EL];
              from_frag<T>(kf[nb][st], lo);
              from_frag<T>(kf[nb][st + KS / 2], hi);
#pragma unroll
              for (int e = 0; e < EL; ++e) {
                const int i = st * KW + G * EL + e;
                const float c = a.cos[crow + i], sn = a.sin[crow + i];
                const float x0 = lo[e], x1 = hi[e];
                lo[e] = x0 * c - x1 * sn;
                hi[e] = x0 * sn + x1 * c;
              }
              kf[nb][st] = to_frag<T>(lo);
              kf[nb][st + KS / 2] = to_frag<T>(hi);
            }
          }
        }
        // S^T = K Q^T: lane holds keys kb + 4G + i of head column col
        f32x4 sc = zero4();
#pragma unroll
        for (int st = 0; st < KS; ++st) sc = mfma16(kf[nb][st], qf[st], sc);
        float x[4], mt = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool vis = col < GQ && kb + 4 * G + i < np;
          x[i] = vis ? sc[i] * c2 : -INFINITY;
          mt = fmaxf(mt, x[i]);
        }
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = m_run == -INFINITY ? (m_new == -INFINITY ? 1.f : 0.f) : exp2f(m_run - m_new);
        float pr4[4], ps = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr4[i] = x[i] == -INFINITY ? 0.f : exp2f(x[i] - m_new);
          ps += pr4[i];
        }
        l_run = l_run * alpha + ps;
        m_run = m_new;
        if constexpr (PV_MFMA) {
          // P^T (B operand): lane (head col, G) holds keys 4G..4G+3 of its
          // column, exactly the scores' layout; V rows go to the wave's LDS
          // slot as they are and come back transposed (ds_read_b64_tr_b16:
          // lane a of group G addresses key 4G + a/4, dims 16 mb + 4 (a % 4)
          // and receives dims 16 mb + a of keys 4G .. 4G+3: the V^T operand)
          T *slot = sVb[wave];
#pragma unroll
          for (int u = 0; u < VPB; ++u) {  // (field by field: an aggregate copy keeps vw out of registers)
            const uint32_t w0 = vw[nb][u].x, w1 = vw[nb][u].y, w2 = vw[nb][u].z, w3 = vw[nb][u].w;
            *reinterpret_cast<uint4 *>(slot + (vr + KPI * u) * VP + e0) = uint4{w0, w1, w2, w3};
          }
          const uint32_t p01 = (uint32_t)f32_to_bf16(pr4[0]) | ((uint32_t)f32_to_bf16(pr4[1]) << 16);
          const uint32_t p23 = (uint32_t)f32_to_bf16(pr4[2]) | ((uint32_t)f32_to_bf16(pr4[3]) << 16);
          const v4i16 pb = __builtin_bit_cast(v4i16, uint2{p01, p23});
          wave_sync();
          const T *vb = slot + (4 * G + col / 4) * VP + 4 * (col % 4);
#pragma unroll
          for (int mb = 0; mb < D / 16; ++mb) {
            const v4i16 vt = lds_read_tr16(vb + 16 * mb);
            oacc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pb, oacc[mb] * alpha, 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (col < GQ) sPr[wave][4 * G + i][col] = pr4[i];
          if (col < GQ && G == 0) sAl[wave][col] = alpha;
          wave_sync();
          // O[h][dims] += p[key][h] V[key][dims] for this lane's keys vr + KPI u
          float al[GQ];
#pragma unroll
          for (int h = 0; h < GQ; ++h) al[h] = sAl[wave][h];
#pragma unroll
          for (int h = 0; h < GQ; ++h)
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] *= al[h];
#pragma unroll
          for (int u = 0; u < VPB; ++u) {
            float v[EPL];
            unpack16<T>(vw[nb][u], v);
            const int key = vr + KPI * u;
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
              const float prh = sPr[wave][key][h];
#pragma unroll
              for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(prh, v[e], acc[h][e]);
            }
          }
        }
        wave_sync();  // the slot is read before the next block rewrites it
        }
      }
    };
    for (int b0 = split * DW + wave; b0 < n_blk; b0 += VW * NB) {
      FT kf[NB][KS];
      uint4 vw[NB][VPB];
      load_batch(b0, kf, vw);
      compute_batch(b0, kf, vw);
    }
    __syncthreads();  // sList is read before the next pass rewrites it
  }

  // the wave's totals: the sum over its lanes of each column, O over its key slots
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (lane < GQ) {  // lanes 0..GQ-1: column = head, G = 0
    sM[wave][lane] = m_run;
    sL[wave][lane] = l_run;
  }
  if constexpr (PV_MFMA) {
    if (col < GQ) {  // lane (head col, G) holds dims 16 mb + 4 G + i
#pragma unroll
      for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sAcc[wave][col][16 * mb + 4 * G + i] = oacc[mb][i];
    }
  } else {
#pragma unroll
  for (int o = LPK; o < 64; o <<= 1)
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], o, 64);
  }
  if (!PV_MFMA && lane < LPK) {
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sAcc[wave][h][e0 + e] = acc[h][e];
  }
  __syncthreads();
  for (int i = tid; i < GQ * D; i += NT) {
    const int h = i / D, dd = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < DW; ++w) M = fmaxf(M, sM[w][h]);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < DW; ++w) {
      const float wt = sM[w][h] == -INFINITY ? 0.f : exp2f(sM[w][h] - M);
      L += wt * sL[w][h];
      o += wt * sAcc[w][h][dd];
    }
    const int64_t row = (int64_t)q * a.h_q + kvh * GQ + h;
    if (ns == 1) {
      const float out = bad ? __builtin_nanf("") : o / L;
      static_cast<T *>(a.O)[row * D + dd] = Elem<T>::from_f32(out);
    } else {  // partials for attend_combine_kernel (NaN sum: an id outside the bank)
      so.o[(row * ns + split) * D + dd] = o;
      if (dd == 0) {
        so.m[row * ns + split] = M;
        so.l[row * ns + split] = bad ? __builtin_nanf("") : L;
      }
    }
  }
}

bool decode_ok(const AttendArgs &a) {
  const int g = a.h_q / a.h_kv;
  return a.T == 1 && (g == 1 || g == 2 || g == 4 || g == 8) && a.k <= MAX_K;
}

template <typename T, int D>
hipError_t launch_decode(const AttendArgs &a, int ns, const SplitOut &so, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)a.n_q * a.h_kv * ns)), block(64 * DW);
  switch (a.h_q / a.h_kv) {
    case 1: hipLaunchKernelGGL((attend_decode_kernel<T, D, 1>), grid, block, 0, s, a, ns, so); break;
    case 2: hipLaunchKernelGGL((attend_decode_kernel<T, D, 2>), grid, block, 0, s, a, ns, so); break;
    case 4: hipLaunchKernelGGL((attend_decode_kernel<T, D, 4>), grid, block, 0, s, a, ns, so); break;
    default: hipLaunchKernelGGL((attend_decode_kernel<T, D, 8>), grid, block, 0, s, a, ns, so); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ns == 1) return e;
  const int64_t rows = (int64_t)a.n_q * a.h_q;
  const int64_t n = rows * D;
  hipLaunchKernelGGL((attend_combine_kernel<T, D>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, rows, ns, so,
                     a.O);
  return hipGetLastError();
}

// Workgroups per (query, KV head) of the decode kernel: enough to give every
// compute unit one (a workgroup's gather is bound by its compute unit's
// memory throughput), each split keeping at least two blocks per wave of the
// estimated keys.  A function of the call's sizes only, so that the layer's
// call and the call on its selection split alike.
int decode_splits(const AttendArgs &a) {
  if (a.kv_host) return 1;
  const int64_t wgs = (int64_t)a.n_q * a.h_kv;
  const int64_t est_keys = std::min<int64_t>((int64_t)a.k * std::max(1, a.max_doc_chunks), a.n_chunks) + a.L_loc;
  const int64_t blocks = (est_keys + 15) / 16;
  int64_t ns = device_cu_count() / std::max<int64_t>(1, wgs);
  ns = std::min<int64_t>(ns, blocks / (2 * DW));
  return (int)std::max<int64_t>(1, std::min<int64_t>(ns, 4));
}

struct Plan {
  int wgw, n_rb, n_rbg, n_split;
};

// 32-key k-steps per gathered tile of the many-row kernel: bf16 128 keys,
// fp32 64 (more bytes in flight per round trip of the tile pipeline; fp32's
// 128-key tile would not fit in LDS)
template <typename T> constexpr int att_nk() { return sizeof(T) == 2 ? 4 : 2; }
// two waves per row block, each taking one half of every tile's keys (two
// waves per SIMD for latency hiding, merged through LDS at the end)
constexpr int ATT_KH = 2;

Plan plan(const AttendArgs &a) {
  Plan p;
  const int g = a.h_q / a.h_kv;
  const int R = a.T * g;
  p.n_rb = (R + 15) / 16;
  p.wgw = p.n_rb >= 4 ? 4 : 1;
  p.n_rbg = (p.n_rb + p.wgw - 1) / p.wgw;
  const int64_t base = (int64_t)a.n_q * a.h_kv * p.n_rbg;
  const int64_t est_keys = std::min<int64_t>((int64_t)a.k * std::max(1, a.max_doc_chunks), a.n_chunks) + a.L_loc;
  const int64_t tiles = (est_keys + KT0 - 1) / KT0;
  // keys/values in host memory: the host link bounds the gather, and a
  // workgroup per (query, KV head, row group) keeps enough rows in flight
  // while leaving the GPU to a concurrent router scan
  const int64_t waves = base * p.wgw;
  int64_t ns = a.kv_host ? 1 : ((int64_t)SPLIT_MUL * device_cu_count() + waves - 1) / waves;
  ns = std::min<int64_t>(ns, std::max<int64_t>(1, tiles / MIN_TILES));
  ns = std::max<int64_t>(1, std::min<int64_t>(ns, 64));
  p.n_split = (int)ns;
  return p;
}

template <typename T, int D, int WGW>
hipError_t launch_kernel(const AttendArgs &a, const Plan &p, const SplitOut &so, hipStream_t s) {
  const int64_t grid = (int64_t)a.n_q * a.h_kv * p.n_rbg * p.n_split;
  hipLaunchKernelGGL((attend_kernel<T, D, WGW, att_nk<T>(), ATT_KH>), dim3((unsigned)grid), dim3(64 * WGW * ATT_KH), 0, s, a,
                     p.n_split, p.n_rbg, so);
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

int attend_splits(const AttendArgs &a) { return decode_ok(a) ? decode_splits(a) : plan(a).n_split; }

size_t attend_ws_bytes(const AttendArgs &a) {
  const int ns = attend_splits(a);
  if (ns == 1) return 0;
  const size_t rows = (size_t)a.n_q * a.T * a.h_q;
  return rows * ns * (a.d + 2) * sizeof(float);
}

hipError_t launch_attend(const AttendArgs &a, void *ws, hipStream_t s) {
  const size_t rows = (size_t)a.n_q * a.T * a.h_q;
  const int ns = attend_splits(a);
  SplitOut so{nullptr, nullptr, nullptr};
  if (ns > 1) {
    float *base = static_cast<float *>(ws);
    so.o = base;
    so.m = base + rows * ns * a.d;
    so.l = so.m + rows * ns;
  }
  if (decode_ok(a)) {
    if (a.dtype == 0) return a.d == 64 ? launch_decode<float, 64>(a, ns, so, s) : launch_decode<float, 128>(a, ns, so, s);
    return a.d == 64 ? launch_decode<bf16_t, 64>(a, ns, so, s) : launch_decode<bf16_t, 128>(a, ns, so, s);
  }
  const Plan p = plan(a);
  if (a.dtype == 0) return a.d == 64 ? dispatch_wgw<float, 64>(a, p, so, s) : dispatch_wgw<float, 128>(a, p, so, s);
  return a.d == 64 ? dispatch_wgw<bf16_t, 64>(a, p, so, s) : dispatch_wgw<bf16_t, 128>(a, p, so, s);
}

}  // namespace msa
