"""Plain fp64 CPU oracle of the MSA routed-layer hot path.

TEST INFRASTRUCTURE.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of bench.py may import this module.  The product path
(the HIP library and its binding) never imports, links or calls it, and this
module imports nothing from the product path.

Every function is the plain definition, in float64, in the order the MSA pages
give it.  Sources (cited by page title and section, never by line):

* [LH] Lighthouse AI-research digest, "MSA: Memory Sparse Attention for
  Efficient End-to-End Memory Model Scaling to 100M Tokens".
* [HD] hotdry blog, "EverMind MSA router sparse attention architecture".
* [CS] gitcode/CSDN article on MSA ("four technical breakthroughs").
* [WC] wiselychen blog, "MSA: 4B model beats a 235B RAG system".

Readings taken where the pages are silent:
  R1 document score = max over the document's chunk scores;
  R2 RoPE is applied to K and Q only (not V, not the router vectors K^R/Q^R);
  R3 RoPE is applied per token at its in-document position, before pooling;
  R4 rotate-half pairing (i, i + d/2), theta_i = base**(-2i/d), base 10000;
  R5 local token s sits at global position pos0 + s with pos0 = k; the query
     tokens are the last T local tokens;
  R6 a partial last chunk is the mean of the tokens it holds;
  R7 cos(x, y) = 0 when either norm is 0;
  R8 top-k ties go to the lower document index; output sorted by descending
     score;
  R9 attention scale 1/sqrt(d), no bias on pooled keys; memory keys are visible
     to every query token, local keys causally; q-head h reads KV head
     h // (H_q / H_kv).
  R10 the router projectors are plain linear maps without bias (Q^R = x W_QR^T,
     K^R = h W_KR^T per token, before pooling); their outputs are stored in
     the bank dtype (rounded once) like every other stored tensor.
  R11 Memory Interleave: round r routes with every active token of the layer
     (T0 + append * r), then attends only the tokens new in that round (T0,
     then ``append``) over the selected documents plus the whole causal local
     context; local token s stays at global position pos0 + s in every round.

Parity is pinned for every function by tests/test_oracle_pins.py (interleave
by the hand-derived tests/golden/interleave_tiny.json and by its slices and
positions); none is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# storage rounding (the oracle's own; shares nothing with the generator or GPU)
def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bfloat16 value (ties to even), returned as fp64.

    bfloat16 keeps 8 significant bits: write x = m * 2**e with 0.5 <= |m| < 1,
    round m * 2**8 to an integer (ties to even) and scale back.  Exact for the
    normal range, which is all these inputs use.
    """
    x = np.asarray(x, dtype=F64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0), e - 8)


def round_store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round exact values to the bank storage dtype ('f32' or 'bf16')."""
    if dtype == "f32":
        return np.asarray(x, dtype=F64).astype(np.float32).astype(F64)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Router projection ([HD] core architecture of the learnable memory routing
# layer: the router projectors map hidden states to Q^R and, per memory token,
# to K^R; [HD] parameter advice: router width 2-4x the head dimension).
def project(X: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Y[..., o] = sum_i X[..., i] * W[o, i] in fp64 (W: one row per output
    feature), unrounded; R10."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    return X @ W.T


# RoPE ([LH] Component 2, document-wise and global RoPE; [HD] key engineering
# details, position encoding).  Formula not printed on the pages: reading R4.
def rope_theta(d: int, base: float = 10000.0) -> np.ndarray:
    """theta_i = base ** (-2 i / d), i < d/2."""
    i = np.arange(d // 2, dtype=F64)
    return np.power(F64(base), -2.0 * i / d)


def rope_cos_sin(pos, d: int, base: float = 10000.0) -> Tuple[np.ndarray, np.ndarray]:
    """cos and sin of pos * theta_i: shape pos.shape + (d/2,)."""
    a = np.asarray(pos, dtype=F64)[..., None] * rope_theta(d, base)
    return np.cos(a), np.sin(a)


def rope_apply(x: np.ndarray, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate-half RoPE of x[..., d] at positions ``pos`` (broadcast over x[..., 0]).

    (x_i, x_{i+d/2}) -> (x_i cos a_i - x_{i+d/2} sin a_i, x_i sin a_i + x_{i+d/2} cos a_i).
    """
    x = np.asarray(x, dtype=F64)
    d = x.shape[-1]
    c, s = rope_cos_sin(pos, d, base)
    lo, hi = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([lo * c - hi * s, lo * s + hi * c], axis=-1)


# ---------------------------------------------------------------------------
# bank layout and chunk-mean pooling ([HD] core architecture of the memory
# routing layer: split each document into fixed-size chunks and average the
# tokens of each chunk into K-bar, V-bar and K-bar^R; [LH] Component 1, steps
# 1-3; [LH] Component 2 for the per-document positions).
def bank_layout(doc_lens: Sequence[int], chunk: int) -> Dict[str, np.ndarray]:
    """Token and chunk offsets of a bank of contiguous documents."""
    L = np.asarray(doc_lens, dtype=np.int64)
    n_ch = (L + chunk - 1) // chunk
    tok_off = np.concatenate([[0], np.cumsum(L)]).astype(np.int64)
    ch_off = np.concatenate([[0], np.cumsum(n_ch)]).astype(np.int64)
    chunk_doc = np.repeat(np.arange(L.shape[0], dtype=np.int64), n_ch)
    return {"doc_tok_off": tok_off, "doc_chunk_off": ch_off, "chunk_doc": chunk_doc,
            "n_chunks": int(ch_off[-1])}


def pool(doc_lens: Sequence[int], chunk: int, K: np.ndarray, V: np.ndarray, KR: np.ndarray,
         dtype: str, base: float = 10000.0) -> Dict[str, np.ndarray]:
    """Chunk-mean pooling with document-wise RoPE.

    K, V: [n_tok][H_kv][d]; KR: [n_tok][H_r][d_r], tokens of the documents in
    bank order.  For document i and chunk j covering in-document tokens
    [j*C, min(L_i, (j+1)*C)):
        Kbar_ij  = mean_t R(t - start_i) K_t      (positions restart at 0 per document)
        Vbar_ij  = mean_t V_t
        KRbar_ij = mean_t KR_t                    (router keys carry no RoPE, R2)
    Returns exact means ("*_exact"), the stored (rounded) values, the inverse
    norms 1/||stored KRbar_ij,h|| (0 for a zero row, R7) and the layout.
    Layouts: kbar/vbar [H_kv][n_chunks][d], krbar [n_chunks][H_r][d_r].
    """
    lay = bank_layout(doc_lens, chunk)
    H_kv, d = K.shape[1], K.shape[2]
    H_r, d_r = KR.shape[1], KR.shape[2]
    N = lay["n_chunks"]
    kbar = np.zeros((H_kv, N, d))
    vbar = np.zeros((H_kv, N, d))
    krbar = np.zeros((N, H_r, d_r))
    c = 0
    for i, Li in enumerate(np.asarray(doc_lens, dtype=np.int64)):
        t0 = int(lay["doc_tok_off"][i])
        pos = np.arange(Li, dtype=F64)
        Krot = rope_apply(K[t0:t0 + Li].astype(F64), pos[:, None], base)  # [Li][H][d]
        for j0 in range(0, int(Li), chunk):
            j1 = min(int(Li), j0 + chunk)
            kbar[:, c, :] = Krot[j0:j1].mean(axis=0)
            vbar[:, c, :] = V[t0 + j0:t0 + j1].astype(F64).mean(axis=0)
            krbar[c] = KR[t0 + j0:t0 + j1].astype(F64).mean(axis=0)
            c += 1
    assert c == N
    krs = round_store(krbar, dtype)
    nrm = np.linalg.norm(krs, axis=-1)
    inv = np.where(nrm > 0, 1.0 / np.where(nrm > 0, nrm, 1.0), 0.0)
    return {"kbar_exact": kbar, "vbar_exact": vbar, "krbar_exact": krbar,
            "kbar": round_store(kbar, dtype), "vbar": round_store(vbar, dtype), "krbar": krs,
            "kr_inv_norm": inv, **lay}


# ---------------------------------------------------------------------------
# routing ([LH] Component 1, key formula for S_ij: mean over heads of the
# cosine, then max over query tokens; [HD] core architecture: cosine
# similarity, mean-pooled over heads, then max over tokens)
def cosine(x: np.ndarray, y: np.ndarray) -> np.ndarray:
    """cos(x, y) over the last axis (broadcast); 0 where either norm is 0 (R7)."""
    x = np.asarray(x, dtype=F64)
    y = np.asarray(y, dtype=F64)
    nx = np.linalg.norm(x, axis=-1)
    ny = np.linalg.norm(y, axis=-1)
    den = nx * ny
    dot = np.sum(x * y, axis=-1)
    return np.where(den > 0, dot / np.where(den > 0, den, 1.0), 0.0)


def _unit(x: np.ndarray) -> np.ndarray:
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)


def chunk_scores(QR: np.ndarray, krbar: np.ndarray, block: int = 2048) -> np.ndarray:
    """S[q, c] = max_t  mean_h  cos(QR[q, t, h], krbar[c, h]).

    QR: [n_q][T][H_r][d_r]; krbar: [n_chunks][H_r][d_r] (stored values).
    Chunks are visited in blocks only to bound memory.
    """
    QR = np.asarray(QR, dtype=F64)
    kr = np.asarray(krbar, dtype=F64)
    qn = _unit(QR)                                  # [n_q][T][H][d]
    n_q, T, H, _ = QR.shape
    N = kr.shape[0]
    S = np.empty((n_q, N))
    for a in range(0, N, block):
        b = min(N, a + block)
        kn = _unit(kr[a:b])                         # [n][H][d]
        # cos[q, t, n, h] for every query token, chunk and head
        cos = np.einsum("qthd,nhd->qtnh", qn, kn)
        S[:, a:b] = cos.mean(axis=3).max(axis=1)    # mean over heads, then max over tokens
    return S


def doc_scores(S: np.ndarray, doc_chunk_off: np.ndarray) -> np.ndarray:
    """Per-document score: max over the document's chunks (reading R1)."""
    off = np.asarray(doc_chunk_off, dtype=np.int64)
    n_docs = off.shape[0] - 1
    out = np.empty((S.shape[0], n_docs))
    for i in range(n_docs):
        out[:, i] = S[:, off[i]:off[i + 1]].max(axis=1)
    return out


def topk(s_doc: np.ndarray, k: int) -> Dict[str, np.ndarray]:
    """The k highest-scoring documents per query ([LH] Component 1, Top-k
    document selection; [HD] Top-k selection mechanism), sorted by descending
    score, ties to the lower index (R8).  ``gap`` = s_(k) - s_(k+1) (inf when
    k = n_docs) tells whether the selected set is unique up to 4e-3.
    """
    s = np.asarray(s_doc, dtype=F64)
    n_q, n = s.shape
    idx = np.empty((n_q, k), dtype=np.int64)
    val = np.empty((n_q, k))
    gap = np.empty(n_q)
    for q in range(n_q):
        order = sorted(range(n), key=lambda i: (-s[q, i], i))
        idx[q] = order[:k]
        val[q] = s[q, order[:k]]
        gap[q] = s[q, order[k - 1]] - s[q, order[k]] if k < n else math.inf
    return {"idx": idx, "val": val, "gap": gap}


# ---------------------------------------------------------------------------
# sparse attention ([LH] Component 1, last step: concatenate the selected
# documents' compressed KV with the query's local KV and attend; [HD] core
# architecture, Top-k paragraph; [LH] Component 2 and [HD] position encoding:
# the active context uses global RoPE starting at position k; [CS] Document-
# wise RoPE paragraph: background -> query -> generation causal order)
def selected_chunks(doc_chunk_off: np.ndarray, idx_row: Sequence[int]) -> np.ndarray:
    """Chunk ids of the selected documents, documents in rank order."""
    off = np.asarray(doc_chunk_off, dtype=np.int64)
    return np.concatenate([np.arange(off[i], off[i + 1]) for i in idx_row]).astype(np.int64)


def attend(Q: np.ndarray, K_loc: np.ndarray, V_loc: np.ndarray, kbar: np.ndarray, vbar: np.ndarray,
           doc_chunk_off: np.ndarray, idx: np.ndarray, pos0: int, scale: Optional[float] = None,
           base: float = 10000.0) -> np.ndarray:
    """O[q, t, h] for the T query tokens (the last T of the L_loc local tokens).

    Q: [n_q][T][H_q][d]; K_loc, V_loc: [n_q][L_loc][H_kv][d] (before RoPE);
    kbar, vbar: [H_kv][n_chunks][d] (stored; document-wise RoPE already in
    kbar); idx: [n_q][k] selected documents.
    Keys of query q, KV head g: [kbar rows of the selected documents' chunks ;
    R(pos0 + s) K_loc_s for s < L_loc]; values: [vbar rows ; V_loc_s].
    Query token t is local token s_t = L_loc - T + t at position pos0 + s_t; it
    sees every memory key and the local keys s <= s_t.  logits = scale *
    <R(pos0 + s_t) Q, key>, softmax with the max subtracted, O = sum p * value.
    """
    Q = np.asarray(Q, dtype=F64)
    K_loc = np.asarray(K_loc, dtype=F64)
    V_loc = np.asarray(V_loc, dtype=F64)
    n_q, T, H_q, d = Q.shape
    L_loc, H_kv = K_loc.shape[1], K_loc.shape[2]
    g = H_q // H_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    s_t = L_loc - T + np.arange(T)
    O = np.empty((n_q, T, H_q, d))
    for q in range(n_q):
        ch = selected_chunks(doc_chunk_off, idx[q])
        n_mem = ch.shape[0]
        k_loc = rope_apply(K_loc[q], (pos0 + np.arange(L_loc))[:, None], base)   # [L_loc][H_kv][d]
        q_rot = rope_apply(Q[q], (pos0 + s_t)[:, None], base)                    # [T][H_q][d]
        visible = np.concatenate([np.ones((T, n_mem), dtype=bool),
                                  np.arange(L_loc)[None, :] <= s_t[:, None]], axis=1)
        for h in range(H_q):
            kv = h // g
            keys = np.concatenate([np.asarray(kbar[kv][ch], dtype=F64), k_loc[:, kv]], axis=0)
            vals = np.concatenate([np.asarray(vbar[kv][ch], dtype=F64), V_loc[q, :, kv]], axis=0)
            logits = scale * (q_rot[:, h] @ keys.T)                               # [T][n_mem + L_loc]
            logits = np.where(visible, logits, -np.inf)
            m = logits.max(axis=1, keepdims=True)
            p = np.exp(logits - m)
            O[q, :, h] = (p @ vals) / p.sum(axis=1, keepdims=True)
    return O


# ---------------------------------------------------------------------------
# one routed layer and the interleave loop
def layer_forward(QR: np.ndarray, Q: np.ndarray, K_loc: np.ndarray, V_loc: np.ndarray,
                  bank: Dict[str, np.ndarray], k: int, pos0: int, scale: Optional[float] = None,
                  base: float = 10000.0) -> Dict[str, np.ndarray]:
    """Route (scan + document max), top-k, sparse attention ([LH] overall
    architecture diagram; [WC] mechanism 3, online routing then sparse
    generation).  ``bank`` is the output of ``pool``.
    """
    S = chunk_scores(QR, bank["krbar"])
    s_doc = doc_scores(S, bank["doc_chunk_off"])
    sel = topk(s_doc, k)
    O = attend(Q, K_loc, V_loc, bank["kbar"], bank["vbar"], bank["doc_chunk_off"], sel["idx"], pos0,
               scale, base)
    return {"s_chunk": S, "s_doc": s_doc, **sel, "O": O}


def interleave(layers: Sequence[Dict[str, np.ndarray]], banks: Sequence[Dict[str, np.ndarray]],
               T0: int, append: int, rounds: int, k: int, pos0: int, scale: Optional[float] = None,
               base: float = 10000.0) -> list:
    """Memory Interleave: rounds of route -> top-k -> attend, re-routing after
    each round of generated tokens ([HD] sparse strategy: routing alternates
    with generation and is redone each round; [HD] parameters: 2-3 rounds;
    [WC] mechanism 4).

    ``layers[l]`` holds that layer's Q, K_loc, V_loc, QR over the whole
    context (T0 + append * (rounds - 1) tokens): the tokens appended after a
    round are the next ``append`` rows.  Round r routes with every active
    token (T0 + append * r), then attends the tokens new in that round (T0 in
    round 0, ``append`` afterwards) over the selected documents plus the full
    causal local context (reading R11).  Returns results[r][l] =
    layer_forward output.
    """
    out = []
    for r in range(rounds):
        L_act = T0 + append * r
        T_new = T0 if r == 0 else append
        res_r = []
        for li, inp in enumerate(layers):
            res = layer_forward(inp["QR"][:, :L_act], inp["Q"][:, L_act - T_new:L_act], inp["K_loc"][:, :L_act],
                                inp["V_loc"][:, :L_act], banks[li], k, pos0, scale, base)
            res_r.append(res)
        out.append(res_r)
    return out
