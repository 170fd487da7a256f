"""Seeded synthetic workloads for the MSA routed-layer hot path.

The five workloads mirror the shapes the MSA pages discuss: a memory bank of
documents, each split into fixed-size chunks ("chunk-mean pooling", hotdry
blog, section on the learnable memory routing layer), router heads for the
cosine scan, GQA attention heads, a local causal context, and top-k.

Everything here is input construction (document lengths, which documents are
planted "gold", raw per-token K / V / K^R and query tensors).  None of the
method's arithmetic lives here; the oracle and the HIP path each implement it
on their own.

Recipe (values are the counter generator of ``synth.rng``):
* document lengths: integers uniform on [a, b] inclusive, drawn until the
  bank total is reached; the last document is truncated to hit the total;
  documents are contiguous in bank order;
* raw K, V, K^R per token and Q, K_loc, V_loc, Q^R per query token:
  approximately N(0,1), rounded once to the storage dtype;
* planted gold: for query q and router head h, u_qh = normalise(mean over the
  router tokens of Q^R[q,t,h]); every raw router key of a gold document of q
  becomes store(0.5 * x + (mix * sqrt(d_r)) * u_qh) -- a shift toward the mean
  query direction with mixing weight ``mix`` (0.5), sqrt(d_r) standing in for
  the expected norm of an N(0,1) key.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

from . import rng

QUERY_STRIDE = 1 << 20  # counter stride per query: values independent of context length


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str            # 'f32' or 'bf16' (storage); accumulation is fp32
    doc_lens: np.ndarray  # int64 [n_docs]
    chunk: int
    h_kv: int
    d: int
    h_r: int
    d_r: int
    h_q: int
    n_q: int
    T: int                # query tokens attended: the last T of the local context
    L_loc: int            # local causal context length (first round)
    T_route: int          # router query tokens: the last T_route of the local context
    k: int
    pos0: int             # global RoPE offset of local token 0 (= k)
    gold: np.ndarray      # int64 [n_q][n_gold] (may have n_gold = 0)
    seed: int
    n_layers: int = 1
    rounds: int = 1
    append: int = 0       # tokens appended per layer after each round
    rope_base: float = 10000.0
    mix: float = 0.5

    # ---- derived layout -------------------------------------------------
    @property
    def n_docs(self) -> int:
        return int(self.doc_lens.shape[0])

    @property
    def n_tok(self) -> int:
        return int(self.doc_lens.sum())

    @property
    def doc_tok_off(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.doc_lens)]).astype(np.int64)

    @property
    def doc_n_chunks(self) -> np.ndarray:
        return ((self.doc_lens + self.chunk - 1) // self.chunk).astype(np.int64)

    @property
    def doc_chunk_off(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.doc_n_chunks)]).astype(np.int64)

    @property
    def n_chunks(self) -> int:
        return int(self.doc_n_chunks.sum())

    @property
    def L_max(self) -> int:
        return self.L_loc + self.append * max(0, self.rounds - 1)

    @property
    def max_pos(self) -> int:
        return int(max(int(self.doc_lens.max()), self.pos0 + self.L_max))

    @property
    def gold_cg(self) -> np.float32:
        return np.float32(self.mix * math.sqrt(self.d_r))

    def gold_owner(self) -> np.ndarray:
        """int32 [n_docs]: the query a document is gold for, or -1."""
        own = np.full(self.n_docs, -1, dtype=np.int32)
        for q in range(self.gold.shape[0]):
            for doc in self.gold[q]:
                own[int(doc)] = q
        return own


# ---------------------------------------------------------------------------
def _doc_lengths(seed: int, total: int, lo: int, hi: int) -> np.ndarray:
    g = np.random.default_rng(np.random.SeedSequence([seed, 101]))
    lens = []
    acc = 0
    while acc < total:
        n = int(g.integers(lo, hi + 1))
        n = min(n, total - acc)
        lens.append(n)
        acc += n
    return np.asarray(lens, dtype=np.int64)


def _gold(seed: int, n_docs: int, n_q: int, n_gold: int) -> np.ndarray:
    if n_gold == 0:
        return np.zeros((n_q, 0), dtype=np.int64)
    g = np.random.default_rng(np.random.SeedSequence([seed, 202]))
    pick = g.choice(n_docs, size=n_q * n_gold, replace=False)  # distinct across queries
    return np.sort(pick.reshape(n_q, n_gold), axis=1).astype(np.int64)


# the five workloads by name; the number is each one's default seed
WORKLOADS = {"tiny-f32": 0, "prefill-16k": 1, "prefill-1m": 2, "decode-100m": 3, "interleave-10mx18": 4}


def make_workload(name: str, seed: Optional[int] = None, bank_tokens: Optional[int] = None,
                  n_layers: Optional[int] = None, n_q: Optional[int] = None) -> Workload:
    """Workload ``name``; ``bank_tokens`` / ``n_layers`` / ``n_q`` shrink it.

    tiny-f32: fp32 layer, 64 docs x 512 tokens, chunk 64, 2 router / 2 KV /
       4 q heads of dim 64, 16 query tokens, k=4, 4 gold docs.
    prefill-16k: 16K-token bank, 32 docs x 512, chunk 128, 8 router heads x
       128, 32 q / 8 KV heads x 128, bf16, 128 causal query tokens, k=8, 4 gold.
    prefill-1m: 1M-token bank, doc lengths U[256,4096], 256 query tokens, k=16,
       8 gold.
    decode-100m: 100M-token bank, doc lengths U[512,8192], 16 queries x 1
       decode token, k=16, 8 gold docs per query (distinct across queries).
    interleave-10mx18: 10M-token bank per layer x 18 routed layers,
       U[256,4096], prefill 512, 3 interleave rounds appending 64 tokens, k=8,
       no gold.
    """
    if name not in WORKLOADS:
        raise ValueError(f"unknown workload {name!r}; one of {sorted(WORKLOADS)}")
    s = WORKLOADS[name] if seed is None else seed
    if name == "tiny-f32":
        total = bank_tokens or 64 * 512
        lens = np.full(total // 512, 512, dtype=np.int64) if total % 512 == 0 else _doc_lengths(s, total, 512, 512)
        w = Workload(name, "f32", lens, 64, 2, 64, 2, 64, 4, n_q or 1, 16, 16, 16, 4, 4,
                     np.zeros((0, 0), np.int64), s)
        n_gold = 4
    elif name == "prefill-16k":
        total = bank_tokens or 32 * 512
        lens = np.full(total // 512, 512, dtype=np.int64) if total % 512 == 0 else _doc_lengths(s, total, 512, 512)
        w = Workload(name, "bf16", lens, 128, 8, 128, 8, 128, 32, n_q or 1, 128, 128, 128, 8, 8,
                     np.zeros((0, 0), np.int64), s)
        n_gold = 4
    elif name == "prefill-1m":
        lens = _doc_lengths(s, bank_tokens or 1_000_000, 256, 4096)
        w = Workload(name, "bf16", lens, 128, 8, 128, 8, 128, 32, n_q or 1, 256, 256, 256, 16, 16,
                     np.zeros((0, 0), np.int64), s)
        n_gold = 8
    elif name == "decode-100m":
        lens = _doc_lengths(s, bank_tokens or 100_000_000, 512, 8192)
        w = Workload(name, "bf16", lens, 128, 8, 128, 8, 128, 32, n_q or 16, 1, 1, 1, 16, 16,
                     np.zeros((0, 0), np.int64), s)
        n_gold = 8
    else:  # interleave-10mx18
        lens = _doc_lengths(s, bank_tokens or 10_000_000, 256, 4096)
        w = Workload(name, "bf16", lens, 128, 8, 128, 8, 128, 32, n_q or 1, 512, 512, 512,
                     8, 8, np.zeros((0, 0), np.int64), s, n_layers=n_layers or 18, rounds=3, append=64)
        n_gold = 0
    n_gold = min(n_gold, w.n_docs // max(1, w.n_q))
    w.gold = _gold(s, w.n_docs, w.n_q, n_gold)
    return w


# ---------------------------------------------------------------------------
# host generation of raw inputs
def query_tensor(w: Workload, role: int, heads: int, dim: int, layer: int = 0,
                 tokens: Optional[int] = None) -> np.ndarray:
    """[n_q][tokens][heads][dim] stored values (fp32 array) of a query-side role."""
    L = w.L_max if tokens is None else tokens
    key = rng.stream_key(w.seed, role, layer)
    out = np.empty((w.n_q, L, heads, dim), dtype=np.float32)
    for q in range(w.n_q):
        out[q] = rng.normal_stored(key, q * QUERY_STRIDE * heads * dim, L * heads * dim, w.dtype).reshape(L, heads, dim)
    return out


def query_inputs(w: Workload, layer: int = 0) -> dict:
    """Q, K_loc, V_loc and Q^R over the whole local context (L_max tokens)."""
    return {
        "Q": query_tensor(w, rng.ROLE_Q, w.h_q, w.d, layer),
        "K_loc": query_tensor(w, rng.ROLE_KLOC, w.h_kv, w.d, layer),
        "V_loc": query_tensor(w, rng.ROLE_VLOC, w.h_kv, w.d, layer),
        "QR": query_tensor(w, rng.ROLE_QR, w.h_r, w.d_r, layer),
    }


def gold_uhat(w: Workload, QR: np.ndarray) -> np.ndarray:
    """fp32 [n_q][h_r][d_r]: unit mean router-query direction per query and head."""
    toks = QR[:, w.L_loc - w.T_route:w.L_loc].astype(np.float64)
    m = toks.mean(axis=1)
    n = np.linalg.norm(m, axis=-1, keepdims=True)
    return (m / np.where(n > 0, n, 1.0)).astype(np.float32)


def bank_raw(w: Workload, role: int, tok0: int, tok1: int, layer: int = 0,
             uhat: Optional[np.ndarray] = None) -> np.ndarray:
    """Raw per-token tensor of ``role`` for bank tokens [tok0, tok1): [n][H][d].

    Router keys of gold documents get the planted shift (needs ``uhat``).
    """
    H, D = (w.h_r, w.d_r) if role == rng.ROLE_KR else (w.h_kv, w.d)
    key = rng.stream_key(w.seed, role, layer)
    x = rng.normal_stored(key, tok0 * H * D, (tok1 - tok0) * H * D, w.dtype).reshape(tok1 - tok0, H, D)
    if role == rng.ROLE_KR and w.gold.size:
        if uhat is None:
            raise ValueError("router keys of a bank with gold documents need uhat")
        off = w.doc_tok_off
        owner = w.gold_owner()
        for doc in np.nonzero(owner >= 0)[0]:
            a, b = max(int(off[doc]), tok0), min(int(off[doc + 1]), tok1)
            if a < b:
                x[a - tok0:b - tok0] = rng.plant_fast(x[a - tok0:b - tok0], uhat[owner[doc]], w.gold_cg, w.dtype)
    return x


def doc_tokens(w: Workload, role: int, doc: int, layer: int = 0, uhat=None) -> np.ndarray:
    off = w.doc_tok_off
    return bank_raw(w, role, int(off[doc]), int(off[doc + 1]), layer, uhat)


def scores_for_topk(seed: int, n_q: int, n_docs: int, tie_frac: float = 0.25) -> np.ndarray:
    """Synthetic fp32 document scores with planted exact ties (isolated top-k tests)."""
    key = rng.stream_key(seed, rng.ROLE_SCORES)
    s = rng.normal_f32(key, 0, n_q * n_docs).reshape(n_q, n_docs)
    # quantise a fraction of entries onto a coarse grid so that many values tie
    g = np.random.default_rng(np.random.SeedSequence([seed, 303]))
    m = g.random((n_q, n_docs)) < tie_frac
    s = np.where(m, np.round(s * 8.0) / 8.0, s).astype(np.float32)
    return s


# ---- router-projector inputs (hidden states and seeded projector weights) ----
def hidden_states(seed: int, role: int, n: int, hidden: int, layer: int = 0) -> np.ndarray:
    """bf16-stored N(0,1) hidden states [n][hidden] (memory tokens or queries)."""
    key = rng.stream_key(seed, role, layer)
    return rng.normal_stored(key, 0, n * hidden, "bf16").reshape(n, hidden)


def projector_weights(seed: int, role: int, hidden: int, out: int, layer: int = 0) -> np.ndarray:
    """bf16-stored projector W [out][hidden] with entries N(0, 1/hidden): the
    projected features of N(0,1) hidden states are about N(0,1)."""
    key = rng.stream_key(seed, role, layer)
    w = rng.normal_stored(key, 0, out * hidden, "f32").reshape(out, hidden) * np.float32(1.0 / np.sqrt(hidden))
    return rng.store_round(w.astype(np.float32), "bf16")
