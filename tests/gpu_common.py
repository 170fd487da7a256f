"""Helpers shared by the GPU parity tests (not a test module).

Inputs come from synth/ (seeded, identical for both sides); expected values
come only from oracle/.  Nothing produced by the HIP path is ever fed to the
oracle: step-isolated tests feed oracle-pooled banks and oracle-chosen
document sets *into* the HIP path instead.
"""
from __future__ import annotations

import math
import sys
from typing import Optional

import numpy as np
import torch

import oracle as O
from synth import rng, workloads as W
from long_context_memory_msa_amd import _lib as L, memory as M


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Upload fp32 values (exactly representable in ``dtype``) as a contiguous tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    return t.to(M.TORCH_DTYPE[dtype]).contiguous()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def host_inputs(w: W.Workload, layer: int = 0):
    qi = W.query_inputs(w, layer)
    uh = W.gold_uhat(w, qi["QR"]) if w.gold.size else None
    K = W.bank_raw(w, rng.ROLE_K, 0, w.n_tok, layer)
    V = W.bank_raw(w, rng.ROLE_V, 0, w.n_tok, layer)
    KR = W.bank_raw(w, rng.ROLE_KR, 0, w.n_tok, layer, uh)
    return qi, K, V, KR


def oracle_bank(w: W.Workload, K, V, KR):
    return O.pool(w.doc_lens, w.chunk, K, V, KR, w.dtype, w.rope_base)


def gpu_bank_pooled(w: W.Workload, K, V, KR, device, n_slabs: int = 1):
    """Pool host raw tensors on the GPU, in ``n_slabs`` contiguous document ranges."""
    bank = M.Bank(w.doc_lens, w.chunk, w.h_kv, w.d, w.h_r, w.d_r, w.dtype, device)
    rope = M.Rope(w.max_pos, w.d, w.rope_base, device)
    off = w.doc_tok_off
    cuts = np.linspace(0, w.n_docs, n_slabs + 1).astype(int)
    for a, b in zip(cuts[:-1], cuts[1:]):
        t0, t1 = int(off[a]), int(off[b])
        bank.pool(dev(K[t0:t1], w.dtype, device), dev(V[t0:t1], w.dtype, device), dev(KR[t0:t1], w.dtype, device),
                  int(a), int(b), rope)
    torch.cuda.synchronize()
    return bank, rope


def gpu_bank_from_oracle(w: W.Workload, ob: dict, device):
    """A device bank holding the oracle's stored (rounded) pooled values."""
    bank = M.Bank(w.doc_lens, w.chunk, w.h_kv, w.d, w.h_r, w.d_r, w.dtype, device)
    rope = M.Rope(w.max_pos, w.d, w.rope_base, device)
    bank.kbar.copy_(dev(ob["kbar"], w.dtype, device))
    bank.vbar.copy_(dev(ob["vbar"], w.dtype, device))
    bank.krbar.copy_(dev(ob["krbar"], w.dtype, device))
    bank.kr_inv_norm.copy_(torch.from_numpy(ob["kr_inv_norm"].astype(np.float32)))
    bank.chunk_doc.copy_(torch.from_numpy(ob["chunk_doc"].astype(np.int32)))
    torch.cuda.synchronize()
    return bank, rope


def bf16_spacing(x: np.ndarray) -> np.ndarray:
    """Distance between adjacent bfloat16 values at |x| (2^(e-8) for x = m 2^e)."""
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, e - 8)


def assert_attention_close(got: np.ndarray, want: np.ndarray, max_abs: float = 2e-2, mean_abs: float = 1e-3):
    err = np.abs(got - want)
    assert np.all(np.isfinite(got)), "non-finite attention output"
    assert err.max() <= max_abs, f"max abs error {err.max():.3g} > {max_abs}"
    assert err.mean() <= mean_abs, f"mean abs error {err.mean():.3g} > {mean_abs}"
    return err.max(), err.mean()


def topk_set_valid(gpu_idx: np.ndarray, s_oracle: np.ndarray, k: int, slack: float = 4e-3) -> None:
    """A top-k selection made on the GPU's own scores, against the oracle's
    scores: k distinct documents, each scoring at least the oracle's k-th best
    minus ``slack``, and every document that scores more than the k-th best
    plus ``slack`` (a clear winner) among them."""
    for q in range(gpu_idx.shape[0]):
        row = gpu_idx[q]
        assert len(set(row.tolist())) == k and np.all((row >= 0) & (row < s_oracle.shape[1])), (q, row)
        kth = np.sort(s_oracle[q])[::-1][k - 1]
        assert np.all(s_oracle[q, row] >= kth - slack), (q, row, kth)
        winners = np.flatnonzero(s_oracle[q] > kth + slack)
        assert set(winners.tolist()) <= set(row.tolist()), (q, winners, row)


def check_topk_property(s_doc: np.ndarray, idx: np.ndarray, val: np.ndarray, k: int) -> None:
    """idx is the first k of the (descending score, ascending index) order of
    the GPU's own s_doc, and val the scores of those documents (bit-exact)."""
    for q in range(s_doc.shape[0]):
        order = np.lexsort((np.arange(s_doc.shape[1]), -s_doc[q].astype(np.float64)))[:k]
        assert idx[q].tolist() == order.tolist(), q
        assert np.array_equal(val[q], s_doc[q, idx[q]])


def run_layer(bank, rope, w: W.Workload, QR, Q, K_loc, V_loc, device, events=None):
    """msa_layer_forward on the workload's first round; returns (O, idx, val, s_doc)."""
    n_q = w.n_q
    O_ = torch.empty((n_q, w.T, w.h_q, w.d), dtype=M.TORCH_DTYPE[w.dtype], device=device)
    idx = torch.empty((n_q, w.k), dtype=torch.int32, device=device)
    val = torch.empty((n_q, w.k), dtype=torch.float32, device=device)
    s_doc = torch.empty((n_q, w.n_docs), dtype=torch.float32, device=device)
    nb = L.msa_layer_workspace_bytes(bank.c, n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k)
    ws = M.workspace(nb, device)
    L.msa_layer_forward(bank.c, Q, K_loc, V_loc, QR, n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k, w.pos0,
                        L.default_scale(w.d), rope.c, O_, idx, val, s_doc, ws, nb, events)
    torch.cuda.synchronize()
    return O_, idx, val, s_doc


def query_views(w: W.Workload, qi: dict, device):
    """Device tensors for one round: QR over the router tokens, Q over the T query tokens."""
    QR = dev(qi["QR"][:, w.L_loc - w.T_route:w.L_loc], w.dtype, device)
    Q = dev(qi["Q"][:, w.L_loc - w.T:w.L_loc], w.dtype, device)
    Kl = dev(qi["K_loc"][:, :w.L_loc], w.dtype, device)
    Vl = dev(qi["V_loc"][:, :w.L_loc], w.dtype, device)
    return QR, Q, Kl, Vl
