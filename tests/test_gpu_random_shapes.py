"""The routed layer over seeded random shapes, against the fp64 oracle.

Each case draws (from its own seed) a bank of random document lengths, the
storage type, chunk size, KV / query / router head shapes, k, the number of
queries, the attended and router token counts and the local context, so
that the scan kernels (single-token, one row block, few-row streaming,
tiled many-row), the top-k forms (single pass, sliced pass 1 with the final
selection in the attention, two passes for larger k) and the attention
kernels (single-token decode, many rows with and without key splits) meet
in combinations the fixed-shape tests do not list.  The checks are those of
the layer tests: router scores within 2e-3 of the oracle's, the selection
the exact top-k of the GPU's own scores and valid against the oracle's,
attention on the GPU's own selection within 2e-2 max / 1e-3 mean, and the
layer halves bit-equal to the whole layer.

Method: Lighthouse digest, Component 1 (key formula, top-k, concatenated
memory and local KV) and Component 2 (document-wise RoPE); hotdry blog, core
architecture of the learnable memory routing layer.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from synth import workloads as W
from long_context_memory_msa_amd import _lib as L, memory as M

from gpu_common import (assert_attention_close, check_topk_property, gpu_bank_pooled, host, host_inputs, log,
                        oracle_bank, query_views, run_layer, topk_set_valid)

N_CASES = 48
MAX_TOKENS = 60_000   # the oracle pools every token in fp64


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def random_case(i: int) -> W.Workload:
    """Case i: family i % 6 fixes what the case must exercise, its seed draws the rest.

    0: single-token queries over a bank of several 512-document slices, small
       k (sliced pass 1, final selection in the attention, decode attention);
    1: many attended rows with key splits over a mid-size bank;
    2: k above the in-attention selection's limit (the whole top-k first);
    3: bf16 router of 128-dim heads with 32-64 router rows per query (one
       query: the few-row streaming scan; several: the tiled many-row scan);
    4: fp32 storage;
    5: banks of one to seven documents (every document possibly selected).
    """
    r = np.random.default_rng(7_000 + i)
    fam = i % 6
    dtype = "f32" if fam == 4 else ("bf16" if fam in (0, 3) else str(r.choice(["bf16", "bf16", "f32"])))
    chunk = int(r.choice([64, 128]))
    d = int(r.choice([64, 128]))
    h_kv = int(r.choice([1, 2, 4, 8]))
    h_q = h_kv * int(r.choice([1, 2, 4, 8]))
    if fam == 3:
        d_r, h_r = 128, int(r.choice([1, 2, 4, 8]))
    else:
        d_r = int(r.choice([64, 128, 256] if dtype == "bf16" else [64, 128]))
        h_r = int(r.choice([h for h in (1, 2, 4, 8, 16) if h * d_r <= 1024]))
    n_docs = {0: int(r.integers(513, 1100)), 1: int(r.integers(20, 300)), 2: int(r.integers(40, 700)),
              3: int(r.integers(10, 600)), 4: int(r.integers(2, 600)), 5: int(r.integers(1, 8))}[fam]
    max_len = max(1, min(3_000, MAX_TOKENS // n_docs))
    lens = r.integers(1, max_len + 1, size=n_docs).astype(np.int64)
    if fam == 2:
        k = int(r.integers(33, min(n_docs, 256) + 1))
    elif fam == 5:
        k = int(r.integers(1, n_docs + 1))
    else:
        k = int(r.integers(1, min(n_docs, 32) + 1))
    n_q = int(r.choice([1, 2, 5, 16, 20]))
    if fam == 3 and (i // 6) % 2 == 0:
        n_q = 1  # 32-64 rows of one query: the few-row streaming scan
    T = 1 if fam == 0 else (int(r.choice([16, 33, 64])) if fam == 1 else int(r.choice([1, 4, 16, 33])))
    L_loc = T + int(r.integers(0, 80 if fam == 1 else 40))
    if fam == 0:
        T_route = 1
    elif fam == 3:
        T_route = int(r.choice([32, 48, 64]))
        L_loc = max(L_loc, T_route)
    else:
        T_route = min(int(r.choice([1, T, 16, 32])), L_loc)
    base = W.make_workload("tiny-f32" if dtype == "f32" else "prefill-16k")
    return dataclasses.replace(base, dtype=dtype, doc_lens=lens, chunk=chunk, h_kv=h_kv, d=d, h_r=h_r, d_r=d_r,
                               h_q=h_q, n_q=n_q, T=T, L_loc=L_loc, T_route=T_route, k=k, pos0=k,
                               gold=np.zeros((n_q, 0), np.int64), seed=7_000 + i)


def test_random_cases_are_varied():
    """The draw covers every scan, top-k and attention form named above."""
    ws = [random_case(i) for i in range(N_CASES)]
    assert any(w.dtype == "f32" for w in ws) and any(w.dtype == "bf16" for w in ws)
    assert any(w.n_docs > 512 and w.k <= 32 for w in ws)          # sliced pass 1, selection in the attention
    assert any(w.k > 32 for w in ws)                               # the whole top-k before the attention
    assert any(w.T == 1 for w in ws) and any(w.T > 1 for w in ws)  # decode and many-row attention
    assert any(w.T_route == 1 for w in ws)
    assert any(w.dtype == "bf16" and w.d_r == 128 and w.T_route >= 32 and w.T_route % 16 == 0
               and w.n_q * w.T_route <= 64 for w in ws)                       # few-row streaming scan
    assert any(w.dtype == "bf16" and w.d_r == 128 and w.T_route >= 32 and w.T_route % 16 == 0
               and w.n_q * w.T_route > 64 for w in ws)                        # tiled many-row scan
    assert all(w.n_tok <= MAX_TOKENS for w in ws)


def _halves(bank, rope, w, QR, Q, Kl, Vl, device):
    """msa_layer_route then msa_layer_select_attend on the same workspace."""
    O_ = torch.empty((w.n_q, w.T, w.h_q, w.d), dtype=M.TORCH_DTYPE[w.dtype], device=device)
    idx = torch.empty((w.n_q, w.k), dtype=torch.int32, device=device)
    val = torch.empty((w.n_q, w.k), dtype=torch.float32, device=device)
    s_doc = torch.empty((w.n_q, w.n_docs), dtype=torch.float32, device=device)
    nb = L.msa_layer_workspace_bytes(bank.c, w.n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k)
    ws = M.workspace(nb, device)
    L.msa_layer_route(bank.c, QR, w.n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k, s_doc, ws, nb)
    L.msa_layer_select_attend(bank.c, Q, Kl, Vl, w.n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k, w.pos0,
                              L.default_scale(w.d), rope.c, O_, idx, val, s_doc, ws, nb)
    torch.cuda.synchronize()
    return O_, idx, val, s_doc


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(N_CASES))
def test_layer_random_shape(device, case):
    w = random_case(case)
    log(f"random case {case}: {w.dtype} docs={w.n_docs} chunks={w.n_chunks} chunk={w.chunk} h_kv={w.h_kv} "
        f"h_q={w.h_q} d={w.d} h_r={w.h_r} d_r={w.d_r} k={w.k} n_q={w.n_q} T={w.T} L_loc={w.L_loc} "
        f"t_r={w.T_route}")
    qi, K, V, KR = host_inputs(w)
    ob = oracle_bank(w, K, V, KR)
    sl = slice(w.L_loc - w.T, w.L_loc)
    want = O.layer_forward(qi["QR"][:, w.L_loc - w.T_route:w.L_loc], qi["Q"][:, sl], qi["K_loc"][:, :w.L_loc],
                           qi["V_loc"][:, :w.L_loc], ob, w.k, w.pos0, base=w.rope_base)
    bank, rope = gpu_bank_pooled(w, K, V, KR, device, 1)
    QR, Q, Kl, Vl = query_views(w, qi, device)
    out, idx, val, s_doc = run_layer(bank, rope, w, QR, Q, Kl, Vl, device)
    assert np.abs(host(s_doc) - want["s_doc"]).max() <= 2e-3
    gi = idx.cpu().numpy()
    check_topk_property(s_doc.cpu().numpy(), gi, val.cpu().numpy(), w.k)
    for q in range(w.n_q):
        if want["gap"][q] > 4e-3:
            assert set(gi[q].tolist()) == set(want["idx"][q].tolist()), q
    topk_set_valid(gi, want["s_doc"], w.k)
    o_ref = O.attend(qi["Q"][:, sl], qi["K_loc"][:, :w.L_loc], qi["V_loc"][:, :w.L_loc], ob["kbar"], ob["vbar"],
                     ob["doc_chunk_off"], gi, w.pos0, base=w.rope_base)
    assert_attention_close(host(out), o_ref)
    for x, y in zip(_halves(bank, rope, w, QR, Q, Kl, Vl, device), (out, idx, val, s_doc)):
        assert torch.equal(x, y)
