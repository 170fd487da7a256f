"""msa_layer_forward_noalloc (the layer with its workspace in the library's
static device array) against msa_layer_forward with a caller-owned workspace:
identical outputs, call after call on the same array, the later calls smaller
than the first (the array keeps the previous call's contents)."""
import dataclasses

import numpy as np
import pytest
import torch

from synth import workloads as W
from long_context_memory_msa_amd import _lib as L, memory as M

from gpu_common import gpu_bank_pooled, host_inputs, log, query_views, run_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _noalloc(bank, rope, w, QR, Q, Kl, Vl, device, with_scores=True):
    O_ = torch.empty((w.n_q, w.T, w.h_q, w.d), dtype=M.TORCH_DTYPE[w.dtype], device=device)
    idx = torch.empty((w.n_q, w.k), dtype=torch.int32, device=device)
    val = torch.empty((w.n_q, w.k), dtype=torch.float32, device=device)
    s_doc = torch.empty((w.n_q, w.n_docs), dtype=torch.float32, device=device) if with_scores else None
    assert L.msa_layer_workspace_bytes(bank.c, w.n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k) <= L.STATIC_WORKSPACE_BYTES
    L.msa_layer_forward_noalloc(bank.c, Q, Kl, Vl, QR, w.n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k, w.pos0,
                                L.default_scale(w.d), rope.c, O_, idx, val, s_doc)
    torch.cuda.synchronize()
    return O_, idx, val, s_doc


def _case(w, device):
    qi, K, V, KR = host_inputs(w)
    bank, rope = gpu_bank_pooled(w, K, V, KR, device, 1)
    return (bank, rope, w) + tuple(query_views(w, qi, device))


def _same(got, want):
    for x, y in zip(got, want):
        if x is not None:
            assert torch.equal(x, y)


def test_noalloc_layer_equals_layer_forward_call_after_call(device):
    # layers of every scan and top-k form on the same array, largest workspace
    # first and each later one smaller: the many-row (atomic-key) scan of the
    # 16K-token prefill layer, the decode layer (single-writer scan,
    # single-pass top-k), a bank of 9,000 documents (top-k pass 1 completes
    # the scores, the attention makes the final selection), fewer queries on
    # a smaller bank; then the first again (its keys and records must not
    # depend on what the others left)
    g = np.random.default_rng(11)
    lens = g.integers(8, 41, size=9_000).astype(np.int64)
    sliced = dataclasses.replace(W.make_workload("decode-100m", bank_tokens=200_000), doc_lens=lens, chunk=64, h_kv=2,
                                 d=64, h_r=2, d_r=64, h_q=4, k=16, pos0=16, gold=np.zeros((16, 0), dtype=np.int64))
    rows = W.make_workload("prefill-16k")
    decode = W.make_workload("decode-100m", bank_tokens=700_000)
    small = dataclasses.replace(W.make_workload("decode-100m", bank_tokens=300_000), n_q=5,
                                gold=np.zeros((5, 0), np.int64))
    def ws_of(w):
        return L.msa_layer_workspace_bytes(_bank_c(w), w.n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k)

    # largest workspace first, each later call smaller, then the first one again
    order = sorted((rows, decode, sliced, small), key=ws_of, reverse=True)
    sizes = [ws_of(w) for w in order]
    assert all(b < a for a, b in zip(sizes, sizes[1:])), sizes
    for i, w in enumerate(order + [order[0]]):
        log(f"noalloc call {i}: {w.name} docs={w.n_docs} chunks={w.n_chunks} n_q={w.n_q} t_r={w.T_route} "
            f"ws={ws_of(w)}")
        bank, rope, w, QR, Q, Kl, Vl = _case(w, device)
        want = run_layer(bank, rope, w, QR, Q, Kl, Vl, device)
        got = _noalloc(bank, rope, w, QR, Q, Kl, Vl, device)
        _same(got, want)
        got2 = _noalloc(bank, rope, w, QR, Q, Kl, Vl, device, with_scores=False)   # no s_doc output
        _same(got2, want)


def _bank_c(w):
    lay = L.msa_bank_layout(w.doc_lens, w.chunk)
    return L.MsaBank(M.ABI_DTYPE[w.dtype], w.n_docs, w.chunk, w.h_kv, w.d, w.h_r, w.d_r, lay["max_doc_len"],
                     lay["max_doc_chunks"], 0, 0, 0, lay["n_chunks"], 16, 16, None, None, 16, 16, 16, 16, 16)
