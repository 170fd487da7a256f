"""Tiered bank (pooled keys/values in pinned host memory, read by the GPU over
the host link) and the two-stream decode pipeline, through the C ABI.

The tiered bank's pooled rows equal the HBM bank's; its routing (scores,
top-k) is the same kernels on the same values, so it must match value for
value; its attention gathers with a different split plan (one workgroup per
query and KV head), so its output is checked against the fp64 oracle on the
selected documents.  The pipeline reproduces msa_layer_forward on the same
bank value for value (same kernels, same plan).
"""
import numpy as np
import pytest
import torch

import oracle as O
from synth import workloads as W
from long_context_memory_msa_amd import _lib as L, memory as M
from long_context_memory_msa_amd.pipeline import DecodePipeline

from gpu_common import assert_attention_close, dev, gpu_bank_pooled, host, host_inputs, log, query_views, run_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _tiered_bank(w, K, V, KR, rope, device):
    bank = M.Bank(w.doc_lens, w.chunk, w.h_kv, w.d, w.h_r, w.d_r, w.dtype, device, kv_host=True)
    assert not bank.kbar.is_cuda and bank.kbar.is_pinned()
    bank.pool(dev(K, w.dtype, device), dev(V, w.dtype, device), dev(KR, w.dtype, device), 0, w.n_docs, rope)
    torch.cuda.synchronize()
    return bank


def test_device_pointer_rejects_unpinned():
    with pytest.raises(L.MsaError):
        L.msa_device_pointer(np.zeros(64, np.float32).ctypes.data)


def test_tiered_bank_equals_hbm_bank(device):
    w = W.make_workload("prefill-1m", bank_tokens=150_000)
    log(f"tiered layer: docs={w.n_docs} chunks={w.n_chunks}")
    qi, K, V, KR = host_inputs(w)
    ref, rope = gpu_bank_pooled(w, K, V, KR, device, 1)
    tb = _tiered_bank(w, K, V, KR, rope, device)
    # pooled rows written over the host link: identical to the HBM bank's, and to the oracle within the bf16 bar
    assert torch.equal(tb.kbar, ref.kbar.cpu()) and torch.equal(tb.vbar, ref.vbar.cpu())
    assert torch.equal(tb.krbar, ref.krbar) and torch.equal(tb.kr_inv_norm, ref.kr_inv_norm)
    ob = O.pool(w.doc_lens, w.chunk, K, V, KR, w.dtype, w.rope_base)
    kb = tb.kbar.float().numpy().astype(np.float64)
    assert np.all(np.abs(kb - ob["kbar"]) <= 2.0 ** -7 * np.abs(ob["kbar"]) + 1e-5 * np.abs(ob["kbar"]).max())
    QR, Q, Kl, Vl = query_views(w, qi, device)
    got = run_layer(tb, rope, w, QR, Q, Kl, Vl, device)
    want = run_layer(ref, rope, w, QR, Q, Kl, Vl, device)
    for x, y in zip(got[1:], want[1:]):          # idx, val, s_doc
        assert torch.equal(x, y)
    gi = got[1].cpu().numpy()
    o_ref = O.attend(qi["Q"][:, w.L_loc - w.T:w.L_loc], qi["K_loc"][:, :w.L_loc], qi["V_loc"][:, :w.L_loc],
                     ob["kbar"], ob["vbar"], ob["doc_chunk_off"], gi, w.pos0, base=w.rope_base)
    assert_attention_close(host(got[0]), o_ref)
    assert tb.bytes_resident() < ref.bytes_resident() / 2


@pytest.mark.parametrize("kv_host", [False, True])
def test_decode_pipeline_equals_layer_forward(device, kv_host):
    # four independent query batches (the seeded query inputs of four layers)
    # through the two-stream pipeline, two steps in flight at a time
    w = W.make_workload("decode-100m", bank_tokens=700_000)
    log(f"pipeline kv_host={kv_host}: docs={w.n_docs} chunks={w.n_chunks} n_q={w.n_q}")
    qi0, K, V, KR = host_inputs(w)
    ref, rope = gpu_bank_pooled(w, K, V, KR, device, 1)
    bank = _tiered_bank(w, K, V, KR, rope, device) if kv_host else ref
    batches = [query_views(w, W.query_inputs(w, layer), device) for layer in range(4)]
    # two slots: the second pair reuses the first pair's buffers (host-side wait)
    pipe = DecodePipeline(bank, rope, w.n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k, w.pos0, device=device, slots=2)
    for pair in ((0, 1), (2, 3)):
        slots = [pipe.step(*batches[i]) for i in pair]
        pipe.synchronize()
        for i, s in zip(pair, slots):
            O_, idx, val, s_doc = run_layer(bank, rope, w, *batches[i], device)
            assert torch.equal(pipe.idx[s], idx) and torch.equal(pipe.val[s], val)
            assert torch.equal(pipe.s_doc[s], s_doc)
            assert torch.equal(pipe.O[s], O_)


@pytest.mark.parametrize("route_streams,slots,cap", [(1, 3, 0), (2, 3, 1), (3, 4, 1), (2, 4, 2)])
def test_decode_pipeline_streams_and_slots(device, route_streams, slots, cap):
    # more steps in flight than slots (the host waits before reusing one), the
    # scans spread over 1-3 route streams with full or capped grids: the
    # steps whose slots were not reused equal the layer forward
    w = W.make_workload("decode-100m", bank_tokens=700_000)
    log(f"pipeline streams={route_streams} slots={slots} cap={cap}: chunks={w.n_chunks}")
    qi0, K, V, KR = host_inputs(w)
    bank, rope = gpu_bank_pooled(w, K, V, KR, device, 1)
    n_steps = slots + 2
    batches = [query_views(w, W.query_inputs(w, layer), device) for layer in range(n_steps)]
    pipe = DecodePipeline(bank, rope, w.n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k, w.pos0, device=device,
                          slots=slots, route_streams=route_streams, max_wg_per_cu=cap)
    got = [pipe.step(*b) for b in batches]
    pipe.synchronize()
    for i in range(n_steps - slots, n_steps):
        O_, idx, val, s_doc = run_layer(bank, rope, w, *batches[i], device)
        s = got[i]
        assert torch.equal(pipe.idx[s], idx) and torch.equal(pipe.val[s], val), i
        assert torch.equal(pipe.s_doc[s], s_doc) and torch.equal(pipe.O[s], O_), i
