"""GPU parity of every hot-path step against the fp64 oracle, at sizes the
oracle finishes in seconds (several tiles, ragged tails, all five workload
shapes), through the C ABI.

Tolerances (written here, applied elementwise):
  pooled fp32      per (chunk, head) row: max |gpu - exact| <= 1e-5 * max |exact row|
  pooled bf16      |gpu - exact| <= one bf16 spacing at the exact value + 1e-5 * max |exact row|
  inverse norms    |gpu - 1/||gpu row||| <= 2e-6 relative (property); vs oracle 1e-5 (fp32) / 2e-4 (bf16)
  router scores    |gpu - oracle| <= 2e-3 (s_chunk and s_doc)
  top-k            bit-exact on identical scores; on scores the GPU computed itself the set is
                   identical where the oracle's k-th vs (k+1)-th gap exceeds 4e-3, else every pick
                   is within 4e-3 of the oracle's k-th score
  attention        max |gpu - oracle| <= 2e-2 and mean <= 1e-3
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from synth import rng, workloads as W
from long_context_memory_msa_amd import _lib as L, memory as M

from gpu_common import (assert_attention_close, bf16_spacing, check_topk_property, dev, gpu_bank_from_oracle,
                        gpu_bank_pooled, host, host_inputs, log, oracle_bank, query_views, run_layer, topk_set_valid)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _wl(name, bank_tokens=None, **kw):
    w = W.make_workload(name, bank_tokens=bank_tokens)
    return dataclasses.replace(w, **kw) if kw else w


# small versions of the five workloads: (workload, bank tokens) -- ragged where the law allows
SMALL = {
    "tiny": ("tiny-f32", None),
    "16k": ("prefill-16k", None),
    "1m": ("prefill-1m", 150_000),
    "decode": ("decode-100m", 700_000),
    "interleave": ("interleave-10mx18", 120_000),
}


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d,base,max_pos", [(128, 10000.0, 8192), (64, 10000.0, 600), (128, 500000.0, 4096)])
def test_rope_table(device, d, base, max_pos):
    log(f"rope d={d} base={base} max_pos={max_pos}")
    r = M.Rope(max_pos, d, base, device)
    torch.cuda.synchronize()
    c, s = O.rope_cos_sin(np.arange(max_pos), d, base)
    assert np.abs(host(r.cos) - c).max() <= 6e-8
    assert np.abs(host(r.sin) - s).max() <= 6e-8


def _check_pool(w, ob, bank):
    kb, vb, krb = host(bank.kbar), host(bank.vbar), host(bank.krbar)
    for got, name in ((kb, "kbar"), (vb, "vbar"), (krb, "krbar")):
        exact = ob[name + "_exact"]
        if w.dtype == "f32":
            err = np.abs(got - exact).max(axis=-1)
            ref = np.abs(exact).max(axis=-1)
            assert np.all(err <= 1e-5 * ref + 1e-30), f"{name}: worst row rel err {np.max(err / ref):.3g}"
        else:
            # one bf16 spacing (the final rounding of a perturbed fp32 mean may land on the
            # neighbour) plus the fp32 accumulation slack of the row, as in the fp32 bound
            slack = 1e-5 * np.abs(exact).max(axis=-1, keepdims=True)
            err = np.abs(got - exact)
            bad = err > bf16_spacing(exact) + slack
            assert not bad.any(), f"{name}: {bad.sum()} elements beyond one bf16 spacing (worst {err[bad].max():.3g})"
    inv = host(bank.kr_inv_norm)
    own = 1.0 / np.linalg.norm(krb, axis=-1)
    assert np.all(np.abs(inv - own) <= 2e-6 * own)
    tol = 1e-5 if w.dtype == "f32" else 2e-4
    assert np.all(np.abs(inv - ob["kr_inv_norm"]) <= tol * ob["kr_inv_norm"])
    assert np.array_equal(bank.chunk_doc.cpu().numpy(), ob["chunk_doc"])


@pytest.mark.parametrize("name,n_slabs", [("tiny", 1), ("16k", 2), ("1m", 3), ("interleave", 1)])
def test_pool(device, name, n_slabs):
    wname, bt = SMALL[name]
    w = _wl(wname, bt)
    log(f"pool {name} docs={w.n_docs} chunks={w.n_chunks} slabs={n_slabs}")
    qi, K, V, KR = host_inputs(w)
    ob = oracle_bank(w, K, V, KR)
    bank, _ = gpu_bank_pooled(w, K, V, KR, device, n_slabs)
    _check_pool(w, ob, bank)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pool_edge_lengths(device, dtype):
    # lengths around the chunk size, single-token documents, one long document
    base = _wl("tiny-f32") if dtype == "f32" else _wl("prefill-16k")
    C = base.chunk
    lens = np.array([1, C - 1, C, C + 1, 3 * C + 5, 2, C // 2, 7 * C], dtype=np.int64)
    w = dataclasses.replace(base, doc_lens=lens, gold=np.zeros((1, 0), np.int64))
    log(f"pool edge {dtype} lens={lens.tolist()}")
    qi, K, V, KR = host_inputs(w)
    ob = oracle_bank(w, K, V, KR)
    bank, _ = gpu_bank_pooled(w, K, V, KR, device, 2)
    _check_pool(w, ob, bank)


# bf16 head shapes: rows of whole 1 KB pieces (h_kv d and h_r d_r multiples of
# 512: one wave per piece, 3 to 16 pieces) and rows that are not (the head-row
# kernel), on ragged documents
@pytest.mark.parametrize("h_kv,d,h_r,d_r", [(8, 64, 8, 64), (4, 128, 4, 256), (8, 128, 2, 256), (16, 128, 8, 128),
                                             (8, 64, 4, 128), (4, 128, 8, 64), (2, 64, 2, 64), (4, 64, 2, 128)])
def test_pool_head_shapes(device, h_kv, d, h_r, d_r):
    base = _wl("prefill-16k")
    C = base.chunk
    lens = np.array([1, C - 1, C, C + 1, 2 * C + 5, 5, C // 2, 5 * C - 3], dtype=np.int64)
    w = dataclasses.replace(base, doc_lens=lens, h_kv=h_kv, d=d, h_r=h_r, d_r=d_r, h_q=h_kv,
                            gold=np.zeros((1, 0), np.int64))
    log(f"pool shapes h_kv={h_kv} d={d} h_r={h_r} d_r={d_r}")
    qi, K, V, KR = host_inputs(w)
    ob = oracle_bank(w, K, V, KR)
    bank, _ = gpu_bank_pooled(w, K, V, KR, device, 2)
    _check_pool(w, ob, bank)


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,t_r,n_q", [("tiny", 16, 1), ("16k", 128, 1), ("16k", 1, 1), ("16k", 5, 3),
                                          ("16k", 40, 2), ("16k", 16, 3), ("16k", 1, 37), ("16k", 48, 3),
                                          ("16k", 64, 5), ("1m", 256, 1),
                                          # few many-row blocks (17-64 rows): the streaming scan
                                          ("16k", 32, 1), ("16k", 32, 2), ("16k", 48, 1), ("16k", 64, 1),
                                          ("1m", 64, 1),
                                          ("decode", 1, 16)])
def test_route_isolated(device, name, t_r, n_q):
    wname, bt = SMALL[name]
    w = _wl(wname, bt)
    if n_q != w.n_q:
        w = dataclasses.replace(w, n_q=n_q, gold=np.zeros((n_q, 0), np.int64))
    log(f"route {name} t_r={t_r} n_q={n_q} chunks={w.n_chunks}")
    qi, K, V, KR = host_inputs(w)
    ob = oracle_bank(w, K, V, KR)
    QRh = qi["QR"][:, :t_r]
    S = O.chunk_scores(QRh, ob["krbar"])
    sd = O.doc_scores(S, ob["doc_chunk_off"])
    bank, _ = gpu_bank_from_oracle(w, ob, device)
    s_doc = torch.empty((n_q, w.n_docs), dtype=torch.float32, device=device)
    s_chunk = torch.empty((n_q, w.n_chunks), dtype=torch.float32, device=device)
    nb = L.msa_route_workspace_bytes(bank.c, n_q, t_r)
    ws = M.workspace(nb, device)
    L.msa_route_score(bank.c, dev(QRh, w.dtype, device), n_q, t_r, s_doc, s_chunk, ws, nb)
    torch.cuda.synchronize()
    assert np.abs(host(s_chunk) - S).max() <= 2e-3
    assert np.abs(host(s_doc) - sd).max() <= 2e-3
    # without the optional chunk output
    s_doc2 = torch.empty_like(s_doc)
    L.msa_route_score(bank.c, dev(QRh, w.dtype, device), n_q, t_r, s_doc2, None, ws, nb)
    torch.cuda.synchronize()
    assert torch.equal(s_doc, s_doc2)
    # a persistent grid capped at 1 or 2 workgroups per compute unit: the
    # same tiles, other waves -- identical scores
    for cap in (1, 2):
        s_doc3, s_chunk3 = torch.empty_like(s_doc), torch.empty_like(s_chunk)
        L.msa_route_score(bank.c, dev(QRh, w.dtype, device), n_q, t_r, s_doc3, s_chunk3, ws, nb, max_wg_per_cu=cap)
        torch.cuda.synchronize()
        assert torch.equal(s_doc, s_doc3) and torch.equal(s_chunk, s_chunk3), cap


# every router head shape the ABI admits (h_r in 1..16, d_r 64 / 128 / 256 --
# 256 for bf16 --, fp32 and bf16), few rows (decode scan) and many rows per
# query (tiled scan), on a small
# ragged bank of the prefill workload's document law (several 128-chunk tiles)
@pytest.mark.parametrize("dtype,h_r,d_r,t_r,n_q", [
    ("bf16", 1, 128, 48, 2), ("bf16", 2, 128, 32, 3), ("bf16", 4, 128, 64, 1), ("bf16", 2, 128, 1, 16),
    ("bf16", 4, 64, 1, 5), ("bf16", 16, 64, 32, 2), ("bf16", 16, 64, 1, 16), ("f32", 16, 64, 16, 1),
    ("f32", 4, 128, 5, 2), ("f32", 8, 128, 48, 1),
    ("bf16", 4, 256, 1, 16), ("bf16", 2, 256, 48, 2), ("bf16", 1, 256, 16, 3),
    ("bf16", 8, 128, 32, 2), ("bf16", 1, 128, 64, 1), ("bf16", 2, 128, 48, 1)])
def test_route_head_shapes(device, dtype, h_r, d_r, t_r, n_q):
    w = _wl("prefill-1m", 60_000)
    # one small attention head: K/V do not enter the routing
    w = dataclasses.replace(w, dtype=dtype, h_r=h_r, d_r=d_r, h_kv=1, d=64, h_q=1, n_q=n_q,
                            gold=np.zeros((n_q, 0), np.int64))
    log(f"route shapes {dtype} h_r={h_r} d_r={d_r} t_r={t_r} n_q={n_q} chunks={w.n_chunks}")
    qi = W.query_inputs(w)
    KR = W.bank_raw(w, rng.ROLE_KR, 0, w.n_tok)
    zeros = np.zeros((w.n_tok, w.h_kv, w.d), np.float32)
    ob = O.pool(w.doc_lens, w.chunk, zeros, zeros, KR, w.dtype, w.rope_base)
    QRh = qi["QR"][:, :t_r]
    S = O.chunk_scores(QRh, ob["krbar"])
    sd = O.doc_scores(S, ob["doc_chunk_off"])
    bank, _ = gpu_bank_from_oracle(w, ob, device)
    s_doc = torch.empty((n_q, w.n_docs), dtype=torch.float32, device=device)
    s_chunk = torch.empty((n_q, w.n_chunks), dtype=torch.float32, device=device)
    nb = L.msa_route_workspace_bytes(bank.c, n_q, t_r)
    ws = M.workspace(nb, device)
    L.msa_route_score(bank.c, dev(QRh, w.dtype, device), n_q, t_r, s_doc, s_chunk, ws, nb)
    torch.cuda.synchronize()
    assert np.abs(host(s_chunk) - S).max() <= 2e-3
    assert np.abs(host(s_doc) - sd).max() <= 2e-3


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n_q,n_docs,k", [(1, 7, 1), (1, 7, 7), (3, 2048, 16), (2, 5000, 256), (16, 23048, 16),
                                          (2, 8192, 32), (1, 6000, 8), (3, 2049, 32), (2, 40, 32),
                                          (4, 4099, 64), (1, 300, 256), (1, 24576, 256),
                                          # above 24K documents per query: the two-pass path
                                          (2, 24577, 16), (3, 60000, 64), (1, 100000, 256)])
def test_topk_isolated(device, n_q, n_docs, k):
    log(f"topk n_q={n_q} n_docs={n_docs} k={k}")
    s = W.scores_for_topk(1000 + n_docs + k, n_q, n_docs)
    want = O.topk(s.astype(np.float64), k)
    sd = torch.from_numpy(s).to(device)
    idx = torch.empty((n_q, k), dtype=torch.int32, device=device)
    val = torch.empty((n_q, k), dtype=torch.float32, device=device)
    nb = L.msa_topk_workspace_bytes(n_q, n_docs, k)
    ws = M.workspace(nb, device)
    L.msa_topk(sd, n_q, n_docs, k, idx, val, ws, nb)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), want["idx"])
    assert np.array_equal(val.cpu().numpy().astype(np.float64), want["val"])


# ---------------------------------------------------------------------------
def _attend_case(w, device, idx_h, T=None, L_loc=None, idx_dev=None):
    """The oracle's attention over idx_h and the GPU's over idx_dev (default idx_h)."""
    T = T or w.T
    L_loc = L_loc or w.L_loc
    idx_dev = idx_h if idx_dev is None else idx_dev
    qi, K, V, KR = host_inputs(w)
    ob = oracle_bank(w, K, V, KR)
    Qh = qi["Q"][:, L_loc - T:L_loc]
    Klh, Vlh = qi["K_loc"][:, :L_loc], qi["V_loc"][:, :L_loc]
    want = O.attend(Qh, Klh, Vlh, ob["kbar"], ob["vbar"], ob["doc_chunk_off"], idx_h, w.pos0, base=w.rope_base)
    bank, rope = gpu_bank_from_oracle(w, ob, device)
    k = idx_h.shape[1]
    out = torch.empty((w.n_q, T, w.h_q, w.d), dtype=M.TORCH_DTYPE[w.dtype], device=device)
    nb = L.msa_attend_workspace_bytes(bank.c, w.n_q, T, L_loc, w.h_q, k)
    ws = M.workspace(nb, device)
    L.msa_sparse_attend(bank.c, dev(Qh, w.dtype, device), dev(Klh, w.dtype, device), dev(Vlh, w.dtype, device),
                        w.n_q, T, L_loc, w.h_q, torch.from_numpy(idx_dev.astype(np.int32)).to(device), k, w.pos0,
                        L.default_scale(w.d), rope.c, out, ws, nb)
    torch.cuda.synchronize()
    return host(out), want


@pytest.mark.parametrize("name", ["tiny", "16k", "1m", "decode"])
def test_attend_isolated(device, name):
    wname, bt = SMALL[name]
    w = _wl(wname, bt)
    g = np.random.default_rng(7)
    idx_h = np.stack([g.choice(w.n_docs, size=w.k, replace=False) for _ in range(w.n_q)])
    log(f"attend {name} n_q={w.n_q} T={w.T} L_loc={w.L_loc} k={w.k}")
    got, want = _attend_case(w, device, idx_h)
    e = assert_attention_close(got, want)
    log(f"  max {e[0]:.3g} mean {e[1]:.3g}")


def test_attend_all_documents_is_dense(device):
    # k = n_docs: attention over the whole compressed memory plus the local context
    w = _wl("tiny-f32")
    idx_h = np.random.default_rng(3).permutation(w.n_docs)[None, :]
    w = dataclasses.replace(w, k=w.n_docs, pos0=w.n_docs)
    got, want = _attend_case(w, device, idx_h)
    assert_attention_close(got, want)


@pytest.mark.parametrize("name,T,L_loc", [("prefill-16k", 1, 1), ("prefill-16k", 1, 37), ("prefill-16k", 3, 70),
                                           ("prefill-16k", 50, 50), ("prefill-16k", 64, 640),
                                           ("prefill-16k", 3, 640), ("tiny-f32", 40, 90), ("tiny-f32", 3, 130)])
def test_attend_shapes(device, name, T, L_loc):
    # decode and partial prefill over long local contexts (causal tails, several
    # key tiles; fp32: four-row-block and one-row-block workgroups; 3 tokens over
    # 640 local keys: ten key splits, merged eight at a time then two)
    w = _wl(name)
    w = dataclasses.replace(w, T=T, L_loc=L_loc, T_route=min(L_loc, 128), rounds=1, append=0)
    idx_h = np.random.default_rng(T + L_loc).choice(w.n_docs, size=(1, w.k), replace=False)
    got, want = _attend_case(w, device, idx_h, T, L_loc)
    assert_attention_close(got, want)


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "16k", "1m", "decode"])
def test_layer_end_to_end(device, name):
    wname, bt = SMALL[name]
    w = _wl(wname, bt)
    log(f"layer {name} docs={w.n_docs} chunks={w.n_chunks} n_q={w.n_q} T={w.T}")
    qi, K, V, KR = host_inputs(w)
    ob = oracle_bank(w, K, V, KR)
    want = O.layer_forward(qi["QR"][:, w.L_loc - w.T_route:w.L_loc], qi["Q"][:, w.L_loc - w.T:w.L_loc],
                           qi["K_loc"][:, :w.L_loc], qi["V_loc"][:, :w.L_loc], ob, w.k, w.pos0, base=w.rope_base)
    bank, rope = gpu_bank_pooled(w, K, V, KR, device, 2)
    QR, Q, Kl, Vl = query_views(w, qi, device)
    out, idx, val, s_doc = run_layer(bank, rope, w, QR, Q, Kl, Vl, device)
    sd = host(s_doc)
    assert np.abs(sd - want["s_doc"]).max() <= 2e-3
    gi = idx.cpu().numpy()
    # the selection is exactly the top-k of the GPU's own document scores (values included)
    check_topk_property(s_doc.cpu().numpy(), gi, val.cpu().numpy(), w.k)
    for q in range(w.n_q):
        if want["gap"][q] > 4e-3:
            assert set(gi[q].tolist()) == set(want["idx"][q].tolist())
    topk_set_valid(gi, want["s_doc"], w.k)
    for q in range(w.n_q):
        if w.gold.size and set(w.gold[q].tolist()) <= set(want["idx"][q].tolist()):
            assert set(w.gold[q].tolist()) <= set(gi[q].tolist()), "planted gold not recovered"
    # attention against the oracle's attention over the GPU's own selection (every query)
    o_ref = O.attend(qi["Q"][:, w.L_loc - w.T:w.L_loc], qi["K_loc"][:, :w.L_loc], qi["V_loc"][:, :w.L_loc],
                     ob["kbar"], ob["vbar"], ob["doc_chunk_off"], gi, w.pos0, base=w.rope_base)
    e = assert_attention_close(host(out), o_ref)
    log(f"  attention on the layer's own selection: max {e[0]:.3g} mean {e[1]:.3g}")


def test_bank_append_equals_one_pass_encoding(device):
    # incremental update: half the documents encoded into a bank with spare
    # capacity, routed (checked against the oracle on that half), then the
    # rest appended and pooled in place -- the result equals the bank encoded
    # in one pass, value for value, and so does the layer over it
    wname, bt = SMALL["1m"]
    w = _wl(wname, bt)
    qi, K, V, KR = host_inputs(w)
    full, rope = gpu_bank_pooled(w, K, V, KR, device, 2)
    half = w.n_docs // 2
    t1 = int(w.doc_tok_off[half])
    log(f"append: {half} + {w.n_docs - half} docs, {w.n_chunks} chunks")
    bank = M.Bank(w.doc_lens[:half], w.chunk, w.h_kv, w.d, w.h_r, w.d_r, w.dtype, device,
                  cap_docs=w.n_docs + 3, cap_chunks=w.n_chunks + 50)
    bank.pool(dev(K[:t1], w.dtype, device), dev(V[:t1], w.dtype, device), dev(KR[:t1], w.dtype, device), 0, half,
              rope)
    wh = dataclasses.replace(w, doc_lens=w.doc_lens[:half], gold=np.zeros((w.n_q, 0), np.int64))
    QR, Q, Kl, Vl = query_views(w, qi, device)
    _, _, _, s_half = run_layer(bank, rope, wh, QR, Q, Kl, Vl, device)
    obh = O.pool(wh.doc_lens, w.chunk, K[:t1], V[:t1], KR[:t1], w.dtype, w.rope_base)
    S = O.chunk_scores(qi["QR"][:, w.L_loc - w.T_route:w.L_loc], obh["krbar"])
    assert np.abs(host(s_half) - O.doc_scores(S, obh["doc_chunk_off"])).max() <= 2e-3
    a, b = bank.append(w.doc_lens[half:])
    assert (a, b) == (half, w.n_docs) and bank.n_chunks == w.n_chunks
    bank.pool(dev(K[t1:], w.dtype, device), dev(V[t1:], w.dtype, device), dev(KR[t1:], w.dtype, device), a, b, rope)
    torch.cuda.synchronize()
    n = w.n_chunks
    assert torch.equal(bank.kbar[:, :n], full.kbar) and torch.equal(bank.vbar[:, :n], full.vbar)
    assert torch.equal(bank.krbar[:n], full.krbar) and torch.equal(bank.kr_inv_norm[:n], full.kr_inv_norm)
    assert torch.equal(bank.chunk_doc[:n], full.chunk_doc)
    assert torch.equal(bank.doc_chunk_off[:w.n_docs + 1], full.doc_chunk_off)
    got = run_layer(bank, rope, w, QR, Q, Kl, Vl, device)
    ref = run_layer(full, rope, w, QR, Q, Kl, Vl, device)
    for x, y in zip(got, ref):
        assert torch.equal(x, y)
    # re-pooling an existing range in place leaves it unchanged
    t0, t2 = int(w.doc_tok_off[2]), int(w.doc_tok_off[5])
    bank.pool(dev(K[t0:t2], w.dtype, device), dev(V[t0:t2], w.dtype, device), dev(KR[t0:t2], w.dtype, device), 2, 5,
              rope)
    torch.cuda.synchronize()
    assert torch.equal(bank.kbar[:, :n], full.kbar) and torch.equal(bank.krbar[:n], full.krbar)


def test_layer_equals_composition_and_is_deterministic(device):
    w = _wl("decode-100m", 300_000)
    qi, K, V, KR = host_inputs(w)
    bank, rope = gpu_bank_pooled(w, K, V, KR, device, 1)
    QR, Q, Kl, Vl = query_views(w, qi, device)
    o1, i1, v1, s1 = run_layer(bank, rope, w, QR, Q, Kl, Vl, device)
    o2, i2, v2, s2 = run_layer(bank, rope, w, QR, Q, Kl, Vl, device)
    assert torch.equal(o1, o2) and torch.equal(i1, i2) and torch.equal(v1, v2) and torch.equal(s1, s2)
    # the same three steps through the individual entry points
    s_doc = torch.empty_like(s1)
    nb0 = L.msa_route_workspace_bytes(bank.c, w.n_q, w.T_route)
    ws0 = M.workspace(nb0, device)
    L.msa_route_score(bank.c, QR, w.n_q, w.T_route, s_doc, None, ws0, nb0)
    idx = torch.empty_like(i1)
    val = torch.empty_like(v1)
    nb = L.msa_topk_workspace_bytes(w.n_q, w.n_docs, w.k)
    ws = M.workspace(nb, device)
    L.msa_topk(s_doc, w.n_q, w.n_docs, w.k, idx, val, ws, nb)
    out = torch.empty_like(o1)
    nb2 = L.msa_attend_workspace_bytes(bank.c, w.n_q, w.T, w.L_loc, w.h_q, w.k)
    ws2 = M.workspace(nb2, device)
    L.msa_sparse_attend(bank.c, Q, Kl, Vl, w.n_q, w.T, w.L_loc, w.h_q, idx, w.k, w.pos0, L.default_scale(w.d),
                        rope.c, out, ws2, nb2)
    torch.cuda.synchronize()
    assert torch.equal(s_doc, s1) and torch.equal(idx, i1) and torch.equal(val, v1) and torch.equal(out, o1)


def _layer_halves(bank, rope, w, QR, Q, Kl, Vl, device):
    """msa_layer_route on one stream, msa_layer_select_attend on another after an event."""
    n_q = w.n_q
    O_ = torch.empty((n_q, w.T, w.h_q, w.d), dtype=M.TORCH_DTYPE[w.dtype], device=device)
    idx = torch.empty((n_q, w.k), dtype=torch.int32, device=device)
    val = torch.empty((n_q, w.k), dtype=torch.float32, device=device)
    s_doc = torch.empty((n_q, w.n_docs), dtype=torch.float32, device=device)
    nb = L.msa_layer_workspace_bytes(bank.c, n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k)
    ws = M.workspace(nb, device)
    rs, ts = torch.cuda.Stream(device=device), torch.cuda.Stream(device=device)
    rs.wait_stream(torch.cuda.current_stream())
    L.msa_layer_route(bank.c, QR, n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k, s_doc, ws, nb, rs)
    ev = torch.cuda.Event()
    ev.record(rs)
    ts.wait_event(ev)
    L.msa_layer_select_attend(bank.c, Q, Kl, Vl, n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k, w.pos0,
                              L.default_scale(w.d), rope.c, O_, idx, val, s_doc, ws, nb, ts)
    torch.cuda.synchronize()
    return O_, idx, val, s_doc


# the halves against the whole layer: single-writer scan with single-pass top-k
# (decode small), many-row tiled scan (16k, 128 router rows), atomic keys
# (16k, 5 router rows), and the fp32 decode scan (tiny)
@pytest.mark.parametrize("name,t_r", [("decode", 1), ("16k", 128), ("16k", 5), ("tiny", 16)])
def test_layer_halves_equal_layer_forward(device, name, t_r):
    wname, bt = SMALL[name]
    w = _wl(wname, bt, T_route=t_r)
    log(f"layer halves {name} t_r={t_r} docs={w.n_docs}")
    qi, K, V, KR = host_inputs(w)
    bank, rope = gpu_bank_pooled(w, K, V, KR, device, 1)
    QR, Q, Kl, Vl = query_views(w, qi, device)
    want = run_layer(bank, rope, w, QR, Q, Kl, Vl, device)
    got = _layer_halves(bank, rope, w, QR, Q, Kl, Vl, device)
    for x, y in zip(got, want):
        assert torch.equal(x, y)


@pytest.mark.parametrize("k", [16, 32])
def test_layer_sliced_topk_selected_in_attention(device, k):
    # more documents than one top-k workgroup holds (8,192), small k: the layer
    # runs top-k pass 1 only (completing the document scores from the scan's
    # records itself) and every attention workgroup selects its query's
    # documents from the candidates; it must equal the separate route / top-k
    # / attend calls bit for bit, and the oracle
    g = np.random.default_rng(11)
    lens = g.integers(8, 41, size=9_000).astype(np.int64)  # one chunk per document
    w = _wl("decode-100m", 200_000, doc_lens=lens, chunk=64, h_kv=2, d=64, h_r=2, d_r=64, h_q=4, n_q=4, k=k, pos0=k,
            gold=np.zeros((4, 0), dtype=np.int64))
    assert w.n_docs > 8192 and w.n_chunks == w.n_docs
    _check_sliced_layer(w, device)


@pytest.mark.parametrize("n_q,t_r,long_chunks", [(20, 1, 40), (3, 4, 40), (20, 1, 130)])
def test_layer_sliced_multi_unit_documents(device, n_q, t_r, long_chunks):
    # the same sliced layer with documents of 1-4 chunks and, every 500th, one
    # of 40 chunks (two or three 32-chunk units: the resolve's first round of
    # record loads) or 130 chunks (five or six units: its later rounds)
    # crossing 32-chunk units; 20 single-token queries (a second, partial
    # block of 16) and 3 queries of 4 router tokens (a row block each)
    g = np.random.default_rng(12 + n_q + long_chunks)
    lens = g.integers(1, 65, size=8_400).astype(np.int64)
    lens[::500] = long_chunks * 16 - 3
    w = _wl("decode-100m", 200_000, doc_lens=lens, chunk=16, h_kv=2, d=64, h_r=2, d_r=64, h_q=4, n_q=n_q, k=16,
            pos0=16, T_route=t_r, L_loc=t_r, gold=np.zeros((n_q, 0), dtype=np.int64))
    assert w.n_docs > 8192 and w.n_chunks > 2 * w.n_docs
    _check_sliced_layer(w, device)


@pytest.mark.parametrize("t_r", [1, 4, 32])
def test_layer_few_slices_selected_in_attention(device, t_r):
    # 2,000 documents (four 512-document slices of the top-k pass) and k = 8:
    # the layer runs top-k pass 1 alone and the attention workgroups make the
    # final selection, after the single-writer scan (one router token), the
    # atomic-key scan (4 tokens) and the many-row scan (32 tokens)
    g = np.random.default_rng(30 + t_r)
    lens = g.integers(8, 41, size=2_000).astype(np.int64)
    n_q = 3
    w = _wl("decode-100m", 200_000, doc_lens=lens, chunk=64, h_kv=2, d=64, h_r=2, d_r=128 if t_r == 32 else 64,
            h_q=4, n_q=n_q, k=8, pos0=8, T_route=t_r, L_loc=t_r, gold=np.zeros((n_q, 0), dtype=np.int64))
    assert 1536 < w.n_docs <= 2048
    _check_sliced_layer(w, device)


def _check_sliced_layer(w, device):
    log(f"sliced layer k={w.k}: docs={w.n_docs} chunks={w.n_chunks} n_q={w.n_q} t_r={w.T_route}")
    qi, K, V, KR = host_inputs(w)
    ob = oracle_bank(w, K, V, KR)
    bank, rope = gpu_bank_pooled(w, K, V, KR, device, 1)
    QR, Q, Kl, Vl = query_views(w, qi, device)
    o1, i1, v1, s1 = run_layer(bank, rope, w, QR, Q, Kl, Vl, device)
    s_doc = torch.empty_like(s1)
    nb0 = L.msa_route_workspace_bytes(bank.c, w.n_q, w.T_route)
    L.msa_route_score(bank.c, QR, w.n_q, w.T_route, s_doc, None, M.workspace(nb0, device), nb0)
    idx, val = torch.empty_like(i1), torch.empty_like(v1)
    nb = L.msa_topk_workspace_bytes(w.n_q, w.n_docs, w.k)
    L.msa_topk(s_doc, w.n_q, w.n_docs, w.k, idx, val, M.workspace(nb, device), nb)
    out = torch.empty_like(o1)
    nb2 = L.msa_attend_workspace_bytes(bank.c, w.n_q, w.T, w.L_loc, w.h_q, w.k)
    L.msa_sparse_attend(bank.c, Q, Kl, Vl, w.n_q, w.T, w.L_loc, w.h_q, idx, w.k, w.pos0, L.default_scale(w.d),
                        rope.c, out, M.workspace(nb2, device), nb2)
    torch.cuda.synchronize()
    assert torch.equal(s_doc, s1) and torch.equal(idx, i1) and torch.equal(val, v1)
    # the layer's attention (its own selection, the workgroup shape for a GPU to
    # itself) and the standalone call's (the shape that runs beside other
    # streams) sum the same terms in another order: equal to a bf16 rounding
    assert torch.allclose(out.float(), o1.float(), rtol=2.0 ** -7, atol=1e-6)
    for x, y in zip(_layer_halves(bank, rope, w, QR, Q, Kl, Vl, device), (o1, i1, v1, s1)):
        assert torch.equal(x, y)
    want = O.layer_forward(qi["QR"][:, w.L_loc - w.T_route:w.L_loc], qi["Q"][:, w.L_loc - w.T:w.L_loc],
                           qi["K_loc"][:, :w.L_loc], qi["V_loc"][:, :w.L_loc], ob, w.k, w.pos0, base=w.rope_base)
    assert np.abs(host(s1) - want["s_doc"]).max() <= 2e-3
    gi = i1.cpu().numpy()
    check_topk_property(s1.cpu().numpy(), gi, v1.cpu().numpy(), w.k)
    for q in range(w.n_q):
        if want["gap"][q] > 4e-3:
            assert set(gi[q].tolist()) == set(want["idx"][q].tolist())
    topk_set_valid(gi, want["s_doc"], w.k)
    o_ref = O.attend(qi["Q"][:, w.L_loc - w.T:w.L_loc], qi["K_loc"][:, :w.L_loc], qi["V_loc"][:, :w.L_loc],
                     ob["kbar"], ob["vbar"], ob["doc_chunk_off"], gi, w.pos0, base=w.rope_base)
    assert_attention_close(host(o1), o_ref)


# degenerate banks through the whole layer against the oracle: a single
# one-token document, a bank smaller than one 16-chunk tile with every
# document selected, documents ending exactly on tile edges, and one long
# document spanning many tiles among short ones; decode (one router token)
# and many-row (32 router tokens) scans
@pytest.mark.parametrize("lens,k,t_r", [
    ([1], 1, 1), ([1], 1, 32),
    ([3, 200, 129, 1, 64], 5, 1), ([3, 200, 129, 1, 64], 5, 32),
    ([16 * 128] * 3 + [128] * 5, 4, 1),
    ([40, 100 * 128 + 7, 300, 2, 4000], 3, 1), ([40, 100 * 128 + 7, 300, 2, 4000], 3, 32)])
def test_layer_degenerate_banks(device, lens, k, t_r):
    lens = np.asarray(lens, dtype=np.int64)
    n_q = 2
    w = _wl("prefill-16k", None, doc_lens=lens, k=k, pos0=k, n_q=n_q, T=8, L_loc=max(32, t_r), T_route=t_r,
            gold=np.zeros((n_q, 0), np.int64))
    log(f"degenerate bank lens={lens.tolist()} k={k} t_r={t_r} chunks={w.n_chunks}")
    qi, K, V, KR = host_inputs(w)
    ob = oracle_bank(w, K, V, KR)
    want = O.layer_forward(qi["QR"][:, w.L_loc - w.T_route:w.L_loc], qi["Q"][:, w.L_loc - w.T:w.L_loc],
                           qi["K_loc"][:, :w.L_loc], qi["V_loc"][:, :w.L_loc], ob, w.k, w.pos0, base=w.rope_base)
    bank, rope = gpu_bank_pooled(w, K, V, KR, device, 1)
    QR, Q, Kl, Vl = query_views(w, qi, device)
    out, idx, val, s_doc = run_layer(bank, rope, w, QR, Q, Kl, Vl, device)
    assert np.abs(host(s_doc) - want["s_doc"]).max() <= 2e-3
    gi = idx.cpu().numpy()
    check_topk_property(s_doc.cpu().numpy(), gi, val.cpu().numpy(), w.k)
    topk_set_valid(gi, want["s_doc"], w.k)
    o_ref = O.attend(qi["Q"][:, w.L_loc - w.T:w.L_loc], qi["K_loc"][:, :w.L_loc], qi["V_loc"][:, :w.L_loc],
                     ob["kbar"], ob["vbar"], ob["doc_chunk_off"], gi, w.pos0, base=w.rope_base)
    assert_attention_close(host(out), o_ref)


# the decode scan's 32-chunk units (pairs of tiles, the document open at the
# end of the first tile carried into the second): documents of exactly one
# tile or one pair, documents ending one chunk before or after a tile or pair
# edge, one-chunk documents, a document crossing from one pair into the next,
# odd tile counts (a last pair of one tile, full or partial, whose last
# documents start inside it) and a last tile of one chunk; one
# and two row blocks of single-token queries (t_r = 1) and one query per row
# block (t_r = 16)
@pytest.mark.parametrize("chunks", [
    [16] * 7, [32] * 3 + [1], [15, 17, 1, 31, 33, 16, 2], [1] * 47, [5, 100, 3, 1], [16, 32, 16], [33],
    [17, 15], [31, 1, 32, 30, 2, 1], [16] * 6 + [8, 8], [16] * 6 + [3, 10, 3], [40, 8, 8]])
@pytest.mark.parametrize("t_r,n_q", [(1, 16), (1, 20), (16, 2)])
def test_route_pair_units(device, chunks, t_r, n_q):
    base = _wl("prefill-16k")
    lens = np.asarray(chunks, dtype=np.int64) * base.chunk
    lens[-1] -= 5  # a partial last chunk
    w = dataclasses.replace(base, doc_lens=lens, n_q=n_q, gold=np.zeros((n_q, 0), np.int64))
    log(f"route pair units chunks={chunks} t_r={t_r} n_q={n_q}")
    qi, K, V, KR = host_inputs(w)
    ob = oracle_bank(w, K, V, KR)
    QRh = qi["QR"][:, :t_r]
    S = O.chunk_scores(QRh, ob["krbar"])
    sd = O.doc_scores(S, ob["doc_chunk_off"])
    bank, _ = gpu_bank_from_oracle(w, ob, device)
    s_doc = torch.full((n_q, w.n_docs), float("nan"), dtype=torch.float32, device=device)
    s_chunk = torch.empty((n_q, w.n_chunks), dtype=torch.float32, device=device)
    nb = L.msa_route_workspace_bytes(bank.c, n_q, t_r)
    ws = M.workspace(nb, device)
    L.msa_route_score(bank.c, dev(QRh, w.dtype, device), n_q, t_r, s_doc, s_chunk, ws, nb)
    torch.cuda.synchronize()
    assert np.abs(host(s_chunk) - S).max() <= 2e-3
    assert np.abs(host(s_doc) - sd).max() <= 2e-3
    # and through the pipeline's capped grid
    s_doc2 = torch.full_like(s_doc, float("nan"))
    L.msa_route_score(bank.c, dev(QRh, w.dtype, device), n_q, t_r, s_doc2, None, ws, nb, max_wg_per_cu=1)
    torch.cuda.synchronize()
    assert torch.equal(s_doc, s_doc2)


def test_scan_read_probe_runs(device):
    # the bandwidth probe reads the bank in the scan's pattern and writes one
    # finite record per pair of 16-chunk tiles (its values carry no meaning),
    # as the scan does
    w = _wl("decode-100m", 700_000)
    qi, K, V, KR = host_inputs(w)
    bank, _ = gpu_bank_pooled(w, K, V, KR, device, 1)
    n_units = (w.n_chunks + 31) // 32
    nb = L.msa_route_workspace_bytes(bank.c, 1, 1)
    ws = torch.full((nb // 4,), float("nan"), dtype=torch.float32, device=device)
    L.msa_scan_read_probe(bank.c, ws, nb)
    torch.cuda.synchronize()
    assert torch.isfinite(ws[:n_units * 32]).all()
    assert not torch.isfinite(ws[n_units * 32:]).any()


@pytest.mark.parametrize("n_q", [1, 2])
def test_interleave_small(device, n_q):
    # the interleave driver on 2 layers of a small bank against the oracle's loop
    # (two queries: the driver's per-round slices are strided and copied)
    from long_context_memory_msa_amd.interleave import interleave

    w = W.make_workload("interleave-10mx18", bank_tokens=120_000, n_layers=2, n_q=n_q)
    banks, layers, ob_banks, hosts = [], [], [], []
    for layer in range(w.n_layers):
        qi = W.query_inputs(w, layer)
        K = W.bank_raw(w, rng.ROLE_K, 0, w.n_tok, layer)
        V = W.bank_raw(w, rng.ROLE_V, 0, w.n_tok, layer)
        KR = W.bank_raw(w, rng.ROLE_KR, 0, w.n_tok, layer)
        ob_banks.append(oracle_bank(w, K, V, KR))
        bank, rope = gpu_bank_pooled(w, K, V, KR, device, 1)
        banks.append(bank)
        hosts.append(qi)
        layers.append({k_: dev(v, w.dtype, device) for k_, v in qi.items()})
    res = interleave(banks, rope, layers, w.L_loc, w.append, w.rounds, w.k, w.pos0, w.h_q, want_scores=True)
    torch.cuda.synchronize()
    want = O.interleave(hosts, ob_banks, w.L_loc, w.append, w.rounds, w.k, w.pos0, base=w.rope_base)
    for r in range(w.rounds):
        for layer in range(w.n_layers):
            g_, o_ = res[r][layer], want[r][layer]
            assert np.abs(host(g_["s_doc"]) - o_["s_doc"]).max() <= 2e-3
            gi = g_["idx"].cpu().numpy()
            check_topk_property(g_["s_doc"].cpu().numpy(), gi, g_["val"].cpu().numpy(), w.k)
            for qq in range(w.n_q):
                if o_["gap"][qq] > 4e-3:
                    assert set(gi[qq].tolist()) == set(o_["idx"][qq].tolist())
            topk_set_valid(gi, o_["s_doc"], w.k)
            # the round's attention against the oracle's over the GPU's own selection
            L_act = w.L_loc + w.append * r
            T_new = w.L_loc if r == 0 else w.append
            qi = hosts[layer]
            o_ref = O.attend(qi["Q"][:, L_act - T_new:L_act], qi["K_loc"][:, :L_act], qi["V_loc"][:, :L_act],
                             ob_banks[layer]["kbar"], ob_banks[layer]["vbar"], ob_banks[layer]["doc_chunk_off"], gi,
                             w.pos0, base=w.rope_base)
            assert_attention_close(host(g_["O"]), o_ref)


# Memory Interleave re-routing: a round whose router tokens are the previous
# round's T0 plus t_new new ones, routed from the previous scores and the new
# tokens only (msa_layer_forward_reroute), against the oracle's routing over
# all T0 + t_new tokens; many-row (wide) and few-row scans for the new tokens,
# a bank sliced for the top-k, in place and not
@pytest.mark.parametrize("name,T0,t_new,n_q", [("16k", 96, 32, 1), ("16k", 64, 5, 2), ("decode", 7, 1, 16),
                                                ("sliced", 3, 16, 4), ("interleave", 512, 64, 1),
                                                ("16k", 96, 80, 1)])
def test_layer_reroute_equals_routing_every_token(device, name, T0, t_new, n_q):
    L_act = T0 + t_new
    if name == "sliced":
        g = np.random.default_rng(21)
        lens = g.integers(8, 41, size=9_000).astype(np.int64)
        w = _wl("decode-100m", 200_000, doc_lens=lens, chunk=64, h_kv=2, d=64, h_r=2, d_r=64, h_q=4, k=16, pos0=16)
    else:
        wname, bt = SMALL[name]
        w = _wl(wname, bt)
    w = dataclasses.replace(w, n_q=n_q, T=t_new, L_loc=L_act, T_route=L_act, gold=np.zeros((n_q, 0), np.int64))
    log(f"reroute {name}: docs={w.n_docs} chunks={w.n_chunks} n_q={n_q} T0={T0} t_new={t_new}")
    qi, K, V, KR = host_inputs(w)
    ob = oracle_bank(w, K, V, KR)
    bank, rope = gpu_bank_pooled(w, K, V, KR, device, 1)
    QR, Q, Kl, Vl = query_views(w, qi, device)          # QR over all L_act router tokens
    # the previous round's document scores: the first T0 router tokens
    prev = torch.empty((n_q, w.n_docs), dtype=torch.float32, device=device)
    nb0 = L.msa_route_workspace_bytes(bank.c, n_q, T0)
    L.msa_route_score(bank.c, QR[:, :T0].contiguous(), n_q, T0, prev, None, M.workspace(nb0, device), nb0)
    # the new tokens' own scores (same scan arithmetic per token), for the exact fold
    new = torch.empty_like(prev)
    nb1 = L.msa_route_workspace_bytes(bank.c, n_q, t_new)
    L.msa_route_score(bank.c, QR[:, T0:].contiguous(), n_q, t_new, new, None, M.workspace(nb1, device), nb1)
    torch.cuda.synchronize()
    outs = []
    for in_place in (False, True):
        O_ = torch.empty((n_q, t_new, w.h_q, w.d), dtype=M.TORCH_DTYPE[w.dtype], device=device)
        idx = torch.empty((n_q, w.k), dtype=torch.int32, device=device)
        val = torch.empty((n_q, w.k), dtype=torch.float32, device=device)
        p = prev.clone()
        s_doc = p if in_place else torch.empty_like(prev)
        nb = L.msa_layer_workspace_bytes(bank.c, n_q, t_new, t_new, L_act, w.h_q, w.k)
        L.msa_layer_forward_reroute(bank.c, Q, Kl, Vl, QR[:, T0:].contiguous(), n_q, t_new, t_new, L_act, w.h_q, w.k,
                                    w.pos0, L.default_scale(w.d), rope.c, p, O_, idx, val, s_doc,
                                    M.workspace(nb, device), nb)
        torch.cuda.synchronize()
        if not in_place:
            assert torch.equal(p, prev)                  # the input scores are left as they were
        outs.append((O_, idx, val, s_doc))
    for x, y in zip(*outs):
        assert torch.equal(x, y)
    O_, idx, val, s_doc = outs[0]
    assert torch.equal(s_doc, torch.maximum(prev, new))  # the fold, exactly
    # against the oracle's routing over every router token of the round
    S = O.chunk_scores(qi["QR"][:, :L_act], ob["krbar"])
    sd_o = O.doc_scores(S, ob["doc_chunk_off"])
    assert np.abs(host(s_doc) - sd_o).max() <= 2e-3
    gi = idx.cpu().numpy()
    check_topk_property(s_doc.cpu().numpy(), gi, val.cpu().numpy(), w.k)
    topk_set_valid(gi, sd_o, w.k)
    o_ref = O.attend(qi["Q"][:, L_act - t_new:L_act], qi["K_loc"][:, :L_act], qi["V_loc"][:, :L_act], ob["kbar"],
                     ob["vbar"], ob["doc_chunk_off"], gi, w.pos0, base=w.rope_base)
    assert_attention_close(host(O_), o_ref)
    # where the whole round's routing and the new tokens' take the same scan
    # (the tiled many-row scan both ways), the layer over all tokens is identical
    def tiled(rows_per_query):
        return rows_per_query % 16 == 0 and rows_per_query >= 32 and n_q * rows_per_query > 64

    if tiled(L_act) and tiled(t_new):
        full = run_layer(bank, rope, w, QR, Q, Kl, Vl, device)
        for x, y in zip((O_, idx, val, s_doc), full):
            assert torch.equal(x, y)


# single-token queries (the decode attention kernel) over every GQA grouping it
# takes (1, 2, 4, 8 query heads per KV head), fp32 and bf16, head dims 64 and
# 128, short and long local contexts
@pytest.mark.parametrize("name,h_kv,h_q,L_loc", [("tiny", 2, 2, 5), ("tiny", 2, 4, 1), ("tiny", 1, 8, 40),
                                                 ("16k", 8, 8, 3), ("16k", 4, 16, 1), ("16k", 2, 16, 70),
                                                 ("decode", 8, 32, 1), ("decode", 8, 64, 9)])
def test_attend_single_token_heads(device, name, h_kv, h_q, L_loc):
    wname, bt = SMALL[name]
    w = _wl(wname, bt)
    n_q = min(w.n_q, 3) if name != "decode" else w.n_q
    w = dataclasses.replace(w, h_kv=h_kv, h_q=h_q, n_q=n_q, T=1, L_loc=L_loc, T_route=1,
                            gold=np.zeros((n_q, 0), np.int64))
    g = np.random.default_rng(h_q + L_loc)
    idx_h = np.stack([g.choice(w.n_docs, size=w.k, replace=False) for _ in range(n_q)])
    log(f"attend T=1 {name} h_kv={h_kv} h_q={h_q} L_loc={L_loc} n_q={n_q} k={w.k}")
    got, want = _attend_case(w, device, idx_h, 1, L_loc)
    assert_attention_close(got, want)


# single-token queries selecting more than 64 documents: the decode kernel's
# chunk prefix over several groups of 64 ranks, memory keys over several
# 1,024-key passes, k up to the ABI's 256
@pytest.mark.parametrize("k", [100, 256])
def test_attend_single_token_many_documents(device, k):
    w = _wl("prefill-1m", 600_000)
    n_q = 3
    assert w.n_docs >= k
    w = dataclasses.replace(w, n_q=n_q, T=1, L_loc=9, T_route=1, k=k, pos0=k, gold=np.zeros((n_q, 0), np.int64))
    g = np.random.default_rng(k)
    idx_h = np.stack([g.choice(w.n_docs, size=k, replace=False) for _ in range(n_q)])
    log(f"attend T=1 k={k} docs={w.n_docs} n_q={n_q}")
    got, want = _attend_case(w, device, idx_h, 1, 9)
    assert_attention_close(got, want)


# a document id outside [0, n_docs) in one query's idx: that query's output is
# NaN throughout (the kernel's own check; the host cannot read idx), the other
# queries' outputs are as with valid ids
@pytest.mark.parametrize("name,T", [("decode", 1), ("16k", 8)])
def test_attend_invalid_document_id_gives_nan(device, name, T):
    wname, bt = SMALL[name]
    w = _wl(wname, bt)
    n_q = 3
    w = dataclasses.replace(w, n_q=n_q, T=T, L_loc=max(T, 4), T_route=1, gold=np.zeros((n_q, 0), np.int64))
    g = np.random.default_rng(5)
    idx_h = np.stack([g.choice(w.n_docs, size=w.k, replace=False) for _ in range(n_q)])
    log(f"attend invalid id {name} T={T}")
    for bad in (w.n_docs, -1):
        ib = idx_h.copy()
        ib[1, w.k // 2] = bad
        got, want = _attend_case(w, device, np.where(ib < 0, 0, np.minimum(ib, w.n_docs - 1)), T, w.L_loc,
                                 idx_dev=ib)
        assert np.isnan(got[1]).all()
        for q in (0, 2):
            assert_attention_close(got[q:q + 1], want[q:q + 1])
