"""GPU parity at the workloads' full sizes, in the launch configuration bench.py
times.

* 1M-token bank (prefill-1m): the whole layer against the oracle.
* 100M-token bank (decode-100m): the bank is generated and pooled on the
  GPU slab by slab; the oracle regenerates a sample of documents (first, last,
  gold, random; >= 4096 chunks) from the same counter generator and checks
  their pooled rows and router scores; top-k is checked by its defining
  property on the GPU's own scores plus planted-gold recovery; attention runs
  at full size on test-chosen documents and is checked for sampled queries.
* 18 routed layers x 10M tokens with 3 Memory Interleave rounds (interleave-10mx18):
  per-layer banks on the GPU, the interleave driver, sampled pooled rows and
  router scores for sampled layers and rounds, top-k properties everywhere,
  the attention of sampled layers in every round on the layer's own selection,
  and full-shape attention (prefill and a later round) on test-chosen
  documents, all against the oracle.
Tolerances as in test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

import oracle as O
from synth import device as sdev, rng, workloads as W
from long_context_memory_msa_amd import _lib as L, memory as M, offline
from long_context_memory_msa_amd.interleave import interleave

from gpu_common import assert_attention_close, bf16_spacing, check_topk_property, dev, host, log, topk_set_valid

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def build_bank(w, layer, uhat_dev, device):
    bank = M.Bank(w.doc_lens, w.chunk, w.h_kv, w.d, w.h_r, w.d_r, w.dtype, device)
    rope = M.Rope(w.max_pos, w.d, w.rope_base, device)
    offline.encode_bank(bank, rope, lambda a, b, K, V, KR: sdev.fill_raw_slab(w, layer, a, b, K, V, KR, uhat_dev),
                        8_000_000, w.h_kv, w.d, w.h_r, w.d_r)
    return bank, rope


def sample_docs(w, n_random, seed, extra=()):
    g = np.random.default_rng(seed)
    docs = {0, w.n_docs - 1, *[int(x) for x in extra]}
    docs |= set(g.choice(w.n_docs, size=min(n_random, w.n_docs), replace=False).tolist())
    return sorted(docs)


def oracle_docs(w, docs, layer, uhat):
    """Oracle pooling of the sampled documents, from regenerated raw tokens."""
    out = {}
    for doc in docs:
        K = W.doc_tokens(w, rng.ROLE_K, doc, layer)
        V = W.doc_tokens(w, rng.ROLE_V, doc, layer)
        KR = W.doc_tokens(w, rng.ROLE_KR, doc, layer, uhat)
        out[doc] = O.pool([int(w.doc_lens[doc])], w.chunk, K, V, KR, w.dtype, w.rope_base)
    return out


def check_pooled_rows(w, bank, ob_docs):
    off = w.doc_chunk_off
    kb, vb, krb, inv = bank.kbar, bank.vbar, bank.krbar, bank.kr_inv_norm
    n = 0
    for doc, ob in ob_docs.items():
        a, b = int(off[doc]), int(off[doc + 1])
        n += b - a
        for got, name in ((host(kb[:, a:b]), "kbar"), (host(vb[:, a:b]), "vbar"), (host(krb[a:b]), "krbar")):
            exact = ob[name + "_exact"]
            slack = 1e-5 * np.abs(exact).max(axis=-1, keepdims=True)
            assert np.all(np.abs(got - exact) <= bf16_spacing(exact) + slack), (doc, name)
        gi = host(inv[a:b])
        assert np.all(np.abs(gi - ob["kr_inv_norm"]) <= 2e-4 * ob["kr_inv_norm"]), doc
        assert np.all(bank.chunk_doc[a:b].cpu().numpy() == doc)
    return n


def compact_bank(ob_docs, docs):
    """A bank of just ``docs`` (in that order) built from per-document oracle pools."""
    kbar = np.concatenate([ob_docs[d]["kbar"] for d in docs], axis=1)
    vbar = np.concatenate([ob_docs[d]["vbar"] for d in docs], axis=1)
    counts = [ob_docs[d]["kbar"].shape[1] for d in docs]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return kbar, vbar, off


# ---------------------------------------------------------------------------
def test_full_1m_bank_layer(device):
    w = W.make_workload("prefill-1m")
    log(f"1M bank: {w.n_docs} docs, {w.n_chunks} chunks")
    qi = W.query_inputs(w)
    uh = W.gold_uhat(w, qi["QR"])
    K = W.bank_raw(w, rng.ROLE_K, 0, w.n_tok)
    V = W.bank_raw(w, rng.ROLE_V, 0, w.n_tok)
    KR = W.bank_raw(w, rng.ROLE_KR, 0, w.n_tok, uhat=uh)
    ob = O.pool(w.doc_lens, w.chunk, K, V, KR, w.dtype, w.rope_base)
    want = O.layer_forward(qi["QR"][:, :w.L_loc], qi["Q"][:, :w.L_loc], qi["K_loc"][:, :w.L_loc],
                           qi["V_loc"][:, :w.L_loc], ob, w.k, w.pos0, base=w.rope_base)
    bank, rope = build_bank(w, 0, torch.from_numpy(uh).to(device), device)
    del K, V, KR
    for name in ("kbar", "vbar", "krbar"):
        exact = ob[name + "_exact"]
        got = host(getattr(bank, name))
        slack = 1e-5 * np.abs(exact).max(axis=-1, keepdims=True)
        assert np.all(np.abs(got - exact) <= bf16_spacing(exact) + slack), name
    QR, Q = dev(qi["QR"][:, :w.L_loc], w.dtype, device), dev(qi["Q"][:, :w.L_loc], w.dtype, device)
    Kl, Vl = dev(qi["K_loc"][:, :w.L_loc], w.dtype, device), dev(qi["V_loc"][:, :w.L_loc], w.dtype, device)
    out = torch.empty((1, w.T, w.h_q, w.d), dtype=torch.bfloat16, device=device)
    idx = torch.empty((1, w.k), dtype=torch.int32, device=device)
    val = torch.empty((1, w.k), dtype=torch.float32, device=device)
    s_doc = torch.empty((1, w.n_docs), dtype=torch.float32, device=device)
    nb = L.msa_layer_workspace_bytes(bank.c, 1, w.T, w.T_route, w.L_loc, w.h_q, w.k)
    ws = M.workspace(nb, device)
    L.msa_layer_forward(bank.c, Q, Kl, Vl, QR, 1, w.T, w.T_route, w.L_loc, w.h_q, w.k, w.pos0,
                        L.default_scale(w.d), rope.c, out, idx, val, s_doc, ws, nb)
    torch.cuda.synchronize()
    assert np.abs(host(s_doc) - want["s_doc"]).max() <= 2e-3
    gi = idx.cpu().numpy()
    check_topk_property(s_doc.cpu().numpy(), gi, val.cpu().numpy(), w.k)
    if want["gap"][0] > 4e-3:
        assert set(gi[0].tolist()) == set(want["idx"][0].tolist())
    topk_set_valid(gi, want["s_doc"], w.k)
    # the layer's attention against the oracle's over the layer's own selection
    o_ref = O.attend(qi["Q"][:, :w.L_loc], qi["K_loc"][:, :w.L_loc], qi["V_loc"][:, :w.L_loc], ob["kbar"],
                     ob["vbar"], ob["doc_chunk_off"], gi, w.pos0, base=w.rope_base)
    e = assert_attention_close(host(out), o_ref)
    log(f"  attention on the layer's own selection: max {e[0]:.3g} mean {e[1]:.3g}")


# ---------------------------------------------------------------------------
def test_full_100m_bank_decode(device):
    w = W.make_workload("decode-100m")
    log(f"100M bank: {w.n_docs} docs, {w.n_chunks} chunks")
    qi = W.query_inputs(w)
    uh = W.gold_uhat(w, qi["QR"])
    bank, rope = build_bank(w, 0, torch.from_numpy(uh).to(device), device)
    QR = dev(qi["QR"], w.dtype, device)
    Q, Kl, Vl = dev(qi["Q"], w.dtype, device), dev(qi["K_loc"], w.dtype, device), dev(qi["V_loc"], w.dtype, device)

    # the layer in bench.py's launch configuration
    out = torch.empty((w.n_q, 1, w.h_q, w.d), dtype=torch.bfloat16, device=device)
    idx = torch.empty((w.n_q, w.k), dtype=torch.int32, device=device)
    val = torch.empty((w.n_q, w.k), dtype=torch.float32, device=device)
    s_doc = torch.empty((w.n_q, w.n_docs), dtype=torch.float32, device=device)
    nb = L.msa_layer_workspace_bytes(bank.c, w.n_q, 1, 1, 1, w.h_q, w.k)
    ws = M.workspace(nb, device)
    L.msa_layer_forward(bank.c, Q, Kl, Vl, QR, w.n_q, 1, 1, 1, w.h_q, w.k, w.pos0, L.default_scale(w.d), rope.c,
                        out, idx, val, s_doc, ws, nb)
    torch.cuda.synchronize()
    sd, gi, gv = s_doc.cpu().numpy(), idx.cpu().numpy(), val.cpu().numpy()
    check_topk_property(sd, gi, gv, w.k)
    for q in range(w.n_q):
        assert set(w.gold[q].tolist()) <= set(gi[q].tolist()), f"query {q}: planted gold not recovered"

    # sampled documents: pooled rows and router scores against the oracle
    docs = sample_docs(w, 110, 31, extra=list(w.gold[0]) + list(w.gold[7]))
    ob_docs = oracle_docs(w, docs, 0, uh)
    n_ch = check_pooled_rows(w, bank, ob_docs)
    log(f"  pooled rows checked: {len(docs)} documents, {n_ch} chunks")
    assert n_ch >= 4096
    for doc in docs:
        S = O.chunk_scores(qi["QR"], ob_docs[doc]["krbar"])
        assert np.abs(sd[:, doc] - S.max(axis=1)).max() <= 2e-3, doc

    # attention at full size on test-chosen documents (gold + random), sampled queries checked
    g = np.random.default_rng(5)
    choice = np.stack([np.concatenate([w.gold[q], g.choice(np.setdiff1d(np.arange(w.n_docs), w.gold[q]), 8,
                                                            replace=False)]) for q in range(w.n_q)])
    choice = np.stack([g.permutation(r) for r in choice]).astype(np.int32)
    out2 = torch.empty_like(out)
    nb2 = L.msa_attend_workspace_bytes(bank.c, w.n_q, 1, 1, w.h_q, w.k)
    ws2 = M.workspace(nb2, device)
    L.msa_sparse_attend(bank.c, Q, Kl, Vl, w.n_q, 1, 1, w.h_q, torch.from_numpy(choice).to(device), w.k, w.pos0,
                        L.default_scale(w.d), rope.c, out2, ws2, nb2)
    torch.cuda.synchronize()
    got = host(out2)
    for q in (0, 5, 10, 15):
        sel = [int(x) for x in choice[q]]
        obs = oracle_docs(w, sel, 0, uh)
        kbar, vbar, off = compact_bank(obs, sel)
        want = O.attend(qi["Q"][q:q + 1], qi["K_loc"][q:q + 1], qi["V_loc"][q:q + 1], kbar, vbar, off,
                        np.arange(w.k)[None, :], w.pos0, base=w.rope_base)
        assert_attention_close(got[q:q + 1], want)
    # the layer's attention is the same kernel on the layer's own selection
    out3 = torch.empty_like(out)
    L.msa_sparse_attend(bank.c, Q, Kl, Vl, w.n_q, 1, 1, w.h_q, idx, w.k, w.pos0, L.default_scale(w.d), rope.c, out3,
                        ws2, nb2)
    torch.cuda.synchronize()
    assert torch.equal(out3, out)


# ---------------------------------------------------------------------------
def test_full_interleave_18_layers(device):
    w = W.make_workload("interleave-10mx18")
    log(f"interleave: {w.n_layers} layers x {w.n_docs} docs, {w.n_chunks} chunks, {w.rounds} rounds")
    banks, layers, hosts = [], [], []
    for layer in range(w.n_layers):
        bank, rope = build_bank(w, layer, None, device)
        banks.append(bank)
        qi = W.query_inputs(w, layer)
        hosts.append(qi)
        layers.append({k_: dev(v, w.dtype, device) for k_, v in qi.items()})
    res = interleave(banks, rope, layers, w.L_loc, w.append, w.rounds, w.k, w.pos0, w.h_q, want_scores=True)
    torch.cuda.synchronize()
    for r in range(w.rounds):
        for layer in range(w.n_layers):
            x = res[r][layer]
            check_topk_property(x["s_doc"].cpu().numpy(), x["idx"].cpu().numpy(), x["val"].cpu().numpy(), w.k)
            assert torch.isfinite(x["O"].float()).all()
    # sampled layers: pooled rows and router scores of every round
    for layer in (0, w.n_layers - 1):
        docs = sample_docs(w, 20, 40 + layer)
        ob_docs = oracle_docs(w, docs, layer, None)
        check_pooled_rows(w, banks[layer], ob_docs)
        for r in range(w.rounds):
            L_act = w.L_loc + w.append * r
            sd = res[r][layer]["s_doc"].cpu().numpy()
            for doc in docs:
                S = O.chunk_scores(hosts[layer]["QR"][:, :L_act], ob_docs[doc]["krbar"])
                assert np.abs(sd[:, doc] - S.max(axis=1)).max() <= 2e-3, (layer, r, doc)
    # every round of sampled layers: the layer's attention on its own selection
    # against the oracle's (pooled rows of the selected documents regenerated
    # from the counter generator)
    for layer in (0, 7, w.n_layers - 1):
        qi = hosts[layer]
        for r in range(w.rounds):
            L_act = w.L_loc + w.append * r
            T_new = w.L_loc if r == 0 else w.append
            sel = [int(x) for x in res[r][layer]["idx"].cpu().numpy()[0]]
            obs = oracle_docs(w, sel, layer, None)
            kbar, vbar, off = compact_bank(obs, sel)
            want = O.attend(qi["Q"][:, L_act - T_new:L_act], qi["K_loc"][:, :L_act], qi["V_loc"][:, :L_act], kbar,
                            vbar, off, np.arange(w.k)[None, :], w.pos0, base=w.rope_base)
            e = assert_attention_close(host(res[r][layer]["O"]), want)
            log(f"  layer {layer} round {r}: attention on its own selection, max {e[0]:.3g} mean {e[1]:.3g}")
    # full-shape attention against the oracle on test-chosen documents: prefill
    # (round 0) and the last round
    layer = 3
    sel = [int(x) for x in np.random.default_rng(9).choice(w.n_docs, size=w.k, replace=False)]
    obs = oracle_docs(w, sel, layer, None)
    kbar, vbar, off = compact_bank(obs, sel)
    qi = hosts[layer]
    idx_d = torch.from_numpy(np.array([sel], dtype=np.int32)).to(device)
    for r in (0, w.rounds - 1):
        L_act = w.L_loc + w.append * r
        T_new = w.L_loc if r == 0 else w.append
        out = torch.empty((1, T_new, w.h_q, w.d), dtype=torch.bfloat16, device=device)
        nb = L.msa_attend_workspace_bytes(banks[layer].c, 1, T_new, L_act, w.h_q, w.k)
        ws = M.workspace(nb, device)
        L.msa_sparse_attend(banks[layer].c, layers[layer]["Q"][:, L_act - T_new:L_act].contiguous(),
                            layers[layer]["K_loc"][:, :L_act].contiguous(), layers[layer]["V_loc"][:, :L_act].contiguous(),
                            1, T_new, L_act, w.h_q, idx_d, w.k, w.pos0, L.default_scale(w.d), rope.c, out, ws, nb)
        torch.cuda.synchronize()
        want = O.attend(qi["Q"][:, L_act - T_new:L_act], qi["K_loc"][:, :L_act], qi["V_loc"][:, :L_act], kbar, vbar,
                        off, np.arange(w.k)[None, :], w.pos0, base=w.rope_base)
        assert_attention_close(host(out), want)
