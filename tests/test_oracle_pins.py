"""Pins of the fp64 oracle against things other than itself.

Each test checks the oracle against a closed form, an invariant, a library
routine (SciPy, NumPy lexsort, torch's scaled_dot_product_attention and
bfloat16 conversion), a brute-force loop, or the hand-derived fixture in
tests/golden/, chosen so that a plausible slip (a dropped term, a wrong sign,
a swapped reduction order, a wrong head or position index) fails one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.spatial.distance as ssd
import torch
import torch.nn.functional as F

import oracle as O
from synth import rng, workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------------------
# RoPE
def test_rope_theta_closed_form():
    th = O.rope_theta(64, 10000.0)
    assert th[0] == 1.0
    assert th[16] == pytest.approx(0.01, rel=1e-15)          # 10000 ** (-32/64)
    assert th[8] == pytest.approx(0.1, rel=1e-15)            # 10000 ** (-16/64)
    th2 = O.rope_theta(128, 500000.0)
    assert th2[32] == pytest.approx(500000.0 ** -0.5, rel=1e-15)


def test_rope_d2_is_plane_rotation():
    # d = 2: (1, 0) at position p -> (cos p, sin p) (counter-clockwise)
    for p in (0.0, 1.0, 2.5, 7.0):
        y = O.rope_apply(np.array([1.0, 0.0]), p)
        assert y == pytest.approx([math.cos(p), math.sin(p)], abs=1e-15)
        y = O.rope_apply(np.array([0.0, 1.0]), p)
        assert y == pytest.approx([-math.sin(p), math.cos(p)], abs=1e-15)


def test_rope_matches_complex_multiplication():
    d, base = 128, 10000.0
    x = _rand((5, d), 1)
    pos = np.array([0, 1, 17, 511, 8191], dtype=np.float64)
    z = x[:, : d // 2] + 1j * x[:, d // 2:]
    freq = np.array([base ** (-(2.0 * i) / d) for i in range(d // 2)])
    zr = z * np.exp(1j * pos[:, None] * freq[None, :])
    want = np.concatenate([zr.real, zr.imag], axis=1)
    assert np.allclose(O.rope_apply(x, pos), want, atol=1e-12, rtol=0)


def test_rope_identity_norm_relative_composition():
    d = 64
    x, y = _rand(d, 2), _rand(d, 3)
    assert np.array_equal(O.rope_apply(x, 0.0), x)
    for p in (3.0, 100.0, 4095.0):
        assert np.linalg.norm(O.rope_apply(x, p)) == pytest.approx(np.linalg.norm(x), rel=1e-13)
    p, pp = 37.0, 1234.0
    lhs = O.rope_apply(x, p) @ O.rope_apply(y, pp)
    rhs = x @ O.rope_apply(y, pp - p)
    assert lhs == pytest.approx(rhs, rel=1e-11)
    assert np.allclose(O.rope_apply(O.rope_apply(x, p), pp), O.rope_apply(x, p + pp), atol=1e-11)


# ---------------------------------------------------------------------------
# storage rounding
def test_round_bf16_matches_torch_and_ties_to_even():
    x = np.random.default_rng(4).standard_normal(100000).astype(np.float32).astype(np.float64)
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x), want)
    one = 1.0
    assert O.round_bf16(np.array([one + 2.0 ** -8]))[0] == 1.0                    # tie -> even (down)
    assert O.round_bf16(np.array([one + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6     # tie -> even (up)
    assert O.round_bf16(np.array([one + 2.0 ** -8 + 2.0 ** -30]))[0] == 1.0 + 2.0 ** -7
    assert O.round_bf16(np.array([-3.0]))[0] == -3.0


# ---------------------------------------------------------------------------
# pooling
def test_pool_hand_example_partial_chunks_and_positions():
    # docs of 3 and 5 tokens, chunk 2: chunks (0,1)(2) | (3,4)(5,6)(7)
    lens = [3, 5]
    n = 8
    V = np.arange(1, n + 1, dtype=np.float64).reshape(n, 1, 1) * np.ones((1, 1, 2))
    KR = 2.0 * V
    K = np.zeros((n, 1, 2))
    K[:, 0, 0] = 1.0                                # unit vector (1, 0) at every token
    b = O.pool(lens, 2, K, V, KR, "f32")
    assert b["n_chunks"] == 5
    assert np.array_equal(b["doc_chunk_off"], [0, 2, 5])
    assert np.array_equal(b["chunk_doc"], [0, 0, 1, 1, 1])
    assert np.allclose(b["vbar_exact"][0, :, 0], [1.5, 3.0, 4.5, 6.5, 8.0])
    assert np.allclose(b["krbar_exact"][:, 0, 0], [3.0, 6.0, 9.0, 13.0, 16.0])
    # positions restart at 0 in each document: rotated (1,0) at p is (cos p, sin p)
    want = np.array([[(math.cos(0) + math.cos(1)) / 2, (math.sin(0) + math.sin(1)) / 2],
                     [math.cos(2), math.sin(2)],
                     [(math.cos(0) + math.cos(1)) / 2, (math.sin(0) + math.sin(1)) / 2],
                     [(math.cos(2) + math.cos(3)) / 2, (math.sin(2) + math.sin(3)) / 2],
                     [math.cos(4), math.sin(4)]])
    assert np.allclose(b["kbar_exact"][0], want, atol=1e-15)


def test_pool_constant_chunk1_and_whole_doc():
    lens = [7, 130, 64, 1]
    n = sum(lens)
    c = _rand((1, 2, 8), 5)
    K = np.repeat(c, n, axis=0)
    b = O.pool(lens, 64, K, K, K, "f32")
    assert b["n_chunks"] == sum((L + 63) // 64 for L in lens)
    assert np.allclose(b["vbar_exact"], np.broadcast_to(c.transpose(1, 0, 2), b["vbar_exact"].shape))
    assert np.allclose(b["krbar_exact"], np.broadcast_to(c, b["krbar_exact"].shape))
    # chunk 1: pooled K is the rotated token itself at its in-document position
    K = _rand((n, 2, 8), 6)
    b1 = O.pool(lens, 1, K, K, K, "f32")
    pos = np.concatenate([np.arange(L) for L in lens]).astype(np.float64)
    assert np.allclose(b1["kbar_exact"].transpose(1, 0, 2), O.rope_apply(K, pos[:, None]), atol=1e-14)
    assert np.allclose(b1["vbar_exact"].transpose(1, 0, 2), K)
    # chunk >= every length: one chunk per document, the document mean
    bw = O.pool(lens, 256, K, K, K, "f32")
    off = np.concatenate([[0], np.cumsum(lens)])
    for i in range(len(lens)):
        assert np.allclose(bw["krbar_exact"][i], K[off[i]:off[i + 1]].mean(axis=0))


def test_pool_inverse_norms_from_stored_values():
    KR = np.zeros((2, 2, 4))
    KR[:, 0, :2] = [3.0, 4.0]
    b = O.pool([2], 2, np.zeros((2, 1, 4)), np.zeros((2, 1, 4)), KR, "bf16")
    assert b["kr_inv_norm"][0, 0] == pytest.approx(0.2, rel=1e-15)
    assert b["kr_inv_norm"][0, 1] == 0.0             # zero row -> 0, so its cosine is 0
    x = np.full((1, 1, 4), 1.0 + 2.0 ** -8 + 2.0 ** -20)  # rounds up to 1 + 2**-7 in bf16
    b = O.pool([1], 1, np.zeros((1, 1, 4)), np.zeros((1, 1, 4)), x, "bf16")
    assert b["krbar"][0, 0, 0] == 1.0 + 2.0 ** -7
    assert b["kr_inv_norm"][0, 0] == pytest.approx(1.0 / (2.0 * (1.0 + 2.0 ** -7)), rel=1e-15)


# ---------------------------------------------------------------------------
# routing
def test_cosine_against_scipy_and_invariants():
    x, y = _rand((50, 32), 7), _rand((50, 32), 8)
    got = O.cosine(x, y)
    want = np.array([1.0 - ssd.cosine(x[i], y[i]) for i in range(50)])
    assert np.allclose(got, want, atol=1e-14)
    assert np.allclose(O.cosine(x, x), 1.0)
    assert np.allclose(O.cosine(x, -x), -1.0)
    assert np.allclose(O.cosine(3.0 * x, 0.25 * y), got)
    assert O.cosine(np.zeros(4), np.ones(4)) == 0.0


def test_route_golden_fixture():
    g = json.load(open(os.path.join(GOLDEN, "route_tiny.json")))
    S = O.chunk_scores(np.array(g["QR"], float), np.array(g["krbar"], float))
    assert np.allclose(S, g["S"], atol=1e-15)
    sd = O.doc_scores(S, np.array(g["doc_chunk_off"]))
    assert np.allclose(sd, g["s_doc"], atol=1e-15)
    assert O.topk(sd, 2)["idx"].tolist() == g["top2"]
    assert O.topk(sd, 3)["idx"].tolist() == g["top3"]


def test_route_single_head_single_token_is_one_cosine():
    q = _rand((1, 1, 1, 16), 9)
    kr = _rand((40, 1, 16), 10)
    S = O.chunk_scores(q, kr)
    want = [1.0 - ssd.cosine(q[0, 0, 0], kr[c, 0]) for c in range(40)]
    assert np.allclose(S[0], want, atol=1e-14)


def test_route_identical_vectors_score_one_for_any_head_count():
    kr = _rand((6, 4, 8), 11)
    q = kr[2][None, None]                 # query equals chunk 2 on every head
    S = O.chunk_scores(q, kr)
    assert S[0, 2] == pytest.approx(1.0, abs=1e-14)
    assert np.all(S[0] <= 1.0 + 1e-14)


def test_route_brute_force_loops_and_head_permutation():
    q = _rand((2, 3, 3, 5), 12)
    kr = _rand((7, 3, 5), 13)
    S = O.chunk_scores(q, kr, block=3)
    for qi in range(2):
        for c in range(7):
            best = -math.inf
            for t in range(3):
                acc = 0.0
                for h in range(3):
                    a, b = q[qi, t, h], kr[c, h]
                    acc += sum(a * b) / (math.sqrt(sum(a * a)) * math.sqrt(sum(b * b)))
                best = max(best, acc / 3)
            assert S[qi, c] == pytest.approx(best, abs=1e-14)
    perm = [2, 0, 1]
    assert np.allclose(O.chunk_scores(q[:, :, perm], kr[:, perm]), S, atol=1e-15)


def test_doc_scores_brute_force_and_one_chunk_per_doc():
    S = _rand((3, 20), 14)
    off = np.array([0, 1, 5, 6, 13, 20])
    sd = O.doc_scores(S, off)
    for q in range(3):
        for i in range(5):
            assert sd[q, i] == max(S[q, off[i]:off[i + 1]])
    assert np.array_equal(O.doc_scores(S, np.arange(21)), S)


# ---------------------------------------------------------------------------
# top-k
def test_topk_against_lexsort_with_ties():
    s = np.round(_rand((4, 300), 15) * 4) / 4          # many exact ties
    for k in (1, 5, 64, 300):
        r = O.topk(s, k)
        for q in range(4):
            order = np.lexsort((np.arange(300), -s[q]))  # by -score, then index
            assert r["idx"][q].tolist() == order[:k].tolist()
            assert np.array_equal(r["val"][q], s[q, order[:k]])
    r = O.topk(np.array([[0.5, 0.7, 0.7, 0.1, 0.7]]), 4)
    assert r["idx"].tolist() == [[1, 2, 4, 0]]
    assert r["gap"][0] == pytest.approx(0.5 - 0.1)
    assert math.isinf(O.topk(np.array([[0.1, 0.2]]), 2)["gap"][0])


# ---------------------------------------------------------------------------
# attention
def _bank(seed, lens, H_kv, d, chunk=4):
    n = sum(lens)
    K, V = _rand((n, H_kv, d), seed), _rand((n, H_kv, d), seed + 1)
    return O.pool(lens, chunk, K, V, _rand((n, H_kv, d), seed + 2), "f32")


def _sdpa_reference(Q, K_loc, V_loc, bank, idx, pos0):
    """torch SDPA (fp64, CPU) on the explicit concatenation with an explicit mask."""
    n_q, T, H_q, d = Q.shape
    L_loc, H_kv = K_loc.shape[1], K_loc.shape[2]
    out = np.empty(Q.shape)
    s_t = L_loc - T + np.arange(T)
    for q in range(n_q):
        ch = np.concatenate([np.arange(bank["doc_chunk_off"][i], bank["doc_chunk_off"][i + 1]) for i in idx[q]])
        kmem = bank["kbar"][:, ch]                                     # [H_kv][n][d]
        vmem = bank["vbar"][:, ch]
        kl = O.rope_apply(K_loc[q], (pos0 + np.arange(L_loc))[:, None]).transpose(1, 0, 2)
        vl = V_loc[q].transpose(1, 0, 2)
        qr = O.rope_apply(Q[q], (pos0 + s_t)[:, None]).transpose(1, 0, 2)  # [H_q][T][d]
        keys = np.concatenate([kmem, kl], axis=1)
        vals = np.concatenate([vmem, vl], axis=1)
        mask = np.concatenate([np.ones((T, ch.size), bool), np.arange(L_loc)[None] <= s_t[:, None]], axis=1)
        o = F.scaled_dot_product_attention(torch.from_numpy(qr)[None], torch.from_numpy(keys)[None],
                                           torch.from_numpy(vals)[None], attn_mask=torch.from_numpy(mask),
                                           enable_gqa=True)
        out[q] = o[0].numpy().transpose(1, 0, 2)
    return out


def test_attend_matches_torch_sdpa_gqa_causal():
    lens = [5, 9, 4, 12, 3]
    H_kv, H_q, d = 2, 6, 8
    bank = _bank(20, lens, H_kv, d)
    n_q, T, L_loc, pos0 = 2, 3, 5, 3
    Q, Kl, Vl = _rand((n_q, T, H_q, d), 30), _rand((n_q, L_loc, H_kv, d), 31), _rand((n_q, L_loc, H_kv, d), 32)
    idx = np.array([[3, 0, 4], [1, 2, 0]])
    got = O.attend(Q, Kl, Vl, bank["kbar"], bank["vbar"], bank["doc_chunk_off"], idx, pos0)
    want = _sdpa_reference(Q, Kl, Vl, bank, idx, pos0)
    assert np.allclose(got, want, atol=1e-12)


def test_attend_all_documents_equals_dense_memory_attention():
    lens = [6, 2, 9, 4]
    bank = _bank(40, lens, 1, 8)
    Q, Kl, Vl = _rand((1, 2, 2, 8), 41), _rand((1, 3, 1, 8), 42), _rand((1, 3, 1, 8), 43)
    got = O.attend(Q, Kl, Vl, bank["kbar"], bank["vbar"], bank["doc_chunk_off"], np.array([[2, 0, 3, 1]]), 4)
    dense = _sdpa_reference(Q, Kl, Vl, bank, np.array([[0, 1, 2, 3]]), 4)   # bank order
    assert np.allclose(got, dense, atol=1e-12)


def test_attend_zero_query_is_mean_of_visible_values_per_kv_head():
    lens = [4, 4, 8]
    H_kv, g, d = 2, 3, 4
    bank = _bank(50, lens, H_kv, d)
    bank["vbar"][0] = 0.0
    bank["vbar"][1] = 100.0
    L_loc, T = 4, 4
    Vl = np.zeros((1, L_loc, H_kv, d))
    Vl[0, :, 0] = np.arange(L_loc)[:, None]          # local values 0, 1, 2, 3 on KV head 0
    Vl[0, :, 1] = 100.0
    Q = np.zeros((1, T, H_kv * g, d))
    idx = np.array([[1, 0]])                        # 2 memory chunks
    got = O.attend(Q, _rand((1, L_loc, H_kv, d), 51), Vl, bank["kbar"], bank["vbar"], bank["doc_chunk_off"], idx, 2)
    for t in range(T):
        n_vis = 2 + t + 1
        for h in range(H_kv * g):
            want = 100.0 if h // g == 1 else sum(range(t + 1)) / n_vis
            assert np.allclose(got[0, t, h], want, atol=1e-12)


def test_attend_query_position_is_pos0_plus_local_index():
    # one memory key and one local key; logits written with complex rotations
    d, pos0 = 4, 7
    bank = _bank(60, [1], 1, d, chunk=1)
    kmem, vmem = bank["kbar"][0, 0], bank["vbar"][0, 0]
    q, kl, vl = _rand(d, 61), _rand(d, 62), _rand(d, 63)

    def rot(x, p):
        z = (x[: d // 2] + 1j * x[d // 2:]) * np.exp(1j * p * O.rope_theta(d))
        return np.concatenate([z.real, z.imag])

    a = rot(q, pos0) @ kmem / 2.0                    # query at pos0 + 0 vs memory key (no extra rotation)
    b = rot(q, pos0) @ rot(kl, pos0) / 2.0            # local key 0 at pos0
    want = (math.exp(a) * vmem + math.exp(b) * vl) / (math.exp(a) + math.exp(b))
    got = O.attend(q[None, None, None], kl[None, None, None], vl[None, None, None], bank["kbar"], bank["vbar"],
                   bank["doc_chunk_off"], np.array([[0]]), pos0)
    assert np.allclose(got[0, 0, 0], want, atol=1e-13)


# ---------------------------------------------------------------------------
# end to end: planted gold documents are recovered
def _oracle_layer(w):
    qi = W.query_inputs(w)
    uh = W.gold_uhat(w, qi["QR"])
    K = W.bank_raw(w, rng.ROLE_K, 0, w.n_tok)
    V = W.bank_raw(w, rng.ROLE_V, 0, w.n_tok)
    KR = W.bank_raw(w, rng.ROLE_KR, 0, w.n_tok, uhat=uh)
    bank = O.pool(w.doc_lens, w.chunk, K, V, KR, w.dtype, w.rope_base)
    res = O.layer_forward(qi["QR"][:, w.L_loc - w.T_route:w.L_loc], qi["Q"][:, w.L_loc - w.T:w.L_loc],
                          qi["K_loc"][:, :w.L_loc], qi["V_loc"][:, :w.L_loc], bank, w.k, w.pos0)
    return res


@pytest.mark.parametrize("name", ["tiny-f32", "prefill-16k"])
def test_planted_gold_recovered(name):
    w = W.make_workload(name)
    res = _oracle_layer(w)
    for q in range(w.n_q):
        assert set(w.gold[q].tolist()) <= set(res["idx"][q].tolist())


@pytest.mark.slow
def test_planted_gold_recovered_decode_shape():
    # the 100M-token decode workload's shape (16 queries x 1 token, k=16, 8 gold each) on a 2M-token bank
    w = W.make_workload("decode-100m", bank_tokens=2_000_000)
    res = _oracle_layer(w)
    for q in range(w.n_q):
        assert set(w.gold[q].tolist()) <= set(res["idx"][q].tolist())


# ---- router projection (R10) -------------------------------------------------
def test_project_brute_force_tiny():
    rng_ = np.random.default_rng(11)
    X = rng_.standard_normal((3, 5))
    Wt = rng_.standard_normal((4, 5))
    want = np.array([[sum(X[r, i] * Wt[o, i] for i in range(5)) for o in range(4)] for r in range(3)])
    assert np.allclose(O.project(X, Wt), want, rtol=1e-14, atol=1e-14)


def test_project_identity_permutation_and_scaling_are_exact():
    rng_ = np.random.default_rng(12)
    X = O.round_bf16(rng_.standard_normal((7, 128)))
    assert np.array_equal(O.project(X, np.eye(128)), X)
    perm = rng_.permutation(128)
    P = np.eye(128)[perm] * 0.25                     # output o reads input perm[o], scaled by 2^-2
    assert np.array_equal(O.project(X, P), X[:, perm] * 0.25)


def test_project_is_linear_and_batches_leading_axes():
    rng_ = np.random.default_rng(13)
    X1, X2 = rng_.standard_normal((2, 3, 64)), rng_.standard_normal((2, 3, 64))
    Wt = rng_.standard_normal((128, 64))
    Y = O.project(2.0 * X1 - 3.0 * X2, Wt)
    assert np.allclose(Y, 2.0 * O.project(X1, Wt) - 3.0 * O.project(X2, Wt), atol=1e-11)
    assert O.project(X1, Wt).shape == (2, 3, 128)
    # a zero row of W gives a zero output feature
    Wz = Wt.copy()
    Wz[5] = 0.0
    assert np.all(O.project(X1, Wz)[..., 5] == 0.0)


# ---- Memory Interleave (hotdry blog, sparse strategy and parameters; Lighthouse
# digest, Component 3) ----------------------------------------------------------
def _interleave_fixture():
    with open(os.path.join(GOLDEN, "interleave_tiny.json")) as f:
        g = json.load(f)
    bank = {name: np.array(g[name], dtype=np.float64) for name in ("krbar", "kbar", "vbar")}
    bank["doc_chunk_off"] = np.array(g["doc_chunk_off"], dtype=np.int64)
    layer = {name: np.array(g[name], dtype=np.float64) for name in ("QR", "Q", "K_loc", "V_loc")}
    return g, bank, layer


def test_interleave_golden_fixture():
    # hand-derived two-round example: round 1 re-routes with all active tokens
    # (the new token alone would pick [C, B], no re-routing [A, B]), attends only
    # the new token at position pos0 + 1 over the whole causal local context
    g, bank, layer = _interleave_fixture()
    res = O.interleave([layer], [bank], g["T0"], g["append"], g["rounds"], g["k"], g["pos0"], scale=g["scale"])
    assert len(res) == g["rounds"] == 2 and all(len(r) == 1 for r in res)
    for r, want in enumerate(g["rounds_expected"]):
        got = res[r][0]
        assert np.allclose(got["s_doc"], want["s_doc"], atol=1e-15, rtol=0), r
        assert got["idx"].tolist() == want["idx"], r
        assert np.allclose(got["val"], want["val"], atol=1e-15, rtol=0), r
        assert np.allclose(got["gap"], want["gap"], atol=1e-15, rtol=0), r
        assert got["O"].shape == np.array(want["O"]).shape, r          # only the new token is attended
        assert np.allclose(got["O"], want["O"], atol=1e-15, rtol=0), r


def test_interleave_rounds_route_all_active_tokens_and_attend_the_new_ones(monkeypatch):
    # every layer call of every round sees exactly: router tokens [0, L_act),
    # query tokens [L_act - T_new, L_act), local context [0, L_act), its own
    # layer's bank, the same k and pos0 -- recorded at the layer_forward boundary
    from oracle import msa_oracle as MO

    T0, append, rounds, k, pos0, n_layers = 5, 2, 3, 2, 2, 2
    L = T0 + append * (rounds - 1)
    layers = [{"QR": _rand((1, L, 2, 4), 200 + 4 * li), "Q": _rand((1, L, 4, 4), 201 + 4 * li),
               "K_loc": _rand((1, L, 2, 4), 202 + 4 * li), "V_loc": _rand((1, L, 2, 4), 203 + 4 * li)}
              for li in range(n_layers)]
    banks = [_bank(210 + li, [3, 5, 2, 7], 2, 4, chunk=2) for li in range(n_layers)]
    for li, b in enumerate(banks):
        b["krbar"] = _rand((b["kbar"].shape[1], 2, 4), 220 + li)
    calls = []
    real = MO.layer_forward

    def spy(QR, Q, K_loc, V_loc, bank, k_, pos0_, scale=None, base=10000.0):
        calls.append((QR, Q, K_loc, V_loc, bank, k_, pos0_))
        return real(QR, Q, K_loc, V_loc, bank, k_, pos0_, scale, base)

    monkeypatch.setattr(MO, "layer_forward", spy)
    out = MO.interleave(layers, banks, T0, append, rounds, k, pos0)
    assert len(calls) == rounds * n_layers
    for r in range(rounds):
        L_act, T_new = T0 + append * r, (T0 if r == 0 else append)
        for li in range(n_layers):
            QR, Q, K_loc, V_loc, bank, k_, pos0_ = calls[r * n_layers + li]
            inp = layers[li]
            assert np.array_equal(QR, inp["QR"][:, :L_act]), (r, li)
            assert np.array_equal(Q, inp["Q"][:, L_act - T_new:L_act]), (r, li)
            assert np.array_equal(K_loc, inp["K_loc"][:, :L_act]) and np.array_equal(V_loc, inp["V_loc"][:, :L_act])
            assert bank is banks[li] and k_ == k and pos0_ == pos0
            assert out[r][li]["O"].shape == (1, T_new, 4, 4)


def test_interleave_rounds_equal_one_causal_prefill_on_their_selection():
    # positions continue across rounds: the tokens new in round r, attended over
    # that round's selection, equal the same rows of one causal prefill of all
    # L_act tokens (local token s at position pos0 + s in both) -- a token
    # placed at pos0 + t of its round, or seeing only the new tokens' local
    # keys, would differ
    T0, append, rounds, k, pos0 = 4, 3, 3, 2, 2
    L = T0 + append * (rounds - 1)
    inp = {"QR": _rand((1, L, 2, 4), 230), "Q": _rand((1, L, 4, 4), 231),
           "K_loc": _rand((1, L, 2, 4), 232), "V_loc": _rand((1, L, 2, 4), 233)}
    bank = _bank(234, [3, 5, 2, 7, 4], 2, 4, chunk=2)
    bank["krbar"] = _rand((bank["kbar"].shape[1], 2, 4), 235)
    out = O.interleave([inp], [bank], T0, append, rounds, k, pos0)
    for r in range(rounds):
        L_act, T_new = T0 + append * r, (T0 if r == 0 else append)
        idx = out[r][0]["idx"]
        full = O.attend(inp["Q"][:, :L_act], inp["K_loc"][:, :L_act], inp["V_loc"][:, :L_act], bank["kbar"],
                        bank["vbar"], bank["doc_chunk_off"], idx, pos0)
        assert np.allclose(out[r][0]["O"], full[:, L_act - T_new:], atol=1e-13, rtol=0), r
        # and the selection is the top-k of the routing over all L_act tokens
        s = O.doc_scores(O.chunk_scores(inp["QR"][:, :L_act], bank["krbar"]), bank["doc_chunk_off"])
        assert np.array_equal(idx, O.topk(s, k)["idx"]), r
