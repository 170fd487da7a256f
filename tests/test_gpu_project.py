"""Router projection (Q^R = x W_QR^T, K^R = h W_KR^T) on the GPU against the
fp64 oracle, and the routed path with a router twice the head width
(h_r = 4 x d_r = 256) fed by it.

Tolerance of the projection (written here, applied elementwise): with
gamma = n u / (1 - n u), u = 2^-24 and n = hidden terms, the fp32 sum is
within gamma * sum_i |x_i w_i| of the exact value and the bf16 rounding adds
at most half a bf16 spacing:
    |Y - exact| <= gamma * sum_i |x_i w_i| + 0.5 * spacing(|exact| + gamma * sum_i |x_i w_i|)
Router scores on the projected inputs: |gpu - oracle| <= 2e-3.
"""
import numpy as np
import pytest
import torch

import oracle as O
from synth import rng, workloads as W
from long_context_memory_msa_amd import _lib as L, memory as M

from gpu_common import bf16_spacing, dev, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _project_gpu(X, Wt, device):
    rows, hidden = X.shape
    out = Wt.shape[0]
    Y = torch.empty((rows, out), dtype=torch.bfloat16, device=device)
    L.msa_router_project(dev(X, "bf16", device), dev(Wt, "bf16", device), rows, hidden, out, Y)
    torch.cuda.synchronize()
    return host(Y)


def _check_projection(X, Wt, Y):
    exact = O.project(X, Wt)
    n = X.shape[1]
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    mag = np.abs(X.astype(np.float64)) @ np.abs(Wt.astype(np.float64)).T
    tol = gamma * mag + 0.5 * bf16_spacing(np.abs(exact) + gamma * mag)
    err = np.abs(Y - exact)
    assert np.all(err <= tol), f"max excess {np.max(err - tol):.3g}"


# rows <= 64 take the skinny kernel (1-4 row tiles, K split over 8 waves, batches of
# 4 or 8 k-steps with a ragged last batch); more rows take the 128 x 128 tiles, and
# from 1024 rows with outputs a multiple of 256 the 256 x 256 tiles (ragged last
# row tile: 1025, 4099)
@pytest.mark.parametrize("rows,hidden,out", [(1, 64, 128), (16, 2560, 1024), (17, 192, 128), (33, 320, 256),
                                             (48, 2560, 1024), (64, 704, 384), (65, 2560, 1024), (200, 640, 256),
                                             (1000, 128, 384), (1025, 128, 512), (2048, 320, 768),
                                             (2000, 192, 384), (4099, 2560, 1024)])
def test_project_isolated(device, rows, hidden, out):
    log(f"project rows={rows} hidden={hidden} out={out}")
    X = W.hidden_states(3, rng.ROLE_HID_MEM, rows, hidden)
    Wt = W.projector_weights(3, rng.ROLE_W_KR, hidden, out)
    Y = _project_gpu(X, Wt, device)
    _check_projection(X, Wt, Y)


def test_projected_route_router_twice_head_width(device):
    # memory-token hidden states -> K^R per token -> pooled bank with h_r = 4 x d_r = 256;
    # query hidden states -> Q^R; route and document reduction against the oracle
    w = W.make_workload("prefill-16k")                      # 32 documents x 512 tokens, chunk 128, bf16
    hidden, h_r, d_r, t_r = 640, 4, 256, 48
    n_q = 2
    log(f"projected route: {w.n_tok} tokens, hidden={hidden}, router {h_r} x {d_r}, t_r={t_r}")
    Hm = W.hidden_states(w.seed, rng.ROLE_HID_MEM, w.n_tok, hidden)
    Hq = W.hidden_states(w.seed, rng.ROLE_HID_Q, n_q * t_r, hidden)
    Wkr = W.projector_weights(w.seed, rng.ROLE_W_KR, hidden, h_r * d_r)
    Wqr = W.projector_weights(w.seed, rng.ROLE_W_QR, hidden, h_r * d_r)
    KR_gpu = _project_gpu(Hm, Wkr, device)
    QR_gpu = _project_gpu(Hq, Wqr, device)
    _check_projection(Hm, Wkr, KR_gpu)
    _check_projection(Hq, Wqr, QR_gpu)
    # oracle side: the same projections, stored in bf16 (R10)
    KR_o = O.round_bf16(O.project(Hm, Wkr)).reshape(w.n_tok, h_r, d_r)
    QR_o = O.round_bf16(O.project(Hq, Wqr)).reshape(n_q, t_r, h_r, d_r)
    zeros = np.zeros((w.n_tok, 1, 64), np.float32)
    ob = O.pool(w.doc_lens, w.chunk, zeros, zeros, KR_o, "bf16")
    S = O.chunk_scores(QR_o, ob["krbar"])
    sd = O.doc_scores(S, ob["doc_chunk_off"])
    # GPU side: projection -> pooling -> scan, never leaving the device
    bank = M.Bank(w.doc_lens, w.chunk, 1, 64, h_r, d_r, "bf16", device)
    rope = M.Rope(w.max_pos, 64, w.rope_base, device)
    X = dev(Hm, "bf16", device)
    KRd = torch.empty((w.n_tok, h_r, d_r), dtype=torch.bfloat16, device=device)
    L.msa_router_project(X, dev(Wkr, "bf16", device), w.n_tok, hidden, h_r * d_r, KRd)
    z = torch.zeros((w.n_tok, 1, 64), dtype=torch.bfloat16, device=device)
    bank.pool(z, z, KRd, 0, w.n_docs, rope)
    QRd = torch.empty((n_q, t_r, h_r, d_r), dtype=torch.bfloat16, device=device)
    L.msa_router_project(dev(Hq, "bf16", device), dev(Wqr, "bf16", device), n_q * t_r, hidden, h_r * d_r, QRd)
    s_doc = torch.empty((n_q, w.n_docs), dtype=torch.float32, device=device)
    s_chunk = torch.empty((n_q, w.n_chunks), dtype=torch.float32, device=device)
    nb = L.msa_route_workspace_bytes(bank.c, n_q, t_r)
    ws = M.workspace(nb, device)
    L.msa_route_score(bank.c, QRd, n_q, t_r, s_doc, s_chunk, ws, nb)
    torch.cuda.synchronize()
    assert np.abs(host(s_chunk) - S).max() <= 2e-3
    assert np.abs(host(s_doc) - sd).max() <= 2e-3
    # the stored router keys: each token's key is within one bf16 spacing (plus
    # the fp32 sum bound) of the oracle's stored one, so the chunk means are
    # within the mean of those bounds, plus one spacing for each side's rounding
    n = hidden
    gamma = n * 2.0 ** -24 / (1 - n * 2.0 ** -24)
    mag = (np.abs(Hm.astype(np.float64)) @ np.abs(Wkr.astype(np.float64)).T).reshape(w.n_tok, h_r, d_r)
    tok_bound = bf16_spacing(KR_o) + gamma * mag
    mean_bound = O.pool(w.doc_lens, w.chunk, zeros, zeros, tok_bound, "f32")["krbar"]
    kb = host(bank.krbar)
    assert np.all(np.abs(kb - ob["krbar"]) <= bf16_spacing(ob["krbar"]) + mean_bound)
