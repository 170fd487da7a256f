"""The C ABI on the CPU: the library loads, exports every entry point that
include/msa.h declares, and rejects invalid arguments on the host (with a
message, before any HIP call) -- no GPU needed."""
import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

import long_context_memory_msa_amd as msa
from long_context_memory_msa_amd import _lib as L

ROOT = Path(__file__).resolve().parents[1]


def declared_symbols():
    text = (ROOT / "include" / "msa.h").read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) >= 12
    lib = ctypes.CDLL(str(L.LIB_PATH))
    for n in names:
        assert hasattr(lib, n), n
        assert hasattr(L, n), f"binding lacks {n}"


def test_abi_version_and_empty_error():
    assert msa.msa_abi_version() == 3
    msa.msa_bank_layout([3], 2)
    assert msa.msa_last_error() == ""


def test_bank_layout_host_helper():
    lens = np.array([5, 128, 129, 1, 300])
    lay = msa.msa_bank_layout(lens, 128)
    assert lay["doc_tok_off"].tolist() == [0, 5, 133, 262, 263, 563]
    assert lay["doc_chunk_off"].tolist() == [0, 1, 2, 4, 5, 8]
    assert lay["n_chunks"] == 8 and lay["max_doc_len"] == 300 and lay["max_doc_chunks"] == 3
    for bad_lens, chunk in (([3, 0, 2], 4), ([], 4), ([4], 0)):
        with pytest.raises(msa.MsaError) as e:
            msa.msa_bank_layout(bad_lens, chunk)
        assert e.value.code == L.MSA_ERR_ARG


class _Fake:
    """Stands in for a device tensor: only its address is ever read."""

    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


A = _Fake(0x10000)      # 16-byte aligned, never dereferenced (validation fails first)
MIS = _Fake(0x10004)    # misaligned


def _bank(**over):
    lay = msa.msa_bank_layout([512] * 4, 128)
    b = L.MsaBank(L.MSA_BF16, 4, 128, 8, 128, 8, 128, 512, 4, 0, 0, 0, lay["n_chunks"], A.addr, A.addr, None, None,
                  A.addr, A.addr, A.addr, A.addr, A.addr)
    for k, v in over.items():
        setattr(b, k, v)
    return b


def _rope(**over):
    r = L.MsaRope(A.addr, A.addr, 4096, 128)
    for k, v in over.items():
        setattr(r, k, v)
    return r


def _code(fn, *a, **kw):
    with pytest.raises(msa.MsaError) as e:
        fn(*a, **kw)
    assert msa.msa_last_error() != ""
    return e.value.code


def test_rope_table_validation():
    assert _code(msa.msa_rope_table, None, A, 16, 128, 1e4, 0) == L.MSA_ERR_ARG
    assert _code(msa.msa_rope_table, A, A, 16, 96, 1e4, 0) == L.MSA_ERR_UNSUPPORTED
    assert _code(msa.msa_rope_table, A, A, 0, 128, 1e4, 0) == L.MSA_ERR_ARG
    assert _code(msa.msa_rope_table, A, A, 16, 128, -1.0, 0) == L.MSA_ERR_ARG


def test_bank_validation():
    for over, code in (({"dtype": 7}, L.MSA_ERR_UNSUPPORTED), ({"d": 96}, L.MSA_ERR_UNSUPPORTED),
                       ({"h_r": 3}, L.MSA_ERR_UNSUPPORTED), ({"n_docs": 0}, L.MSA_ERR_ARG),
                       ({"max_doc_chunks": 9}, L.MSA_ERR_ARG), ({"kbar": None}, L.MSA_ERR_ARG),
                       ({"krbar": MIS.addr}, L.MSA_ERR_ARG), ({"n_chunks": 1}, L.MSA_ERR_ARG),
                       ({"chunk_cap": 15}, L.MSA_ERR_ARG), ({"chunk_cap": -1}, L.MSA_ERR_ARG),
                       ({"d_r": 256, "h_r": 4, "dtype": L.MSA_F32}, L.MSA_ERR_UNSUPPORTED),
                       ({"d_r": 256}, L.MSA_ERR_UNSUPPORTED), ({"d_r": 512, "h_r": 2}, L.MSA_ERR_UNSUPPORTED)):
        assert _code(msa.msa_route_score, _bank(**over), A, 1, 1, A, None, A, 1 << 30, stream=0) == code, over


def test_bank_capacity_host_side():
    # a bank with room for later documents: offsets and counts grow, capacity fixed
    import torch
    lens = [300, 129, 1]
    from long_context_memory_msa_amd.memory import Bank
    b = Bank(lens, 128, 2, 64, 2, 64, "f32", device="cpu", cap_docs=6, cap_chunks=12)
    assert (b.n_docs, b.n_chunks, b.c.chunk_cap) == (3, 6, 12)
    assert tuple(b.kbar.shape) == (2, 12, 64) and tuple(b.krbar.shape) == (12, 2, 64)
    assert b.append([128, 500]) == (3, 5)
    assert (b.n_docs, b.n_chunks, b.c.n_docs, b.c.n_chunks) == (5, 11, 5, 11)
    assert b.doc_lens.tolist() == [300, 129, 1, 128, 500]
    assert b.doc_chunk_off_host[:6].tolist() == [0, 3, 5, 6, 7, 11]
    assert b.doc_tok_off.tolist()[:6] == [0, 300, 429, 430, 558, 1058]
    assert (b.c.max_doc_len, b.c.max_doc_chunks) == (500, 4)
    assert b.append([]) == (5, 5)
    with pytest.raises(ValueError):
        b.append([129])          # 2 more chunks > capacity 12
    with pytest.raises(msa.MsaError) as e:
        b.append([0])            # lengths are validated by the library's layout helper
    assert e.value.code == L.MSA_ERR_ARG and (b.n_docs, b.n_chunks) == (5, 11)
    assert isinstance(b.kbar, torch.Tensor)


def test_router_project_validation():
    ok = dict(X=A, W=A, rows=16, hidden=640, out=1024, Y=A)

    def call(**over):
        a = {**ok, **over}
        return _code(msa.msa_router_project, a["X"], a["W"], a["rows"], a["hidden"], a["out"], a["Y"], 0)

    assert call(X=None) == L.MSA_ERR_ARG
    assert call(Y=MIS) == L.MSA_ERR_ARG
    assert call(rows=-1) == L.MSA_ERR_ARG
    assert call(hidden=100) == L.MSA_ERR_ARG      # not a multiple of 64
    assert call(out=200) == L.MSA_ERR_ARG         # not a multiple of 128
    assert call(hidden=0) == L.MSA_ERR_ARG


def test_route_validation():
    assert _code(msa.msa_route_score, _bank(), None, 1, 1, A, None, A, 1 << 30, stream=0) == L.MSA_ERR_ARG
    assert _code(msa.msa_route_score, _bank(), A, 0, 1, A, None, A, 1 << 30, stream=0) == L.MSA_ERR_ARG
    assert _code(msa.msa_route_score, _bank(), A, 1, 0, A, None, A, 1 << 30, stream=0) == L.MSA_ERR_ARG
    assert _code(msa.msa_route_score, _bank(), MIS, 1, 1, A, None, A, 1 << 30, stream=0) == L.MSA_ERR_ARG
    assert _code(msa.msa_route_score, _bank(), A, 1, 1, None, None, A, 1 << 30, stream=0) == L.MSA_ERR_ARG
    assert _code(msa.msa_route_score, _bank(), A, 1, 1, A, None, A, 1 << 30, stream=0,
                 max_wg_per_cu=-1) == L.MSA_ERR_ARG


def test_topk_validation_and_workspace():
    assert msa.msa_topk_workspace_bytes(2, 5000, 16) == 0                 # one pass per query
    assert msa.msa_topk_workspace_bytes(2, 20000, 16) == 2 * 40 * 16 * 8    # k <= 32: 512-document slices
    assert msa.msa_topk_workspace_bytes(2, 20000, 64) == 2 * 10 * 64 * 8    # larger k: 2048-document slices
    assert msa.msa_topk_workspace_bytes(1, 10, 11) == 0
    assert _code(msa.msa_topk, A, 1, 10, 11, A, A, A, 1 << 20, 0) == L.MSA_ERR_ARG      # k > n_docs
    assert _code(msa.msa_topk, A, 1, 1000, 257, A, A, A, 1 << 20, 0) == L.MSA_ERR_ARG   # k > 256
    assert _code(msa.msa_topk, A, 1, 1000, 0, A, A, A, 1 << 20, 0) == L.MSA_ERR_ARG
    assert _code(msa.msa_topk, A, 1, 20000, 16, A, A, A, 100, 0) == L.MSA_ERR_WORKSPACE
    assert _code(msa.msa_topk, A, 1, 20000, 16, A, A, None, 1 << 20, 0) == L.MSA_ERR_WORKSPACE


def test_attend_validation():
    b = _bank()
    ok = dict(Q=A, K_loc=A, V_loc=A, n_q=1, T=4, L_loc=8, h_q=32, idx=A, k=2, pos0=2, scale=0.1, rope=_rope(),
              O=A, ws=A, ws_bytes=1 << 30)

    def call(**over):
        a = {**ok, **over}
        return _code(msa.msa_sparse_attend, b, a["Q"], a["K_loc"], a["V_loc"], a["n_q"], a["T"], a["L_loc"], a["h_q"],
                     a["idx"], a["k"], a["pos0"], a["scale"], a["rope"], a["O"], a["ws"], a["ws_bytes"], 0)

    assert call(T=9) == L.MSA_ERR_ARG                     # T > L_loc
    assert call(h_q=12) == L.MSA_ERR_ARG                  # not a multiple of h_kv
    assert call(k=5) == L.MSA_ERR_ARG                     # k > n_docs
    assert call(Q=None) == L.MSA_ERR_ARG
    assert call(O=MIS) == L.MSA_ERR_ARG
    assert call(scale=float("nan")) == L.MSA_ERR_ARG
    assert call(rope=_rope(max_pos=9)) == L.MSA_ERR_ARG   # pos0 + L_loc = 10 > 9
    assert call(rope=_rope(d=64)) == L.MSA_ERR_ARG
    assert call(idx=None) == L.MSA_ERR_ARG
    assert msa.msa_attend_workspace_bytes(b, 1, 9, 8, 32, 2) == 0


def test_pool_validation():
    lay = msa.msa_bank_layout([512] * 4, 128)
    tok, ch = lay["doc_tok_off"], lay["doc_chunk_off"]
    b = _bank(doc_tok_off_host=tok.ctypes.data, doc_chunk_off_host=ch.ctypes.data)
    r = _rope(max_pos=512)
    assert _code(msa.msa_pool_memory, b, A, A, A, 0, 5, r, 0) == L.MSA_ERR_ARG          # range beyond n_docs
    assert _code(msa.msa_pool_memory, b, A, A, A, 2, 1, r, 0) == L.MSA_ERR_ARG
    assert _code(msa.msa_pool_memory, b, None, A, A, 0, 1, r, 0) == L.MSA_ERR_ARG
    assert _code(msa.msa_pool_memory, _bank(), A, A, A, 0, 1, r, 0) == L.MSA_ERR_ARG    # no host offsets
    assert _code(msa.msa_pool_memory, b, A, A, A, 0, 1, _rope(max_pos=100), 0) == L.MSA_ERR_ARG
    bad = ch.copy()
    bad[2] += 1
    b2 = _bank(doc_tok_off_host=tok.ctypes.data, doc_chunk_off_host=bad.ctypes.data)
    assert _code(msa.msa_pool_memory, b2, A, A, A, 0, 4, r, 0) == L.MSA_ERR_ARG


def test_layer_validation():
    b = _bank()
    r = _rope()
    args = [b, A, A, A, A, 1, 4, 4, 8, 32, 2, 2, 0.1, r, A, A, A, None, A, 1 << 30]
    assert _code(msa.msa_layer_forward, *args[:19], 16, stream=0) == L.MSA_ERR_WORKSPACE
    bad = list(args)
    bad[7] = 0                                              # t_r = 0
    assert _code(msa.msa_layer_forward, *bad, stream=0) == L.MSA_ERR_ARG
    assert _code(msa.msa_layer_forward, *args, stage_events=[A.addr, 0, A.addr, A.addr], stream=0) == L.MSA_ERR_ARG
    assert msa.msa_layer_workspace_bytes(b, 1, 4, 4, 8, 32, 2) > 0


def test_layer_halves_validation():
    # the two halves check the same sizes and the same workspace as the whole layer
    b = _bank()
    r = _rope()
    big = 1 << 30
    route = [b, A, 1, 4, 4, 8, 32, 2, None, A]
    assert _code(msa.msa_layer_route, *route, 16, stream=0) == L.MSA_ERR_WORKSPACE
    assert _code(msa.msa_layer_route, b, None, *route[2:], big, stream=0) == L.MSA_ERR_ARG     # QR
    assert _code(msa.msa_layer_route, b, A, 1, 4, 0, 8, 32, 2, None, A, big, stream=0) == L.MSA_ERR_ARG  # t_r
    assert _code(msa.msa_layer_route, b, A, 1, 9, 4, 8, 32, 2, None, A, big, stream=0) == L.MSA_ERR_ARG  # T > L_loc
    assert _code(msa.msa_layer_route, b, A, 1, 4, 4, 8, 32, 5, None, A, big, stream=0) == L.MSA_ERR_ARG  # k > n_docs
    tail = [b, A, A, A, 1, 4, 4, 8, 32, 2, 2, 0.1, r, A, A, A, None, A]
    assert _code(msa.msa_layer_select_attend, *tail, 16, stream=0) == L.MSA_ERR_WORKSPACE
    bad = list(tail)
    bad[14] = None                                          # idx
    assert _code(msa.msa_layer_select_attend, *bad, big, stream=0) == L.MSA_ERR_ARG
    bad = list(tail)
    bad[12] = _rope(max_pos=4)                              # rope shorter than pos0 + L_loc
    assert _code(msa.msa_layer_select_attend, *bad, big, stream=0) == L.MSA_ERR_ARG


def test_scan_read_probe_validation():
    b = _bank()
    need = msa.msa_route_workspace_bytes(b, 1, 1)
    assert _code(msa.msa_scan_read_probe, b, A, need - 1, stream=0) == L.MSA_ERR_WORKSPACE
    assert _code(msa.msa_scan_read_probe, b, None, need, stream=0) == L.MSA_ERR_WORKSPACE
    assert _code(msa.msa_scan_read_probe, _bank(dtype=L.MSA_F32), A, need, stream=0) == L.MSA_ERR_UNSUPPORTED
    assert _code(msa.msa_scan_read_probe, _bank(h_r=4), A, need, stream=0) == L.MSA_ERR_UNSUPPORTED


def test_rope_tables_must_be_16_byte_aligned():
    # every device buffer of the ABI is 16-byte aligned, the RoPE tables included
    assert _code(msa.msa_rope_table, MIS, A, 16, 128, 1e4, 0) == L.MSA_ERR_ARG
    assert _code(msa.msa_rope_table, A, MIS, 16, 128, 1e4, 0) == L.MSA_ERR_ARG
    lay = msa.msa_bank_layout([512] * 4, 128)
    tok, ch = lay["doc_tok_off"], lay["doc_chunk_off"]
    b = _bank(doc_tok_off_host=tok.ctypes.data, doc_chunk_off_host=ch.ctypes.data)
    assert _code(msa.msa_pool_memory, b, A, A, A, 0, 1, _rope(max_pos=512, cos=MIS.addr), 0) == L.MSA_ERR_ARG
    assert "rope.cos" in msa.msa_last_error()


def test_layer_noalloc_validation():
    # the allocation-free layer validates like msa_layer_forward and refuses a
    # layer whose workspace exceeds the static array, before any device call
    b = _bank()
    r = _rope()
    args = [b, A, A, A, A, 1, 4, 4, 8, 32, 2, 2, 0.1, r, A, A, A, None]
    bad = list(args)
    bad[7] = 0                                              # t_r = 0
    assert _code(msa.msa_layer_forward_noalloc, *bad, stream=0) == L.MSA_ERR_ARG
    bad = list(args)
    bad[4] = None                                           # QR
    assert _code(msa.msa_layer_forward_noalloc, *bad, stream=0) == L.MSA_ERR_ARG
    assert _code(msa.msa_layer_forward_noalloc, *args, stage_events=[A.addr, 0, A.addr, A.addr],
                 stream=0) == L.MSA_ERR_ARG
    # 200,000 documents of 512 tokens and 64 single-token queries: far more than 16 MiB of workspace
    lay = msa.msa_bank_layout([512] * 200_000, 128)
    big = _bank(n_docs=200_000, n_chunks=lay["n_chunks"])
    need = msa.msa_layer_workspace_bytes(big, 64, 1, 1, 1, 32, 16)
    assert need > L.STATIC_WORKSPACE_BYTES
    e = _code(msa.msa_layer_forward_noalloc, big, A, A, A, A, 64, 1, 1, 1, 32, 16, 16, 0.1, r, A, A, A, None, stream=0)
    assert e == L.MSA_ERR_WORKSPACE and "static workspace" in msa.msa_last_error()


def test_layer_reroute_validation():
    # the re-routing layer checks what msa_layer_forward checks, plus its previous scores
    b = _bank()
    r = _rope()
    big = 1 << 30
    args = [b, A, A, A, A, 1, 4, 4, 8, 32, 2, 2, 0.1, r, A, A, A, A, None, A, big]
    msa.msa_layer_forward_reroute  # exported
    bad = list(args)
    bad[14] = None                                          # s_doc_prev
    assert _code(msa.msa_layer_forward_reroute, *bad, stream=0) == L.MSA_ERR_ARG
    bad = list(args)
    bad[14] = _Fake(0x10002)                                # s_doc_prev not 4-byte aligned
    assert _code(msa.msa_layer_forward_reroute, *bad, stream=0) == L.MSA_ERR_ARG
    bad = list(args)
    bad[7] = 0                                              # t_new = 0
    assert _code(msa.msa_layer_forward_reroute, *bad, stream=0) == L.MSA_ERR_ARG
    assert _code(msa.msa_layer_forward_reroute, *args[:20], 16, stream=0) == L.MSA_ERR_WORKSPACE
