"""ctypes binding of libmsa (include/msa.h): argument marshalling only.

Every function here forwards device pointers (torch tensors' ``data_ptr()``)
and sizes to the C ABI; all computation runs in the HIP kernels.  There is no
fallback: if the library cannot be loaded, importing this module raises.
"""
from __future__ import annotations

import ctypes
import math
from pathlib import Path
from typing import Optional, Sequence

import numpy as np

_HERE = Path(__file__).resolve().parent
LIB_PATH = _HERE / "libmsa.so"

MSA_OK, MSA_ERR_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE, MSA_ERR_DEVICE = range(5)
MSA_F32, MSA_BF16 = 0, 1


class MsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"msa error {code}: {msg}")
        self.code = code


class MsaRope(ctypes.Structure):
    _fields_ = [("cos", ctypes.c_void_p), ("sin", ctypes.c_void_p), ("max_pos", ctypes.c_int32),
                ("d", ctypes.c_int32)]


class MsaBank(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("n_docs", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("h_kv", ctypes.c_int32), ("d", ctypes.c_int32), ("h_r", ctypes.c_int32), ("d_r", ctypes.c_int32),
                ("max_doc_len", ctypes.c_int32), ("max_doc_chunks", ctypes.c_int32), ("chunk_cap", ctypes.c_int32),
                ("kv_host", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("n_chunks", ctypes.c_int64),
                ("doc_tok_off", ctypes.c_void_p), ("doc_chunk_off", ctypes.c_void_p),
                ("doc_tok_off_host", ctypes.c_void_p), ("doc_chunk_off_host", ctypes.c_void_p),
                ("chunk_doc", ctypes.c_void_p), ("kbar", ctypes.c_void_p), ("vbar", ctypes.c_void_p),
                ("krbar", ctypes.c_void_p), ("kr_inv_norm", ctypes.c_void_p)]


ABI_VERSION = 3  # include/msa.h MSA_ABI_VERSION


def _load():
    # torch ships its own HIP runtime: load it first so that libmsa binds to the
    # same runtime instance as torch's streams and allocations (one runtime per
    # process; a second copy would not see torch's streams).
    import torch  # noqa: F401
    if not LIB_PATH.exists():
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(str(LIB_PATH))
    P, I32, I64, SZ, D, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_double, ctypes.c_float
    bank_p, rope_p = ctypes.POINTER(MsaBank), ctypes.POINTER(MsaRope)
    sig = {
        "msa_abi_version": ([], ctypes.c_int),
        "msa_last_error": ([], ctypes.c_char_p),
        "msa_device_pointer": ([P, P], ctypes.c_int),
        "msa_router_project": ([P, P, I64, I32, I32, P, P], ctypes.c_int),
        "msa_bank_layout": ([P, I32, I32, P, P, P, P, P], ctypes.c_int),
        "msa_rope_table": ([P, P, I32, I32, D, P], ctypes.c_int),
        "msa_pool_memory": ([bank_p, P, P, P, I32, I32, rope_p, P], ctypes.c_int),
        "msa_route_workspace_bytes": ([bank_p, I32, I32], SZ),
        "msa_route_score": ([bank_p, P, I32, I32, P, P, P, SZ, I32, P], ctypes.c_int),
        "msa_topk_workspace_bytes": ([I32, I32, I32], SZ),
        "msa_topk": ([P, I32, I32, I32, P, P, P, SZ, P], ctypes.c_int),
        "msa_attend_workspace_bytes": ([bank_p, I32, I32, I32, I32, I32], SZ),
        "msa_sparse_attend": ([bank_p, P, P, P, I32, I32, I32, I32, P, I32, I32, F, rope_p, P, P, SZ, P],
                              ctypes.c_int),
        "msa_layer_workspace_bytes": ([bank_p, I32, I32, I32, I32, I32, I32], SZ),
        "msa_layer_forward": ([bank_p, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, F, rope_p, P, P, P, P, P, SZ,
                               P, P], ctypes.c_int),
        "msa_layer_forward_reroute": ([bank_p, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, F, rope_p, P, P, P, P, P,
                                       P, SZ, P, P], ctypes.c_int),
        "msa_layer_forward_noalloc": ([bank_p, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, F, rope_p, P, P, P, P,
                                       P, P], ctypes.c_int),
        "msa_scan_read_probe": ([bank_p, P, SZ, P], ctypes.c_int),
        "msa_layer_route": ([bank_p, P, I32, I32, I32, I32, I32, I32, P, P, SZ, P], ctypes.c_int),
        "msa_layer_select_attend": ([bank_p, P, P, P, I32, I32, I32, I32, I32, I32, I32, F, rope_p, P, P, P, P, P, SZ,
                                     P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if lib.msa_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} implements ABI {lib.msa_abi_version()}, this binding ABI {ABI_VERSION}: rebuild it")
    return lib


_lib = _load()


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int) -> None:
    if rc != MSA_OK:
        raise MsaError(rc, _lib.msa_last_error().decode())


# ---------------------------------------------------------------------------
def msa_abi_version() -> int:
    return _lib.msa_abi_version()


def msa_device_pointer(host_ptr: int) -> int:
    """Device address of pinned, device-mapped host memory (a torch tensor made
    with pin_memory=True is one)."""
    out = ctypes.c_void_p()
    _check(_lib.msa_device_pointer(ctypes.c_void_p(host_ptr), ctypes.byref(out)))
    return int(out.value)


def msa_last_error() -> str:
    return _lib.msa_last_error().decode()


def msa_bank_layout(doc_lens: Sequence[int], chunk: int) -> dict:
    """Host layout of a bank (prefix offsets, n_chunks, max lengths)."""
    lens = np.ascontiguousarray(doc_lens, dtype=np.int64)
    n = lens.shape[0]
    tok = np.empty(n + 1, dtype=np.int64)
    ch = np.empty(n + 1, dtype=np.int64)
    nc = ctypes.c_int64()
    ml = ctypes.c_int32()
    mc = ctypes.c_int32()
    _check(_lib.msa_bank_layout(lens.ctypes.data, n, chunk, tok.ctypes.data, ch.ctypes.data, ctypes.byref(nc),
                                ctypes.byref(ml), ctypes.byref(mc)))
    return {"doc_tok_off": tok, "doc_chunk_off": ch, "n_chunks": nc.value, "max_doc_len": ml.value,
            "max_doc_chunks": mc.value}


def msa_rope_table(cos, sin, max_pos: int, d: int, base: float = 10000.0, stream=None) -> None:
    _check(_lib.msa_rope_table(_ptr(cos), _ptr(sin), max_pos, d, base, _stream(stream)))


def msa_pool_memory(bank: MsaBank, K, V, KR, doc_begin: int, doc_end: int, rope: MsaRope, stream=None) -> None:
    _check(_lib.msa_pool_memory(ctypes.byref(bank), _ptr(K), _ptr(V), _ptr(KR), doc_begin, doc_end,
                                ctypes.byref(rope), _stream(stream)))


def msa_router_project(X, W, rows: int, hidden: int, out: int, Y, stream=None) -> None:
    _check(_lib.msa_router_project(_ptr(X), _ptr(W), rows, hidden, out, _ptr(Y), _stream(stream)))


def msa_route_workspace_bytes(bank: MsaBank, n_q: int, t_r: int) -> int:
    return _lib.msa_route_workspace_bytes(ctypes.byref(bank), n_q, t_r)


def msa_route_score(bank: MsaBank, QR, n_q: int, t_r: int, s_doc, s_chunk=None, ws=None, ws_bytes: int = 0,
                    stream=None, max_wg_per_cu: int = 0) -> None:
    _check(_lib.msa_route_score(ctypes.byref(bank), _ptr(QR), n_q, t_r, _ptr(s_doc), _ptr(s_chunk), _ptr(ws),
                                ws_bytes, max_wg_per_cu, _stream(stream)))


def msa_topk_workspace_bytes(n_q: int, n_docs: int, k: int) -> int:
    return _lib.msa_topk_workspace_bytes(n_q, n_docs, k)


def msa_topk(s_doc, n_q: int, n_docs: int, k: int, idx, val, ws, ws_bytes: int, stream=None) -> None:
    _check(_lib.msa_topk(_ptr(s_doc), n_q, n_docs, k, _ptr(idx), _ptr(val), _ptr(ws), ws_bytes, _stream(stream)))


def msa_attend_workspace_bytes(bank: MsaBank, n_q: int, T: int, L_loc: int, h_q: int, k: int) -> int:
    return _lib.msa_attend_workspace_bytes(ctypes.byref(bank), n_q, T, L_loc, h_q, k)


def msa_sparse_attend(bank: MsaBank, Q, K_loc, V_loc, n_q: int, T: int, L_loc: int, h_q: int, idx, k: int,
                      pos0: int, scale: float, rope: MsaRope, O, ws, ws_bytes: int, stream=None) -> None:
    _check(_lib.msa_sparse_attend(ctypes.byref(bank), _ptr(Q), _ptr(K_loc), _ptr(V_loc), n_q, T, L_loc, h_q,
                                  _ptr(idx), k, pos0, scale, ctypes.byref(rope), _ptr(O), _ptr(ws), ws_bytes,
                                  _stream(stream)))


def msa_layer_workspace_bytes(bank: MsaBank, n_q: int, T: int, t_r: int, L_loc: int, h_q: int, k: int) -> int:
    return _lib.msa_layer_workspace_bytes(ctypes.byref(bank), n_q, T, t_r, L_loc, h_q, k)


def msa_layer_forward(bank: MsaBank, Q, K_loc, V_loc, QR, n_q: int, T: int, t_r: int, L_loc: int, h_q: int, k: int,
                      pos0: int, scale: float, rope: MsaRope, O, idx, val, s_doc, ws, ws_bytes: int,
                      stage_events: Optional[Sequence[int]] = None, stream=None) -> None:
    ev = None
    if stage_events is not None:
        ev = (ctypes.c_void_p * 4)(*stage_events)
    _check(_lib.msa_layer_forward(ctypes.byref(bank), _ptr(Q), _ptr(K_loc), _ptr(V_loc), _ptr(QR), n_q, T, t_r,
                                  L_loc, h_q, k, pos0, scale, ctypes.byref(rope), _ptr(O), _ptr(idx), _ptr(val),
                                  _ptr(s_doc), _ptr(ws), ws_bytes, ev, _stream(stream)))


def msa_layer_forward_reroute(bank: MsaBank, Q, K_loc, V_loc, QR_new, n_q: int, T: int, t_new: int, L_loc: int,
                              h_q: int, k: int, pos0: int, scale: float, rope: MsaRope, s_doc_prev, O, idx, val, s_doc,
                              ws, ws_bytes: int, stage_events: Optional[Sequence[int]] = None, stream=None) -> None:
    ev = None
    if stage_events is not None:
        ev = (ctypes.c_void_p * 4)(*stage_events)
    _check(_lib.msa_layer_forward_reroute(ctypes.byref(bank), _ptr(Q), _ptr(K_loc), _ptr(V_loc), _ptr(QR_new), n_q,
                                          T, t_new, L_loc, h_q, k, pos0, scale, ctypes.byref(rope), _ptr(s_doc_prev),
                                          _ptr(O), _ptr(idx), _ptr(val), _ptr(s_doc), _ptr(ws), ws_bytes, ev,
                                          _stream(stream)))


STATIC_WORKSPACE_BYTES = 16 << 20  # include/msa.h MSA_STATIC_WORKSPACE_BYTES


def msa_layer_forward_noalloc(bank: MsaBank, Q, K_loc, V_loc, QR, n_q: int, T: int, t_r: int, L_loc: int, h_q: int,
                              k: int, pos0: int, scale: float, rope: MsaRope, O, idx, val, s_doc,
                              stage_events: Optional[Sequence[int]] = None, stream=None) -> None:
    ev = None
    if stage_events is not None:
        ev = (ctypes.c_void_p * 4)(*stage_events)
    _check(_lib.msa_layer_forward_noalloc(ctypes.byref(bank), _ptr(Q), _ptr(K_loc), _ptr(V_loc), _ptr(QR), n_q, T,
                                          t_r, L_loc, h_q, k, pos0, scale, ctypes.byref(rope), _ptr(O), _ptr(idx),
                                          _ptr(val), _ptr(s_doc), ev, _stream(stream)))


def msa_scan_read_probe(bank: MsaBank, ws, ws_bytes: int, stream=None) -> None:
    _check(_lib.msa_scan_read_probe(ctypes.byref(bank), _ptr(ws), ws_bytes, _stream(stream)))


def msa_layer_route(bank: MsaBank, QR, n_q: int, T: int, t_r: int, L_loc: int, h_q: int, k: int, s_doc, ws,
                    ws_bytes: int, stream=None) -> None:
    _check(_lib.msa_layer_route(ctypes.byref(bank), _ptr(QR), n_q, T, t_r, L_loc, h_q, k, _ptr(s_doc), _ptr(ws),
                                ws_bytes, _stream(stream)))


def msa_layer_select_attend(bank: MsaBank, Q, K_loc, V_loc, n_q: int, T: int, t_r: int, L_loc: int, h_q: int, k: int,
                            pos0: int, scale: float, rope: MsaRope, O, idx, val, s_doc, ws, ws_bytes: int,
                            stream=None) -> None:
    _check(_lib.msa_layer_select_attend(ctypes.byref(bank), _ptr(Q), _ptr(K_loc), _ptr(V_loc), n_q, T, t_r, L_loc,
                                        h_q, k, pos0, scale, ctypes.byref(rope), _ptr(O), _ptr(idx), _ptr(val),
                                        _ptr(s_doc), _ptr(ws), ws_bytes, _stream(stream)))


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
