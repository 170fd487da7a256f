"""Device memory plumbing for the C ABI: a pooled bank and RoPE tables held in
torch tensors (torch allocates; the kernels compute).

A bank keeps, per routed layer ([HD] core architecture of the memory routing
layer): pooled keys/values [h_kv][n_chunks][d], pooled router keys
[n_chunks][h_r][d_r], their inverse norms and the document layout.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
ABI_DTYPE = {"f32": _lib.MSA_F32, "bf16": _lib.MSA_BF16}


class Rope:
    """cos/sin tables [max_pos][d/2] fp32, filled by msa_rope_table on the device."""

    def __init__(self, max_pos: int, d: int, base: float = 10000.0, device="cuda", stream=None):
        self.cos = torch.empty((max_pos, d // 2), dtype=torch.float32, device=device)
        self.sin = torch.empty((max_pos, d // 2), dtype=torch.float32, device=device)
        _lib.msa_rope_table(self.cos, self.sin, max_pos, d, base, stream)
        self.c = _lib.MsaRope(self.cos.data_ptr(), self.sin.data_ptr(), max_pos, d)


class Bank:
    """Pooled memory bank of one routed layer, resident in HBM."""

    def __init__(self, doc_lens: Sequence[int], chunk: int, h_kv: int, d: int, h_r: int, d_r: int, dtype: str,
                 device="cuda"):
        lay = _lib.msa_bank_layout(doc_lens, chunk)
        self.dtype = dtype
        self.layout = lay
        self.n_docs = len(doc_lens)
        self.n_chunks = lay["n_chunks"]
        td = TORCH_DTYPE[dtype]
        self.doc_tok_off_host = np.ascontiguousarray(lay["doc_tok_off"])
        self.doc_chunk_off_host = np.ascontiguousarray(lay["doc_chunk_off"])
        self.doc_tok_off = torch.from_numpy(self.doc_tok_off_host).to(device)
        self.doc_chunk_off = torch.from_numpy(self.doc_chunk_off_host).to(device)
        self.chunk_doc = torch.empty(self.n_chunks, dtype=torch.int32, device=device)
        self.kbar = torch.empty((h_kv, self.n_chunks, d), dtype=td, device=device)
        self.vbar = torch.empty((h_kv, self.n_chunks, d), dtype=td, device=device)
        self.krbar = torch.empty((self.n_chunks, h_r, d_r), dtype=td, device=device)
        self.kr_inv_norm = torch.empty((self.n_chunks, h_r), dtype=torch.float32, device=device)
        self.c = _lib.MsaBank(
            ABI_DTYPE[dtype], self.n_docs, chunk, h_kv, d, h_r, d_r, lay["max_doc_len"], lay["max_doc_chunks"], 0,
            self.n_chunks, self.doc_tok_off.data_ptr(), self.doc_chunk_off.data_ptr(),
            self.doc_tok_off_host.ctypes.data, self.doc_chunk_off_host.ctypes.data, self.chunk_doc.data_ptr(),
            self.kbar.data_ptr(), self.vbar.data_ptr(), self.krbar.data_ptr(), self.kr_inv_norm.data_ptr())

    def pool(self, K, V, KR, doc_begin: int, doc_end: int, rope: Rope, stream=None) -> None:
        """Offline pooling of documents [doc_begin, doc_end) from a token slab."""
        _lib.msa_pool_memory(self.c, K, V, KR, doc_begin, doc_end, rope.c, stream)

    def bytes_resident(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.kbar, self.vbar, self.krbar, self.kr_inv_norm, self.chunk_doc, self.doc_tok_off,
                    self.doc_chunk_off))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A device byte buffer of at least ``nbytes`` (256-byte aligned by torch)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
