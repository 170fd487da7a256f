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
    """Pooled memory bank of one routed layer, resident in HBM.

    ``cap_docs`` / ``cap_chunks`` reserve room for documents appended later
    (``append``): the offset arrays hold cap_docs + 1 entries and the chunk
    arrays cap_chunks rows, so new documents are pooled in place without
    moving the ones already encoded.

    ``kv_host=True`` makes a tiered bank: the pooled keys/values (two thirds
    of the bytes) live in pinned host memory that the GPU reads directly,
    only the router keys, their norms and the layout stay in HBM.
    """

    def __init__(self, doc_lens: Sequence[int], chunk: int, h_kv: int, d: int, h_r: int, d_r: int, dtype: str,
                 device="cuda", cap_docs: Optional[int] = None, cap_chunks: Optional[int] = None,
                 kv_host: bool = False):
        lay = _lib.msa_bank_layout(doc_lens, chunk)
        self.dtype = dtype
        self.chunk = chunk
        self.layout = lay
        self.n_docs = len(doc_lens)
        self.n_chunks = lay["n_chunks"]
        cap_docs = self.n_docs if cap_docs is None else int(cap_docs)
        cap_chunks = self.n_chunks if cap_chunks is None else int(cap_chunks)
        if cap_docs < self.n_docs or cap_chunks < self.n_chunks:
            raise ValueError("capacity below the initial documents")
        self.cap_docs, self.cap_chunks = cap_docs, cap_chunks
        td = TORCH_DTYPE[dtype]
        self.doc_tok_off_host = np.zeros(cap_docs + 1, dtype=np.int64)
        self.doc_chunk_off_host = np.zeros(cap_docs + 1, dtype=np.int64)
        self.doc_tok_off_host[:self.n_docs + 1] = lay["doc_tok_off"]
        self.doc_chunk_off_host[:self.n_docs + 1] = lay["doc_chunk_off"]
        self.doc_tok_off = torch.from_numpy(self.doc_tok_off_host).to(device)
        self.doc_chunk_off = torch.from_numpy(self.doc_chunk_off_host).to(device)
        self.chunk_doc = torch.empty(cap_chunks, dtype=torch.int32, device=device)
        self.kv_host = kv_host
        if kv_host:
            self.kbar = torch.empty((h_kv, cap_chunks, d), dtype=td, pin_memory=True)
            self.vbar = torch.empty((h_kv, cap_chunks, d), dtype=td, pin_memory=True)
            kv_ptr = (_lib.msa_device_pointer(self.kbar.data_ptr()), _lib.msa_device_pointer(self.vbar.data_ptr()))
        else:
            self.kbar = torch.empty((h_kv, cap_chunks, d), dtype=td, device=device)
            self.vbar = torch.empty((h_kv, cap_chunks, d), dtype=td, device=device)
            kv_ptr = (self.kbar.data_ptr(), self.vbar.data_ptr())
        self.krbar = torch.empty((cap_chunks, h_r, d_r), dtype=td, device=device)
        self.kr_inv_norm = torch.empty((cap_chunks, h_r), dtype=torch.float32, device=device)
        self.c = _lib.MsaBank(
            ABI_DTYPE[dtype], self.n_docs, chunk, h_kv, d, h_r, d_r, lay["max_doc_len"], lay["max_doc_chunks"],
            cap_chunks, int(kv_host), 0, self.n_chunks, self.doc_tok_off.data_ptr(), self.doc_chunk_off.data_ptr(),
            self.doc_tok_off_host.ctypes.data, self.doc_chunk_off_host.ctypes.data, self.chunk_doc.data_ptr(),
            kv_ptr[0], kv_ptr[1], self.krbar.data_ptr(), self.kr_inv_norm.data_ptr())

    def append(self, doc_lens: Sequence[int]) -> tuple:
        """Add documents at the end of the bank (offsets and counts only);
        returns their range (doc_begin, doc_end) for ``pool``.  Nothing is
        enqueued on the device except the copy of the new offsets."""
        lens = np.asarray(doc_lens, dtype=np.int64)
        if lens.size == 0:
            return self.n_docs, self.n_docs
        # the new documents' own layout (the library's helper validates the
        # lengths), shifted to the end of the bank
        lay = _lib.msa_bank_layout(lens, self.chunk)
        n0, c0 = self.n_docs, self.n_chunks
        n1, c1 = n0 + lens.size, c0 + lay["n_chunks"]
        if n1 > self.cap_docs or c1 > self.cap_chunks:
            raise ValueError(f"bank capacity exceeded: {n1} documents / {c1} chunks "
                             f"(capacity {self.cap_docs} / {self.cap_chunks})")
        self.doc_tok_off_host[n0 + 1:n1 + 1] = self.doc_tok_off_host[n0] + lay["doc_tok_off"][1:]
        self.doc_chunk_off_host[n0 + 1:n1 + 1] = c0 + lay["doc_chunk_off"][1:]
        self.doc_tok_off[n0 + 1:n1 + 1].copy_(torch.from_numpy(self.doc_tok_off_host[n0 + 1:n1 + 1]))
        self.doc_chunk_off[n0 + 1:n1 + 1].copy_(torch.from_numpy(self.doc_chunk_off_host[n0 + 1:n1 + 1]))
        self.n_docs, self.n_chunks = n1, c1
        self.c.n_docs, self.c.n_chunks = n1, c1
        if lay["max_doc_len"] > self.c.max_doc_len:
            self.c.max_doc_len, self.c.max_doc_chunks = lay["max_doc_len"], lay["max_doc_chunks"]
        return n0, n1

    @property
    def doc_lens(self) -> np.ndarray:
        return np.diff(self.doc_tok_off_host[:self.n_docs + 1])

    def pool(self, K, V, KR, doc_begin: int, doc_end: int, rope: Rope, stream=None) -> None:
        """Offline pooling of documents [doc_begin, doc_end) from a token slab."""
        _lib.msa_pool_memory(self.c, K, V, KR, doc_begin, doc_end, rope.c, stream)

    def bytes_resident(self) -> int:
        """Bytes of the bank in HBM (the host tier not counted)."""
        ts = [self.krbar, self.kr_inv_norm, self.chunk_doc, self.doc_tok_off, self.doc_chunk_off]
        if not self.kv_host:
            ts += [self.kbar, self.vbar]
        return sum(t.numel() * t.element_size() for t in ts)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A device byte buffer of at least ``nbytes`` (256-byte aligned by torch)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
