"""Offline encoding of a memory bank in slabs of whole documents.

The pages' first inference stage (wiselychen blog, mechanism 3: encode the
corpus offline once and cache each document's compressed representation)
pools every document's per-token K, V and K^R into the bank.  At 100M tokens
the per-token tensors (about 6 KB per token in bf16) are far larger than HBM,
so they are produced and pooled one slab of whole documents at a time: the
caller's ``fill(doc_begin, doc_end, K, V, KR)`` writes a slab's raw tensors
into reused device buffers and ``msa_pool_memory`` reduces them.
"""
from __future__ import annotations

from typing import Callable, List

import numpy as np
import torch

from .memory import TORCH_DTYPE, Bank, Rope


def slab_ranges(doc_tok_off: np.ndarray, slab_tokens: int) -> List[tuple]:
    """Contiguous document ranges whose token counts stay within ``slab_tokens``
    (a longer single document gets a slab of its own)."""
    out = []
    n_docs = doc_tok_off.shape[0] - 1
    a = 0
    while a < n_docs:
        b = int(np.searchsorted(doc_tok_off, doc_tok_off[a] + slab_tokens, side="right")) - 1
        b = max(b, a + 1)
        b = min(b, n_docs)
        out.append((a, b))
        a = b
    return out


def encode_bank(bank: Bank, rope: Rope, fill: Callable, slab_tokens: int, h_kv: int, d: int, h_r: int, d_r: int,
                time_slabs: bool = False, docs: tuple = None) -> dict:
    """Pool the bank's documents slab by slab -- all of them, or the range
    ``docs`` = (doc_begin, doc_end), e.g. the documents just appended; returns
    the slab count and (optionally) the pooling kernels' time and raw bytes
    read per slab."""
    off = bank.doc_tok_off_host[:bank.n_docs + 1]
    lo, hi = (0, bank.n_docs) if docs is None else docs
    ranges = [(a + lo, b + lo) for a, b in slab_ranges(off[lo:hi + 1] - off[lo], slab_tokens)] if hi > lo else []
    if not ranges:
        return {"slabs": 0, "seconds": [], "raw_bytes": []}
    cap = max(int(off[b] - off[a]) for a, b in ranges)
    td = TORCH_DTYPE[bank.dtype]
    dev = bank.krbar.device
    K = torch.empty((cap, h_kv, d), dtype=td, device=dev)
    V = torch.empty((cap, h_kv, d), dtype=td, device=dev)
    KR = torch.empty((cap, h_r, d_r), dtype=td, device=dev)
    esz = K.element_size()
    times, raw = [], []
    for a, b in ranges:
        fill(a, b, K, V, KR)
        if time_slabs:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        bank.pool(K, V, KR, a, b, rope)
        if time_slabs:
            e1.record()
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
            n = int(off[b] - off[a])
            raw.append(n * (2 * h_kv * d + h_r * d_r) * esz)
    torch.cuda.synchronize()
    del K, V, KR
    return {"slabs": len(ranges), "seconds": times, "raw_bytes": raw}
