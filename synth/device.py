"""Raw per-token bank tensors generated directly on the GPU, slab by slab.

Same values as ``synth.workloads.bank_raw`` (the counter generator is
bit-identical on host and device), so the host can regenerate any sampled
document to check the device-pooled bank.  Input generation only.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import native, rng
from .workloads import Workload


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"synth device generator: {what} failed with code {rc}")


def fill_raw_slab(w: Workload, layer: int, doc_begin: int, doc_end: int, K, V, KR, uhat_dev=None,
                  stream: Optional[int] = None) -> None:
    """Write raw K, V, K^R of documents [doc_begin, doc_end) into the front of the
    device tensors K, V ([n][h_kv][d]) and KR ([n][h_r][d_r]) (stored dtype)."""
    import torch

    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    off = w.doc_tok_off
    t0, t1 = int(off[doc_begin]), int(off[doc_end])
    n = t1 - t0
    bf = 1 if w.dtype == "bf16" else 0
    lib = native.dev_lib()
    for role, buf, H, D in ((rng.ROLE_K, K, w.h_kv, w.d), (rng.ROLE_V, V, w.h_kv, w.d),
                            (rng.ROLE_KR, KR, w.h_r, w.d_r)):
        if buf.numel() < n * H * D:
            raise ValueError("slab buffer too small")
        key = rng.stream_key(w.seed, role, layer)
        _check(lib.synth_dev_fill_normal(buf.data_ptr(), key, t0 * H * D, n * H * D, bf, stream), "fill")
    if w.gold.size:
        if uhat_dev is None:
            raise ValueError("router keys of a bank with gold documents need uhat")
        owner = w.gold_owner()
        esz = KR.element_size()
        for doc in np.nonzero(owner[doc_begin:doc_end] >= 0)[0] + doc_begin:
            a, b = int(off[doc]), int(off[doc + 1])
            ptr = KR.data_ptr() + (a - t0) * w.h_r * w.d_r * esz
            u = uhat_dev[int(owner[doc])]
            _check(lib.synth_dev_plant(ptr, b - a, w.h_r, w.d_r, u.data_ptr(), float(w.gold_cg), bf, stream),
                   "plant")
