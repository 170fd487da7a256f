"""Decode steps of independent query batches, the router scans of
consecutive steps and the top-k and attention of earlier steps overlapping.

The router scan of a step streams the whole bank and is bound by HBM
bandwidth; the top-k and the sparse attention after it are short,
latency-bound kernels.  Independent query batches (other requests, other
layers' queries) can therefore share the GPU, on three streams:

  route stream A: route_score(s)   (even steps) -> mark routed(s)
  route stream B: route_score(s+1) (odd steps)  -> mark routed(s+1)
  tail stream:    [wait routed(s)] topk(s) -> sparse_attend(s) -> mark done(s)

Each scan's persistent grid is capped at one workgroup per compute unit
(max_wg_per_cu = 1): a scan that holds two or three workgroups on every
compute unit keeps the kernels of other streams waiting until its waves
retire (measured: a 1M-element add on a second stream took 6.6 us alone and
220 us beside the full-grid scan, 10 us beside the capped one), whereas one
capped scan streams nearly as fast as the full grid (≈ 1-2 % slower alone).
Two scans in flight hide each other's start and ragged end and the few
microseconds between consecutive kernels of one stream; the tail runs in
the room they leave.  Measured at the 100M-token decode workload: one route
stream with the full grid 308-312 us per step, two route streams with capped
grids 294-296 us (one route stream, capped: 310 us; three route streams:
297-305 us; the route/select-attend layer halves on two route streams:
300-309 us, and 284-292 us with their scan capped too, which takes the
resolve kernel off the route streams).

The pages load the selected documents' pooled rows asynchronously while the
search goes on (hotdry blog, key engineering details: tiered storage and
asynchronous prefetch; wiselychen blog, mechanism 3); with a tiered bank
(``Bank(kv_host=True)``) the attention's gather runs over the host link, a
different resource from the scans' HBM streams, and the same streams overlap
it.

Outputs rotate over `slots` buffers: step s writes slot s % slots, which
stays valid until step s + slots is issued.  The route streams never wait on
the GPU: before reusing a slot the host waits for the tail that last read it
(long finished when the slots outnumber the steps in flight), and the
caller's stream is waited on only while it still has work queued (a
cross-stream wait on a route stream delayed each scan by 10-20 us).  All
computation runs in the library's kernels; this module only orders launches
on streams.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from .memory import TORCH_DTYPE, Bank, Rope, workspace


class DecodePipeline:
    def __init__(self, bank: Bank, rope: Rope, n_q: int, T: int, t_r: int, L_loc: int, h_q: int, k: int, pos0: int,
                 scale: Optional[float] = None, device="cuda", slots: int = 4, route_streams: int = 2,
                 max_wg_per_cu: int = 1):
        self.bank, self.rope = bank, rope
        self.n_q, self.T, self.t_r, self.L_loc, self.h_q, self.k, self.pos0 = n_q, T, t_r, L_loc, h_q, k, pos0
        d = bank.c.d
        self.scale = _lib.default_scale(d) if scale is None else scale
        c = bank.c
        self.ws_route_n = _lib.msa_route_workspace_bytes(c, n_q, t_r)
        self.ws_topk_n = _lib.msa_topk_workspace_bytes(n_q, c.n_docs, k)
        self.ws_attend_n = _lib.msa_attend_workspace_bytes(c, n_q, T, L_loc, h_q, k)
        self.ws_route = [workspace(self.ws_route_n, device) for _ in range(route_streams)]
        self.ws_topk = workspace(self.ws_topk_n, device)
        self.ws_attend = workspace(self.ws_attend_n, device)
        td = TORCH_DTYPE[bank.dtype]
        self.s_doc = [torch.empty((n_q, c.n_docs), dtype=torch.float32, device=device) for _ in range(slots)]
        self.idx = [torch.empty((n_q, k), dtype=torch.int32, device=device) for _ in range(slots)]
        self.val = [torch.empty((n_q, k), dtype=torch.float32, device=device) for _ in range(slots)]
        self.O = [torch.empty((n_q, T, h_q, d), dtype=td, device=device) for _ in range(slots)]
        self.route_streams = [torch.cuda.Stream(device=device) for _ in range(route_streams)]
        self.tail_stream = torch.cuda.Stream(device=device)
        self.max_wg_per_cu = max_wg_per_cu
        self.routed = [torch.cuda.Event() for _ in range(slots)]
        self.done = [torch.cuda.Event() for _ in range(slots)]
        self.slots = slots
        self.issued = 0

    def step(self, QR, Q, K_loc, V_loc) -> int:
        """Issue one decode step; returns its output slot.  The inputs must stay
        alive (and unchanged) until the step has run."""
        s = self.issued % self.slots
        r = self.issued % len(self.route_streams)
        c = self.bank.c
        rs, ts = self.route_streams[r], self.tail_stream
        if self.issued >= self.slots:
            self.done[s].synchronize()  # the tail of step - slots has read s_doc[s] and written idx/O[s]
        cur = torch.cuda.current_stream()
        if not cur.query():
            rs.wait_stream(cur)  # the caller's inputs are still being produced
        _lib.msa_route_score(c, QR, self.n_q, self.t_r, self.s_doc[s], None, self.ws_route[r], self.ws_route_n, rs,
                             max_wg_per_cu=self.max_wg_per_cu)
        self.routed[s].record(rs)
        ts.wait_event(self.routed[s])
        _lib.msa_topk(self.s_doc[s], self.n_q, c.n_docs, self.k, self.idx[s], self.val[s], self.ws_topk,
                      self.ws_topk_n, ts)
        _lib.msa_sparse_attend(c, Q, K_loc, V_loc, self.n_q, self.T, self.L_loc, self.h_q, self.idx[s], self.k,
                               self.pos0, self.scale, self.rope.c, self.O[s], self.ws_attend, self.ws_attend_n, ts)
        self.done[s].record(ts)
        self.issued += 1
        return s

    def synchronize(self) -> None:
        for rs in self.route_streams:
            rs.synchronize()
        self.tail_stream.synchronize()
