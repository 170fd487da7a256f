"""Memory Interleave over the routed layers: rounds of route -> top-k ->
attend, re-routing after each round of newly generated tokens (hotdry blog,
sparse strategy: routing alternates with generation and is redone each round;
hotdry blog, parameters: 2-3 rounds; Lighthouse digest, Component 3).

Round r of layer l routes with all active tokens of the layer's context
(T0 + append * r), then attends the tokens that are new in this round (T0 in
round 0, ``append`` afterwards) over the selected documents plus the whole
causal local context.  Appending is the caller's: the context tensors hold the
whole final context and each round uses a prefix of it.

The router score is a max over router tokens, so a later round's document
scores are the max of the previous round's and the new tokens' own: round 0
runs msa_layer_forward over its T0 tokens, later rounds
msa_layer_forward_reroute over the ``append`` new ones with the layer's
previous scores -- the same scores as routing all active tokens again, for a
fraction of the scan.  This module is a host loop over those calls; all
computation runs in the kernels.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import torch

from . import _lib
from .memory import TORCH_DTYPE, Bank, Rope, workspace


def _contig(t: torch.Tensor) -> torch.Tensor:
    return t if t.is_contiguous() else t.contiguous()


def interleave(banks: Sequence[Bank], rope: Rope, layers: Sequence[Dict[str, torch.Tensor]], T0: int, append: int,
               rounds: int, k: int, pos0: int, h_q: int, scale: Optional[float] = None,
               want_scores: bool = False, stream=None) -> List[List[Dict[str, torch.Tensor]]]:
    """Run ``rounds`` interleave rounds over all layers.

    ``layers[l]`` holds device tensors Q [n_q][L][h_q][d], K_loc / V_loc
    [n_q][L][h_kv][d] and QR [n_q][L][h_r][d_r] over the whole context
    (L >= T0 + append * (rounds - 1)).  Returns out[r][l] = {O, idx, val
    [, s_doc]}.  Every copy, allocation and layer call runs on ``stream`` (a
    torch.cuda.Stream; None = the current stream): the caller orders the
    writes of ``layers`` before it and its uses of the outputs after it.
    """
    if not banks or len(banks) != len(layers):
        raise ValueError("one bank per layer is required")
    n_q = layers[0]["Q"].shape[0]
    d = layers[0]["Q"].shape[-1]
    scale = _lib.default_scale(d) if scale is None else scale
    dev = layers[0]["Q"].device
    td = TORCH_DTYPE[banks[0].dtype]
    # one workspace for the largest round (rounds after the first route only
    # their new tokens)
    nb = max(_lib.msa_layer_workspace_bytes(b.c, n_q, T0 if r == 0 else append, T0 if r == 0 else append,
                                            T0 + append * r, h_q, k)
             for b in banks for r in range(rounds))
    # the copies of strided slices and the output tensors are made on the
    # stream the layer calls run on, so that the allocator and the kernels see
    # one order of work
    strm = torch.cuda.current_stream(dev) if stream is None else stream
    if not isinstance(strm, torch.cuda.Stream):
        raise TypeError("stream must be a torch.cuda.Stream (or None for the current stream)")
    with torch.cuda.stream(strm):
        return _rounds(banks, rope, layers, T0, append, rounds, k, pos0, h_q, scale, want_scores, strm, nb, n_q, d,
                       dev, td)


def _rounds(banks, rope, layers, T0, append, rounds, k, pos0, h_q, scale, want_scores, stream, nb, n_q, d, dev, td):
    ws = workspace(nb, dev)
    out = []
    prev = [None] * len(banks)  # each layer's document scores after the previous round
    for r in range(rounds):
        L_act = T0 + append * r
        T_new = T0 if r == 0 else append
        res_r = []
        for li, (bank, inp) in enumerate(zip(banks, layers)):
            O = torch.empty((n_q, T_new, h_q, d), dtype=td, device=dev)
            idx = torch.empty((n_q, k), dtype=torch.int32, device=dev)
            val = torch.empty((n_q, k), dtype=torch.float32, device=dev)
            s_doc = torch.empty((n_q, bank.n_docs), dtype=torch.float32, device=dev)
            Q = _contig(inp["Q"][:, L_act - T_new:L_act])
            K_loc, V_loc = _contig(inp["K_loc"][:, :L_act]), _contig(inp["V_loc"][:, :L_act])
            if r == 0:
                _lib.msa_layer_forward(bank.c, Q, K_loc, V_loc, _contig(inp["QR"][:, :L_act]), n_q, T_new, L_act,
                                       L_act, h_q, k, pos0, scale, rope.c, O, idx, val, s_doc, ws, nb, None, stream)
            else:
                _lib.msa_layer_forward_reroute(bank.c, Q, K_loc, V_loc, _contig(inp["QR"][:, L_act - T_new:L_act]),
                                               n_q, T_new, T_new, L_act, h_q, k, pos0, scale, rope.c, prev[li], O,
                                               idx, val, s_doc, ws, nb, None, stream)
            prev[li] = s_doc
            res = {"O": O, "idx": idx, "val": val}
            if want_scores:
                res["s_doc"] = s_doc
            res_r.append(res)
        out.append(res_r)
    return out
