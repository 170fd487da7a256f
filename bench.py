#!/usr/bin/env python3
"""Throughput of one MSA routed layer over a 100M-token memory bank on one MI355X.

Workload (decode): 100,000,000 bank tokens in documents of U[512, 8192]
tokens, chunk 128 (about 793K chunks), 8 router heads x 128, 32 query / 8 KV
heads x 128, bf16 storage with fp32 accumulation, 16 independent queries x 1
decode token, k = 16, 8 planted gold documents per query.  The pooled bank
(Kbar^R 1.6 GB, Kbar/Vbar 3.2 GB) is resident in HBM before timing; the raw
per-token tensors (614 GB) are generated on the device and pooled slab by slab
beforehand (the offline stage).

A step is one pass of the routed layer over one batch of 16 queries: router
scan with the fused document max, top-k, sparse attention (plus split merge).
Two timed regions of --steps steps each: sequential msa_layer_forward calls
on one stream (per-stage events: layer latency, the scan's HBM roofline), then
independent batches through the decode pipeline (two route streams whose
scans overlap, the top-k and attention of earlier batches on a third); the
pipelined rate is the throughput `value`.  The same line carries the Memory
Interleave workload (18 routed layers x 10M-token banks, 3 rounds; MFMA-bound)
as the `interleave` record, the tiered bank (Kbar/Vbar in pinned host memory,
pipelined decode), the incremental append of the last 10% of the documents and
the router projector GEMM as the `tiered`, `append` and `project` records, and
the fp64 oracle's rate on the host's cores as `cpu_baseline` (timed first,
before the GPU is used).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import resource
import statistics
import sys
import time

# the oracle baseline runs one single-threaded process per core: no BLAS
# thread pools of its own (set before NumPy is imported)
for _v in ("OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ[_v] = "1"

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "memory tokens routed/sec/GPU + MSA layer latency @100M-token bank; % HBM peak"
HBM_PEAK_GBS = 8000.0


class Events:
    """Timing events for msa_layer_forward's stage_events: torch's own events, so
    they belong to the same HIP runtime as the stream the library launches on.
    ``h`` holds the raw hipEvent_t handles."""

    def __init__(self, n: int):
        import torch

        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in self.ev:          # materialise the underlying hipEvent_t
            e.record()
        torch.cuda.synchronize()
        self.h = [e.cuda_event for e in self.ev]
        self._by_handle = dict(zip(self.h, self.ev))

    def ms(self, a: int, b: int) -> float:
        return self._by_handle[a].elapsed_time(self._by_handle[b])

    def close(self):
        self.ev = []


def route_traffic(bytes_per_launch: int):
    """HBM bytes per router-scan launch from the committed counter passes, or None
    when the kernel source changed since they were taken (see profiles/)."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "route_scan_100M_decode_traffic.txt")
    try:
        kv = {}
        for line in open(path):
            if "=" in line and not line.startswith("#"):
                k, v = line.strip().split("=", 1)
                kv[k] = v
        src = b"".join(open(os.path.join(ROOT, "long_context_memory_msa_amd", "csrc", f), "rb").read()
                       for f in ("route.hip", "msa_device.hpp"))
        if hashlib.sha256(src).hexdigest()[:16] != kv["kernel_source_sha256_16"]:
            return None
        return (float(kv["fetch_kib"]) * float(kv["fetch_factor"]) +
                float(kv["write_kib"]) * float(kv["write_factor"])) * 1024.0
    except (OSError, KeyError, ValueError):
        return None


def pct(xs) -> list:
    """p10, p50, p90 of a list of times."""
    ys = sorted(xs)
    return [ys[int(round(f * (len(ys) - 1)))] for f in (0.1, 0.5, 0.9)]


def attend_roofline(w, bank, gi, attend_ms: float) -> dict:
    """Attention stage against both rooflines: algorithmic FLOPs
    4 * H_q * d * sum over rows of the visible keys (selected documents' pooled
    rows + causal local keys) over the bf16 MFMA peak, and the gathered pooled
    K/V rows + Q, local K/V and O bytes over the HBM peak."""
    off = bank.doc_chunk_off_host
    n_mem = [sum(int(off[d + 1] - off[d]) for d in gi[q]) for q in range(w.n_q)]
    vis = sum(n_mem[q] + (w.L_loc - w.T + t + 1) for q in range(w.n_q) for t in range(w.T))
    flop = 4.0 * w.h_q * w.d * vis
    esz = 2 if w.dtype == "bf16" else 4
    nbytes = (sum(n_mem) * w.h_kv * w.d * 2 + w.n_q * w.T * w.h_q * w.d * 2
              + w.n_q * w.L_loc * w.h_kv * w.d * 2) * esz
    sec = attend_ms * 1e-3
    return {"flop": flop, "bytes": nbytes, "TFLOP/s": flop / sec / 1e12, "mfma_frac": flop / sec / 2.5e15,
            "GB/s": nbytes / sec / 1e9, "hbm_frac": nbytes / sec / 1e9 / HBM_PEAK_GBS,
            "note": "stage time includes the in-kernel top-k selection and the split merge"}


def run_pipelined(bank, rope, w, scale, dev, QR, Q, Kl, Vl, idx, O_, args) -> float:
    """Wall time of --steps independent decode steps through the decode
    pipeline; the last step's output must equal msa_layer_forward's."""
    import torch

    from long_context_memory_msa_amd.pipeline import DecodePipeline

    pipe = DecodePipeline(bank, rope, w.n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k, w.pos0, scale, dev)
    for _ in range(args.warmup):
        pipe.step(QR, Q, Kl, Vl)
    pipe.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        last = pipe.step(QR, Q, Kl, Vl)
    pipe.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if not (torch.equal(pipe.idx[last], idx) and torch.equal(pipe.O[last], O_)):
        raise RuntimeError("pipelined step differs from msa_layer_forward")
    return wall


_CPU_JOB = {}  # inputs of the oracle scan, inherited by the forked workers


def _scan_block(bounds):
    """Worker: the oracle's router scores of chunks [a, b) (fp64, single thread)."""
    import oracle as O

    a, b = bounds
    return O.chunk_scores(_CPU_JOB["QR"], _CPU_JOB["krbar"][a:b])


def _pool_block(bounds):
    """Worker: the oracle's pooling of sample documents [a, b) (fp64, single thread)."""
    import oracle as O

    a, b = bounds
    j = _CPU_JOB
    t0, t1 = int(j["tok_off"][a]), int(j["tok_off"][b])
    O.pool(j["lens"][a:b], j["chunk"], j["K"][t0:t1], j["V"][t0:t1], j["KR"][t0:t1], j["dtype"], j["base"])
    return t1 - t0


def cpu_pool_baseline(w, qi, n_docs: int, workers: int) -> dict:
    """The fp64 oracle's offline pooling (oracle.pool) on the raw tokens of the
    bank's first ``n_docs`` documents, one contiguous document range per forked
    single-threaded worker; the rate is extrapolated to the whole bank (the
    oracle's pooling time is linear in the tokens)."""
    import multiprocessing

    import numpy as np

    from synth import rng, workloads as W

    lens = w.doc_lens[:n_docs]
    tok_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    n_tok = int(tok_off[-1])
    _CPU_JOB.update(lens=lens, tok_off=tok_off, chunk=w.chunk, dtype=w.dtype, base=w.rope_base,
                    K=W.bank_raw(w, rng.ROLE_K, 0, n_tok), V=W.bank_raw(w, rng.ROLE_V, 0, n_tok),
                    KR=W.bank_raw(w, rng.ROLE_KR, 0, n_tok, uhat=W.gold_uhat(w, qi["QR"])))
    cuts = np.unique(np.linspace(0, n_docs, min(workers, n_docs) + 1).astype(np.int64))
    blocks = [(int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:])]
    pool = multiprocessing.get_context("fork").Pool(len(blocks))
    pool.map(int, range(len(blocks)))
    t0 = time.perf_counter()
    done = sum(pool.map(_pool_block, blocks, chunksize=1))
    dt = time.perf_counter() - t0
    pool.close()
    pool.join()
    _CPU_JOB.clear()
    rate = done / dt
    return {
        "value": rate,
        "unit": "tokens/s",
        "cores": len(blocks),
        "kind": "oracle",
        "extrapolated_s_whole_bank": w.n_tok / rate,
        "sample": (f"oracle pooling (fp64 NumPy: chunk means with document-wise RoPE, stored rounding, inverse "
                   f"norms) of the raw K, V, K^R tokens of the first {n_docs} documents ({done} tokens) in "
                   f"{len(blocks)} forked single-threaded processes, {dt:.2f} s wall; whole-bank time "
                   f"extrapolated per token"),
    }


def cpu_baseline(w, qi, n_docs: int, workers: int) -> dict:
    """The fp64 oracle's layer forward on the first ``n_docs`` documents of the
    bank (pooled-shape synthetic values; the oracle's time does not depend on
    them) on this host's cores: the router scan (oracle.chunk_scores) over
    contiguous chunk blocks in ``workers`` forked single-threaded processes,
    then the document max, top-k and attention (oracle functions) here.  Runs
    before this process touches the GPU (the workers are forked from it)."""
    import multiprocessing

    import numpy as np

    import oracle as O
    from synth import rng

    n_docs = w.n_docs if n_docs < 0 else min(n_docs, w.n_docs)
    lens = w.doc_lens[:n_docs]
    lay = O.bank_layout(lens, w.chunk)
    N = lay["n_chunks"]
    g = 1.0 / np.sqrt(w.chunk)
    bank = {
        "krbar": rng.normal_stored(rng.stream_key(w.seed, rng.ROLE_POOLED_KR), 0, N * w.h_r * w.d_r,
                                   w.dtype).reshape(N, w.h_r, w.d_r) * np.float32(g),
        "kbar": rng.normal_stored(rng.stream_key(w.seed, rng.ROLE_POOLED_K), 0, N * w.h_kv * w.d,
                                  w.dtype).reshape(w.h_kv, N, w.d) * np.float32(g),
        "vbar": rng.normal_stored(rng.stream_key(w.seed, rng.ROLE_POOLED_V), 0, N * w.h_kv * w.d,
                                  w.dtype).reshape(w.h_kv, N, w.d) * np.float32(g),
        "doc_chunk_off": lay["doc_chunk_off"],
    }
    QR = qi["QR"][:, w.L_loc - w.T_route:w.L_loc]
    Q = qi["Q"][:, w.L_loc - w.T:w.L_loc]
    _CPU_JOB.update(QR=QR, krbar=bank["krbar"])
    cuts = np.linspace(0, N, workers + 1).astype(np.int64)
    blocks = [(int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    pool = multiprocessing.get_context("fork").Pool(len(blocks))   # workers start before the timed region
    pool.map(int, range(len(blocks)))                              # ... and are all up
    r0s, r0c = resource.getrusage(resource.RUSAGE_SELF), resource.getrusage(resource.RUSAGE_CHILDREN)
    t0 = time.perf_counter()
    S = np.concatenate(pool.map(_scan_block, blocks, chunksize=1), axis=1)
    s_doc = O.doc_scores(S, bank["doc_chunk_off"])
    sel = O.topk(s_doc, w.k)
    O.attend(Q, qi["K_loc"][:, :w.L_loc], qi["V_loc"][:, :w.L_loc], bank["kbar"], bank["vbar"],
             bank["doc_chunk_off"], sel["idx"], w.pos0, base=w.rope_base)
    dt = time.perf_counter() - t0
    pool.close()
    pool.join()
    r1s, r1c = resource.getrusage(resource.RUSAGE_SELF), resource.getrusage(resource.RUSAGE_CHILDREN)
    _CPU_JOB.clear()
    cpu = sum((getattr(r1, f) - getattr(r0, f)) for r0, r1 in ((r0s, r1s), (r0c, r1c))
              for f in ("ru_utime", "ru_stime"))
    tokens = int(lens.sum())
    return {
        "value": tokens / dt,
        "unit": "tokens/s",
        "cores": len(blocks),
        "kind": "oracle",
        "sample": (f"oracle layer forward (fp64 NumPy) over the first {n_docs} documents ({tokens} tokens, {N} "
                   f"chunks) of the same bank layout and query batch: router scan (oracle.chunk_scores) over "
                   f"{len(blocks)} chunk blocks in as many forked single-threaded processes, then document max, "
                   f"top-k and attention in one; {dt:.2f} s wall, {cpu:.1f} s CPU "
                   f"({cpu / dt:.1f} cores busy on average); {len(os.sched_getaffinity(0))} host cores available"),
    }


def interleave_measure(args, n_passes: int) -> dict:
    """18 routed layers x 10M-token banks, 3 rounds of route -> top-k -> attend
    (prefill 512 tokens, then 64 appended per round), ``n_passes`` timed passes
    over the 54 layer calls: throughput, per-call latency per round, and the
    MFMA rooflines of the router scan and of attention from the stage events
    (median pass)."""
    import numpy as np
    import torch

    from synth import device as sdev, workloads as W
    from long_context_memory_msa_amd import _lib as L, memory as M, offline

    dev = torch.device("cuda:0")
    w = W.make_workload("interleave-10mx18")
    print(f"[bench] {w.name}: {w.n_layers} layers x {w.n_tok} tokens, {w.n_docs} docs, {w.n_chunks} chunks",
          file=sys.stderr, flush=True)
    banks, layers = [], []
    rope = None
    for layer in range(w.n_layers):
        bank = M.Bank(w.doc_lens, w.chunk, w.h_kv, w.d, w.h_r, w.d_r, w.dtype, dev)
        rope = rope or M.Rope(w.max_pos, w.d, w.rope_base, dev)
        offline.encode_bank(bank, rope, lambda a, b, K, V, KR, l=layer: sdev.fill_raw_slab(w, l, a, b, K, V, KR),
                            args.slab_tokens, w.h_kv, w.d, w.h_r, w.d_r)
        banks.append(bank)
        qi = W.query_inputs(w, layer)
        layers.append({k: torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(dev).to(torch.bfloat16)
                       for k, v in qi.items()})
    calls = [(r, l) for r in range(w.rounds) for l in range(w.n_layers)]
    shapes = {}   # round -> (active tokens, new tokens: attended, and routed by the scan)
    for r in range(w.rounds):
        L_act = w.L_loc + w.append * r
        shapes[r] = (L_act, w.L_loc if r == 0 else w.append)
    nb = max(L.msa_layer_workspace_bytes(banks[0].c, 1, T, T, La, w.h_q, w.k) for La, T in shapes.values())
    ws = M.workspace(nb, dev)
    outs = {r: torch.empty((1, shapes[r][1], w.h_q, w.d), dtype=torch.bfloat16, device=dev) for r in shapes}
    idxs = {c: torch.empty((1, w.k), dtype=torch.int32, device=dev) for c in calls}
    val = torch.empty((1, w.k), dtype=torch.float32, device=dev)
    sdoc = [torch.empty((1, w.n_docs), dtype=torch.float32, device=dev) for _ in range(w.n_layers)]
    scale = L.default_scale(w.d)

    def run(events=None):
        # round 0 routes its 512 tokens; later rounds scan only the 64 new
        # tokens and fold in the layer's previous document scores (the same
        # scores as routing every active token again)
        for i, (r, l) in enumerate(calls):
            La, T = shapes[r]
            inp = layers[l]
            ev = None if events is None else events[4 * i:4 * i + 4]
            if r == 0:
                L.msa_layer_forward(banks[l].c, inp["Q"][:, La - T:La], inp["K_loc"][:, :La], inp["V_loc"][:, :La],
                                    inp["QR"][:, :La], 1, T, La, La, w.h_q, w.k, w.pos0, scale, rope.c, outs[r],
                                    idxs[(r, l)], val, sdoc[l], ws, nb, ev)
            else:
                L.msa_layer_forward_reroute(banks[l].c, inp["Q"][:, La - T:La], inp["K_loc"][:, :La],
                                            inp["V_loc"][:, :La], inp["QR"][:, La - T:La], 1, T, T, La, w.h_q, w.k,
                                            w.pos0, scale, rope.c, sdoc[l], outs[r], idxs[(r, l)], val, sdoc[l], ws,
                                            nb, ev)

    for _ in range(max(1, args.warmup)):
        run()
    torch.cuda.synchronize()
    passes = []
    for _ in range(max(1, n_passes)):
        ev = Events(4 * len(calls))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(ev.h)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        route = [ev.ms(ev.h[4 * i], ev.h[4 * i + 1]) for i in range(len(calls))]
        attend = [ev.ms(ev.h[4 * i + 2], ev.h[4 * i + 3]) for i in range(len(calls))]
        layer = [ev.ms(ev.h[4 * i], ev.h[4 * i + 3]) for i in range(len(calls))]
        passes.append((wall, route, attend, layer))
        ev.close()
    passes.sort(key=lambda p: p[0])
    wall, route, attend, layer = passes[len(passes) // 2]
    off = w.doc_chunk_off
    route_flop = attn_flop = 0.0
    for (r, l) in calls:
        La, T = shapes[r]
        route_flop += 2.0 * T * w.n_chunks * w.h_r * w.d_r   # the router tokens this call scans
        sel = idxs[(r, l)].cpu().numpy()[0]
        n_mem = int(sum(off[d + 1] - off[d] for d in sel))
        visible = sum(n_mem + (La - T + t) + 1 for t in range(T))
        attn_flop += 4.0 * w.h_q * w.d * visible
    peak = 2.5e15
    per_round = {f"round{r}": {"router_tokens": shapes[r][0], "tokens_scanned": shapes[r][1],
                               "tokens_attended": shapes[r][1],
                               "layer_call_ms_p50": statistics.median(
                                   layer[i] for i, c in enumerate(calls) if c[0] == r),
                               "route_ms_p50": statistics.median(route[i] for i, c in enumerate(calls) if c[0] == r),
                               "attend_ms_p50": statistics.median(
                                   attend[i] for i, c in enumerate(calls) if c[0] == r)}
                 for r in range(w.rounds)}
    del banks, layers, ws
    torch.cuda.empty_cache()
    return {
        "workload": "18 routed layers x 10M tokens, docs U[256,4096], chunk 128, prefill 512 + 2 x 64, k=8",
        "value": w.n_tok * len(calls) / wall,
        "unit": "memory tokens routed/s",
        "ms_per_interleave": wall * 1e3,
        "passes": len(passes),
        "n_chunks_per_layer": w.n_chunks,
        "layer_calls": len(calls),
        "rounds": per_round,
        "route": {"ms_total": sum(route), "tflop": route_flop / 1e12,
                  "mfma_frac": route_flop / (sum(route) * 1e-3) / peak, "peak_tflops": peak / 1e12,
                  "round0_mfma_frac": sum(2.0 * shapes[0][1] * w.n_chunks * w.h_r * w.d_r for c in calls if c[0] == 0)
                  / (sum(route[i] for i, c in enumerate(calls) if c[0] == 0) * 1e-3) / peak,
                  "note": "rounds after the first scan only their 64 new router tokens and fold in the previous "
                          "round's document scores; tflop counts the tokens scanned"},
        "attend": {"ms_total": sum(attend), "tflop": attn_flop / 1e12,
                   "mfma_frac": attn_flop / (sum(attend) * 1e-3) / peak, "peak_tflops": peak / 1e12},
    }


def bench_interleave(args) -> int:
    """The interleave workload's own line (not the headline)."""
    rec = interleave_measure(args, args.steps)
    out = {"metric": "Memory Interleave: memory tokens routed/sec over 18 layers x 3 rounds (10M-token banks)",
           "value": rec.pop("value"), "unit": "tokens/s", "n_gpus": 1, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": rec.pop("workload")}, **rec}
    print(json.dumps(out), flush=True)
    return 0


def project_measure(args) -> dict:
    """Router projection GEMM (Y = X W^T, bf16, fp32 accumulation): the
    encoding-time projection of a 256K-token slab of memory hidden states
    (hidden 2560 -> router 4 x 256) and the decode-time projection of 16 query
    tokens; MFMA roofline of the slab GEMM."""
    import torch

    from synth import rng, workloads as W
    from long_context_memory_msa_amd import _lib as L

    dev = torch.device("cuda:0")
    hidden, out = 2560, 1024
    res = {}
    for name, rows in (("encode_slab", 262144), ("decode_query", 16)):
        X = torch.from_numpy(W.hidden_states(9, rng.ROLE_HID_MEM, rows, hidden)).to(dev).to(torch.bfloat16)
        Wt = torch.from_numpy(W.projector_weights(9, rng.ROLE_W_KR, hidden, out)).to(dev).to(torch.bfloat16)
        Y = torch.empty((rows, out), dtype=torch.bfloat16, device=dev)
        for _ in range(max(1, args.warmup)):
            L.msa_router_project(X, Wt, rows, hidden, out, Y)
        torch.cuda.synchronize()
        n = max(5, args.steps)
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for i in range(n):
            e0[i].record()
            L.msa_router_project(X, Wt, rows, hidden, out, Y)
            e1[i].record()
        torch.cuda.synchronize()
        ms = statistics.median(e0[i].elapsed_time(e1[i]) for i in range(n))
        flop = 2.0 * rows * hidden * out
        res[name] = {"rows": rows, "ms": ms, "tflops": flop / (ms * 1e-3) / 1e12,
                     "mfma_frac": flop / (ms * 1e-3) / 2.5e15}
    rec = {
        "metric": "router projection GEMM (hidden 2560 -> 4 x 256), bf16 MFMA",
        "value": res["encode_slab"]["tflops"],
        "unit": "TFLOP/s",
        "roofline": {"bound": "mfma", "achieved": res["encode_slab"]["tflops"], "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": res["encode_slab"]["mfma_frac"]},
        "cases": res,
        "data": "synthetic",
    }
    return rec


def append_measure(args) -> dict:
    """Incremental update of the 100M-token bank: encode the first 90% of the
    documents into a bank with room for all, append the rest, pool only the
    appended range; report the pooling rate of the appended range and the
    decode layer time before and after (the scan grows with the bank)."""
    import numpy as np
    import torch

    from synth import device as sdev, workloads as W
    from long_context_memory_msa_amd import _lib as L, memory as M, offline

    dev = torch.device("cuda:0")
    w = W.make_workload("decode-100m", bank_tokens=args.bank_tokens)
    qi = W.query_inputs(w)
    uhat = torch.from_numpy(W.gold_uhat(w, qi["QR"])).to(dev)
    td = M.TORCH_DTYPE[w.dtype]

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).to(td).contiguous()

    QR = up(qi["QR"][:, w.L_loc - w.T_route:w.L_loc])
    Q = up(qi["Q"][:, w.L_loc - w.T:w.L_loc])
    Kl = up(qi["K_loc"][:, :w.L_loc])
    Vl = up(qi["V_loc"][:, :w.L_loc])
    n0 = int(w.n_docs * 0.9)
    bank = M.Bank(w.doc_lens[:n0], w.chunk, w.h_kv, w.d, w.h_r, w.d_r, w.dtype, dev, cap_docs=w.n_docs,
                  cap_chunks=w.n_chunks)
    rope = M.Rope(w.max_pos, w.d, w.rope_base, dev)
    fill = lambda a, b, K, V, KR: sdev.fill_raw_slab(w, 0, a, b, K, V, KR, uhat)
    offline.encode_bank(bank, rope, fill, args.slab_tokens, w.h_kv, w.d, w.h_r, w.d_r)
    scale = L.default_scale(w.d)

    def layer_ms():
        O_ = torch.empty((w.n_q, w.T, w.h_q, w.d), dtype=td, device=dev)
        idx = torch.empty((w.n_q, w.k), dtype=torch.int32, device=dev)
        val = torch.empty((w.n_q, w.k), dtype=torch.float32, device=dev)
        nb = L.msa_layer_workspace_bytes(bank.c, w.n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k)
        ws = M.workspace(nb, dev)
        run = lambda ev=None: L.msa_layer_forward(bank.c, Q, Kl, Vl, QR, w.n_q, w.T, w.T_route, w.L_loc, w.h_q,
                                                  w.k, w.pos0, scale, rope.c, O_, idx, val, None, ws, nb, ev)
        for _ in range(3):
            run()
        ev = Events(4 * 10)
        for i in range(10):
            run(ev.h[4 * i:4 * i + 4])
        torch.cuda.synchronize()
        t = statistics.median(ev.ms(ev.h[4 * i], ev.h[4 * i + 3]) for i in range(10))
        ev.close()
        return t, idx.cpu().numpy()

    before, _ = layer_ms()
    a, b = bank.append(w.doc_lens[n0:])
    enc = offline.encode_bank(bank, rope, fill, args.slab_tokens, w.h_kv, w.d, w.h_r, w.d_r, time_slabs=True,
                              docs=(a, b))
    after, idx = layer_ms()
    n_new = int(w.doc_tok_off[b] - w.doc_tok_off[a])
    ch_new = int(w.doc_chunk_off[b] - w.doc_chunk_off[a])
    pooled = ch_new * ((2 * w.h_kv * w.d + w.h_r * w.d_r) * 2 + 4 * w.h_r + 4)
    secs = sum(enc["seconds"])
    gold_ok = float(np.mean([set(w.gold[q].tolist()) <= set(idx[q].tolist()) for q in range(w.n_q)]))
    rec = {
        "metric": "incremental bank append: pooling rate of the appended documents",
        "value": (sum(enc["raw_bytes"]) + pooled) / secs / 1e9,
        "unit": "GB/s",
        "appended": {"docs": b - a, "tokens": n_new, "chunks": ch_new, "pool_ms": secs * 1e3,
                     "tokens_per_s": n_new / secs},
        "layer_ms_before": before, "layer_ms_after": after,
        "bank_tokens_before": int(w.doc_tok_off[a]), "bank_tokens_after": int(w.doc_tok_off[b]),
        "gold_recovered_after": gold_ok,
        "data": "synthetic",
    }
    return rec


def tiered_measure(args) -> dict:
    """The 100M-token decode layer with a tiered bank: pooled keys/values in
    pinned host memory (read by the attention over the host link), router keys
    in HBM.  Steps of the same query batch run through the decode pipeline
    (attention of step s during the routing of later steps); one sequential step
    with stage events gives the breakdown."""
    import numpy as np
    import torch

    from synth import device as sdev, workloads as W
    from long_context_memory_msa_amd import _lib as L, memory as M, offline
    from long_context_memory_msa_amd.pipeline import DecodePipeline

    dev = torch.device("cuda:0")
    w = W.make_workload("decode-100m", bank_tokens=args.bank_tokens)
    print(f"[bench] tiered {w.name}: {w.n_tok} tokens, {w.n_docs} docs, {w.n_chunks} chunks", file=sys.stderr,
          flush=True)
    qi = W.query_inputs(w)
    uhat = torch.from_numpy(W.gold_uhat(w, qi["QR"])).to(dev)
    td = M.TORCH_DTYPE[w.dtype]

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).to(td).contiguous()

    QR = up(qi["QR"][:, w.L_loc - w.T_route:w.L_loc])
    Q = up(qi["Q"][:, w.L_loc - w.T:w.L_loc])
    Kl = up(qi["K_loc"][:, :w.L_loc])
    Vl = up(qi["V_loc"][:, :w.L_loc])
    bank = M.Bank(w.doc_lens, w.chunk, w.h_kv, w.d, w.h_r, w.d_r, w.dtype, dev, kv_host=True)
    rope = M.Rope(w.max_pos, w.d, w.rope_base, dev)
    t0 = time.perf_counter()
    offline.encode_bank(bank, rope, lambda a, b, K, V, KR: sdev.fill_raw_slab(w, 0, a, b, K, V, KR, uhat),
                        args.slab_tokens, w.h_kv, w.d, w.h_r, w.d_r)
    print(f"[bench] tiered bank encoded in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    scale = L.default_scale(w.d)

    # sequential steps (one stream, stage events)
    O_ = torch.empty((w.n_q, w.T, w.h_q, w.d), dtype=td, device=dev)
    idx = torch.empty((w.n_q, w.k), dtype=torch.int32, device=dev)
    val = torch.empty((w.n_q, w.k), dtype=torch.float32, device=dev)
    nb = L.msa_layer_workspace_bytes(bank.c, w.n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k)
    ws = M.workspace(nb, dev)
    n_seq = 10
    for _ in range(3):
        L.msa_layer_forward(bank.c, Q, Kl, Vl, QR, w.n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k, w.pos0, scale,
                            rope.c, O_, idx, val, None, ws, nb)
    torch.cuda.synchronize()
    ev = Events(4 * n_seq)
    for i in range(n_seq):
        L.msa_layer_forward(bank.c, Q, Kl, Vl, QR, w.n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k, w.pos0, scale,
                            rope.c, O_, idx, val, None, ws, nb, ev.h[4 * i:4 * i + 4])
    torch.cuda.synchronize()
    st = {name: statistics.median(ev.ms(ev.h[4 * i + a], ev.h[4 * i + b]) for i in range(n_seq))
          for name, a, b in (("route", 0, 1), ("topk", 1, 2), ("attend", 2, 3), ("layer", 0, 3))}
    ev.close()
    off = w.doc_chunk_off
    gi = idx.cpu().numpy()
    n_sel = sum(int(off[d + 1] - off[d]) for q in range(w.n_q) for d in gi[q])
    gathered = n_sel * w.h_kv * w.d * 2 * 2   # K and V rows of the selected chunks, bf16

    # pipelined steps
    pipe = DecodePipeline(bank, rope, w.n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k, w.pos0, scale, dev)
    for _ in range(args.warmup):
        pipe.step(QR, Q, Kl, Vl)
    pipe.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        pipe.step(QR, Q, Kl, Vl)
    pipe.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    rec = {
        "metric": "memory tokens routed/sec, tiered bank (Kbar/Vbar in pinned host memory), pipelined decode",
        "value": w.n_tok / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": "100M-token bank, decode 16 queries x 1 token, k=16; Kbar/Vbar in host memory",
                   "n_chunks": w.n_chunks},
        "sequential_stage_ms": st,
        "attend_gather": {"bytes": gathered, "GB/s": gathered / (st["attend"] * 1e-3) / 1e9},
        "hbm_bytes": bank.bytes_resident(),
        "host_bytes": bank.kbar.numel() * bank.kbar.element_size() * 2,
    }
    return rec


def bench_secondary(args, measure) -> int:
    """A secondary workload's own line (not the headline)."""
    print(json.dumps(measure(args)), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sequential-only", action="store_true",
                    help="decode: time only the sequential msa_layer_forward steps (for kernel profiles)")
    ap.add_argument("--cpu-docs", type=int, default=-1,
                    help="oracle baseline sample: first N documents (-1 = the whole bank, 0 = skip)")
    ap.add_argument("--bank-tokens", type=int, default=None, help="smaller bank for a quick look (not the metric)")
    ap.add_argument("--slab-tokens", type=int, default=8_000_000)
    ap.add_argument("--workload", choices=["decode100m", "interleave", "tiered", "append", "project"],
                    default="decode100m",
                    help="decode100m: the headline layer (default); interleave: 18 routed layers x 10M tokens, "
                         "3 Memory Interleave rounds (MFMA-bound prefill report); tiered: the decode layer with "
                         "Kbar/Vbar in host memory, decode pipeline; append: the last 10%% of the documents "
                         "appended to an encoded bank; project: the router projection GEMM")
    ap.add_argument("--no-interleave", action="store_true",
                    help="decode: leave out the Memory Interleave sub-record (18 layers x 10M tokens)")
    ap.add_argument("--no-secondary", action="store_true",
                    help="decode: leave out the tiered-bank, append and projector sub-records")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (reference kernel for HBM counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); a bank would shard by whole documents, one shard per GPU, with a "
              f"global top-k merge of the per-GPU candidates.", file=sys.stderr)
        return 2

    import numpy as np

    from synth import workloads as W

    # the oracle baseline runs first: its workers are forked from this process,
    # which must not have touched the GPU yet
    cpu_rec = None
    if args.workload == "decode100m" and args.cpu_docs != 0 and not args.copy_calibration:
        w = W.make_workload("decode-100m", bank_tokens=args.bank_tokens)
        workers = max(1, len(os.sched_getaffinity(0)))
        print(f"[bench] timing the oracle on {workers} host cores ...", file=sys.stderr, flush=True)
        qi = W.query_inputs(w)
        cpu_rec = cpu_baseline(w, qi, args.cpu_docs, workers)
        cpu_rec["pool"] = cpu_pool_baseline(w, qi, 8 * workers, workers)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return 0

    from synth import device as sdev
    from long_context_memory_msa_amd import _lib as L, memory as M, offline

    dev = torch.device("cuda:0")
    if args.workload == "interleave":
        return bench_interleave(args)
    if args.workload == "tiered":
        return bench_secondary(args, tiered_measure)
    if args.workload == "append":
        return bench_secondary(args, append_measure)
    if args.workload == "project":
        return bench_secondary(args, project_measure)
    w = W.make_workload("decode-100m", bank_tokens=args.bank_tokens)
    print(f"[bench] {w.name}: {w.n_tok} tokens, {w.n_docs} docs, {w.n_chunks} chunks", file=sys.stderr, flush=True)

    # ---- queries (host-generated, uploaded) and the pooled bank (device) -------
    qi = W.query_inputs(w)
    uhat = torch.from_numpy(W.gold_uhat(w, qi["QR"])).to(dev)
    td = M.TORCH_DTYPE[w.dtype]

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).to(td).contiguous()

    QR = up(qi["QR"][:, w.L_loc - w.T_route:w.L_loc])
    Q = up(qi["Q"][:, w.L_loc - w.T:w.L_loc])
    Kl = up(qi["K_loc"][:, :w.L_loc])
    Vl = up(qi["V_loc"][:, :w.L_loc])
    bank = M.Bank(w.doc_lens, w.chunk, w.h_kv, w.d, w.h_r, w.d_r, w.dtype, dev)
    rope = M.Rope(w.max_pos, w.d, w.rope_base, dev)
    t0 = time.perf_counter()
    enc = offline.encode_bank(bank, rope, lambda a, b, K, V, KR: sdev.fill_raw_slab(w, 0, a, b, K, V, KR, uhat),
                              args.slab_tokens, w.h_kv, w.d, w.h_r, w.d_r, time_slabs=True)
    esz = 2 if w.dtype == "bf16" else 4
    pooled_bytes = w.n_chunks * ((2 * w.h_kv * w.d + w.h_r * w.d_r) * esz + 4 * w.h_r + 4)
    pool_s = sum(enc["seconds"])
    pool_gbs = (sum(enc["raw_bytes"]) + pooled_bytes) / pool_s / 1e9
    print(f"[bench] bank encoded in {time.perf_counter() - t0:.1f} s ({enc['slabs']} slabs, pool kernels "
          f"{pool_s * 1e3:.1f} ms, {pool_gbs:.0f} GB/s)", file=sys.stderr, flush=True)

    O_ = torch.empty((w.n_q, w.T, w.h_q, w.d), dtype=td, device=dev)
    idx = torch.empty((w.n_q, w.k), dtype=torch.int32, device=dev)
    val = torch.empty((w.n_q, w.k), dtype=torch.float32, device=dev)
    nb = L.msa_layer_workspace_bytes(bank.c, w.n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k)
    ws = M.workspace(nb, dev)
    scale = L.default_scale(w.d)

    def step(events=None):
        L.msa_layer_forward(bank.c, Q, Kl, Vl, QR, w.n_q, w.T, w.T_route, w.L_loc, w.h_q, w.k, w.pos0, scale,
                            rope.c, O_, idx, val, None, ws, nb, events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = Events(4 * args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev.h[4 * i:4 * i + 4])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    route = [ev.ms(ev.h[4 * i], ev.h[4 * i + 1]) for i in range(args.steps)]
    topk = [ev.ms(ev.h[4 * i + 1], ev.h[4 * i + 2]) for i in range(args.steps)]
    attend = [ev.ms(ev.h[4 * i + 2], ev.h[4 * i + 3]) for i in range(args.steps)]
    layer = [ev.ms(ev.h[4 * i], ev.h[4 * i + 3]) for i in range(args.steps)]
    ev.close()

    # the scan's access pattern without its arithmetic (read-only probe), same launches
    n_probe = max(10, args.steps // 2)
    pws_n = L.msa_route_workspace_bytes(bank.c, 1, 1)
    pws = M.workspace(pws_n, dev)
    for _ in range(3):
        L.msa_scan_read_probe(bank.c, pws, pws_n)
    pev = Events(2 * n_probe)
    for i in range(n_probe):
        torch.cuda.current_stream().record_event(pev.ev[2 * i])
        L.msa_scan_read_probe(bank.c, pws, pws_n)
        torch.cuda.current_stream().record_event(pev.ev[2 * i + 1])
    torch.cuda.synchronize()
    probe_ms = statistics.median(pev.ms(pev.h[2 * i], pev.h[2 * i + 1]) for i in range(n_probe))
    pev.close()

    # planted gold documents must be among each query's selection
    gi = idx.cpu().numpy()
    gold_ok = float(np.mean([set(w.gold[q].tolist()) <= set(gi[q].tolist()) for q in range(w.n_q)]))
    ms_seq = wall / args.steps * 1e3

    # pipelined steps: the same batch issued as independent steps, two in flight
    # (--sequential-only: skipped, value from the sequential steps; for profiles)
    if args.sequential_only:
        wall_p = wall
    else:
        wall_p = run_pipelined(bank, rope, w, scale, dev, QR, Q, Kl, Vl, idx, O_, args)
    ms_step = wall_p / args.steps * 1e3
    route_ms = statistics.mean(route)
    scan_bytes = w.n_chunks * (w.h_r * w.d_r * esz + 4 * w.h_r + 4)   # K^R rows + inverse norms + chunk->doc
    achieved = scan_bytes / (route_ms * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": w.n_tok / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": ("100M-token memory bank, one routed layer, decode: 16 queries x 1 token, k=16, "
                                "docs U[512,8192], chunk 128, 8 router heads x 128, 32 q / 8 KV heads x 128"),
                   "bank_tokens": w.n_tok, "n_docs": w.n_docs, "n_chunks": w.n_chunks, "queries": w.n_q,
                   "query_tokens": w.T, "k": w.k, "chunk": w.chunk},
        "pipelined": (None if args.sequential_only else
                      {"streams": 3, "overlap": "router scans of steps s and s+1 on two streams (grids capped at "
                                                "one workgroup per CU), top-k + attention of earlier steps on a "
                                                "third"}),
        "sequential": {"ms_per_step": ms_seq, "value": w.n_tok / (ms_seq * 1e-3)},
        "layer_latency_ms": statistics.median(layer),
        "stage_ms": {"route": statistics.median(route), "topk": statistics.median(topk),
                     "attend": statistics.median(attend)},
        "route_ms_p10_p50_p90": pct(route),
        "layer_ms_p10_p50_p90": pct(layer),
        "attend_roofline": attend_roofline(w, bank, gi, statistics.median(attend)),
        "route_tokens_per_s": w.n_tok / (route_ms * 1e-3),
        "roofline": {"bound": "hbm", "kernel": "route_scan", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": route_traffic(scan_bytes),
                     "bytes_per_launch": scan_bytes,
                     "pattern_floor": {"kernel": "scan_read_probe", "ms": probe_ms,
                                       "GB/s": scan_bytes / (probe_ms * 1e-3) / 1e9,
                                       "frac_of_peak": scan_bytes / (probe_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                       "scan_frac_of_floor": probe_ms / route_ms}},
        "pool": {"slabs": enc["slabs"], "GB/s": pool_gbs, "frac": pool_gbs / HBM_PEAK_GBS,
                 "tokens_per_s": w.n_tok / pool_s},
        "gold_recovered": gold_ok,
    }
    if not (args.no_interleave and args.no_secondary):
        del bank, ws  # the sub-records below build their own banks and inputs
        torch.cuda.empty_cache()
    # the secondary workloads run after the headline is measured; one that
    # raises records its error in its own field instead of losing the line
    subs = []
    if not args.no_interleave:
        subs.append(("interleave", lambda a: interleave_measure(a, 3)))   # the MFMA-bound workload
    if not args.no_secondary:
        subs += [("tiered", tiered_measure), ("append", append_measure), ("project", project_measure)]
    for name, measure in subs:
        print(f"[bench] {name} ...", file=sys.stderr, flush=True)
        try:
            sub = measure(args)
            rec[name] = {k: v for k, v in sub.items() if k not in ("n_gpus", "steps", "warmup", "dtype", "data")}
        except Exception as exc:  # noqa: BLE001 -- reported on the line, the headline stands
            rec[name] = {"error": f"{type(exc).__name__}: {exc}"}
            print(f"[bench] {name} failed: {exc!r}", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if cpu_rec is not None:
        rec["cpu_baseline"] = cpu_rec
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
