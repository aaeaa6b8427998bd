#!/usr/bin/env python3
"""Benchmark of one compressed-attention layer step on one MI355X.

Default workload: CSA decode, bf16, batch 32 at a 131072-token context
(32768 compressed entries, m=4; 64 index heads x 128; top-1024; 64 query heads
x 512 sharing the KV; window of 128 raw tokens; the new token's group is
compressed in the step).  A step = csa_compress + csa_index_topk +
csa_sparse_mqa through the C ABI, replayed from captured HIP graphs over R
input replicas (>= 1 GiB touched in rotation, so the 256 MB Infinity Cache
cannot serve repeats).  Inputs are resident in HBM before timing starts.

Printed: ONE JSON line with tokens/s (= B*Tq / step time), the roofline of
the call that takes longest alone (for the default decode step the lightning
indexer, HBM-bound: algorithmic bytes per launch over its HIP-event-timed
average duration; for a prefill chunk the MFMA-bound indexer or attention),
the oracle timed on the host's cores, and the other workloads as secondary
entries.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s
# counter-based HBM traffic of the indexer, measured by rocprofv3 on this
# workload and kept with the source digest of the kernel it was taken on
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_traffic_csa_decode_128K.txt")
TRAFFIC_WORKLOAD = "csa_decode_bf16_B32_ctx128K"  # the workload those counters were taken on
INDEXER_SOURCES = ["long_context_compressed_06_amd/csrc/indexer.hip", "long_context_compressed_06_amd/csrc/common.h",
                   "long_context_compressed_06_amd/csrc/kernels.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(wl) -> dict:
    """Unique HBM bytes the method must move once per step (overheads like
    scores, histograms and split-K partials excluded), and the indexer's share.

    Per sequence: the index keys visible to its last query (each read once),
    every query's index query and head weights, its q and fp32 output, its
    selection written and read back, the distinct entry rows attended (at most
    the visible entries; for one query, its selected rows), the distinct raw
    positions its windows cover, the new groups' logits and entry writes.  For
    a block of queries that share a cache (a prefill chunk) rows reused across
    queries count once: their re-reads are served by the caches."""
    es = 2 if wl.dtype == "bf16" else 4
    t_last = wl.q_pos0 + wl.Tq - 1
    nv_max = min(wl.N, (t_last + 1) // wl.m)
    win_span = min(wl.W + wl.Tq - 1, t_last + 1) if wl.W > 0 else 0
    per_query = wl.H * wl.d * es + wl.H * wl.d * 4
    if wl.mode == "csa":
        if wl.index_fmt == "mx4":
            # FP4 keys: dI/2 code bytes + dI/32 scale bytes per row; the element-type
            # index queries are read once by the quantiser
            key_row = wl.dI // 2 + wl.dI // 32
        else:
            key_row = wl.dI * es
        iq = wl.HI * wl.dI * es + wl.HI * 4
        indexer = nv_max * key_row + wl.Tq * iq
        sel_rows = min(sum(min(wl.k, min(wl.N, (wl.q_pos0 + ti + 1) // wl.m)) for ti in range(wl.Tq)), nv_max)
        step = indexer + wl.Tq * (per_query + 2 * wl.k * 4) + (sel_rows + win_span) * wl.d * es
    else:
        indexer = 0
        step = wl.Tq * per_query + (nv_max + win_span) * wl.d * es
    step += wl.G_new * wl.m * 4 + wl.G_new * wl.d * es  # new groups: logits, entry writes
    return {"step": step * wl.B, "indexer": indexer * wl.B}


def attention_bytes(wl) -> int:
    """Unique HBM bytes of one attention call (decode): per query its q, the
    fp32 output and lse, its selection read (CSA), the rows it attends (the
    selected or all visible entries, plus its window's raw rows)."""
    assert wl.Tq == 1
    es = 2 if wl.dtype == "bf16" else 4
    nv = min(wl.N, (wl.q_pos0 + 1) // wl.m)
    rows = (min(wl.k, nv) if wl.mode == "csa" else nv) + min(wl.W, wl.q_pos0 + 1)
    per_query = wl.H * wl.d * es + wl.H * wl.d * 4 + wl.H * 4 + (wl.k * 4 if wl.mode == "csa" else 0)
    return wl.B * (per_query + rows * wl.d * es)


def indexer_source_digest() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in INDEXER_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def indexer_traffic():
    """Counter-based bytes per indexer launch, or None when the profile is
    missing or was taken on different kernel source."""
    try:
        fields = dict(line.split(":", 1) for line in open(TRAFFIC_FILE) if ":" in line and not line.startswith(" "))
    except OSError:
        return None
    fields = {k.strip(): v.strip() for k, v in fields.items()}
    if fields.get("indexer_source_sha256") != indexer_source_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def replicas_for(x: dict) -> int:
    foot = sum(v.numel() * v.element_size() for v in x.values() if hasattr(v, "numel"))
    return max(2, min(8, math.ceil((1 << 30) / max(foot, 1)) + 1))


def clone_inputs(x):
    return {k: (v.clone() if hasattr(v, "clone") else v) for k, v in x.items()}


def capture(fn):
    import torch

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def time_graphs(graphs, steps, warmup, multi=None, per_multi=1):
    """Average ms per step over exactly `steps` steps.  `multi` (optional) is
    one graph holding `per_multi` consecutive steps; it is replayed while at
    least `per_multi` steps remain, the single-step graphs do the rest."""
    import torch

    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    left, i = steps, 0
    while multi is not None and left >= per_multi:
        multi.replay()
        left -= per_multi
    while left > 0:
        graphs[i % len(graphs)].replay()
        left -= 1
        i += 1
    end.record()
    end.synchronize()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA peak
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 (MXFP4) MFMA peak


def algorithmic_flops(wl) -> dict:
    """Indexer 2*n_vis*H_I*d_I and attention 4*(min(k, n_vis) + window)*H*d FLOPs per query, summed."""
    idx = att = 0
    for ti in range(wl.Tq):
        t = wl.q_pos0 + ti
        nv = min(wl.N, (t + 1) // wl.m)
        n_win = min(wl.W, t + 1)
        idx += 2 * nv * wl.HI * wl.dI
        att += 4 * ((min(wl.k, nv) if wl.mode == "csa" else nv) + n_win) * wl.H * wl.d
    return {"indexer": idx * wl.B, "attention": att * wl.B}


def attention_call(csa, wl, s, x):
    """The step's attention call alone (on the step's own selection for CSA)."""
    if wl.mode == "csa":
        return lambda: csa.csa_sparse_mqa(x["q"], x["entries"], s.topk_idx, x["raw"], wl.N, wl.m, wl.W, wl.q_pos0,
                                          wl.raw_pos0, scale=wl.scale, out=s.out, lse=s.lse, workspace=s.mqa_ws)
    return lambda: csa.hca_dense_mqa(x["q"], x["entries"], x["raw"], wl.N, wl.m, wl.W, wl.q_pos0, wl.raw_pos0,
                                     scale=wl.scale, out=s.out, lse=s.lse, workspace=s.mqa_ws)


def hbm_rooflines(wl, r) -> dict:
    """HBM rates of the decode step's indexer and attention calls timed alone."""
    out = {}
    if "indexer_ms" in r:
        b = algorithmic_bytes(wl)["indexer"]
        ach = b / (r["indexer_ms"] * 1e-3) / 1e9
        out["indexer"] = {"kernel": "k_index_mx4_dma (lightning indexer, FP4 keys)" if wl.index_fmt == "mx4"
                          else "k_index_dma (lightning indexer, bf16 keys)", "bound": "hbm", "achieved": ach,
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": checked_frac(ach / HBM_PEAK_GBS,
                                                                                      wl.name + " indexer"),
                          "bytes_per_launch": b, "avg_launch_us": r["indexer_ms"] * 1e3}
    if "attention_ms" in r:
        b = attention_bytes(wl)
        ach = b / (r["attention_ms"] * 1e-3) / 1e9
        out["attention"] = {"kernel": "k_mqa_wide + k_combine16 (one attention call)", "bound": "hbm",
                            "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": checked_frac(ach / HBM_PEAK_GBS, wl.name + " attention"),
                            "bytes_per_launch": b, "avg_launch_us": r["attention_ms"] * 1e3}
    return out


def mfma_rooflines(wl, r) -> dict:
    """MFMA rates of a prefill chunk's indexer and attention timed alone."""
    out = {}
    fl = algorithmic_flops(wl)
    for kern in ("indexer", "attention"):
        if kern + "_ms" not in r:
            continue
        tf = fl[kern] / (r[kern + "_ms"] * 1e-3) / 1e12
        # (an FP4 indexer against the FP4 peak, everything else against bf16's)
        pk = MFMA_FP4_PEAK_TFLOPS if kern == "indexer" and wl.index_fmt == "mx4" else MFMA_BF16_PEAK_TFLOPS
        name = {"indexer": "k_index_prefill_mx4 (FP4 keys)" if wl.index_fmt == "mx4" else "k_index_prefill",
                "attention": "k_mqa_wide + k_combine16 (one attention call)"}[kern]
        out[kern] = {"kernel": name, "bound": "mfma", "achieved": tf, "peak": pk, "unit": "TFLOP/s",
                     "frac": checked_frac(tf / pk, wl.name + " " + kern), "flops_per_launch": fl[kern],
                     "avg_launch_ms": r[kern + "_ms"]}
    return out


def bench_workload(wl, steps, warmup, with_kernel=True, with_mfma=False):
    import torch

    import long_context_compressed_06_amd as csa
    from workloads import make_inputs

    x0 = make_inputs(wl, "cuda")
    if wl.index_fmt == "mx4":
        # the cache holds the keys' FP4 form (quantised when they entered it)
        csa.AttentionStep.quantize_index_keys(x0)
        del x0["k_idx"]
        torch.cuda.synchronize()
    R = replicas_for(x0)
    xs = [x0] + [clone_inputs(x0) for _ in range(R - 1)]
    steps_ = [csa.AttentionStep.for_workload(wl) for _ in xs]
    for s, x in zip(steps_, xs):
        s(x)
    torch.cuda.synchronize()
    graphs = [capture(lambda s=s, x=x: s(x)) for s, x in zip(steps_, xs)]
    # one graph with a step on every replica in turn (fewer graph launches)
    multi = capture(lambda: [s(x) for s, x in zip(steps_, xs)])
    ms = time_graphs(graphs, steps, warmup, multi, R)
    res = {"ms_per_step": ms, "replicas": R}
    if with_kernel and wl.Tq == 1:
        # the lightning indexer and the attention call alone, same launch
        # configuration, 8 launches per graph over the replicas, timed with HIP
        # events on the stream they run on
        if wl.mode == "csa":
            sc = [torch.empty((wl.B, wl.Tq, wl.N), dtype=torch.float32, device="cuda") for _ in xs]
            if wl.index_fmt == "mx4":
                idx_call = [lambda x=x, o=o: csa.csa_index_scores_mx4(x["q_idx"], x["w_idx"], x["k_codes"],
                                                                      x["k_scales"], wl.N, wl.m, wl.q_pos0, scores=o)
                            for x, o in zip(xs, sc)]
            else:
                idx_call = [lambda x=x, o=o: csa.csa_index_scores(x["q_idx"], x["w_idx"], x["k_idx"], wl.N, wl.m,
                                                                  wl.q_pos0, scores=o) for x, o in zip(xs, sc)]
            kg = [capture(f) for f in idx_call]
            km = capture(lambda: [idx_call[i % R]() for i in range(8)])
            res["indexer_ms"] = time_graphs(kg, steps, warmup, km, 8)
            del sc, kg, km
        att_call = [attention_call(csa, wl, s, x) for s, x in zip(steps_, xs)]
        kg = [capture(f) for f in att_call]
        km = capture(lambda: [att_call[i % R]() for i in range(8)])
        res["attention_ms"] = time_graphs(kg, steps, warmup, km, 8)
        del kg, km
    if with_mfma and wl.mode == "csa":
        # the two MFMA-bound kernels alone (prefill chunks), each timed from graphs over the replicas
        sc = [torch.empty((wl.B, wl.Tq, wl.N), dtype=torch.float32, device="cuda") for _ in xs]
        if wl.index_fmt == "mx4":
            idx_call = [lambda x=x, o=o: csa.csa_index_scores_mx4(x["q_idx"], x["w_idx"], x["k_codes"],
                                                                  x["k_scales"], wl.N, wl.m, wl.q_pos0, scores=o)
                        for x, o in zip(xs, sc)]
        else:
            idx_call = [lambda x=x, o=o: csa.csa_index_scores(x["q_idx"], x["w_idx"], x["k_idx"], wl.N, wl.m,
                                                              wl.q_pos0, scores=o) for x, o in zip(xs, sc)]
        res["indexer_ms"] = time_graphs([capture(f) for f in idx_call], max(3, steps // 4), 2)
        del sc
        att_call = [attention_call(csa, wl, s, x) for s, x in zip(steps_, xs)]
        res["attention_ms"] = time_graphs([capture(f) for f in att_call], max(3, steps // 4), 2)
    del graphs, steps_, xs, x0
    torch.cuda.empty_cache()
    return res


LOOP_LAYERS = 2  # layer states alternating in the decode loop (the keys of one do not fit the Infinity Cache)


def loop_bytes(sq) -> int:
    """Algorithmic bytes of one decode cycle (m steps per layer, every layer): per step the
    visible index keys, index query and weights, the selected and window rows, q, the fp32
    output, the appended raw row and logit; per cycle one group's compression (its logits,
    the entry write) and the appended index key."""
    es = 2 if sq.dtype == "bf16" else 4
    row_i = (sq.dI // 2 + sq.dI // 32) if sq.index_fmt == "mx4" else sq.dI * es
    lg = sq.d * 4 if sq.pool == "channel" else 4        # one token's pooling logits
    total = 0
    for j in range(sq.m):
        t = sq.T + j
        nv = (t + 1) // sq.m
        total += nv * row_i + sq.HI * sq.dI * es + sq.HI * 4
        total += (min(sq.k, nv) + min(sq.W, t + 1)) * sq.d * es + sq.H * sq.d * es + sq.H * sq.d * 4 + 2 * sq.k * 4
        total += sq.d * es + lg
        if sq.index_keys == "pooled":  # the token's index key (and its logits) into their ring
            total += sq.dI * es + (sq.dI * 4 if sq.pool == "channel" else 0)
    total += sq.m * lg + sq.d * es + row_i
    if sq.index_keys == "pooled":      # the group's index-key rows (and logits) read by the compressor
        total += sq.m * sq.dI * es + (sq.m * sq.dI * 4 if sq.pool == "channel" else 0)
    return total * sq.B * LOOP_LAYERS


def bench_loop(sq, cycles, warmup):
    """Decode loop with cache maintenance: LOOP_LAYERS layers resumed at position T, one graph of m
    decode steps on each (positions T .. T+m-1; the m-th emits a group), replayed."""
    import torch

    import long_context_compressed_06_amd as csa

    B, m, R_ = sq.B, sq.m, None
    g = torch.Generator(device="cuda")
    g.manual_seed(sq.seed_base + 11)
    rn = lambda *shape, std=1.0: torch.randn(shape, generator=g, device="cuda") * std
    layers = []
    for _ in range(LOOP_LAYERS):
        L = csa.StreamingLayer(mode=sq.mode, B=B, H=sq.H, d=sq.d, m=m, W=sq.W, capacity=sq.T + m, chunk=1,
                               dtype=sq.torch_dtype, k=sq.k, HI=sq.HI, dI=sq.dI, index_fmt=sq.index_fmt,
                               scale=sq.scale, pool=sq.pool, index_keys=sq.index_keys)
        N0 = sq.T // m
        L.entries[:, :N0] = rn(B, N0, sq.d).to(L.entries.dtype)
        kI = rn(B, N0, sq.dI, std=sq.dI ** -0.5).to(sq.torch_dtype)
        if sq.index_fmt == "mx4":
            c, s_ = csa.csa_mx4_quantize(kI)
            L.k_codes[:, :N0], L.k_scales[:, :N0] = c, s_
        else:
            L.k_idx[:, :N0] = kI
        del kI
        half = rn(B, L.R, sq.d).to(sq.torch_dtype)
        L.raw_ring[:, :L.R], L.raw_ring[:, L.R:] = half, half
        lg = rn(B, L.R, L.logit_ring.shape[2])
        L.logit_ring[:, :L.R], L.logit_ring[:, L.R:] = lg, lg
        if sq.index_keys == "pooled":
            kt = rn(B, L.R, sq.dI, std=sq.dI ** -0.5).to(sq.torch_dtype)
            L.kidx_ring[:, :L.R], L.kidx_ring[:, L.R:] = kt, kt
            if sq.pool == "channel":
                kl = rn(B, L.R, sq.dI)
                L.kidx_logit_ring[:, :L.R], L.kidx_logit_ring[:, L.R:] = kl, kl
        R_ = L.R
        layers.append(L)
    # per-step inputs (one token per sequence)
    steps_in = []
    for j in range(m):
        x = {"raw": rn(B, 1, sq.d).to(sq.torch_dtype),
             "logits": rn(B, 1, sq.d) if sq.pool == "channel" else rn(B, 1),
             "q": rn(B, 1, sq.H, sq.d).to(sq.torch_dtype),
             "k_idx_tokens": rn(B, 1, sq.dI, std=sq.dI ** -0.5).to(sq.torch_dtype), "k_idx_logits": rn(B, 1, sq.dI),
             "q_idx": rn(B, 1, sq.HI, sq.dI, std=sq.dI ** -0.5).to(sq.torch_dtype),
             "w_idx": torch.rand((B, 1, sq.HI), generator=g, device="cuda"),
             "k_idx_new": rn(B, 1, sq.dI, std=sq.dI ** -0.5).to(sq.torch_dtype)}
        steps_in.append(x)
    outs = [(torch.empty((B, 1, sq.H, sq.d), device="cuda"), torch.empty((B, 1, sq.H), device="cuda"),
             torch.empty((B, 1, sq.k), dtype=torch.int32, device="cuda")) for _ in range(m * LOOP_LAYERS)]

    def cycle():
        for L in layers:
            L.resume(sq.T)
        for j in range(m):
            x = steps_in[j]
            for li, L in enumerate(layers):
                o, l_, ti = outs[j * LOOP_LAYERS + li]
                kw = {}
                if sq.index_keys == "pooled":
                    kw["k_idx_tokens"] = x["k_idx_tokens"]
                    if sq.pool == "channel":
                        kw["k_idx_logits"] = x["k_idx_logits"]
                elif L.plan(1).g_new:
                    kw["k_idx_new"] = x["k_idx_new"]
                L.step(x["raw"], x["logits"], x["q"], q_idx=x["q_idx"], w_idx=x["w_idx"], out=o, lse=l_,
                       topk_idx=ti, **kw)

    cycle()
    torch.cuda.synchronize()
    graph = capture(cycle)
    ms = time_graphs([graph], cycles, warmup)
    del graph, layers, steps_in, outs
    torch.cuda.empty_cache()
    return {"ms_per_cycle": ms, "ring_positions": R_}


def bench_prefill(sq, reps, warmup):
    """A whole prefill from position 0 through the streaming layer (chunks of sq.chunks), one graph."""
    import torch

    import long_context_compressed_06_amd as csa

    g = torch.Generator(device="cuda")
    g.manual_seed(sq.seed_base + 11)
    rn = lambda shape, std=1.0: torch.randn(shape, generator=g, device="cuda") * std
    B, T = sq.B, sq.T
    dt = sq.torch_dtype
    x = {"raw": rn((B, T, sq.d)).to(dt), "logits": rn((B, T)), "q": rn((B, T, sq.H, sq.d)).to(dt),
         "k_idx": rn((B, T // sq.m, sq.dI), sq.dI ** -0.5).to(dt),
         "q_idx": rn((B, T, sq.HI, sq.dI), sq.dI ** -0.5).to(dt),
         "w_idx": torch.rand((B, T, sq.HI), generator=g, device="cuda")}
    sched = sq.schedule()
    C = max(sched)
    layer = csa.StreamingLayer(mode=sq.mode, B=B, H=sq.H, d=sq.d, m=sq.m, W=sq.W, capacity=T, chunk=C, dtype=dt,
                               k=sq.k, HI=sq.HI, dI=sq.dI, index_fmt=sq.index_fmt, scale=sq.scale)
    out = torch.empty((B, C, sq.H, sq.d), device="cuda")
    lse = torch.empty((B, C, sq.H), device="cuda")
    idx = torch.empty((B, C, sq.k), dtype=torch.int32, device="cuda")
    # contiguous per-chunk inputs, prepared once
    chunks, p = [], 0
    for n in sched:
        chunks.append({k: x[k][:, p:p + n].contiguous() for k in ("raw", "logits", "q", "q_idx", "w_idx")})
        p += n

    def prefill():
        layer.resume(0)
        p = 0
        for n, c in zip(sched, chunks):
            pl = layer.plan(n)
            layer.step(c["raw"], c["logits"], c["q"], k_idx_new=x["k_idx"][:, pl.g0:pl.g0 + pl.g_new],
                       q_idx=c["q_idx"], w_idx=c["w_idx"], out=out[:, :n], lse=lse[:, :n], topk_idx=idx[:, :n])
            p += n

    prefill()
    torch.cuda.synchronize()
    graph = capture(prefill)
    ms = time_graphs([graph], reps, warmup)
    del graph, layer, x, chunks
    torch.cuda.empty_cache()
    return {"ms_per_prefill": ms, "chunks": len(sched), "chunk": C}


def ragged_bytes(rs) -> int:
    """Algorithmic bytes of one stack step at the starting positions: per layer and sequence the visible
    index keys (CSA), index query and weights, the attended rows (selected or all visible entries plus the
    window), q, the fp32 output, the appended raw row and logit; one group's compression every m tokens."""
    es = 2 if rs.dtype == "bf16" else 4
    total = 0
    for spec in rs.specs():
        m = spec["m"]
        for t in rs.lengths:
            nv = (t + 1) // m
            row = rs.H * rs.d * es + rs.H * rs.d * 4 + rs.d * es + 4
            if spec["mode"] == "csa":
                row += nv * spec["dI"] * es + spec["HI"] * spec["dI"] * es + spec["HI"] * 4
                row += (min(spec["k"], nv) + rs.W) * rs.d * es + 2 * spec["k"] * 4
                row += (m * 4 + rs.d * es + spec["dI"] * es) / m
            else:
                row += (nv + rs.W) * rs.d * es + (m * 4 + rs.d * es) / m
            total += row
    return int(total)


def bench_ragged(rs, steps, warmup):
    """Ragged decode through a stack of layers: one captured stack step replayed for every token, the
    positions advancing on the GPU (groups are emitted whenever a sequence completes one)."""
    import torch

    import long_context_compressed_06_amd as csa

    g = torch.Generator(device="cuda")
    g.manual_seed(rs.seed_base + 11)
    dt = torch.bfloat16 if rs.dtype == "bf16" else torch.float32
    B = rs.B
    cap = max(rs.lengths) + steps + warmup + 256
    stack = csa.HybridStack(rs.specs(), B=B, H=rs.H, d=rs.d, W=rs.W, capacity=cap, dtype=dt)
    pos = torch.tensor(rs.lengths, dtype=torch.int64, device="cuda")
    inputs = []
    for L in stack.layers:
        for t in [L.entries] + ([L.k_idx] if L.mode == "csa" else []):
            sc = t.shape[-1] ** -0.5 if t is not L.entries else 1.0
            for part in t.view(-1, t.shape[-1]).split(1 << 20):  # (bounded temporaries; any cache layout)
                part.copy_(torch.randn(part.shape, generator=g, device="cuda") * sc)
        L.raw_ring.copy_(torch.randn(L.raw_ring.shape, generator=g, device="cuda"))
        L.logit_ring.copy_(torch.randn(L.logit_ring.shape, generator=g, device="cuda"))
        L.pos.copy_(pos)
        x = {"raw": torch.randn((B, 1, rs.d), generator=g, device="cuda").to(dt),
             "logits": torch.randn((B, 1), generator=g, device="cuda"),
             "q": torch.randn((B, 1, rs.H, rs.d), generator=g, device="cuda").to(dt)}
        if L.mode == "csa":
            x.update(k_idx_tok=(torch.randn((B, 1, L.dI), generator=g, device="cuda") * L.dI ** -0.5).to(dt),
                     q_idx=(torch.randn((B, 1, L.HI, L.dI), generator=g, device="cuda") * L.dI ** -0.5).to(dt),
                     w_idx=torch.rand((B, 1, L.HI), generator=g, device="cuda"))
        inputs.append(x)
    stack.step(inputs)  # (first launches outside the capture)
    torch.cuda.synchronize()
    graph = capture(lambda: stack.step(inputs))
    ms = time_graphs([graph], steps, warmup)
    del graph, stack, inputs
    torch.cuda.empty_cache()
    return {"ms_per_step": ms}


def stream_ceiling_gbs(fronts: int, reps=10) -> float:
    """Measured streaming-read reference on the same GPU: csa_stream_read over 2 GiB (beyond the 256 MB
    Infinity Cache) as `fronts` concurrent fronts, bytes read per second."""
    import torch

    import long_context_compressed_06_amd as csa

    buf = torch.empty(1 << 31, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    for _ in range(2):
        csa.csa_stream_read(buf, fronts, sink)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        csa.csa_stream_read(buf, fronts, sink)
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b) / reps
    del buf, sink
    torch.cuda.empty_cache()
    return (1 << 31) / (ms * 1e-3) / 1e9


# the prefill chunk's oracle baseline runs on these query rows (its first and
# last 128): every row of the chunk would take minutes of host time
PREFILL_BASELINE_ROWS = 128


def cpu_baseline(wl, min_seconds=10.0, max_reps=40):
    """The oracle, as it stands, on the same workload's inputs (host copies):
    the whole step, or for a block of many queries a stated subset of rows."""
    import torch

    import oracle
    from workloads import make_inputs

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from chain import host_inputs, oracle_step

    x = make_inputs(wl, "cuda")
    xh = host_inputs(x)
    del x
    torch.cuda.empty_cache()
    rows = None
    n_rows = wl.B * wl.Tq
    if wl.Tq > 2 * PREFILL_BASELINE_ROWS:
        rows = [(0, PREFILL_BASELINE_ROWS), (wl.Tq - PREFILL_BASELINE_ROWS, wl.Tq)]
        n_rows = wl.B * 2 * PREFILL_BASELINE_ROWS
    reps, t0 = 0, time.perf_counter()
    while reps < max_reps:
        oracle_step(wl, xh, rows)
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    el = time.perf_counter() - t0
    what = (f"whole step of the {wl.name} workload (all {wl.B} sequences: compression, "
            + (f"indexer over {wl.N} entries, top-{wl.k}, attention)" if wl.mode == "csa"
               else f"dense attention over {wl.N} entries)"))
    if rows is not None:
        what = (f"query rows 0-{PREFILL_BASELINE_ROWS - 1} and {wl.Tq - PREFILL_BASELINE_ROWS}-{wl.Tq - 1} of the "
                f"{wl.name} workload ({n_rows} of {wl.B * wl.Tq} rows; compression of all new groups, indexer over "
                f"up to {wl.N} entries, top-{wl.k}, attention), tokens/s = rows/s")
    return {"value": n_rows * reps / el, "unit": "tokens/s", "cores": oracle.default_threads(), "kind": "oracle",
            "sample": f"{what} repeated {reps}x in {el:.1f} s"}


def checked_frac(frac: float, what: str) -> float:
    """A fraction of a peak above 1 means the bytes or FLOPs counted are wrong."""
    assert frac <= 1.0, f"{what}: fraction {frac:.3f} of the peak is above 1"
    return frac


# secondary workloads that also get an oracle baseline (the 1M decodes and the prefill chunk)
BASELINE_ALSO = ("c3", "c5", "c4")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2", help="c2 (default; the metric's configuration) or another config")
    ap.add_argument("--also", default="c3,c5,c4,c2x,c5x,c4x,l2,l2x,l2c,p1,r1,r1p,r2",
                    help="secondary workloads ('' for none); c4: the 64K prefill chunk (tokens/s and the MFMA "
                         "fractions of its indexer and attention); c2x/c5x/c4x: FP4 (MXFP4) indexer operands; "
                         "l2/l2x/l2c: decode loops with cache maintenance (l2c: per-channel pooling, pooled "
                         "index keys); p1: a whole chunked prefill from 0; r1/r2: ragged decode (lengths "
                         "96K..158K) through one CSA layer / a CSA + HCA stack, one graph per token; r1p: r1 with "
                         "caches in 64-row pages")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for the HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log("bench.py measures one GPU: the library has no multi-GPU path (one process, one MI355X). Use --gpus 1.")
        sys.exit(2)

    import torch

    from workloads import CONFIGS, LOOPS, PREFILLS, RAGGED

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = CONFIGS[args.workload]
    log(f"[bench] {wl}")
    r = bench_workload(wl, args.steps, args.warmup, with_kernel=wl.Tq == 1, with_mfma=wl.Tq > 1)
    ab = algorithmic_bytes(wl)
    toks = wl.B * wl.Tq / (r["ms_per_step"] * 1e-3)
    line = {
        "metric": "compressed-attn decode tokens/s + % HBM roofline at 128K and 1M ctx",
        "value": toks,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "context": wl.T, "m": wl.m, "entries": wl.N, "top_k": wl.k,
                   "index_heads": wl.HI, "index_dim": wl.dI, "heads": wl.H, "head_dim": wl.d, "window": wl.W,
                   "input_replicas": r["replicas"], "graph_replay": "one graph per pass over the replicas"},
        "step_hbm": {"algorithmic_bytes": ab["step"],
                     "achieved_GBs": ab["step"] / (r["ms_per_step"] * 1e-3) / 1e9,
                     "frac": checked_frac(ab["step"] / (r["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, wl.name)},
    }
    # the roofline of the call that takes the longest alone (the dominant kernel)
    kern = mfma_rooflines(wl, r) if wl.Tq > 1 else hbm_rooflines(wl, r)
    if kern:
        dom = max(kern, key=lambda k: r[k + "_ms"])
        line["roofline"] = dict(kern[dom], traffic=None)
        if dom == "indexer" and wl.Tq == 1 and wl.index_fmt == "elem":
            c1, c32 = stream_ceiling_gbs(1), stream_ceiling_gbs(32)
            line["roofline"]["traffic"] = indexer_traffic() if wl.name == TRAFFIC_WORKLOAD else None
            line["roofline"]["measured_ceiling"] = {"what": "csa_stream_read of 2 GiB on the same GPU (the "
                                                            "indexer's LDS-DMA load path), bytes read per second",
                                                    "one_front_GBs": c1, "32_fronts_GBs": c32}
            line["roofline"]["frac_of_measured_ceiling"] = line["roofline"]["achieved"] / c32
        line["kernels"] = kern
    also = {}
    for name in [a for a in args.also.split(",") if a and a != args.workload]:
        if name in RAGGED:
            rs = RAGGED[name]
            log(f"[bench] also {rs.name}")
            r2 = bench_ragged(rs, max(16, args.steps), max(4, args.warmup // 2))
            b2 = ragged_bytes(rs)
            also[rs.name] = {"tokens_per_s": rs.B / (r2["ms_per_step"] * 1e-3), "ms_per_step": r2["ms_per_step"],
                             "layers": "+".join(s["mode"] for s in rs.specs()),
                             "page_rows": [s.get("page_rows", 0) for s in rs.specs()],
                             "step_hbm_frac": checked_frac(b2 / (r2["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                                           rs.name),
                             "algorithmic_bytes": b2,
                             "step": f"one token of each of {rs.B} sequences (lengths {min(rs.lengths)}.."
                                     f"{max(rs.lengths)}) through every layer, one captured graph replayed per "
                                     f"token, positions advancing on the GPU"}
            continue
        if name in PREFILLS:
            sq = PREFILLS[name]
            log(f"[bench] also {sq}")
            r2 = bench_prefill(sq, 3, 1)
            also[sq.name] = {"tokens_per_s": sq.B * sq.T / (r2["ms_per_prefill"] * 1e-3),
                             "ms_per_prefill": r2["ms_per_prefill"],
                             "prefill": f"{sq.B} x {sq.T} tokens from position 0 in {r2['chunks']} chunks of "
                                        f"{r2['chunk']}: append, compress, index-key append, index + top-k, "
                                        f"attention per chunk"}
            continue
        if name in LOOPS:
            sq = LOOPS[name]
            log(f"[bench] also {sq}")
            r2 = bench_loop(sq, max(5, args.steps // 4), max(2, args.warmup // 4))
            toks = sq.B * sq.m * LOOP_LAYERS
            b2 = loop_bytes(sq)
            also[sq.name] = {"tokens_per_s": toks / (r2["ms_per_cycle"] * 1e-3),
                             "ms_per_layer_step": r2["ms_per_cycle"] / (sq.m * LOOP_LAYERS),
                             "step_hbm_frac": checked_frac(b2 / (r2["ms_per_cycle"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                                           sq.name),
                             "algorithmic_bytes_per_cycle": b2,
                             "cycle": f"{sq.m} decode steps x {LOOP_LAYERS} layers from position {sq.T}, "
                                      f"ring of {r2['ring_positions']} positions, one group emitted per layer"}
            continue
        w2 = CONFIGS[name]
        log(f"[bench] also {w2}")
        prefill = w2.Tq > 1
        r2 = bench_workload(w2, max(10, args.steps // 2) if not prefill else max(5, args.steps // 5), args.warmup,
                            with_kernel=not prefill, with_mfma=prefill)
        b2 = algorithmic_bytes(w2)["step"]
        also[w2.name] = {"tokens_per_s": w2.B * w2.Tq / (r2["ms_per_step"] * 1e-3), "ms_per_step": r2["ms_per_step"],
                         "step_hbm_frac": checked_frac(b2 / (r2["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, w2.name),
                         "algorithmic_bytes": b2}
        for kern, v in (mfma_rooflines(w2, r2) if prefill else hbm_rooflines(w2, r2)).items():
            also[w2.name][kern + ("_mfma" if prefill else "_hbm")] = v
        if not args.no_cpu_baseline and name in BASELINE_ALSO:
            log(f"[bench] cpu baseline (oracle) {w2.name}")
            also[w2.name]["cpu_baseline"] = cpu_baseline(w2)
    if also:
        line["also"] = also
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")  # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
