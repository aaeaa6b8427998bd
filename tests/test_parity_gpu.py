"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case prints its name, shape and seed before touching the GPU.  Inputs
are seeded synthetic tensors drawn on the GPU; the oracle receives host copies
taken before the step runs.  Rules (tests/helpers.py): bf16 max 2e-2 / mean
2e-3 absolute, fp32 1e-5 normwise per row, top-k rule T, bookkeeping exact.
The chain is compared on every row: its out and lse against the oracle's
attention evaluated on the GPU's own selection (once that selection passed
rule T), so a legal near-tie swap is neither an error nor a row left
unchecked.  The attention kernel is also run alone on the oracle's own
selection and compared with the oracle's output.
"""
import sys

import numpy as np
import pytest
import torch

from chain import host_inputs, oracle_attention_on, oracle_step
from helpers import assert_close, check_topk, nvis_rows, to_np
from workloads import CONFIGS, Workload, make_inputs, scaled

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    import long_context_compressed_06_amd as m

    m.lib()
    assert torch.cuda.is_available(), "no GPU visible"
    return m


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def run_and_check(csa, wl: Workload, entries_capacity=None):
    say(wl)
    x = make_inputs(wl, "cuda", entries_capacity=entries_capacity)
    xh = host_inputs(x)
    if wl.index_fmt == "mx4":  # the cache holds the keys' FP4 form
        csa.AttentionStep.quantize_index_keys(x)
    step = csa.AttentionStep.for_workload(wl)
    out = step(x)
    torch.cuda.synchronize()
    ref = oracle_step(wl, xh)
    # a1: compressed entries against the unrounded oracle value
    if ref["e"] is not None:
        assert_close(x["entries"][:, wl.g0:wl.N], ref["e"], wl.dtype, "entries")
    if wl.mode == "csa":
        gidx = to_np(step.topk_idx)
        swapped = check_topk(gidx, ref["idx"], ref["scores"], nvis_rows(wl), wl.k, "topk")
        # the chain, every row: out and lse against the oracle's attention on the GPU's own selection
        ro, rl = oracle_attention_on(xh["q"], ref["entries"], gidx, xh["raw"], wl.raw_pos0, wl.W, wl.q_pos0,
                                     wl.scale)
        assert_close(out, ro, wl.dtype, "chain out")
        assert_close(step.lse, rl, wl.dtype, "chain lse", row_dims=1)
        # the attention kernel alone on the oracle's own selection
        ridx = torch.from_numpy(np.ascontiguousarray(ref["idx"])).cuda()
        lse2 = torch.empty(x["q"].shape[:3], device="cuda")
        o2 = csa.csa_sparse_mqa(x["q"], x["entries"], ridx, x["raw"], wl.N, wl.m, wl.W, wl.q_pos0, wl.raw_pos0,
                                scale=wl.scale, lse=lse2)
        torch.cuda.synchronize()
        assert_close(o2, ref["out"], wl.dtype, "attention(oracle idx)")
        assert_close(lse2, ref["lse"], wl.dtype, "attention(oracle idx) lse", row_dims=1)
        say(f"top-k rows with a legal near-tie swap: {swapped} of {gidx.shape[0] * gidx.shape[1]}")
    else:
        assert_close(out, ref["out"], wl.dtype, "out")
        assert_close(step.lse, ref["lse"], wl.dtype, "lse", row_dims=1)
    return x, step, ref


# ---------------------------------------------------------------- full configs
def test_c1_tiny_prefill_fp32(csa):
    run_and_check(csa, CONFIGS["c1"])


def test_c2_csa_decode_128k(csa):
    run_and_check(csa, CONFIGS["c2"])


def test_c3_hca_decode_1m(csa):
    run_and_check(csa, CONFIGS["c3"])


def test_c4_csa_prefill_chunk_all_rows(csa):
    """All 4096 query rows of the 64K prefill chunk against the oracle (about 2.3 TFLOP of fp64 oracle work)."""
    run_and_check(csa, CONFIGS["c4"])


def test_c5_csa_decode_1m_stress(csa):
    run_and_check(csa, CONFIGS["c5"])


def test_c2x_csa_decode_128k_fp4_indexer(csa):
    run_and_check(csa, CONFIGS["c2x"])


def test_c5x_csa_decode_1m_stress_fp4_indexer(csa):
    run_and_check(csa, CONFIGS["c5x"])


def test_c4x_csa_prefill_chunk_fp4_indexer_all_rows(csa):
    """The 64K prefill chunk with FP4 index operands (the query-blocked FP4 indexer), all 4096 rows."""
    run_and_check(csa, CONFIGS["c4x"])


# ------------------------------------------------------- small and ragged shapes
SMALL = [
    # name, dtype, B, T, Tq, m, d, H, W, k, HI, dI
    ("csa_bf16_ragged", "bf16", 2, 1003, 37, 4, 128, 64, 16, 50, 64, 128),
    ("csa_bf16_k_ge_n", "bf16", 1, 300, 9, 4, 64, 16, 8, 2048, 16, 64),
    ("csa_f32_m1", "f32", 2, 200, 11, 1, 32, 8, 5, 17, 4, 32),
    ("csa_f32_d512", "f32", 1, 700, 3, 4, 512, 20, 33, 100, 17, 128),
    ("csa_bf16_no_window", "bf16", 3, 500, 4, 4, 256, 64, 0, 64, 64, 128),
    ("csa_bf16_w1_h1", "bf16", 2, 4097, 2, 4, 512, 1, 1, 1000, 1, 32),
    ("csa_bf16_early_queries", "bf16", 1, 40, 40, 4, 128, 8, 3, 5, 4, 32),
    ("csa_bf16_big_row", "bf16", 1, 4 * 40000, 1, 4, 128, 16, 128, 1024, 64, 128),
    ("csa_bf16_prefill_blocks", "bf16", 2, 2403, 100, 4, 128, 16, 8, 64, 20, 64),
    ("csa_bf16_prefill_d32", "bf16", 1, 1000, 70, 4, 64, 8, 4, 50, 4, 32),
    ("csa_bf16_many_queries", "bf16", 2, 1300, 300, 4, 256, 8, 16, 40, 16, 32),
    ("csa_bf16_fp4_indexer", "bf16:mx4", 2, 4 * 2000 + 3, 5, 4, 128, 16, 16, 300, 64, 128),
    ("hca_bf16_ragged", "bf16", 2, 128 * 77 + 5, 3, 128, 512, 64, 128, 0, 0, 0),
    # d = 512 bf16 with few queries: head groups of 16 (a partial group here), one split per query below
    ("csa_bf16_d512_h20", "bf16", 2, 3001, 3, 4, 512, 20, 33, 200, 17, 128),
    ("csa_bf16_d512_one_split", "bf16", 1, 2000, 70, 4, 512, 64, 16, 100, 16, 64),
    ("hca_bf16_many_queries", "bf16", 1, 128 * 10 + 600, 600, 128, 128, 16, 32, 0, 0, 0),
    ("hca_f32_m1_w0", "f32", 1, 150, 150, 1, 64, 4, 0, 0, 0, 0),
    ("hca_bf16_window_only", "bf16", 1, 100, 100, 128, 128, 64, 16, 0, 0, 0),
    # one query over 30016 rows of d = 512: more splits than one batch of the split-K merge
    ("hca_bf16_many_splits", "bf16", 1, 4 * 30000, 1, 4, 512, 64, 16, 0, 0, 0),
    # the 32-head-wavefront kernel with a partial second head group (heads >= H: clamped query rows,
    # nothing stored), split and unsplit queries
    ("csa_bf16_d512_h48", "bf16", 2, 3001, 3, 4, 512, 48, 33, 200, 17, 128),
    ("hca_bf16_d512_h40", "bf16", 1, 128 * 40 + 7, 2, 128, 512, 40, 16, 0, 0, 0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes(csa, case):
    name, dt, B, T, Tq, m, d, H, W, k, HI, dI = case
    dt, _, fmt = dt.partition(":")
    wl = Workload(name, dt, B=B, T=T, Tq=Tq, m=m, d=d, H=H, W=W, k=k, HI=HI, dI=dI,
                  seed_base=90000 + 1000 * SMALL.index(case), index_fmt=fmt or "elem")
    run_and_check(csa, wl, entries_capacity=wl.N + 40)


# ----------------------------------------------------------------- exact ties
def test_topk_exact_integer_scores(csa):
    """Small-integer index keys and dyadic head weights make every score exact in
    float32, with many ties: the selection must equal the oracle's bit for bit."""
    wl = Workload("ties", "bf16", B=2, T=4 * 3000, Tq=3, m=4, d=128, H=16, W=4, k=700, HI=16, dI=32, seed_base=77000)
    say(wl)
    g = torch.Generator(device="cuda").manual_seed(77001)
    x = make_inputs(wl, "cuda")
    x["k_idx"] = torch.randint(-2, 3, x["k_idx"].shape, generator=g, device="cuda").to(torch.bfloat16)
    x["q_idx"] = torch.randint(-2, 3, x["q_idx"].shape, generator=g, device="cuda").to(torch.bfloat16)
    x["w_idx"] = torch.randint(0, 5, x["w_idx"].shape, generator=g, device="cuda").float() * 0.25
    xh = host_inputs(x)
    step = csa.AttentionStep.for_workload(wl)
    step(x)
    torch.cuda.synchronize()
    ref = oracle_step(wl, xh)
    assert np.array_equal(to_np(step.topk_idx), ref["idx"])


@pytest.mark.parametrize("n_entries,tq", [(20000, 2), (70000, 2), (20000, 256)],
                         ids=["filter_20k", "filter_70k", "one_pass_20k"])
def test_topk_all_scores_equal(csa, n_entries, tq):
    """Zero index queries make every visible score 0: all keys tie, more pairs
    than the LDS holds share the k-th digit, and the kept set must be the
    first k visible entries (ties go to the lower index)."""
    wl = Workload("equal", "bf16", B=1, T=4 * n_entries, Tq=tq, m=4, d=128, H=8, W=4, k=1000, HI=16, dI=32,
                  seed_base=76000)
    say(wl)
    x = make_inputs(wl, "cuda")
    x["q_idx"].zero_()
    xh = host_inputs(x)
    step = csa.AttentionStep.for_workload(wl)
    step(x)
    torch.cuda.synchronize()
    ref = oracle_step(wl, xh)
    got = to_np(step.topk_idx)
    assert np.array_equal(got, ref["idx"])
    assert np.array_equal(got[0, 0], np.arange(wl.k))


@pytest.mark.parametrize("tq", [5, 80], ids=["few_queries", "query_blocked"])
def test_scores_out_and_masking(csa, tq):
    wl = Workload("scores", "bf16", B=2, T=4 * 700 + 3, Tq=tq, m=4, d=128, H=16, W=4, k=64, HI=64, dI=128,
                  seed_base=78000)
    say(wl)
    x = make_inputs(wl, "cuda")
    xh = host_inputs(x)
    sc = torch.empty((wl.B, wl.Tq, wl.N), device="cuda")
    csa.csa_index_topk(x["q_idx"], x["w_idx"], x["k_idx"], wl.N, wl.m, wl.k, wl.q_pos0, scores_out=sc)
    torch.cuda.synchronize()
    ref = oracle_step(wl, xh)["scores"]
    got = to_np(sc)
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    fin = np.isfinite(ref)
    rel = np.abs(got[fin] - ref[fin]).max() / np.abs(ref[fin]).max()
    assert rel <= 1e-5, rel


# ------------------------------------------------------ poison, empty, determinism
@pytest.mark.parametrize("d", [256, 512])
def test_poisoned_memory_is_never_read(csa, d):
    """Entries and index keys beyond N, and raw rows outside every window, are
    filled with large finite values: outputs must not change by a single bit."""
    wl = Workload("poison", "bf16", B=2, T=4 * 2000 + 2, Tq=4, m=4, d=d, H=64, W=32, k=300, HI=64, dI=128,
                  seed_base=79000)
    say(wl)
    outs = []
    for poison in (False, True):
        x = make_inputs(wl, "cuda", entries_capacity=wl.N + 64)
        if poison:
            x["entries"][:, wl.N:] = 3e4
            x["k_idx"][:, wl.N:] = 3e4
        step = csa.AttentionStep.for_workload(wl)
        step(x)
        torch.cuda.synchronize()
        outs.append((step.out.clone(), step.topk_idx.clone(), step.lse.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d", [64, 512])
def test_empty_and_invisible(csa, d):
    say("empty batch / no visible rows", d)
    q = torch.randn((1, 1, 16, d), device="cuda").to(torch.bfloat16)
    e = torch.randn((1, 8, d), device="cuda").to(torch.bfloat16)
    raw = torch.randn((1, 4, d), device="cuda").to(torch.bfloat16)
    # query at position 2 with m=4: no complete group, W=0: empty row set
    lse = torch.empty((1, 1, 16), device="cuda")
    out = csa.hca_dense_mqa(q, e, raw, 8, 4, 0, 2, 0, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    # zero-sized batch enqueues nothing
    q0 = torch.empty((0, 1, 16, d), device="cuda", dtype=torch.bfloat16)
    csa.hca_dense_mqa(q0, e[:0], raw[:0], 8, 4, 2, 2, 0)


def test_determinism(csa):
    wl = CONFIGS["c5"]
    say(wl, "twice")
    res = []
    for _ in range(2):
        x = make_inputs(wl, "cuda")
        step = csa.AttentionStep.for_workload(wl)
        step(x)
        torch.cuda.synchronize()
        res.append((step.out.clone(), step.topk_idx.clone()))
        del x, step
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


def test_graph_replay_matches_eager(csa):
    wl = CONFIGS["c2"]
    say(wl, "graph replay")
    x = make_inputs(wl, "cuda")
    step = csa.AttentionStep.for_workload(wl)
    step(x)
    torch.cuda.synchronize()
    eager = (step.out.clone(), step.topk_idx.clone(), step.lse.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(x)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(x)
    for i in range(4):
        step.out.fill_(float("nan"))
        step.topk_idx.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, eager[0]) and torch.equal(step.topk_idx, eager[1]), i
        assert torch.equal(step.lse, eager[2]), i
        _ = (x["q"].float() * 2).sum().item()  # unrelated eager work between replays


# ------------------------------------------------ compression: two kernel forms
@pytest.mark.parametrize("dtype,m,d", [("bf16", 4, 512), ("bf16", 4, 128), ("bf16", 1, 256), ("f32", 4, 512),
                                       ("bf16", 8, 256), ("f32", 2, 32)])
def test_compress_forms_bit_identical(csa, dtype, m, d):
    """Small groups are pooled by one wavefront per group without LDS; the ragged
    compression pools the same group with the LDS reduction.  Both compute the
    same weights, round each product once and add the products in row order:
    the entries must agree bit for bit."""
    say("compress forms", dtype, m, d)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    B, G = 5, 3
    g = torch.Generator().manual_seed(4242 + m * 1000 + d)
    raw = (torch.randn((B, G * m, d), generator=g) * 3).to(dt).cuda()
    logits = (torch.randn((B, G * m), generator=g) * 2).cuda()
    out = torch.empty((B, G, d), dtype=dt, device="cuda")
    csa.csa_compress(raw, logits, m, out)
    # the ragged form, one group per call: group gi sits at ring rows 0 .. m-1
    for gi in range(G):
        ring = max(m, 1)
        raw_ring = torch.zeros((B, 2 * ring, d), dtype=dt, device="cuda")
        logit_ring = torch.zeros((B, 2 * ring), dtype=torch.float32, device="cuda")
        raw_ring[:, :m] = raw[:, gi * m:(gi + 1) * m]
        raw_ring[:, ring:ring + m] = raw[:, gi * m:(gi + 1) * m]
        logit_ring[:, :m] = logits[:, gi * m:(gi + 1) * m]
        logit_ring[:, ring:ring + m] = logits[:, gi * m:(gi + 1) * m]
        pos = torch.full((B,), m - 1, dtype=torch.int64, device="cuda")
        cache = torch.empty((B, 1, d), dtype=dt, device="cuda")
        csa.csa_ragged_compress(raw_ring, logit_ring, ring, m, pos, cache)
        torch.cuda.synchronize()
        assert torch.equal(cache[:, 0].view(torch.int16 if dtype == "bf16" else torch.int32),
                           out[:, gi].view(torch.int16 if dtype == "bf16" else torch.int32)), gi


# ------------------------------- compression fused into one of the index call's launches
FUSED = [("elem", "bf16", 4, 512, 1, 1, 3000), ("mx4", "bf16", 4, 512, 1, 1, 3000),
         ("elem", "bf16", 16, 128, 3, 2, 2500), ("mx4", "f32", 8, 256, 2, 4, 1900),
         ("elem", "f32", 4, 64, 5, 1, 40), ("elem", "bf16", 4, 512, 2, 1, 0), ("mx4", "bf16", 4, 512, 1, 3, 0),
         ("elem", "bf16", 4, 128, 100, 2, 3000), ("mx4", "bf16", 4, 512, 90, 1, 2000)]


@pytest.mark.parametrize("case", FUSED, ids=["-".join(map(str, c)) for c in FUSED])
def test_compress_index_topk_fused_bit_identical(csa, case):
    """The fused call gives what csa_compress then the index call give, bit for bit: entries, selection and
    scores.  Both run on one workspace, the fused call after the separate one and then again, so its own
    histogram clear is what resets the selection's counts each time.  Then with hist_zero (no clear: the
    compression in the top-k filter launch for few queries, alone before the indexer for many, the last two
    cases), three times in a row on that workspace and on a zero-filled one: each call must leave the
    histograms zero for the next."""
    fmt, dtype, m, d, Tq, G, N = case
    say("fused compress + index", case)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    B, HI, dI, k = 3, 16, 128, 64
    q_pos0 = max(N * m - Tq, 0)
    g = torch.Generator().manual_seed(9100 + 7 * m + d + N)
    raw = (torch.randn((B, G * m, d), generator=g) * 2).to(dt).cuda()
    logits = torch.randn((B, G * m), generator=g).cuda()
    q_idx = torch.randn((B, Tq, HI, dI), generator=g).to(dt).cuda()
    w_idx = torch.randn((B, Tq, HI), generator=g).cuda()
    k_idx = torch.randn((B, max(N, 1), dI), generator=g).to(dt).cuda()
    ws = torch.empty(max(csa.index_topk_workspace_bytes(B, Tq, N, HI, k), 256), dtype=torch.uint8, device="cuda")
    if fmt == "mx4":
        codes, scales = csa.csa_mx4_quantize(k_idx)
        kargs = (codes, scales)
        sep, fused = csa.csa_index_topk_mx4, csa.csa_compress_index_topk_mx4
    else:
        kargs = (k_idx,)
        sep, fused = csa.csa_index_topk, csa.csa_compress_index_topk

    def outputs():
        return (torch.full((B, G, d), float("nan"), dtype=dt, device="cuda"),
                torch.full((B, Tq, k), -7, dtype=torch.int32, device="cuda"),
                torch.full((B, Tq, N), float("nan"), device="cuda"))

    ea, ia, sa = outputs()
    csa.csa_compress(raw, logits, m, ea)
    sep(q_idx, w_idx, *kargs, N, m, k, q_pos0, topk_idx=ia, scores_out=sa, workspace=ws)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == "bf16" else torch.int32
    for rep in range(2):
        eb, ib, sb = outputs()
        fused(raw, logits, m, eb, q_idx, w_idx, *kargs, N, k, q_pos0, topk_idx=ib, scores_out=sb, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(ea.view(bits), eb.view(bits)), rep
        assert torch.equal(ia, ib), rep
        assert torch.equal(sa.view(torch.int32), sb.view(torch.int32)), rep
    assert not torch.isnan(ea.float()).any()
    ws0 = torch.zeros_like(ws)
    for w in (ws, ws0):
        for rep in range(3):
            eb, ib, sb = outputs()
            fused(raw, logits, m, eb, q_idx, w_idx, *kargs, N, k, q_pos0, topk_idx=ib, scores_out=sb, workspace=w,
                  hist_zero=True)
            torch.cuda.synchronize()
            assert torch.equal(ea.view(bits), eb.view(bits)), ("hist_zero", rep)
            assert torch.equal(ia, ib), ("hist_zero", rep)
            assert torch.equal(sa.view(torch.int32), sb.view(torch.int32)), ("hist_zero", rep)


# ------------------------------------------ top-k first digit: window and end bins
EDGE_CASES = [("elem", 4), ("elem", 256), ("mx4", 4), ("mx4", 256)]


@pytest.mark.parametrize("fmt,tq", EDGE_CASES, ids=[f"{f}-tq{t}" for f, t in EDGE_CASES])
def test_topk_scores_beyond_the_digit_window(csa, fmt, tq):
    """The first radix digit resolves 16 bins per binade inside a window of non-negative scores and
    gathers every score below it (negative, zero, tiny) or above it (huge) in its two end bins,
    whose keys are resolved from the top bit again.  Query rows cycle through four regimes of head
    weights: huge of both signs (the k-th score in the upper end bin), all negative and tiny (the
    lower end bin), and ordinary (an interior bin).  Rule T against the oracle, few-query and
    query-blocked paths, bf16 and FP4 index operands."""
    N = 6000
    wl = Workload("edges", "bf16", B=1, T=4 * N, Tq=tq, m=4, d=128, H=8, W=4, k=500, HI=16, dI=128,
                  seed_base=78000 + tq, index_fmt=fmt)
    say(wl)
    g = torch.Generator(device="cuda").manual_seed(78011 + tq)
    x = make_inputs(wl, "cuda")
    w = torch.rand(x["w_idx"].shape, generator=g, device="cuda")
    regime = torch.arange(tq, device="cuda") % 4
    scale = torch.tensor([2.0 ** 80, -1.0, 2.0 ** -90, 1.0], device="cuda")[regime].view(1, tq, 1)
    sign = torch.where((regime == 0).view(1, tq, 1), torch.sign(torch.rand(w.shape, generator=g, device="cuda") - 0.5),
                       torch.ones_like(w))
    x["w_idx"] = (w * scale * sign).contiguous()
    if fmt == "mx4":
        csa.AttentionStep.quantize_index_keys(x)
    xh = host_inputs(x)
    step = csa.AttentionStep.for_workload(wl)
    step(x)
    torch.cuda.synchronize()
    ref = oracle_step(wl, xh)
    swapped = check_topk(to_np(step.topk_idx), ref["idx"], ref["scores"], nvis_rows(wl), wl.k, "topk")
    say(f"rows with a legal near-tie swap: {swapped} of {tq}")
