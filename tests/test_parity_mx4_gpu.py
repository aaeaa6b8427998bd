"""GPU parity of the FP4 (MXFP4) indexer operands against the CPU oracle.

The quantiser is integer / byte work decided by exact power-of-two scaling of
the bf16 / fp32 inputs: codes and scales must match the oracle bit for bit.
The indexer on MXFP4 operands is compared with the oracle's indexer run on the
oracle's own dequantised operands (exact values): scores normwise 1e-5 per
query row (float32 accumulation of exact block products), selection by rule T.
Both sides quantise the same seeded inputs themselves; nothing the GPU
computes feeds the oracle.
"""
import sys

import numpy as np
import pytest
import torch

from helpers import F32_REL, check_topk, nvis_rows, to_np
from workloads import CONFIGS, Workload, make_inputs

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


def special_blocks():
    """Blocks with exact ties, saturation, zeros, signed zeros and extreme magnitudes."""
    rows = []
    ties = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -2.5, 7.0, 0.0, -0.0, 4.0, -6.0, 0.5] * 2,
                    dtype=np.float32)
    for e in (-30, -3, 0, 5, 40):
        rows.append(ties * np.float32(2.0 ** e))
    rows.append(np.zeros(32, dtype=np.float32))
    z = np.zeros(32, dtype=np.float32)
    z[::2] = -0.0
    rows.append(z)
    big = np.full(32, 3.0e38, dtype=np.float32)
    big[1::2] = -1.0e38
    rows.append(big)
    tiny = np.full(32, 1e-38, dtype=np.float32)  # (below the smallest normal float: subnormal inputs)
    tiny[3] = -3e-38
    rows.append(tiny)
    return np.stack(rows)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mx4_quantize_bit_exact(csa, orc, dtype):
    say("mx4 quantise", dtype)
    g = torch.Generator().manual_seed(501)
    x = torch.randn((700, 128), generator=g) * torch.exp(torch.empty(700, 1).uniform_(-25, 25, generator=g))
    x = torch.cat([x.reshape(-1, 32), torch.from_numpy(special_blocks())])  # rows of one block
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    xd = x.to(tdt)
    codes, scales = csa.csa_mx4_quantize(xd.cuda())
    torch.cuda.synchronize()
    rc, rs = orc.mx4_quantize(xd.float().numpy())
    np.testing.assert_array_equal(to_np(scales), rs)
    np.testing.assert_array_equal(to_np(codes), rc)


MX_CASES = [
    # name, B, T, Tq, m, HI, dI, k, cap_extra
    ("decode_ragged", 3, 4 * 3001 + 2, 1, 4, 64, 128, 256, 40),
    ("decode_k_ge_n", 2, 4 * 300, 1, 4, 64, 128, 1024, 0),
    ("queries_causal_d64", 2, 4 * 500, 37, 4, 16, 64, 64, 8),
    ("queries_early_d32", 1, 70, 70, 4, 4, 32, 5, 0),
    ("decode_m1_heads20", 2, 2500, 2, 1, 20, 128, 300, 16),
    ("queries_causal_d128", 2, 4 * 700 + 3, 40, 4, 64, 128, 128, 8),
    ("queries_early_d128", 1, 70, 70, 4, 8, 128, 5, 0),
    # the query-blocked kernel: several workgroups of queries, a ragged last one, key tiles past N
    ("prefill_blocks_d128", 2, 4 * 2100 + 3, 150, 4, 64, 128, 256, 8),
    ("prefill_blocks_heads20", 1, 4 * 900, 77, 4, 20, 128, 64, 0),
]


def run_mx4(csa, orc, wl: Workload, cap_extra: int, scale_offset: int = 0):
    say(wl, "mx4 indexer", f"scale offset {scale_offset}")
    x = make_inputs(wl, "cuda", entries_capacity=wl.N + cap_extra)
    qc, qs = csa.csa_mx4_quantize(x["q_idx"].contiguous())  # (the same block routine the indexer runs inside)
    kc, ks = csa.csa_mx4_quantize(x["k_idx"].contiguous())
    if scale_offset:  # scales at an address that is not a multiple of 4 bytes
        buf = torch.zeros(ks.numel() + scale_offset, dtype=torch.uint8, device="cuda")
        ks = buf[scale_offset:].view(ks.shape)
        ks.copy_(csa.csa_mx4_quantize(x["k_idx"].contiguous())[1])
    sc = torch.empty((wl.B, wl.Tq, wl.N), dtype=torch.float32, device="cuda")
    idx = csa.csa_index_topk_mx4(x["q_idx"], x["w_idx"], kc, ks, wl.N, wl.m, wl.k, wl.q_pos0, scores_out=sc)
    torch.cuda.synchronize()
    # the oracle quantises the same inputs itself
    rqc, rqs = orc.mx4_quantize(x["q_idx"].float().cpu().numpy())
    rkc, rks = orc.mx4_quantize(x["k_idx"][:, : wl.N].float().cpu().numpy())
    np.testing.assert_array_equal(to_np(qc), rqc)
    np.testing.assert_array_equal(to_np(kc)[:, : wl.N], rkc)
    q = orc.mx4_dequantize(rqc, rqs)
    k = orc.mx4_dequantize(rkc, rks)
    ref = orc.index_scores(q, x["w_idx"].cpu().numpy(), k, wl.m, wl.q_pos0)
    got = to_np(sc)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), "finiteness of scores differs"
    if ref.size:
        # masked entries are -inf on both sides: take differences only where finite
        diff = np.zeros_like(ref)
        diff[fin] = got[fin] - ref[fin]
        err = np.abs(diff).max(axis=2)
        scale = np.abs(np.where(fin, ref, 0.0)).max(axis=2)
        worst = (err / np.maximum(scale, 1e-30)).max()
        assert np.all(err <= F32_REL * np.maximum(scale, 1e-30)), f"scores: worst {worst:.3e}"
    ridx = orc.topk(ref, wl.k, wl.m, wl.q_pos0)
    swapped = check_topk(idx, ridx, ref, nvis_rows(wl), wl.k, "mx4 topk")
    say(f"rows with a legal near-tie swap: {swapped}")


@pytest.mark.parametrize("case", MX_CASES, ids=[c[0] for c in MX_CASES])
def test_index_topk_mx4(csa, orc, case):
    name, B, T, Tq, m, HI, dI, k, cap_extra = case
    wl = Workload(name, "bf16", B=B, T=T, Tq=Tq, m=m, d=128, H=8, W=4, k=k, HI=HI, dI=dI,
                  seed_base=70000 + 1000 * MX_CASES.index(case))
    run_mx4(csa, orc, wl, cap_extra)


def test_index_topk_mx4_unaligned_scales(csa, orc):
    """Key scales at an odd address (read a byte at a time rather than as dwords)."""
    wl = Workload("mx4_scales_odd", "bf16", B=2, T=4 * 1500 + 1, Tq=3, m=4, d=128, H=8, W=4, k=200, HI=64, dI=128,
                  seed_base=78000)
    run_mx4(csa, orc, wl, 4, scale_offset=1)


def test_index_topk_mx4_decode_128k(csa, orc):
    """The 128K decode shape (32 sequences, 32768 entries, 64 index heads x 128, top-1024)."""
    run_mx4(csa, orc, CONFIGS["c2"], 0)


def test_index_topk_mx4_nothing_visible(csa, orc):
    wl = Workload("mx4_invisible", "bf16", B=2, T=3, Tq=3, m=4, d=128, H=8, W=4, k=16, HI=64, dI=128,
                  seed_base=79000)
    say(wl)
    run_mx4(csa, orc, wl, 8)


@pytest.mark.parametrize("shape", [(3, 4 * 3001 + 2, 1, 64), (2, 4 * 2100 + 3, 150, 64), (1, 4 * 900, 77, 20)],
                         ids=["decode", "prefill_blocks", "prefill_heads20"])
def test_index_scores_mx4_equals_index_topk_scores(csa, shape):
    """csa_index_scores_mx4 runs the same indexer as csa_index_topk_mx4: identical scores, bit for bit."""
    B, T, Tq, HI = shape
    wl = Workload("mx4_scores_only", "bf16", B=B, T=T, Tq=Tq, m=4, d=128, H=8, W=4, k=64, HI=HI, dI=128,
                  seed_base=79500 + T)
    x = make_inputs(wl, "cuda")
    kc, ks = csa.csa_mx4_quantize(x["k_idx"].contiguous())
    a = torch.empty((wl.B, wl.Tq, wl.N), dtype=torch.float32, device="cuda")
    csa.csa_index_topk_mx4(x["q_idx"], x["w_idx"], kc, ks, wl.N, wl.m, wl.k, wl.q_pos0, scores_out=a)
    b = csa.csa_index_scores_mx4(x["q_idx"], x["w_idx"], kc, ks, wl.N, wl.m, wl.q_pos0)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
