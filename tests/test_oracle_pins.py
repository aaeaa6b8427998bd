"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test ties one oracle function to a closed form, a library routine on a
special case, an invariant, a brute-force enumeration or a count the pages
state.  They are chosen so that a plausible slip (a dropped normalisation, a
wrong group / head / row index, a wrong sign, a transposed operand, an
off-by-one in causality or in the window) fails at least one of them.

Pin status per oracle function:
  compress      -- pinned: library mean (uniform logits), selection (one-hot),
                   closed-form weights 1:2:3:4, shift invariance, identity at m=1,
                   convexity.
  round_bf16    -- pinned: torch's float32->bfloat16 conversion, hand-checked ties.
  n_visible     -- pinned: brute-force enumeration, the page's 1M-token counts.
  index_scores  -- pinned: numpy matmul + ReLU at one head, linearity in w,
                   head-permutation invariance, causal mask positions.
  topk          -- pinned: brute-force full sort, tie-heavy inputs, k >= n_visible.
  mx4_quantize /
  mx4_dequantize -- pinned: E2M1 values from the bit-field definition, E8M0
                   scale as a power of two, exact round trip of representable
                   blocks, brute-force nearest value with ties to the even
                   mantissa, hand-checked ties and saturation, the block
                   maximum landing on 4 or 6 (the scale exponent), power-of-two
                   equivariance, zero blocks.
  sparse_mqa /
  dense_mqa     -- pinned: torch SDPA (causal MQA and banded window), scipy
                   softmax / logsumexp on basis rows, two-row closed form,
                   permutation invariance, CSA == HCA when k >= n_visible.
The whole path against a trained model is parity unpinned: the pages print no
numeric example and no weights exist.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# compress
# --------------------------------------------------------------------------
def test_compress_uniform_logits_is_group_mean(orc):
    r = rng(1)
    B, G, m, d = 3, 5, 4, 16
    raw = r.standard_normal((B, G * m, d)).astype(np.float32)
    logits = np.full((B, G * m), 0.37, dtype=np.float32)
    out = orc.compress(raw, logits, m)
    ref = raw.astype(np.float64).reshape(B, G, m, d).mean(axis=2)
    np.testing.assert_allclose(out, ref, rtol=1e-14, atol=1e-14)


def test_compress_one_hot_logit_selects_token(orc):
    r = rng(2)
    B, G, m, d = 2, 6, 4, 8
    raw = r.standard_normal((B, G * m, d)).astype(np.float32)
    logits = np.zeros((B, G * m), dtype=np.float32)
    pick = r.integers(0, m, size=(B, G))
    for b in range(B):
        for g in range(G):
            logits[b, g * m + pick[b, g]] = 60.0
    out = orc.compress(raw, logits, m)
    for b in range(B):
        for g in range(G):
            np.testing.assert_allclose(out[b, g], raw[b, g * m + pick[b, g]], rtol=0, atol=1e-24)


def test_compress_closed_form_weights(orc):
    # logits log(1..4) give softmax weights exactly 0.1, 0.2, 0.3, 0.4
    r = rng(3)
    B, G, m, d = 1, 3, 4, 5
    raw = r.standard_normal((B, G * m, d)).astype(np.float32)
    logits = np.tile(np.log(np.arange(1, 5, dtype=np.float64)).astype(np.float32), G)[None]
    out = orc.compress(raw, logits, m)
    a = np.exp(logits.astype(np.float64).reshape(G, m))
    a = a / a.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(a, np.tile([0.1, 0.2, 0.3, 0.4], (G, 1)), rtol=1e-6)
    ref = np.einsum("gi,gix->gx", a, raw[0].astype(np.float64).reshape(G, m, d))
    np.testing.assert_allclose(out[0], ref, rtol=1e-13, atol=1e-14)


def test_compress_shift_invariance_and_convexity(orc):
    r = rng(4)
    B, G, m, d = 2, 4, 128, 12
    raw = r.standard_normal((B, G * m, d)).astype(np.float32)
    logits = r.standard_normal((B, G * m)).astype(np.float32)
    shift = np.repeat(r.uniform(-500, 500, size=(B, G)), m, axis=1).astype(np.float32)
    a = orc.compress(raw, logits, m)
    b = orc.compress(raw, (logits.astype(np.float64) + shift).astype(np.float32), m)
    # the shifted logits are rounded to float32, so compare loosely; exact shift below
    assert np.max(np.abs(a - b)) < 1e-3
    # logits on a 2^-10 grid with |z| < 8: z + 1000 is exact in float32 (its ulp there is 2^-14), the shift
    # cancels exactly in z - max z, so the entries must be identical bit for bit
    zq = (np.round(logits.astype(np.float64) * 1024) / 1024).astype(np.float32)
    assert np.all(np.abs(zq) < 8)
    zs = zq + np.float32(1000.0)
    assert np.array_equal(zs.astype(np.float64) - 1000.0, zq.astype(np.float64))
    np.testing.assert_array_equal(orc.compress(raw, zs, m), orc.compress(raw, zq, m))
    grp = raw.astype(np.float64).reshape(B, G, m, d)
    assert np.all(a <= grp.max(axis=2) + 1e-12) and np.all(a >= grp.min(axis=2) - 1e-12)


def test_compress_m1_identity(orc):
    r = rng(5)
    raw = r.standard_normal((2, 9, 7)).astype(np.float32)
    logits = r.standard_normal((2, 9)).astype(np.float32)
    np.testing.assert_array_equal(orc.compress(raw, logits, 1), raw.astype(np.float64))


# per-channel pooling logits (the pages leave the form of the softmax weights open)
def test_compress_channels_equal_logits_reduce_to_token_logits(orc):
    r = rng(41)
    B, G, m, d = 2, 5, 4, 24
    raw = r.standard_normal((B, G * m, d)).astype(np.float32)
    z = r.standard_normal((B, G * m)).astype(np.float32)
    zc = np.repeat(z[:, :, None], d, axis=2)
    np.testing.assert_allclose(orc.compress_channels(raw, zc, m), orc.compress(raw, z, m), rtol=1e-14, atol=1e-15)
    r2 = rng(42)
    raw = r2.standard_normal((1, 2 * 128, 8)).astype(np.float32)
    z = r2.standard_normal((1, 2 * 128)).astype(np.float32)
    np.testing.assert_allclose(orc.compress_channels(raw, np.repeat(z[:, :, None], 8, axis=2), 128),
                               orc.compress(raw, z, 128), rtol=1e-13, atol=1e-15)


def test_compress_channels_closed_form_weights(orc):
    # channel 0: logits log(1..4) -> weights 0.1 0.2 0.3 0.4; channel 1: reversed; channel 2: equal
    raw = np.array([[[1, 10, 3], [2, 20, 5], [4, 40, 7], [8, 80, 11]]], dtype=np.float32)
    lg = np.log(np.array([[1, 4, 5], [2, 3, 5], [3, 2, 5], [4, 1, 5]], dtype=np.float64)).astype(np.float32)[None]
    out = orc.compress_channels(raw, lg, 4)[0, 0]
    want = [0.1 * 1 + 0.2 * 2 + 0.3 * 4 + 0.4 * 8, 0.4 * 10 + 0.3 * 20 + 0.2 * 40 + 0.1 * 80, (3 + 5 + 7 + 11) / 4]
    np.testing.assert_allclose(out, want, rtol=1e-6)  # (the float32 logits of log k carry ~1e-7 error)


def test_compress_channels_one_hot_per_channel(orc):
    r = rng(43)
    B, G, m, d = 2, 3, 4, 10
    raw = r.standard_normal((B, G * m, d)).astype(np.float32)
    z = np.zeros((B, G * m, d), dtype=np.float32)
    pick = r.integers(0, m, size=(B, G, d))
    for b in range(B):
        for g in range(G):
            for x in range(d):
                z[b, g * m + pick[b, g, x], x] = 80.0
    out = orc.compress_channels(raw, z, m)
    for b in range(B):
        for g in range(G):
            for x in range(d):
                assert abs(out[b, g, x] - raw[b, g * m + pick[b, g, x], x]) <= 1e-30


def test_compress_channels_permutation_shift_and_bounds(orc):
    r = rng(44)
    B, G, m, d = 2, 4, 128, 9
    raw = r.standard_normal((B, G * m, d)).astype(np.float32)
    z = (np.round(r.uniform(-2, 2, size=(B, G * m, d)) * 64) / 64).astype(np.float32)  # exact under integer shifts
    out = orc.compress_channels(raw, z, m)
    perm = r.permutation(d)
    np.testing.assert_array_equal(orc.compress_channels(raw[:, :, perm], z[:, :, perm], m), out[:, :, perm])
    shift = np.repeat(r.integers(-300, 300, size=(B, G, 1, d)), m, axis=2).reshape(B, G * m, d).astype(np.float32)
    np.testing.assert_allclose(orc.compress_channels(raw, z + shift, m), out, rtol=1e-13, atol=1e-15)
    grp = raw.astype(np.float64).reshape(B, G, m, d)
    assert np.all(out <= grp.max(axis=2) + 1e-12) and np.all(out >= grp.min(axis=2) - 1e-12)
    np.testing.assert_array_equal(orc.compress_channels(raw[:, :7], z[:, :7], 1), raw[:, :7].astype(np.float64))


def test_compress_batches_and_groups_independent(orc):
    r = rng(6)
    B, G, m, d = 4, 3, 4, 6
    raw = r.standard_normal((B, G * m, d)).astype(np.float32)
    logits = r.standard_normal((B, G * m)).astype(np.float32)
    full = orc.compress(raw, logits, m)
    perm = [2, 0, 3, 1]
    np.testing.assert_array_equal(orc.compress(raw[perm], logits[perm], m), full[perm])
    gp = [1, 2, 0]
    raw_g = raw.reshape(B, G, m, d)[:, gp].reshape(B, G * m, d)
    log_g = logits.reshape(B, G, m)[:, gp].reshape(B, G * m)
    np.testing.assert_array_equal(orc.compress(raw_g, log_g, m), full[:, gp])


# --------------------------------------------------------------------------
# bf16 rounding of the compressed cache
# --------------------------------------------------------------------------
def test_round_bf16_matches_torch_on_float32_values(orc):
    r = rng(7)
    x = np.concatenate([r.standard_normal(20000) * 10.0 ** r.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, -2.5, 3.0e38, 1e-39]]).astype(np.float32)
    mine = orc.round_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(mine, ref)


def test_round_bf16_ties_to_even(orc):
    u = 2.0 ** -7  # bf16 spacing in [1, 2)
    x = np.array([1 + u / 2, 1 + 1.5 * u, 1 + u / 2 + 2 ** -40, -(1 + 1.5 * u)])
    np.testing.assert_array_equal(orc.round_bf16(x), np.array([1.0, 1 + 2 * u, 1 + u, -(1 + 2 * u)],
                                                              dtype=np.float32))


# --------------------------------------------------------------------------
# causal bookkeeping
# --------------------------------------------------------------------------
def test_n_visible_page_counts(orc):
    with open(os.path.join(GOLDEN, "page_counts.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        T, m = case["tokens"], case["m"]
        n = orc.n_visible(T - 1, m, 1 << 40)
        assert n == case["entries"]
        lo, hi = case.get("page_range", [n, n])
        assert lo <= n <= hi


def test_n_visible_brute_force(orc):
    for m in (1, 2, 3, 4, 128):
        for N in (0, 1, 3, 1000):
            for t in range(-2, 300):
                brute = sum(1 for g in range(N) if g * m + m - 1 <= t)
                assert orc.n_visible(t, m, N) == brute, (m, N, t)


def test_window_start(orc):
    for W in (1, 4, 64):
        for t in range(0, 100):
            brute = [p for p in range(0, t + 1) if t - p < W]
            assert orc.window_start(t, W) == brute[0]


# --------------------------------------------------------------------------
# lightning indexer
# --------------------------------------------------------------------------
def _idx_inputs(seed, B, Tq, N, HI, dI):
    r = rng(seed)
    q = (r.standard_normal((B, Tq, HI, dI)) / np.sqrt(dI)).astype(np.float32)
    w = r.uniform(0, 1, (B, Tq, HI)).astype(np.float32)
    k = (r.standard_normal((B, N, dI)) / np.sqrt(dI)).astype(np.float32)
    return q, w, k


def test_index_single_head_is_relu_matmul(orc):
    q, w, k = _idx_inputs(10, 2, 5, 40, 1, 16)
    w[:] = 1.0
    m, q_pos0 = 1, 100  # every entry visible
    s = orc.index_scores(q, w, k, m, q_pos0)
    for b in range(2):
        ref = np.maximum(q[b, :, 0].astype(np.float64) @ k[b].astype(np.float64).T, 0.0)
        np.testing.assert_allclose(s[b], ref, rtol=1e-13, atol=1e-15)


def test_index_one_hot_head_weight(orc):
    q, w, k = _idx_inputs(11, 1, 3, 30, 4, 8)
    for h in range(4):
        wh = np.zeros_like(w)
        wh[..., h] = 1.0
        s = orc.index_scores(q, wh, k, 1, 100)
        ref = np.maximum(q[0, :, h].astype(np.float64) @ k[0].astype(np.float64).T, 0.0)
        np.testing.assert_allclose(s[0], ref, rtol=1e-13, atol=1e-15)


def test_index_linear_in_w_and_head_permutation(orc):
    q, w, k = _idx_inputs(12, 2, 4, 50, 4, 32)
    w2 = rng(13).uniform(-1, 1, w.shape).astype(np.float32)
    s1 = orc.index_scores(q, w, k, 1, 100)
    s2 = orc.index_scores(q, w2, k, 1, 100)
    s12 = orc.index_scores(q, (w.astype(np.float64) + w2).astype(np.float32), k, 1, 100)
    # w + w2 is rounded to float32; linearity holds up to that rounding
    np.testing.assert_allclose(s12, s1 + s2, rtol=1e-6, atol=1e-6)
    perm = [2, 0, 3, 1]
    sp = orc.index_scores(q[:, :, perm], w[:, :, perm], k, 1, 100)
    np.testing.assert_allclose(sp, s1, rtol=1e-13, atol=1e-15)
    # scaling w by a positive constant scales the scores
    np.testing.assert_allclose(orc.index_scores(q, w * np.float32(4.0), k, 1, 100), 4.0 * s1, rtol=1e-13)


def test_index_relu_drops_negative_dots(orc):
    dI = 4
    q = np.array([[[[1, 0, 0, 0], [0, 1, 0, 0]]]], dtype=np.float32)  # B=1,Tq=1,HI=2
    w = np.array([[[2.0, 3.0]]], dtype=np.float32)
    k = np.array([[[1, 1, 0, 0], [-1, 1, 0, 0], [1, -1, 0, 0], [-1, -1, 0, 0]]], dtype=np.float32)
    s = orc.index_scores(q, w, k, 1, 10)
    np.testing.assert_array_equal(s[0, 0], [5.0, 3.0, 2.0, 0.0])


def test_index_causal_mask(orc):
    B, Tq, N, m = 1, 40, 20, 4
    q, w, k = _idx_inputs(14, B, Tq, N, 2, 8)
    q_pos0 = 3
    s = orc.index_scores(q, w, k, m, q_pos0)
    for ti in range(Tq):
        t = q_pos0 + ti
        nv = min(N, (t + 1) // m)
        assert np.all(np.isfinite(s[0, ti, :nv])) and np.all(s[0, ti, nv:] == -np.inf), ti


# --------------------------------------------------------------------------
# top-k
# --------------------------------------------------------------------------
def _brute_topk(s, nv, k):
    order = sorted(range(nv), key=lambda j: (-s[j], j))[:k]
    out = sorted(order) + [-1] * (k - min(k, nv))
    return out


@pytest.mark.parametrize("kind", ["random", "ties"])
def test_topk_equals_brute_force_sort(orc, kind):
    r = rng(20)
    B, Tq, N, m, k = 2, 30, 64, 2, 10
    if kind == "random":
        s = r.standard_normal((B, Tq, N))
    else:
        s = r.integers(0, 3, (B, Tq, N)).astype(np.float64)
    q_pos0 = 0
    for ti in range(Tq):
        nv = min(N, (q_pos0 + ti + 1) // m)
        s[:, ti, nv:] = -np.inf
    idx = orc.topk(s, k, m, q_pos0)
    for b in range(B):
        for ti in range(Tq):
            nv = min(N, (q_pos0 + ti + 1) // m)
            assert list(idx[b, ti]) == _brute_topk(list(s[b, ti]), nv, k), (b, ti)


def test_topk_k_at_least_visible_selects_all(orc):
    s = rng(21).standard_normal((1, 3, 12))
    idx = orc.topk(s, 16, 1, 5)  # n_visible = 6, 7, 8
    for ti, nv in enumerate((6, 7, 8)):
        assert list(idx[0, ti]) == list(range(nv)) + [-1] * (16 - nv)


def test_topk_positive_scaling_invariance(orc):
    q, w, k = _idx_inputs(22, 1, 6, 200, 4, 16)
    s = orc.index_scores(q, w, k, 1, 500)
    s3 = orc.index_scores(q, w * np.float32(0.125), k, 1, 500)
    np.testing.assert_array_equal(orc.topk(s, 17, 1, 500), orc.topk(s3, 17, 1, 500))


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------
def _sdpa_mqa(q, c, mask):
    """torch SDPA in float64 on the CPU; K = V = c shared by every head."""
    Tq, H, d = q.shape
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)  # [H, Tq, d]
    kv = torch.from_numpy(c.astype(np.float64))[None].expand(H, -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kv, kv, attn_mask=torch.from_numpy(mask))
    return o.permute(1, 0, 2).numpy()


def test_hca_m1_no_window_is_causal_mqa(orc):
    r = rng(30)
    T, H, d = 24, 3, 16
    c = r.standard_normal((1, T, d)).astype(np.float32)
    q = r.standard_normal((1, T, H, d)).astype(np.float32)
    entries = orc.compress(c, r.standard_normal((1, T)).astype(np.float32), 1).astype(np.float32)
    out, lse = orc.dense_mqa(q, entries, c, 0, 1, 0, 0)
    mask = np.tril(np.ones((T, T), dtype=bool))
    np.testing.assert_allclose(out[0], _sdpa_mqa(q[0], c[0], mask), rtol=1e-12, atol=1e-12)


def test_csa_m1_k_ge_T_no_window_is_causal_mqa(orc):
    r = rng(31)
    T, H, d = 20, 2, 8
    c = r.standard_normal((1, T, d)).astype(np.float32)
    q = r.standard_normal((1, T, H, d)).astype(np.float32)
    qi, wi, ki = _idx_inputs(32, 1, T, T, 2, 8)
    s = orc.index_scores(qi, wi, ki, 1, 0)
    idx = orc.topk(s, T + 3, 1, 0)
    out, _ = orc.sparse_mqa(q, c, idx, c, 0, 0, 0)
    mask = np.tril(np.ones((T, T), dtype=bool))
    np.testing.assert_allclose(out[0], _sdpa_mqa(q[0], c[0], mask), rtol=1e-12, atol=1e-12)


def test_window_only_is_banded_mqa(orc):
    # t < m-1 for every query: no complete group, only the sliding window
    r = rng(33)
    T, H, d, W = 30, 2, 8, 5
    c = r.standard_normal((1, T, d)).astype(np.float32)
    q = r.standard_normal((1, T, H, d)).astype(np.float32)
    idx = np.full((1, T, 4), -1, dtype=np.int32)
    entries = np.zeros((1, 1, d), dtype=np.float32)
    out, _ = orc.sparse_mqa(q, entries, idx, c, 0, W, 0)
    i = np.arange(T)
    mask = (i[None, :] <= i[:, None]) & (i[:, None] - i[None, :] < W)
    np.testing.assert_allclose(out[0], _sdpa_mqa(q[0], c[0], mask), rtol=1e-12, atol=1e-12)
    out2, _ = orc.dense_mqa(q, entries, c, 0, 128, W, 0)
    np.testing.assert_allclose(out2, out, rtol=0, atol=0)


def test_attention_basis_rows_give_softmax_and_lse(orc):
    r = rng(34)
    n, d, H = 6, 8, 3
    entries = np.eye(d, dtype=np.float32)[None, :n]  # entry j = basis vector e_j
    q = r.standard_normal((1, 1, H, d)).astype(np.float32) * 3
    idx = np.array([[[0, 1, 2, 3, 4, 5, -1, -1]]], dtype=np.int32)
    raw = np.zeros((1, 1, d), dtype=np.float32)
    scale = 0.7
    out, lse = orc.sparse_mqa(q, entries, idx, raw, 0, 0, 0, scale=scale)
    logits = scale * q[0, 0, :, :n].astype(np.float64)
    np.testing.assert_allclose(out[0, 0, :, :n], scipy.special.softmax(logits, axis=1), rtol=1e-13)
    np.testing.assert_array_equal(out[0, 0, :, n:], 0.0)
    np.testing.assert_allclose(out[0, 0].sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(lse[0, 0], scipy.special.logsumexp(logits, axis=1), rtol=1e-14)


def test_attention_two_row_closed_form(orc):
    r = rng(35)
    d, H = 5, 2
    R = r.standard_normal((1, 2, d)).astype(np.float32)
    q = r.standard_normal((1, 1, H, d)).astype(np.float32)
    idx = np.array([[[1, -1, -1]]], dtype=np.int32)  # entry 1 selected
    raw = R[:, :1]  # window of one raw row: position 0
    entries = R
    out, lse = orc.sparse_mqa(q, entries, idx, raw, 0, 1, 0, scale=1.0)
    for h in range(H):
        l1 = float(np.dot(q[0, 0, h].astype(np.float64), R[0, 1].astype(np.float64)))
        l2 = float(np.dot(q[0, 0, h].astype(np.float64), R[0, 0].astype(np.float64)))
        a1 = 1.0 / (1.0 + math.exp(l2 - l1))
        ref = a1 * R[0, 1].astype(np.float64) + (1 - a1) * R[0, 0].astype(np.float64)
        np.testing.assert_allclose(out[0, 0, h], ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[0, 0, h], np.logaddexp(l1, l2), rtol=1e-14)


def test_attention_constant_rows_and_empty(orc):
    r = rng(36)
    d = 6
    row = r.standard_normal(d).astype(np.float32)
    entries = np.tile(row, (1, 10, 1))
    raw = np.tile(row, (1, 4, 1))
    q = r.standard_normal((1, 1, 2, d)).astype(np.float32)
    idx = np.array([[[0, 3, 7, 9]]], dtype=np.int32)
    out, _ = orc.sparse_mqa(q, entries, idx, raw, 0, 4, 3)
    np.testing.assert_allclose(out[0, 0], np.tile(row.astype(np.float64), (2, 1)), rtol=1e-14)
    empty = np.full((1, 1, 4), -1, dtype=np.int32)
    out, lse = orc.sparse_mqa(q, entries, empty, raw, 0, 0, 3)
    assert np.all(out == 0.0) and np.all(lse == -np.inf)


def test_attention_permuting_selection_changes_nothing(orc):
    r = rng(37)
    B, N, d, H, k, W = 2, 40, 16, 4, 12, 3
    entries = r.standard_normal((B, N, d)).astype(np.float32)
    raw = r.standard_normal((B, 5, d)).astype(np.float32)
    q = r.standard_normal((B, 1, H, d)).astype(np.float32)
    idx = np.stack([np.sort(r.choice(N, k, replace=False)) for _ in range(B)])[:, None].astype(np.int32)
    a, la = orc.sparse_mqa(q, entries, idx, raw, 100, W, 104)
    pidx = idx[:, :, r.permutation(k)]
    b, lb = orc.sparse_mqa(q, entries, pidx, raw, 100, W, 104)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(la, lb, rtol=1e-14)
    # a window row added at the raw buffer's far end does not change a W-row window
    raw2 = np.concatenate([r.standard_normal((B, 1, d)).astype(np.float32), raw], axis=1)
    c, _ = orc.sparse_mqa(q, entries, idx, raw2, 99, W, 104)
    np.testing.assert_allclose(c, a, rtol=1e-13, atol=1e-15)


def test_csa_with_k_ge_visible_equals_hca(orc):
    r = rng(38)
    B, T, m, d, H, W = 2, 64, 4, 16, 4, 6
    Tq = 9
    q_pos0 = T - Tq
    N = T // m
    entries = r.standard_normal((B, N, d)).astype(np.float32)
    raw = r.standard_normal((B, T, d)).astype(np.float32)
    q = r.standard_normal((B, Tq, H, d)).astype(np.float32)
    qi, wi, ki = _idx_inputs(39, B, Tq, N, 2, 8)
    s = orc.index_scores(qi, wi, ki, m, q_pos0)
    idx = orc.topk(s, N, m, q_pos0)
    a, la = orc.sparse_mqa(q, entries, idx, raw, 0, W, q_pos0)
    b, lb = orc.dense_mqa(q, entries, raw, 0, m, W, q_pos0)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(la, lb, rtol=1e-14)


# ---------------------------------------------------------------- MXFP4
def e2m1_from_bits(code):
    """E2M1 by its bit fields: sign, 2 exponent bits (bias 1), 1 mantissa bit."""
    s, e, mbit = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = (mbit / 2.0) if e == 0 else (2.0 ** (e - 1)) * (1.0 + mbit / 2.0)
    return -mag if s else mag


def pack_codes(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def test_mx4_element_values_from_bit_fields():
    from oracle import mx4_dequantize
    codes = np.arange(32, dtype=np.uint8) % 16
    out = mx4_dequantize(pack_codes(codes)[None], np.array([[127]], dtype=np.uint8))[0]
    np.testing.assert_array_equal(out, [e2m1_from_bits(int(c)) for c in codes])
    assert sorted(set(abs(float(v)) for v in out)) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_mx4_scale_is_a_power_of_two():
    from oracle import mx4_dequantize
    codes = pack_codes(np.full(32, 2, dtype=np.uint8))  # all 1.0
    for E in (0, 1, 100, 127, 128, 254):
        out = mx4_dequantize(codes[None], np.array([[E]], dtype=np.uint8))[0]
        assert np.all(out == np.float32(math.ldexp(1.0, E - 127)))


def test_mx4_representable_blocks_round_trip():
    from oracle import mx4_dequantize, mx4_quantize
    r = rng(71)
    for trial in range(200):
        e = int(r.integers(-20, 20))
        codes = r.integers(0, 16, 32).astype(np.uint8)
        codes[int(r.integers(0, 32))] = int(r.choice([6, 7, 14, 15]))  # block maximum 4 or 6
        x = mx4_dequantize(pack_codes(codes)[None], np.array([[127 + e]], dtype=np.uint8))
        c2, s2 = mx4_quantize(x)
        assert s2[0, 0] == 127 + e
        np.testing.assert_array_equal(c2[0], pack_codes(codes))


def test_mx4_nearest_value_brute_force():
    from oracle import mx4_dequantize, mx4_quantize
    r = rng(72)
    grid = np.array([e2m1_from_bits(c) for c in range(16)])
    x = (r.standard_normal((300, 32)) * np.exp(r.uniform(-6, 6, (300, 1)))).astype(np.float32)
    codes, scales = mx4_quantize(x)
    deq = mx4_dequantize(codes, scales).astype(np.float64)
    X = np.ldexp(1.0, scales.astype(np.int64) - 127)
    for b in range(x.shape[0]):
        cand = grid * X[b, 0]
        for i in range(32):
            err = np.abs(cand - float(x[b, i]))
            best = err.min()
            ok = [c for c in range(16) if err[c] == best]
            even = [c for c in ok if c % 2 == 0]
            pick = even if even else ok
            assert any(cand[c] == deq[b, i] for c in pick), (b, i, x[b, i], deq[b, i])


def test_mx4_hand_checked_ties_and_saturation():
    from oracle import mx4_dequantize, mx4_quantize
    vals = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -2.5, 7.0, 0.0]
    want = [6.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, -0.0, -2.0, 6.0, 0.0]
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :len(vals)] = vals
    codes, scales = mx4_quantize(x)
    assert scales[0, 0] == 127  # max 7.0: floor(log2 7) - 2 = 0
    out = mx4_dequantize(codes, scales)[0, :len(vals)]
    np.testing.assert_array_equal(out, np.array(want, dtype=np.float32))
    assert (codes[0, 4] & 15) == 8  # -0.25 keeps its sign bit
    assert (codes[0, 6] >> 4) == 0  # +0.0


def test_mx4_block_maximum_lands_on_four_or_six_and_equivariance():
    from oracle import mx4_dequantize, mx4_quantize
    r = rng(73)
    x = (r.standard_normal((200, 32)) * np.exp(r.uniform(-8, 8, (200, 1)))).astype(np.float32)
    codes, scales = mx4_quantize(x)
    deq = mx4_dequantize(codes, scales).astype(np.float64)
    X = np.ldexp(1.0, scales.astype(np.int64) - 127)
    top = np.abs(deq).max(axis=1) / X[:, 0]
    assert set(np.unique(top)) <= {4.0, 6.0}
    for k in (-5, 3):
        c2, s2 = mx4_quantize(x * np.float32(2.0 ** k))
        np.testing.assert_array_equal(c2, codes)
        np.testing.assert_array_equal(s2.astype(int), scales.astype(int) + k)


def test_mx4_zero_block():
    from oracle import mx4_quantize
    codes, scales = mx4_quantize(np.zeros((2, 64), dtype=np.float32))
    assert np.all(codes == 0) and np.all(scales == 0)
