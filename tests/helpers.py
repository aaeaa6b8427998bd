"""Comparison rules shared by the parity tests (test-side logic, no method arithmetic).

Tolerances (fixed by the project statement of the method):
  bf16 inputs, fp32 accumulation: max |err| <= 2e-2 and mean |err| <= 2e-3;
  fp32 inputs: normwise per output row, max |err| <= 1e-5 * max |ref|.
Top-k sets: identical, except that an entry in the symmetric difference must
have an oracle score within 1e-5 (relative, with a floor of 1e-3 of the row's
largest score) of the oracle's k-th score.  Counts, padding and order: exact.
"""
from __future__ import annotations

import numpy as np

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_REL = 1e-5
TOPK_REL = 1e-5


def to_np(t) -> np.ndarray:
    if hasattr(t, "detach"):
        t = t.detach().cpu()
        if t.dtype.is_floating_point:
            t = t.double()
        return t.numpy()
    return np.asarray(t)


def assert_close(got, ref, dtype: str, what: str, row_dims: int = 1):
    """Compare per the dtype's rule.  row_dims: trailing dims forming one 'row' for the fp32 normwise rule."""
    got = to_np(got).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if got.size == 0:
        return
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: finiteness differs"
    assert np.array_equal(got[~fin], ref[~fin]), f"{what}: non-finite values differ"
    err = np.abs(np.where(fin, got - ref, 0.0))
    if dtype == "bf16":
        mx, mean = err.max(), err[fin].mean() if fin.any() else 0.0
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, f"{what}: max {mx:.3e} mean {mean:.3e}"
    else:
        shp = ref.shape[: ref.ndim - row_dims] + (-1,)
        e = err.reshape(shp).max(axis=-1)
        scale = np.abs(np.where(fin, ref, 0.0)).reshape(shp).max(axis=-1)
        bad = e > F32_REL * np.maximum(scale, 1e-30)
        assert not bad.any(), f"{what}: {bad.sum()} rows over 1e-5 normwise, worst {(e / np.maximum(scale, 1e-30)).max():.3e}"


def check_topk(gpu_idx, ref_idx, ref_scores, nvis, k: int, what: str, extra_tol=None) -> int:
    """Rule T.  Returns the number of query rows whose set differs (legal near-tie swaps).
    extra_tol: optional per-row absolute slack added to the near-tie tolerance (a bound on how far the
    scores can move for a documented reason, e.g. one-ulp differences of the stored keys)."""
    g = to_np(gpu_idx).reshape(-1, k)
    r = to_np(ref_idx).reshape(-1, k)
    s = np.asarray(ref_scores).reshape(g.shape[0], -1)
    nvis = np.asarray(nvis).reshape(-1)
    swapped = 0
    for i in range(g.shape[0]):
        n_sel = min(k, int(nvis[i]))
        gi, ri = g[i], r[i]
        assert np.all(gi[n_sel:] == -1), f"{what} row {i}: padding"
        assert np.all(gi[:n_sel] >= 0) and np.all(gi[:n_sel] < nvis[i]), f"{what} row {i}: index out of visible range"
        assert np.all(np.diff(gi[:n_sel]) > 0), f"{what} row {i}: not strictly ascending"
        if np.array_equal(gi, ri):
            continue
        swapped += 1
        sg, sr = set(gi[:n_sel].tolist()), set(ri[:n_sel].tolist())
        row = s[i, : nvis[i]]
        kth = np.sort(row)[::-1][n_sel - 1]
        tol = TOPK_REL * max(abs(kth), 1e-3 * np.abs(row).max())
        if extra_tol is not None:
            tol += float(np.asarray(extra_tol).reshape(-1)[i])
        for j in sg ^ sr:
            assert abs(row[j] - kth) <= tol, f"{what} row {i}: entry {j} score {row[j]!r} vs k-th {kth!r}"
    return swapped


def nvis_rows(wl, B=None, Tq=None, q_pos0=None, N=None):
    B = wl.B if B is None else B
    Tq = wl.Tq if Tq is None else Tq
    q_pos0 = wl.q_pos0 if q_pos0 is None else q_pos0
    N = wl.N if N is None else N
    t = q_pos0 + np.arange(Tq)
    nv = np.minimum(N, (t + 1) // wl.m)
    return np.tile(nv, (B, 1))
