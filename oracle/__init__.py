"""CPU oracle for DeepSeek-V4 hybrid compressed attention (CSA / HCA).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this package.  It shares no
code with the HIP library and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, double accumulation); this
module only builds that file with gcc, marshals numpy arrays through ctypes and
checks argument shapes.  Every function follows the DeepSeek-V4 overview page
(gitcode.csdn.net, section 2.2 "CSA" steps 1-3 and section 2.3 "HCA"):

* ``compress``      -- step 1: softmax-weighted pooling of m adjacent tokens.
* ``index_scores``  -- step 2: lightning indexer, s_j = sum_h w_h ReLU(q_h.k_j)
                       (the form fixed by the project statement of the method).
* ``topk``          -- step 2: keep the top-k entries, ties to the lower index.
* ``sparse_mqa``    -- step 3: shared-KV MQA over the selected entries plus a
                       window of recent raw tokens, one softmax.
* ``dense_mqa``     -- section 2.3: the same attention over every visible entry.
* ``mx4_quantize`` / ``mx4_dequantize`` -- the FP4 indexer operands (section 9,
                       item 5), read as OCP MXFP4; the indexer then runs on the
                       exact dequantised values.

Parity-pin status of each function is listed in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FMA)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-D_GNU_SOURCE", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    L = ctypes.c_long
    D = ctypes.c_double
    lib.oracle_n_visible.argtypes = [L, I, L]
    lib.oracle_n_visible.restype = L
    lib.oracle_window_start.argtypes = [L, I]
    lib.oracle_window_start.restype = L
    lib.oracle_compress.argtypes = [I, I, I, I, P, P, P, I]
    lib.oracle_compress_channels.argtypes = [I, I, I, I, P, P, P, I]
    lib.oracle_round_bf16.argtypes = [L, P, P]
    lib.oracle_index_scores.argtypes = [I, I, I, I, I, I, L, P, P, P, P, I]
    lib.oracle_topk.argtypes = [I, I, I, I, I, L, P, P, I]
    lib.oracle_sparse_mqa.argtypes = [I, I, I, I, I, I, I, L, D, P, P, P, P, L, I, P, P, I]
    lib.oracle_dense_mqa.argtypes = [I, I, I, I, I, I, I, L, D, P, P, P, L, I, P, P, I]
    lib.oracle_mx4_quantize.argtypes = [L, P, P, P]
    lib.oracle_mx4_dequantize.argtypes = [L, P, P, P]
    for f in ("oracle_compress", "oracle_compress_channels", "oracle_round_bf16", "oracle_index_scores", "oracle_topk",
              "oracle_sparse_mqa", "oracle_dense_mqa", "oracle_mx4_quantize", "oracle_mx4_dequantize"):
        getattr(lib, f).restype = None
    _lib = lib
    return lib


def default_threads() -> int:
    """Host threads the oracle uses: the CPU count, capped by OMP_NUM_THREADS if set."""
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def _f32(a) -> np.ndarray:
    """Exact widening of a bf16/fp32 array (numpy or torch, CPU) to a dense float32 array."""
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().cpu().float().numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def n_visible(t: int, m: int, N: int) -> int:
    """Entries visible to a query at position t: complete groups ending at or before t."""
    return int(_load().oracle_n_visible(int(t), int(m), int(N)))


def window_start(t: int, W: int) -> int:
    return int(_load().oracle_window_start(int(t), int(W)))


def compress(raw, logits, m: int, nthreads: int | None = None) -> np.ndarray:
    """raw [B, G*m, d], logits [B, G*m] -> exact pooled entries [B, G, d] (float64)."""
    raw = _f32(raw)
    logits = _f32(logits)
    B, Tm, d = raw.shape
    assert Tm % m == 0 and logits.shape == (B, Tm)
    G = Tm // m
    out = np.empty((B, G, d), dtype=np.float64)
    _load().oracle_compress(B, G, m, d, _ptr(raw), _ptr(logits), _ptr(out), nthreads or default_threads())
    return out


def compress_channels(raw, logits, m: int, nthreads: int | None = None) -> np.ndarray:
    """raw [B, G*m, d], per-channel logits [B, G*m, d] -> exact pooled entries [B, G, d] (float64)."""
    raw = _f32(raw)
    logits = _f32(logits)
    B, Tm, d = raw.shape
    assert Tm % m == 0 and logits.shape == (B, Tm, d)
    G = Tm // m
    out = np.empty((B, G, d), dtype=np.float64)
    _load().oracle_compress_channels(B, G, m, d, _ptr(raw), _ptr(logits), _ptr(out), nthreads or default_threads())
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of float64 values onto the bf16 grid (returned as float32)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(x.shape, dtype=np.float32)
    _load().oracle_round_bf16(x.size, _ptr(x), _ptr(y))
    return y


def index_scores(q_idx, w_idx, k_idx, m: int, q_pos0: int, nthreads: int | None = None) -> np.ndarray:
    """q_idx [B,Tq,HI,dI], w_idx [B,Tq,HI], k_idx [B,N,dI] -> scores [B,Tq,N] float64 (-inf if not visible)."""
    q = _f32(q_idx)
    w = _f32(w_idx)
    k = _f32(k_idx)
    B, Tq, HI, dI = q.shape
    N = k.shape[1]
    assert w.shape == (B, Tq, HI) and k.shape == (B, N, dI)
    s = np.empty((B, Tq, N), dtype=np.float64)
    _load().oracle_index_scores(B, Tq, N, HI, dI, m, int(q_pos0), _ptr(q), _ptr(w), _ptr(k), _ptr(s),
                                nthreads or default_threads())
    return s


def mx4_quantize(x):
    """MXFP4 of x [..., d] (d a multiple of 32) -> (codes uint8 [..., d/2], scales uint8 [..., d/32]).

    OCP microscaling FP4: 32-element blocks with one E8M0 scale, E2M1 elements,
    two codes per byte (even element in the low nibble); the reading of the
    overview page's FP4 indexer operands (section 9, item 5)."""
    x = _f32(x)
    d = x.shape[-1]
    assert d % 32 == 0
    nb = x.size // 32
    codes = np.empty(x.shape[:-1] + (d // 2,), dtype=np.uint8)
    scales = np.empty(x.shape[:-1] + (d // 32,), dtype=np.uint8)
    _load().oracle_mx4_quantize(nb, _ptr(x), _ptr(codes), _ptr(scales))
    return codes, scales


def mx4_dequantize(codes, scales) -> np.ndarray:
    """The exact values of MXFP4 codes [..., d/2] with scales [..., d/32] -> float32 [..., d]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    d = codes.shape[-1] * 2
    assert scales.shape[-1] * 32 == d and codes.shape[:-1] == scales.shape[:-1]
    out = np.empty(codes.shape[:-1] + (d,), dtype=np.float32)
    _load().oracle_mx4_dequantize(scales.size, _ptr(codes), _ptr(scales), _ptr(out))
    return out


def topk(scores: np.ndarray, k: int, m: int, q_pos0: int, nthreads: int | None = None) -> np.ndarray:
    """scores [B,Tq,N] float64 -> idx [B,Tq,k] int32, ascending, -1 padded."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    B, Tq, N = s.shape
    idx = np.empty((B, Tq, k), dtype=np.int32)
    _load().oracle_topk(B, Tq, N, k, m, int(q_pos0), _ptr(s), _ptr(idx), nthreads or default_threads())
    return idx


def _check_window(q_pos0, Tq, W, raw_pos0, raw_len):
    if W > 0 and Tq > 0:
        lo = window_start(q_pos0, W)
        assert raw_pos0 <= lo and raw_pos0 + raw_len >= q_pos0 + Tq, "raw rows do not cover the window"


def sparse_mqa(q, entries, idx, raw, raw_pos0: int, W: int, q_pos0: int, scale: float | None = None,
               nthreads: int | None = None):
    """q [B,Tq,H,d], entries [B,N,d], idx [B,Tq,k], raw [B,raw_len,d] -> (out [B,Tq,H,d], lse [B,Tq,H]) float64."""
    q = _f32(q)
    e = _f32(entries)
    r = _f32(raw)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    B, Tq, H, d = q.shape
    N = e.shape[1]
    k = idx.shape[2]
    raw_len = r.shape[1]
    assert idx.shape[:2] == (B, Tq) and e.shape == (B, N, d) and r.shape[::2] == (B, d)
    assert np.all(idx < N) and np.all(idx >= -1)
    _check_window(q_pos0, Tq, W, raw_pos0, raw_len)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.empty((B, Tq, H, d), dtype=np.float64)
    lse = np.empty((B, Tq, H), dtype=np.float64)
    _load().oracle_sparse_mqa(B, Tq, H, d, N, k, W, int(q_pos0), float(scale), _ptr(q), _ptr(e), _ptr(idx),
                              _ptr(r), int(raw_pos0), raw_len, _ptr(out), _ptr(lse),
                              nthreads or default_threads())
    return out, lse


def dense_mqa(q, entries, raw, raw_pos0: int, m: int, W: int, q_pos0: int, scale: float | None = None,
              nthreads: int | None = None):
    """HCA: attention over all visible entries plus the window -> (out, lse) float64."""
    q = _f32(q)
    e = _f32(entries)
    r = _f32(raw)
    B, Tq, H, d = q.shape
    N = e.shape[1]
    raw_len = r.shape[1]
    assert e.shape == (B, N, d) and r.shape[::2] == (B, d)
    _check_window(q_pos0, Tq, W, raw_pos0, raw_len)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.empty((B, Tq, H, d), dtype=np.float64)
    lse = np.empty((B, Tq, H), dtype=np.float64)
    _load().oracle_dense_mqa(B, Tq, H, d, N, m, W, int(q_pos0), float(scale), _ptr(q), _ptr(e), _ptr(r),
                             int(raw_pos0), raw_len, _ptr(out), _ptr(lse), nthreads or default_threads())
    return out, lse
