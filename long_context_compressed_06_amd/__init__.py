"""Python binding of libcsa.so: DeepSeek-V4 hybrid compressed attention on MI355X.

Thin ctypes layer with the same names as the C ABI (``include/csa.h``).  Each
function checks that the torch tensors it receives are contiguous CUDA (HIP)
tensors of the expected dtype, then passes raw device pointers and the
current stream to the library.  Every step of the path runs in the HIP
kernels; PyTorch only provides device memory and the stream.  If libcsa.so
is missing the import of the library fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa.so")

CSA_F32, CSA_BF16 = 0, 1
_STATUS = {0: "CSA_OK", -1: "CSA_EINVAL", -2: "CSA_EDTYPE", -3: "CSA_EALIGN", -4: "CSA_EWORKSPACE",
           -5: "CSA_EHIP", -6: "CSA_EUNSUPPORTED"}
EXPORTS = ("csa_abi_version", "csa_status_string", "csa_last_error_detail", "csa_compress",
           "csa_index_topk_workspace_bytes", "csa_index_topk", "csa_index_scores", "csa_mqa_workspace_bytes",
           "csa_sparse_mqa", "hca_dense_mqa", "csa_mx4_quantize", "csa_index_topk_mx4", "csa_append_rows",
           "csa_compress_channels", "csa_append_rows_multi", "csa_positions_advance", "csa_ragged_compress",
           "csa_ragged_index_topk", "csa_ragged_index_topk_mx4", "csa_ragged_sparse_mqa", "hca_ragged_dense_mqa", "csa_stream_read",
           "csa_index_topk_noalloc", "csa_index_scores_mx4", "csa_compress_index_topk",
           "csa_compress_index_topk_mx4", "csa_ragged_compress_index_topk", "csa_ragged_compress_index_topk_mx4")


class AppendJob(ctypes.Structure):
    """csa_append_job of include/csa.h."""
    _fields_ = [("B", ctypes.c_int), ("n", ctypes.c_int), ("row_bytes", ctypes.c_int64), ("rows", ctypes.c_void_p),
                ("rows_bstride", ctypes.c_int64), ("dst", ctypes.c_void_p), ("dst_bstride", ctypes.c_int64),
                ("dst_rows", ctypes.c_int64), ("pos0", ctypes.c_int64), ("ring", ctypes.c_int64),
                ("pos", ctypes.c_void_p), ("every", ctypes.c_int64), ("page_table", ctypes.c_void_p),
                ("max_pages", ctypes.c_int), ("page_rows", ctypes.c_int), ("n_pages", ctypes.c_int64)]


class CsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def lib():
    """Load libcsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.csa_abi_version.restype = I
    L.csa_status_string.argtypes = [I]
    L.csa_status_string.restype = ctypes.c_char_p
    L.csa_last_error_detail.restype = ctypes.c_char_p
    L.csa_compress.argtypes = [I, I, I, I, I, P, I64, P, I64, P, I64, P]
    L.csa_compress.restype = I
    L.csa_index_topk_workspace_bytes.argtypes = [I, I, I, I, I]
    L.csa_index_topk_workspace_bytes.restype = SZ
    L.csa_index_topk.argtypes = [I, I, I, I, I, I, I, I, I64, P, P, P, I64, P, P, P, SZ, P]
    L.csa_index_topk.restype = I
    L.csa_index_scores.argtypes = [I, I, I, I, I, I, I, I64, P, P, P, I64, P, P]
    L.csa_index_scores.restype = I
    L.csa_mqa_workspace_bytes.argtypes = [I, I, I, I, I]
    L.csa_mqa_workspace_bytes.restype = SZ
    L.csa_sparse_mqa.argtypes = [I, I, I, I, I, I, I, I, I, I64, F, P, P, I64, P, P, I64, I64, I, P, P, P, SZ, P]
    L.csa_sparse_mqa.restype = I
    L.hca_dense_mqa.argtypes = [I, I, I, I, I, I, I, I, I64, F, P, P, I64, P, I64, I64, I, P, P, P, SZ, P]
    L.hca_dense_mqa.restype = I
    L.csa_mx4_quantize.argtypes = [I, I64, I, P, P, P, P]
    L.csa_mx4_quantize.restype = I
    L.csa_index_topk_mx4.argtypes = [I, I, I, I, I, I, I, I, I64, P, P, P, P, I64, P, P, P, SZ, P]
    L.csa_index_scores_mx4.argtypes = [I, I, I, I, I, I, I, I64, P, P, P, P, I64, P, P]
    L.csa_index_scores_mx4.restype = I
    L.csa_index_topk_mx4.restype = I
    L.csa_append_rows.argtypes = [I, I, I64, P, I64, P, I64, I64, I64, I64, P]
    L.csa_compress_channels.argtypes = [I, I, I, I, I, P, I64, P, I64, P, I64, P]
    L.csa_compress_channels.restype = I
    L.csa_append_rows_multi.argtypes = [I, P, P]
    L.csa_append_rows_multi.restype = I
    L.csa_positions_advance.argtypes = [I, P, I64, P]
    L.csa_positions_advance.restype = I
    L.csa_ragged_compress.argtypes = [I, I, I, I, P, P, I64, P, I64, I64, P, I64, I64, P, I, I, I64, P]
    L.csa_ragged_compress.restype = I
    L.csa_ragged_index_topk.argtypes = [I, I, I, I, I, I, I, P, P, P, P, I64, P, I, I, I64, P, P, P, SZ, P]
    L.csa_ragged_index_topk.restype = I
    L.csa_ragged_index_topk_mx4.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, I64, P, I, I, I64, P, P, P, SZ, P]
    L.csa_ragged_index_topk_mx4.restype = I
    L.csa_ragged_sparse_mqa.argtypes = [I, I, I, I, I, I, I, I, P, F, P, P, I64, P, I, I, I64, P, P, I64, I64, P, P, P,
                                        SZ, P]
    L.csa_ragged_sparse_mqa.restype = I
    L.hca_ragged_dense_mqa.argtypes = [I, I, I, I, I, I, I, P, F, P, P, I64, P, I, I, I64, P, I64, I64, P, P, P, SZ, P]
    L.hca_ragged_dense_mqa.restype = I
    L.csa_index_topk_noalloc.argtypes = [I, I, I, I, I, I, I, I, I64, P, P, P, I64, P, P, P]
    L.csa_index_topk_noalloc.restype = I
    comp = [I, I, I, I, I, P, I64, P, I64, P, I64]  # csa_compress's arguments, without the stream
    L.csa_compress_index_topk.argtypes = comp + [I, I, I, I, I, I64, P, P, P, I64, P, P, P, SZ, I, P]
    L.csa_compress_index_topk.restype = I
    L.csa_compress_index_topk_mx4.argtypes = comp + [I, I, I, I, I, I64, P, P, P, P, I64, P, P, P, SZ, I, P]
    L.csa_compress_index_topk_mx4.restype = I
    rcomp = [I, I, I, I, P, P, I64, P, I64, I64, P, I64, I64, P, I, I, I64]  # csa_ragged_compress's, no stream
    L.csa_ragged_compress_index_topk.argtypes = rcomp + [I, I, I, I, P, P, P, I64, P, I, I, I64, P, P, P, SZ, I, P]
    L.csa_ragged_compress_index_topk.restype = I
    L.csa_ragged_compress_index_topk_mx4.argtypes = rcomp + [I, I, I, I, P, P, P, P, I64, P, I, I, I64, P, P, P, SZ,
                                                             I, P]
    L.csa_ragged_compress_index_topk_mx4.restype = I
    L.csa_stream_read.argtypes = [P, I64, I, P, P]
    L.csa_stream_read.restype = I
    L.csa_append_rows.restype = I
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise CsaError(status, lib().csa_last_error_detail().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    raise TypeError(f"element type {t.dtype} is neither float32 nor bfloat16")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, dtype=None, dims=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimensions, got {t.dim()}")
    if t.stride(-1) != 1:
        raise ValueError(f"{name} needs a packed innermost dimension")


def _bstride(t):
    return t.stride(0)


def _compress_args(raw, logits, m, out) -> tuple:
    """Checks csa_compress's tensors; returns its arguments from dt to out_bstride."""
    _need(raw, "raw", dims=3)
    _need(logits, "logits", torch.float32, 2)
    _need(out, "out", raw.dtype, 3)
    B, Gm, d = raw.shape
    if Gm % m:
        raise ValueError("raw rows must be a multiple of m")
    G = Gm // m
    for t, n in ((raw, "raw"), (out, "out")):
        if t.stride(1) != d:
            raise ValueError(f"{n} rows must be packed")
    if out.shape != (B, G, d) or logits.shape != (B, Gm) or logits.stride(1) != 1:
        raise ValueError("shape mismatch between raw, logits and out")
    return (_dt(raw), B, G, m, d, _p(raw), _bstride(raw), _p(logits), _bstride(logits), _p(out), _bstride(out))


def csa_compress(raw: torch.Tensor, logits: torch.Tensor, m: int, out: torch.Tensor) -> torch.Tensor:
    """raw [B, G*m, d], logits [B, G*m] f32 -> out [B, G, d] (written in place, may be a cache view)."""
    _check(lib().csa_compress(*_compress_args(raw, logits, m, out), _stream(raw)))
    return out


def index_topk_workspace_bytes(B, Tq, N, H_I, k) -> int:
    return int(lib().csa_index_topk_workspace_bytes(B, Tq, N, H_I, k))


def _index_args(q_idx, w_idx, k_idx, N, k, q_pos0, topk_idx, scores_out, workspace) -> tuple:
    """Checks csa_index_topk's tensors (allocating the missing outputs); returns (topk_idx, its arguments from
    Tq to workspace_bytes with m left out)."""
    _need(q_idx, "q_idx", dims=4)
    _need(w_idx, "w_idx", torch.float32, 3)
    _need(k_idx, "k_idx", q_idx.dtype, 3)
    B, Tq, HI, dI = q_idx.shape
    if not q_idx.is_contiguous() or not w_idx.is_contiguous() or k_idx.stride(1) != dI or k_idx.shape[1] < N:
        raise ValueError("q_idx/w_idx must be contiguous and k_idx rows packed with >= N rows")
    if topk_idx is None:
        topk_idx = torch.empty((B, Tq, k), dtype=torch.int32, device=q_idx.device)
    _need(topk_idx, "topk_idx", torch.int32, 3)
    if scores_out is not None:
        _need(scores_out, "scores_out", torch.float32, 3)
        if scores_out.shape != (B, Tq, N) or not scores_out.is_contiguous():
            raise ValueError("scores_out must be a contiguous [B, Tq, N] tensor")
    need = index_topk_workspace_bytes(B, Tq, N, HI, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_idx.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return topk_idx, (Tq, N, HI, dI, k, q_pos0, _p(q_idx), _p(w_idx), _p(k_idx), _bstride(k_idx), _p(topk_idx),
                      _p(scores_out), _p(workspace), ws_bytes)


def csa_index_topk(q_idx, w_idx, k_idx, N: int, m: int, k: int, q_pos0: int, topk_idx=None, scores_out=None,
                   workspace=None) -> torch.Tensor:
    """q_idx [B,Tq,H_I,d_I], w_idx [B,Tq,H_I] f32, k_idx [B,cap,d_I] (first N rows used) -> topk_idx [B,Tq,k] int32."""
    topk_idx, a = _index_args(q_idx, w_idx, k_idx, N, k, q_pos0, topk_idx, scores_out, workspace)
    _check(lib().csa_index_topk(_dt(q_idx), q_idx.shape[0], *a[:4], m, *a[4:], _stream(q_idx)))
    return topk_idx


def _fused_pair(raw, q_idx):
    if raw.dtype != q_idx.dtype or raw.shape[0] != q_idx.shape[0] or raw.device != q_idx.device:
        raise ValueError("raw and q_idx must share the element type, the batch and the device")



def _flags(hist_zero, workspace):
    if hist_zero and workspace is None:
        raise ValueError("hist_zero needs a caller-owned workspace (a fresh one is not zero-filled)")
    return CSA_HIST_ZERO if hist_zero else 0


# flag of the fused calls: the workspace's top-k histograms are zero on entry (a zero-filled workspace, or one whose
# previous call had the same shape: every index call leaves them zero); then nothing is cleared first and, for few
# queries, the compression rides in the top-k filter launch
CSA_HIST_ZERO = 1


def csa_compress_index_topk(raw, logits, m: int, entries_out, q_idx, w_idx, k_idx, N: int, k: int, q_pos0: int,
                            topk_idx=None, scores_out=None, workspace=None, hist_zero=False) -> torch.Tensor:
    """csa_compress(raw, logits, m, entries_out) then csa_index_topk(q_idx, w_idx, k_idx, N, m, k, q_pos0, ...) in
    one call with one launch fewer; returns topk_idx.  entries_out is the attention's cache, not k_idx.
    hist_zero: the given workspace's histograms are zero (CSA_HIST_ZERO): one launch fewer again."""
    _fused_pair(raw, q_idx)
    c = _compress_args(raw, logits, m, entries_out)
    topk_idx, a = _index_args(q_idx, w_idx, k_idx, N, k, q_pos0, topk_idx, scores_out, workspace)
    _check(lib().csa_compress_index_topk(*c, *a, _flags(hist_zero, workspace), _stream(q_idx)))
    return topk_idx


NOALLOC_SCRATCH_BYTES = 16 << 20  # CSA_NOALLOC_SCRATCH_BYTES of include/csa.h


def csa_index_topk_noalloc(q_idx, w_idx, k_idx, N: int, m: int, k: int, q_pos0: int, topk_idx,
                           scores_out=None) -> torch.Tensor:
    """csa_index_topk on the library's static scratch: the call itself allocates nothing (topk_idx, and
    scores_out if wanted, are the caller's).  Calls on one GPU share the scratch and must not overlap."""
    _need(q_idx, "q_idx", dims=4)
    _need(w_idx, "w_idx", torch.float32, 3)
    _need(k_idx, "k_idx", q_idx.dtype, 3)
    _need(topk_idx, "topk_idx", torch.int32, 3)
    B, Tq, HI, dI = q_idx.shape
    if not q_idx.is_contiguous() or not w_idx.is_contiguous() or k_idx.stride(1) != dI or k_idx.shape[1] < N:
        raise ValueError("q_idx/w_idx must be contiguous and k_idx rows packed with >= N rows")
    if topk_idx.shape != (B, Tq, k) or not topk_idx.is_contiguous():
        raise ValueError("topk_idx must be a contiguous [B, Tq, k] tensor")
    if scores_out is not None:
        _need(scores_out, "scores_out", torch.float32, 3)
        if scores_out.shape != (B, Tq, N) or not scores_out.is_contiguous():
            raise ValueError("scores_out must be a contiguous [B, Tq, N] tensor")
    _check(lib().csa_index_topk_noalloc(_dt(q_idx), B, Tq, N, HI, dI, m, k, q_pos0, _p(q_idx), _p(w_idx), _p(k_idx),
                                        _bstride(k_idx), _p(topk_idx), _p(scores_out), _stream(q_idx)))
    return topk_idx


def csa_index_scores(q_idx, w_idx, k_idx, N: int, m: int, q_pos0: int, scores=None) -> torch.Tensor:
    """Lightning indexer only: scores [B,Tq,N] f32, -inf for entries not yet visible."""
    _need(q_idx, "q_idx", dims=4)
    _need(w_idx, "w_idx", torch.float32, 3)
    _need(k_idx, "k_idx", q_idx.dtype, 3)
    B, Tq, HI, dI = q_idx.shape
    if not q_idx.is_contiguous() or not w_idx.is_contiguous() or k_idx.stride(1) != dI or k_idx.shape[1] < N:
        raise ValueError("q_idx/w_idx must be contiguous and k_idx rows packed with >= N rows")
    if scores is None:
        scores = torch.empty((B, Tq, N), dtype=torch.float32, device=q_idx.device)
    _need(scores, "scores", torch.float32, 3)
    if scores.shape != (B, Tq, N) or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous [B, Tq, N] tensor")
    _check(lib().csa_index_scores(_dt(q_idx), B, Tq, N, HI, dI, m, q_pos0, _p(q_idx), _p(w_idx), _p(k_idx),
                                  _bstride(k_idx), _p(scores), _stream(q_idx)))
    return scores


def csa_mx4_quantize(x: torch.Tensor, codes=None, scales=None):
    """MXFP4 of x [..., d] (contiguous, d a multiple of 32) -> (codes uint8 [..., d/2], scales uint8 [..., d/32])."""
    _need(x, "x")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    d = x.shape[-1]
    if codes is None:
        codes = torch.empty(x.shape[:-1] + (d // 2,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1] + (d // 32,), dtype=torch.uint8, device=x.device)
    _need(codes, "codes", torch.uint8)
    _need(scales, "scales", torch.uint8)
    if (codes.shape != x.shape[:-1] + (d // 2,) or scales.shape != x.shape[:-1] + (d // 32,)
            or not codes.is_contiguous() or not scales.is_contiguous()):
        raise ValueError("codes / scales must be contiguous [..., d/2] / [..., d/32] tensors")
    n_rows = x.numel() // d if d else 0
    _check(lib().csa_mx4_quantize(_dt(x), n_rows, d, _p(x), _p(codes), _p(scales), _stream(x)))
    return codes, scales


def csa_index_scores_mx4(q_idx, w_idx, k_codes, k_scales, N: int, m: int, q_pos0: int, scores=None) -> torch.Tensor:
    """FP4 (MXFP4) indexer only: scores [B,Tq,N] f32 (-inf for entries not yet visible); operands as for
    csa_index_topk_mx4."""
    _need(q_idx, "q_idx", dims=4)
    _need(w_idx, "w_idx", torch.float32, 3)
    _need(k_codes, "k_codes", torch.uint8, 3)
    _need(k_scales, "k_scales", torch.uint8, 3)
    B, Tq, HI, dI = q_idx.shape
    rb = dI // 2
    if (w_idx.shape != (B, Tq, HI) or k_codes.shape[2] != rb or k_scales.shape[:2] != k_codes.shape[:2]
            or k_scales.shape[2] != dI // 32):
        raise ValueError("shape mismatch between the index operands")
    if not (q_idx.is_contiguous() and w_idx.is_contiguous()):
        raise ValueError("q_idx and w_idx must be contiguous")
    if k_codes.stride(1) != rb or k_scales.stride(1) != dI // 32 or k_codes.shape[1] < N:
        raise ValueError("k_codes / k_scales rows must be packed, with >= N rows")
    cap = k_codes.stride(0) // rb
    if k_codes.stride(0) != cap * rb or k_scales.stride(0) != cap * (dI // 32):
        raise ValueError("k_codes and k_scales must share one batch stride in rows")
    if scores is None:
        scores = torch.empty((B, Tq, N), dtype=torch.float32, device=q_idx.device)
    _need(scores, "scores", torch.float32, 3)
    if scores.shape != (B, Tq, N) or not scores.is_contiguous():
        raise ValueError("scores must be a contiguous [B, Tq, N] tensor")
    _check(lib().csa_index_scores_mx4(_dt(q_idx), B, Tq, N, HI, dI, m, q_pos0, _p(q_idx), _p(w_idx), _p(k_codes),
                                      _p(k_scales), cap, _p(scores), _stream(q_idx)))
    return scores


def _index_mx4_args(q_idx, w_idx, k_codes, k_scales, N, k, q_pos0, topk_idx, scores_out, workspace) -> tuple:
    """Checks csa_index_topk_mx4's tensors (allocating the missing outputs); returns (topk_idx, its arguments
    from Tq to workspace_bytes with m left out)."""
    _need(q_idx, "q_idx", dims=4)
    _need(w_idx, "w_idx", torch.float32, 3)
    _need(k_codes, "k_codes", torch.uint8, 3)
    _need(k_scales, "k_scales", torch.uint8, 3)
    B, Tq, HI, dI = q_idx.shape
    rb = dI // 2
    if (w_idx.shape != (B, Tq, HI) or k_codes.shape[2] != rb or k_scales.shape[:2] != k_codes.shape[:2]
            or k_scales.shape[2] != dI // 32):
        raise ValueError("shape mismatch between the index operands")
    if not (q_idx.is_contiguous() and w_idx.is_contiguous()):
        raise ValueError("q_idx and w_idx must be contiguous")
    if k_codes.stride(1) != rb or k_scales.stride(1) != dI // 32 or k_codes.shape[1] < N:
        raise ValueError("k_codes / k_scales rows must be packed, with >= N rows")
    cap = k_codes.stride(0) // rb
    if k_codes.stride(0) != cap * rb or k_scales.stride(0) != cap * (dI // 32):
        raise ValueError("k_codes and k_scales must share one batch stride in rows")
    if topk_idx is None:
        topk_idx = torch.empty((B, Tq, k), dtype=torch.int32, device=q_idx.device)
    _need(topk_idx, "topk_idx", torch.int32, 3)
    if scores_out is not None:
        _need(scores_out, "scores_out", torch.float32, 3)
        if scores_out.shape != (B, Tq, N) or not scores_out.is_contiguous():
            raise ValueError("scores_out must be a contiguous [B, Tq, N] tensor")
    need = index_topk_workspace_bytes(B, Tq, N, HI, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_idx.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return topk_idx, (Tq, N, HI, dI, k, q_pos0, _p(q_idx), _p(w_idx), _p(k_codes), _p(k_scales), cap, _p(topk_idx),
                      _p(scores_out), _p(workspace), ws_bytes)


def csa_index_topk_mx4(q_idx, w_idx, k_codes, k_scales, N: int, m: int, k: int, q_pos0: int, topk_idx=None,
                       scores_out=None, workspace=None) -> torch.Tensor:
    """FP4 (MXFP4) indexer + top-k.  q_idx [B,Tq,H_I,d_I] (f32/bf16, quantised inside the call), w_idx
    [B,Tq,H_I] f32, k_codes [B,cap,d_I/2], k_scales [B,cap,d_I/32] (first N rows used) -> topk_idx [B,Tq,k]."""
    topk_idx, a = _index_mx4_args(q_idx, w_idx, k_codes, k_scales, N, k, q_pos0, topk_idx, scores_out, workspace)
    _check(lib().csa_index_topk_mx4(_dt(q_idx), q_idx.shape[0], *a[:4], m, *a[4:], _stream(q_idx)))
    return topk_idx


def csa_compress_index_topk_mx4(raw, logits, m: int, entries_out, q_idx, w_idx, k_codes, k_scales, N: int, k: int,
                                q_pos0: int, topk_idx=None, scores_out=None, workspace=None,
                                hist_zero=False) -> torch.Tensor:
    """csa_compress then csa_index_topk_mx4 in one call with one launch fewer; returns topk_idx.  hist_zero: as
    csa_compress_index_topk."""
    _fused_pair(raw, q_idx)
    c = _compress_args(raw, logits, m, entries_out)
    topk_idx, a = _index_mx4_args(q_idx, w_idx, k_codes, k_scales, N, k, q_pos0, topk_idx, scores_out, workspace)
    _check(lib().csa_compress_index_topk_mx4(*c, *a, _flags(hist_zero, workspace), _stream(q_idx)))
    return topk_idx


def csa_append_rows(rows: torch.Tensor, dst: torch.Tensor, pos0: int, ring: int = 0) -> torch.Tensor:
    """rows [B, n, *row] -> dst [B, cap, *row] at rows pos0.. (ring 0) or into a mirrored ring of `ring`
    positions (dst holds 2*ring slots: position p goes to slots p % ring and p % ring + ring)."""
    _need(rows, "rows")
    _need(dst, "dst", rows.dtype)
    if rows.dim() < 2 or rows.shape[0] != dst.shape[0] or rows.shape[2:] != dst.shape[2:]:
        raise ValueError("rows and dst must be [B, n, ...] and [B, cap, ...] with the same row shape")
    B, n = rows.shape[0], rows.shape[1]
    per_row = 1
    for x in rows.shape[2:]:
        per_row *= x
    es = rows.element_size()
    for t, name in ((rows, "rows"), (dst, "dst")):
        packed = t[0:1].is_contiguous() if t.shape[0] else True
        if not packed:
            raise ValueError(f"{name}: the rows of one batch must be packed")
    _check(lib().csa_append_rows(B, n, per_row * es, _p(rows), rows.stride(0) * es, _p(dst), dst.stride(0) * es,
                                 dst.shape[1], pos0, ring, _stream(rows)))
    return dst


def _pages(pages, B):
    """pages: None, or (page_table [B, max_pages] int32, page_rows, n_pages) -> ctypes arguments."""
    if pages is None:
        return None, 0, 0, 0
    table, page_rows, n_pages = pages
    _need(table, "page_table", torch.int32, 2)
    if table.shape[0] != B or not table.is_contiguous():
        raise ValueError("page_table must be a contiguous [B, max_pages] int32 tensor")
    return _p(table), table.shape[1], page_rows, n_pages


def _append_job(rows: torch.Tensor, dst: torch.Tensor, pos0: int, ring: int, pos=None, every: int = 0,
                pages=None) -> AppendJob:
    _need(rows, "rows")
    _need(dst, "dst", rows.dtype)
    if pages is not None:  # dst is a page pool [n_pages, page_rows, ...]
        if rows.dim() < 2 or rows.shape[2:] != dst.shape[2:] or not dst.is_contiguous():
            raise ValueError("rows [B, n, ...] and a contiguous pool [n_pages, page_rows, ...] with the same row shape")
        per_row = 1
        for x in rows.shape[2:]:
            per_row *= x
        es = rows.element_size()
        if rows.shape[0] and not rows[0:1].is_contiguous():
            raise ValueError("rows: the rows of one batch must be packed")
        pt, mp, pr, npg = _pages(pages, rows.shape[0])
        if pos is not None:
            _need(pos, "pos", torch.int64, 1)
        return AppendJob(rows.shape[0], rows.shape[1], per_row * es, rows.data_ptr(), rows.stride(0) * es,
                         dst.data_ptr(), 0, mp * pr, pos0, ring, None if pos is None else pos.data_ptr(), every,
                         pt, mp, pr, npg)
    if rows.dim() < 2 or rows.shape[0] != dst.shape[0] or rows.shape[2:] != dst.shape[2:]:
        raise ValueError("rows and dst must be [B, n, ...] and [B, cap, ...] with the same row shape")
    per_row = 1
    for x in rows.shape[2:]:
        per_row *= x
    es = rows.element_size()
    for t, name in ((rows, "rows"), (dst, "dst")):
        if t.shape[0] and not t[0:1].is_contiguous():
            raise ValueError(f"{name}: the rows of one batch must be packed")
    if pos is not None:
        _need(pos, "pos", torch.int64, 1)
        if pos.shape[0] != rows.shape[0] or not pos.is_contiguous():
            raise ValueError("pos must be a contiguous [B] int64 tensor")
    return AppendJob(rows.shape[0], rows.shape[1], per_row * es, rows.data_ptr(), rows.stride(0) * es,
                     dst.data_ptr(), dst.stride(0) * es, dst.shape[1], pos0, ring,
                     None if pos is None else pos.data_ptr(), every, None, 0, 0, 0)


def csa_append_rows_multi(jobs) -> None:
    """jobs: (rows, dst, pos0, ring[, pos[, every[, pages]]]) tuples, each as csa_append_rows (pos: per-batch
    device positions added to pos0; every: keep only the token completing a group, at that group's row; pages:
    (page_table, page_rows, n_pages) with dst a page pool); one launch."""
    jobs = list(jobs)
    if not jobs:
        return
    arr = (AppendJob * len(jobs))(*[_append_job(*j) for j in jobs])
    _check(lib().csa_append_rows_multi(len(jobs), ctypes.cast(arr, ctypes.c_void_p), _stream(jobs[0][0])))


def csa_compress_channels(raw: torch.Tensor, logits: torch.Tensor, m: int, out: torch.Tensor) -> torch.Tensor:
    """raw [B, G*m, d], per-channel logits [B, G*m, d] f32 -> out [B, G, d] (written in place)."""
    _need(raw, "raw", dims=3)
    _need(logits, "logits", torch.float32, 3)
    _need(out, "out", raw.dtype, 3)
    B, Gm, d = raw.shape
    if Gm % m:
        raise ValueError("raw rows must be a multiple of m")
    G = Gm // m
    for t, n in ((raw, "raw"), (out, "out"), (logits, "logits")):
        if t.stride(1) != d:
            raise ValueError(f"{n} rows must be packed")
    if out.shape != (B, G, d) or logits.shape != (B, Gm, d):
        raise ValueError("shape mismatch between raw, logits and out")
    _check(lib().csa_compress_channels(_dt(raw), B, G, m, d, _p(raw), _bstride(raw), _p(logits), _bstride(logits),
                                       _p(out), _bstride(out), _stream(raw)))
    return out


def csa_positions_advance(pos: torch.Tensor, delta: int = 1) -> torch.Tensor:
    """pos [B] int64 (device) += delta."""
    _need(pos, "pos", torch.int64, 1)
    if not pos.is_contiguous():
        raise ValueError("pos must be contiguous")
    _check(lib().csa_positions_advance(pos.shape[0], _p(pos), delta, _stream(pos)))
    return pos


def _ragged_pos(pos, B):
    _need(pos, "pos", torch.int64, 1)
    if pos.shape[0] != B or not pos.is_contiguous():
        raise ValueError("pos must be a contiguous [B] int64 tensor")


def _ragged_compress_args(raw_ring, logit_ring, ring, m, pos, out, pages) -> tuple:
    """Checks csa_ragged_compress's tensors; returns its arguments from dt to n_pages."""
    _need(raw_ring, "raw_ring", dims=3)
    _need(logit_ring, "logit_ring", torch.float32)
    _need(out, "out", raw_ring.dtype, 3)
    B, _, d = raw_ring.shape
    _ragged_pos(pos, B)
    if raw_ring.stride(1) != d or out.stride(1) != d or logit_ring.stride(1) != 1:
        raise ValueError("ring and cache rows must be packed")
    pt, mp, pr, npg = _pages(pages, B)
    rows = mp * pr if pages is not None else out.shape[1]
    return (_dt(raw_ring), B, m, d, _p(pos), _p(raw_ring), _bstride(raw_ring), _p(logit_ring), _bstride(logit_ring),
            ring, _p(out), 0 if pages is not None else _bstride(out), rows, pt, mp, pr, npg)


def csa_ragged_compress(raw_ring: torch.Tensor, logit_ring: torch.Tensor, ring: int, m: int, pos: torch.Tensor,
                        out: torch.Tensor, pages=None) -> torch.Tensor:
    """Per sequence, the group its newest token (position pos[b]) completes, pooled out of the mirrored rings
    raw_ring [B, 2*ring, d] / logit_ring [B, 2*ring] into out [B, cap, d] at row (pos[b]+1)/m - 1."""
    _check(lib().csa_ragged_compress(*_ragged_compress_args(raw_ring, logit_ring, ring, m, pos, out, pages),
                                     _stream(raw_ring)))
    return out


def _ragged_index_args(q_idx, w_idx, k_idx, N, k, pos, topk_idx, scores_out, workspace, pages) -> tuple:
    """Checks csa_ragged_index_topk's tensors (allocating the missing outputs); returns (topk_idx, its arguments
    from N to workspace_bytes, with m and pos left out)."""
    _need(q_idx, "q_idx", dims=4)
    _need(w_idx, "w_idx", torch.float32, 3)
    _need(k_idx, "k_idx", q_idx.dtype, 3)
    B, Tq, HI, dI = q_idx.shape
    _ragged_pos(pos, B)
    if Tq != 1 or w_idx.shape != (B, 1, HI) or k_idx.shape[2] != dI or k_idx.stride(1) != dI or (
            pages is None and k_idx.shape[1] < N):
        raise ValueError("shape mismatch between the index operands")
    pt, mp, pr, npg = _pages(pages, B)
    if not (q_idx.is_contiguous() and w_idx.is_contiguous()):
        raise ValueError("q_idx and w_idx must be contiguous")
    if topk_idx is None:
        topk_idx = torch.empty((B, 1, k), dtype=torch.int32, device=q_idx.device)
    need = index_topk_workspace_bytes(B, 1, N, HI, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_idx.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return topk_idx, (N, HI, dI, k, _p(q_idx), _p(w_idx), _p(k_idx), _bstride(k_idx), pt, mp, pr, npg, _p(topk_idx),
                      _p(scores_out), _p(workspace), ws_bytes)


def csa_ragged_index_topk(q_idx, w_idx, k_idx, N: int, m: int, k: int, pos, topk_idx=None, scores_out=None,
                          workspace=None, pages=None) -> torch.Tensor:
    """One query per sequence at position pos[b]: q_idx [B,1,H_I,d_I], w_idx [B,1,H_I], k_idx [B,cap,d_I]."""
    topk_idx, a = _ragged_index_args(q_idx, w_idx, k_idx, N, k, pos, topk_idx, scores_out, workspace, pages)
    _check(lib().csa_ragged_index_topk(_dt(q_idx), q_idx.shape[0], *a[:3], m, a[3], _p(pos), *a[4:],
                                       _stream(q_idx)))
    return topk_idx


def csa_ragged_compress_index_topk(raw_ring, logit_ring, ring: int, m: int, pos, entries_out, q_idx, w_idx, k_idx,
                                   N: int, k: int, topk_idx=None, scores_out=None, workspace=None, entry_pages=None,
                                   pages=None, hist_zero=False) -> torch.Tensor:
    """csa_ragged_compress(raw_ring, logit_ring, ring, m, pos, entries_out, entry_pages) then
    csa_ragged_index_topk(q_idx, w_idx, k_idx, N, m, k, pos, ..., pages) in one call with one launch fewer.
    hist_zero: as csa_compress_index_topk."""
    _fused_pair(raw_ring, q_idx)
    c = _ragged_compress_args(raw_ring, logit_ring, ring, m, pos, entries_out, entry_pages)
    topk_idx, a = _ragged_index_args(q_idx, w_idx, k_idx, N, k, pos, topk_idx, scores_out, workspace, pages)
    _check(lib().csa_ragged_compress_index_topk(*c, *a, _flags(hist_zero, workspace), _stream(q_idx)))
    return topk_idx


def _ragged_index_mx4_args(q_idx, w_idx, k_codes, k_scales, N, k, pos, topk_idx, scores_out, workspace,
                           pages) -> tuple:
    """Checks csa_ragged_index_topk_mx4's tensors (allocating the missing outputs); returns (topk_idx, its
    arguments from N to workspace_bytes, with m and pos left out)."""
    _need(q_idx, "q_idx", dims=4)
    _need(w_idx, "w_idx", torch.float32, 3)
    B, Tq, HI, dI = q_idx.shape
    _ragged_pos(pos, B)
    rb = dI // 2
    if Tq != 1 or k_codes.shape[2] != rb or k_scales.shape[2] != dI // 32 or (pages is None and k_codes.shape[1] < N):
        raise ValueError("shape mismatch between the index operands")
    pt, mp, pr, npg = _pages(pages, B)
    cap = k_codes.stride(0) // rb
    if k_codes.stride(0) != cap * rb or k_scales.stride(0) != cap * (dI // 32):
        raise ValueError("k_codes and k_scales must share one batch stride in rows")
    if topk_idx is None:
        topk_idx = torch.empty((B, 1, k), dtype=torch.int32, device=q_idx.device)
    need = index_topk_workspace_bytes(B, 1, N, HI, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_idx.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return topk_idx, (N, HI, dI, k, _p(q_idx), _p(w_idx), _p(k_codes), _p(k_scales), cap, pt, mp, pr, npg,
                      _p(topk_idx), _p(scores_out), _p(workspace), ws_bytes)


def csa_ragged_index_topk_mx4(q_idx, w_idx, k_codes, k_scales, N: int, m: int, k: int, pos, topk_idx=None,
                              scores_out=None, workspace=None, pages=None) -> torch.Tensor:
    """csa_ragged_index_topk on MXFP4 keys (codes [B,cap,d_I/2], scales [B,cap,d_I/32])."""
    topk_idx, a = _ragged_index_mx4_args(q_idx, w_idx, k_codes, k_scales, N, k, pos, topk_idx, scores_out,
                                         workspace, pages)
    _check(lib().csa_ragged_index_topk_mx4(_dt(q_idx), q_idx.shape[0], *a[:3], m, a[3], _p(pos), *a[4:],
                                           _stream(q_idx)))
    return topk_idx


def csa_ragged_compress_index_topk_mx4(raw_ring, logit_ring, ring: int, m: int, pos, entries_out, q_idx, w_idx,
                                       k_codes, k_scales, N: int, k: int, topk_idx=None, scores_out=None,
                                       workspace=None, entry_pages=None, pages=None,
                                       hist_zero=False) -> torch.Tensor:
    """csa_ragged_compress then csa_ragged_index_topk_mx4 in one call with one launch fewer.  hist_zero: as
    csa_compress_index_topk."""
    _fused_pair(raw_ring, q_idx)
    c = _ragged_compress_args(raw_ring, logit_ring, ring, m, pos, entries_out, entry_pages)
    topk_idx, a = _ragged_index_mx4_args(q_idx, w_idx, k_codes, k_scales, N, k, pos, topk_idx, scores_out,
                                         workspace, pages)
    _check(lib().csa_ragged_compress_index_topk_mx4(*c, *a, _flags(hist_zero, workspace), _stream(q_idx)))
    return topk_idx


def csa_ragged_sparse_mqa(q, entries, topk_idx, raw_ring, ring: int, N: int, m: int, W: int, pos,
                          scale: float | None = None, out=None, lse=None, workspace=None, pages=None):
    """One query per sequence at position pos[b]; window rows from raw_ring (position p at row p % ring);
    pages: (page_table, page_rows, n_pages) with entries a page pool [n_pages, page_rows, d]."""
    B, Tq, H, d, out = _mqa_checks(q, entries, raw_ring, out, lse)
    pt, mp, pr, npg = _pages(pages, B)
    _ragged_pos(pos, B)
    k = topk_idx.shape[2]
    scale = (1.0 / d ** 0.5) if scale is None else scale
    need = mqa_workspace_bytes(B, 1, H, d, k + W)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().csa_ragged_sparse_mqa(_dt(q), B, H, d, N, m, k, W, _p(pos), scale, _p(q), _p(entries),
                                       _bstride(entries), pt, mp, pr, npg, _p(topk_idx), _p(raw_ring),
                                       _bstride(raw_ring), ring, _p(out), _p(lse), _p(workspace), ws_bytes,
                                       _stream(q)))
    return out


def hca_ragged_dense_mqa(q, entries, raw_ring, ring: int, N: int, m: int, W: int, pos, scale: float | None = None,
                         out=None, lse=None, workspace=None, pages=None):
    """HCA with one query per sequence at position pos[b]; window rows from raw_ring; pages as above."""
    B, Tq, H, d, out = _mqa_checks(q, entries, raw_ring, out, lse)
    pt, mp, pr, npg = _pages(pages, B)
    _ragged_pos(pos, B)
    scale = (1.0 / d ** 0.5) if scale is None else scale
    need = mqa_workspace_bytes(B, 1, H, d, N + W)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hca_ragged_dense_mqa(_dt(q), B, H, d, N, m, W, _p(pos), scale, _p(q), _p(entries), _bstride(entries),
                                      pt, mp, pr, npg, _p(raw_ring), _bstride(raw_ring), ring, _p(out), _p(lse),
                                      _p(workspace), ws_bytes, _stream(q)))
    return out


def csa_stream_read(buf: torch.Tensor, fronts: int, sink: torch.Tensor) -> None:
    """Measurement helper: stream-read buf (contiguous, bytes a multiple of 1 KiB x fronts) as `fronts` fronts."""
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    _need(sink, "sink", torch.int32)
    if sink.numel() < 64 or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous int32 tensor of at least 64 elements")
    _check(lib().csa_stream_read(_p(buf), buf.numel() * buf.element_size(), fronts, _p(sink), _stream(buf)))


def mqa_workspace_bytes(B, Tq, H, d, n_rows_max) -> int:
    return int(lib().csa_mqa_workspace_bytes(B, Tq, H, d, n_rows_max))


def _mqa_checks(q, entries, raw, out, lse):
    _need(q, "q", dims=4)
    _need(entries, "entries", q.dtype, 3)
    _need(raw, "raw", q.dtype, 3)
    B, Tq, H, d = q.shape
    if not q.is_contiguous() or entries.stride(1) != d or raw.stride(1) != d:
        raise ValueError("q must be contiguous and entries/raw rows packed")
    if out is None:
        out = torch.empty((B, Tq, H, d), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, 4)
    if out.shape != (B, Tq, H, d) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, Tq, H, d] float32 tensor")
    if lse is not None:
        _need(lse, "lse", torch.float32, 3)
        if lse.shape != (B, Tq, H) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous [B, Tq, H] float32 tensor")
    return B, Tq, H, d, out


def csa_sparse_mqa(q, entries, topk_idx, raw, N: int, m: int, W: int, q_pos0: int, raw_pos0: int,
                   scale: float | None = None, out=None, lse=None, workspace=None):
    """Sparse shared-KV MQA over topk_idx rows plus the raw window -> out [B,Tq,H,d] f32 (and lse if given)."""
    B, Tq, H, d, out = _mqa_checks(q, entries, raw, out, lse)
    _need(topk_idx, "topk_idx", torch.int32, 3)
    if topk_idx.shape[:2] != (B, Tq) or not topk_idx.is_contiguous():
        raise ValueError("topk_idx must be a contiguous [B, Tq, k] tensor")
    k = topk_idx.shape[2]
    scale = (1.0 / d ** 0.5) if scale is None else scale
    need = mqa_workspace_bytes(B, Tq, H, d, k + W)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().csa_sparse_mqa(_dt(q), B, Tq, H, d, N, m, k, W, q_pos0, scale, _p(q), _p(entries),
                                _bstride(entries), _p(topk_idx), _p(raw), _bstride(raw), raw_pos0, raw.shape[1],
                                _p(out), _p(lse), _p(workspace), ws_bytes, _stream(q)))
    return out


def hca_dense_mqa(q, entries, raw, N: int, m: int, W: int, q_pos0: int, raw_pos0: int, scale: float | None = None,
                  out=None, lse=None, workspace=None):
    """Dense shared-KV MQA over all visible entries plus the raw window -> out [B,Tq,H,d] f32."""
    B, Tq, H, d, out = _mqa_checks(q, entries, raw, out, lse)
    scale = (1.0 / d ** 0.5) if scale is None else scale
    need = mqa_workspace_bytes(B, Tq, H, d, N + W)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().hca_dense_mqa(_dt(q), B, Tq, H, d, N, m, W, q_pos0, scale, _p(q), _p(entries), _bstride(entries),
                               _p(raw), _bstride(raw), raw_pos0, raw.shape[1], _p(out), _p(lse), _p(workspace),
                               ws_bytes, _stream(q)))
    return out


from .step import AttentionStep  # noqa: E402  (uses the functions above)
from .stream import StreamingLayer, chunk_plan, ring_size  # noqa: E402
from .ragged import RaggedLayer  # noqa: E402
from .hybrid import HybridStack, alternating  # noqa: E402
