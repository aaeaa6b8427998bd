"""One layer step of hybrid compressed attention, composed from the C-ABI calls.

CSA (DeepSeek-V4 overview page, section 2.2):  compress the new groups ->
lightning indexer + top-k -> sparse shared-KV MQA with the raw window (the
first two in one library call, the compression sharing a launch with the
selection's histogram clear).  With
FP4 indexer operands (section 9, item 5; index_fmt "mx4") the indexer
quantises the index queries to MXFP4 itself and scores them against MXFP4
keys that were quantised once, when they entered the cache
(quantize_index_keys).
HCA (section 2.3):  compress the new group -> dense shared-KV MQA.

The step owns its outputs and workspaces (allocated once, so the step can be
replayed from a captured HIP graph) and only calls the library.
"""
from __future__ import annotations

import torch

from . import csa_compress, csa_compress_index_topk, csa_compress_index_topk_mx4, csa_index_topk, csa_index_topk_mx4, \
    csa_mx4_quantize, csa_sparse_mqa, hca_dense_mqa, index_topk_workspace_bytes, mqa_workspace_bytes


class AttentionStep:
    """Step of one attention layer for a block of Tq new tokens of B sequences.

    Geometry (all positions absolute): queries at q_pos0 .. q_pos0+Tq-1; the
    cache holds N entries after the step, of which g0 .. N-1 are produced by
    this step from raw rows; the raw buffer holds positions raw_pos0 ...
    """

    def __init__(self, *, mode: str, N: int, m: int, W: int, q_pos0: int, raw_pos0: int, g0: int, k: int = 0,
                 scale: float | None = None, index_fmt: str = "elem"):
        assert mode in ("csa", "hca") and index_fmt in ("elem", "mx4")
        self.mode, self.N, self.m, self.W, self.k = mode, N, m, W, k
        self.index_fmt = index_fmt
        self.q_pos0, self.raw_pos0, self.g0 = q_pos0, raw_pos0, g0
        self.scale = scale
        self._ready = False

    def _prepare(self, x: dict):
        q = x["q"]
        B, Tq, H, d = q.shape
        dev = q.device
        self.out = torch.empty((B, Tq, H, d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Tq, H), dtype=torch.float32, device=dev)
        rows_max = (self.k if self.mode == "csa" else self.N) + self.W
        nb = mqa_workspace_bytes(B, Tq, H, d, rows_max)
        self.mqa_ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
        if self.mode == "csa":
            HI = x["q_idx"].shape[2]
            self.topk_idx = torch.empty((B, Tq, self.k), dtype=torch.int32, device=dev)

            nb = index_topk_workspace_bytes(B, Tq, self.N, HI, self.k)
            # zero-filled once: every index call of this one shape leaves its top-k histograms zero, so the fused
            # calls need not clear them (and carry the compression in the top-k filter launch)
            self.idx_ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device=dev)
        self._ready = True

    def __call__(self, x: dict) -> torch.Tensor:
        """x: raw, logits, entries, q (+ q_idx, w_idx, k_idx for CSA) on the GPU.  Returns out."""
        if not self._ready:
            self._prepare(x)
        raw, entries = x["raw"], x["entries"]
        # the new groups' compression rides in one of the index call's launches (CSA) or runs alone (HCA)
        comp = ()
        if self.N > self.g0:
            r0 = self.g0 * self.m - self.raw_pos0
            comp = (raw[:, r0:r0 + (self.N - self.g0) * self.m], x["logits"], self.m, entries[:, self.g0:self.N])
            if self.mode != "csa" or x["q_idx"].dtype != raw.dtype:  # (one element type per fused call)
                csa_compress(*comp)
                comp = ()
        if self.mode == "csa" and self.index_fmt == "mx4":
            args = (x["q_idx"], x["w_idx"], x["k_codes"], x["k_scales"], self.N)
            if comp:
                csa_compress_index_topk_mx4(*comp, *args, self.k, self.q_pos0, topk_idx=self.topk_idx,
                                            workspace=self.idx_ws, hist_zero=True)
            else:
                csa_index_topk_mx4(*args, self.m, self.k, self.q_pos0, topk_idx=self.topk_idx, workspace=self.idx_ws)
        elif self.mode == "csa":
            args = (x["q_idx"], x["w_idx"], x["k_idx"], self.N)
            if comp:
                csa_compress_index_topk(*comp, *args, self.k, self.q_pos0, topk_idx=self.topk_idx,
                                        workspace=self.idx_ws, hist_zero=True)
            else:
                csa_index_topk(*args, self.m, self.k, self.q_pos0, topk_idx=self.topk_idx, workspace=self.idx_ws)
        if self.mode == "csa":
            csa_sparse_mqa(x["q"], entries, self.topk_idx, raw, self.N, self.m, self.W, self.q_pos0, self.raw_pos0,
                           scale=self.scale, out=self.out, lse=self.lse, workspace=self.mqa_ws)
        else:
            hca_dense_mqa(x["q"], entries, raw, self.N, self.m, self.W, self.q_pos0, self.raw_pos0, scale=self.scale,
                          out=self.out, lse=self.lse, workspace=self.mqa_ws)
        return self.out

    @staticmethod
    def quantize_index_keys(x: dict) -> dict:
        """Give x the MXFP4 form of its index keys (k_codes, k_scales), as a cache stores them."""
        x["k_codes"], x["k_scales"] = csa_mx4_quantize(x["k_idx"])
        return x

    @classmethod
    def for_workload(cls, wl) -> "AttentionStep":
        return cls(mode=wl.mode, N=wl.N, m=wl.m, W=wl.W, q_pos0=wl.q_pos0, raw_pos0=wl.raw_pos0, g0=wl.g0, k=wl.k,
                   scale=wl.scale, index_fmt=getattr(wl, "index_fmt", "elem"))
