"""Streaming use of one attention layer: the cache it keeps between steps.

DeepSeek-V4 overview page, section 2.2 (CSA): every m consecutive tokens
become one compressed entry (step 1), the lightning indexer scores a query
against every complete entry through the entries' index keys (step 2), and
the attention reads the selected entries together with a window of raw
tokens (step 3); section 2.3 (HCA): the same with m = 128 and every entry.

A layer keeps, per sequence:
  raw ring    [2R, d]   the raw latents of the last R positions (mirrored: a
                        window of up to R consecutive positions is one plain
                        strided view, so the kernels read it as they read any
                        raw buffer)
  logit ring  [2R]      their pooling logits
  entries     [cap, d]  compressed entries 0 .. N-1
  index keys  [cap, dI] (CSA; or their MXFP4 codes [cap, dI/2] and scale
                        bytes [cap, dI/32] when the indexer runs on FP4)

Prefill from position 0 is a sequence of chunks of up to `chunk` tokens;
decoding is a chunk of one token.  A chunk of n tokens at p0 .. p0+n-1:
  1. appends their raw rows and logits to the rings;
  2. compresses the groups that complete inside the chunk (N .. (p0+n)//m - 1)
     out of the ring;
  3. appends those groups' index keys: one per group given by the caller
     (index_keys="given"), or pooled by the same compressor from per-token
     index keys kept in their own ring (index_keys="pooled"), quantised to
     MXFP4 when the indexer runs on FP4;
  4. runs the indexer and top-k for the chunk's queries (CSA);
  5. runs the attention over the selected (CSA) or all visible (HCA)
     entries plus the raw window, read out of the ring.
Pooling logits are one per token (pool="token") or one per token and
channel (pool="channel", csa_compress_channels); pooled index keys use the
entry's weights with per-token logits and their own per-channel logits with
per-channel pooling.
Every step is a call into libcsa; this module keeps positions and views.
"""
from __future__ import annotations

import dataclasses

import torch

from . import (csa_append_rows_multi, csa_compress, csa_compress_channels, csa_compress_index_topk,
               csa_compress_index_topk_mx4, csa_index_topk, csa_index_topk_mx4,
               csa_mx4_quantize, csa_sparse_mqa, hca_dense_mqa, index_topk_workspace_bytes, mqa_workspace_bytes)


@dataclasses.dataclass(frozen=True)
class ChunkPlan:
    """Bookkeeping of one chunk (positions p0 .. p0+n-1, N entries before it)."""
    p0: int
    n: int
    g0: int          # first group compressed by the chunk (= N before it)
    g_new: int       # groups that complete inside the chunk
    comp_lo: int     # first raw position those groups pool (g0 * m)
    win_lo: int      # first raw position of the earliest query's window
    win_len: int     # raw positions win_lo .. p0+n-1 the attention may read
    ring_oldest: int # oldest position still in the ring after the append


def ring_size(chunk: int, m: int, W: int) -> int:
    """Ring positions a layer needs: a chunk reads back at most max(W, m) - 1 positions before its
    first token (the first query's window, or the first token of the group that token belongs to)."""
    return chunk + max(W, m) - 1


def chunk_plan(p0: int, n: int, N: int, m: int, W: int, R: int) -> ChunkPlan:
    """Plan the chunk of n tokens at p0 when N entries exist (N = p0 // m after whole-group steps)."""
    if n < 1 or p0 < 0:
        raise ValueError("a chunk holds at least one token at a position >= 0")
    if N != p0 // m:
        raise ValueError(f"{N} entries before position {p0}: expected {p0 // m} (groups are emitted as they complete)")
    g_new = (p0 + n) // m - N
    win_lo = max(0, p0 - W + 1)
    plan = ChunkPlan(p0=p0, n=n, g0=N, g_new=g_new, comp_lo=N * m, win_lo=win_lo, win_len=p0 + n - win_lo,
                     ring_oldest=max(0, p0 + n - R))
    if g_new > 0 and plan.comp_lo < plan.ring_oldest:
        raise ValueError("the ring no longer holds the first token of a group to compress")
    if plan.win_lo < plan.ring_oldest:
        raise ValueError("the ring no longer holds the window of the chunk's first query")
    return plan


class StreamingLayer:
    """One CSA or HCA layer's cache for B sequences that advance together."""

    def __init__(self, *, mode: str, B: int, H: int, d: int, m: int, W: int, capacity: int, chunk: int,
                 dtype=torch.bfloat16, k: int = 0, HI: int = 0, dI: int = 0, index_fmt: str = "elem",
                 scale: float | None = None, pool: str = "token", index_keys: str = "given", device="cuda"):
        assert mode in ("csa", "hca") and index_fmt in ("elem", "mx4")
        assert pool in ("token", "channel") and index_keys in ("given", "pooled")
        if mode == "csa" and (k < 1 or HI < 1 or dI < 1):
            raise ValueError("CSA needs k, HI and dI")
        if index_keys == "pooled" and index_fmt == "mx4":
            raise ValueError("pooled index keys are built for element-type index keys only")
        self.pool, self.index_keys = pool, index_keys
        self.mode, self.B, self.H, self.d, self.m, self.W = mode, B, H, d, m, W
        self.k, self.HI, self.dI, self.index_fmt = k, HI, dI, index_fmt
        self.chunk, self.capacity, self.dtype, self.device = chunk, capacity, dtype, device
        self.scale = (1.0 / d ** 0.5) if scale is None else scale
        self.R = ring_size(chunk, m, W)
        self.cap_e = max(1, capacity // m)
        self.raw_ring = torch.zeros((B, 2 * self.R, d), dtype=dtype, device=device)
        self.logit_ring = torch.zeros((B, 2 * self.R, d if pool == "channel" else 1), dtype=torch.float32,
                                      device=device)
        self.entries = torch.zeros((B, self.cap_e, d), dtype=dtype, device=device)
        if mode == "csa":
            if index_fmt == "mx4":
                self.k_codes = torch.zeros((B, self.cap_e, dI // 2), dtype=torch.uint8, device=device)
                self.k_scales = torch.zeros((B, self.cap_e, dI // 32), dtype=torch.uint8, device=device)
            else:
                self.k_idx = torch.zeros((B, self.cap_e, dI), dtype=dtype, device=device)
            if index_keys == "pooled":
                self.kidx_ring = torch.zeros((B, 2 * self.R, dI), dtype=dtype, device=device)
                if pool == "channel":
                    self.kidx_logit_ring = torch.zeros((B, 2 * self.R, dI), dtype=torch.float32, device=device)
            # (the selection's and the attention's plans change with the number of queries: the
            # workspaces cover every chunk length up to `chunk`, at the full entry capacity)
            nb = max(index_topk_workspace_bytes(B, t, self.cap_e, HI, k) for t in range(1, chunk + 1))
            self.idx_ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=device)
        rows_max = (k if mode == "csa" else self.cap_e) + W
        nb = max(mqa_workspace_bytes(B, t, H, d, rows_max) for t in range(1, chunk + 1))
        self.mqa_ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=device)
        self.pos = 0  # tokens consumed
        self.N = 0    # entries complete

    # ---- views of the rings
    def _ring_view(self, ring: torch.Tensor, lo: int, length: int) -> torch.Tensor:
        s = lo % self.R
        return ring[:, s:s + length]

    def resume(self, pos: int):
        """Continue a stream at position `pos` whose state the caller has put in place: entries (and
        index keys) 0 .. pos//m - 1 and the ring's positions max(0, pos-R) .. pos-1 (both mirror slots)."""
        if pos < 0 or pos // self.m > self.cap_e:
            raise ValueError("position outside the layer's capacity")
        self.pos, self.N = pos, pos // self.m

    def plan(self, n: int) -> ChunkPlan:
        return chunk_plan(self.pos, n, self.N, self.m, self.W, self.R)

    def _pool(self, rows: torch.Tensor, logits: torch.Tensor, out: torch.Tensor):
        if self.pool == "channel":
            csa_compress_channels(rows, logits, self.m, out)
        else:
            csa_compress(rows, logits[..., 0], self.m, out)

    def step(self, raw: torch.Tensor, logits: torch.Tensor, q: torch.Tensor, k_idx_new: torch.Tensor | None = None,
             q_idx: torch.Tensor | None = None, w_idx: torch.Tensor | None = None, out: torch.Tensor | None = None,
             lse: torch.Tensor | None = None, topk_idx: torch.Tensor | None = None,
             k_idx_tokens: torch.Tensor | None = None, k_idx_logits: torch.Tensor | None = None):
        """Advance by one chunk.  raw [B, n, d], logits [B, n] f32 (pool "token") or [B, n, d] (pool
        "channel"), q [B, n, H, d]; CSA also q_idx [B, n, HI, dI], w_idx [B, n, HI] and the index keys:
        k_idx_new [B, g_new, dI] (those of the groups completing in the chunk; index_keys "given") or
        k_idx_tokens [B, n, dI] (per token, pooled into the entries' keys; index_keys "pooled", with
        k_idx_logits [B, n, dI] f32 under per-channel pooling).
        Returns (out [B, n, H, d] f32, lse [B, n, H], topk_idx [B, n, k] or None)."""
        B, n = raw.shape[0], raw.shape[1]
        q = q.contiguous()
        if self.mode == "csa":
            q_idx, w_idx = q_idx.contiguous(), w_idx.contiguous()
        if n > self.chunk:
            raise ValueError(f"chunk of {n} tokens above the layer's {self.chunk}")
        p = self.plan(n)
        if p.g0 + p.g_new > self.cap_e:
            raise ValueError("entry capacity exhausted")
        # 1. raw rows and logits (and per-token index keys) into the rings, one launch
        jobs = [(raw, self.raw_ring, p.p0, self.R),
                (logits.reshape(B, n, self.logit_ring.shape[2]), self.logit_ring, p.p0, self.R)]
        if self.mode == "csa" and self.index_keys == "pooled":
            jobs.append((k_idx_tokens, self.kidx_ring, p.p0, self.R))
            if self.pool == "channel":
                jobs.append((k_idx_logits, self.kidx_logit_ring, p.p0, self.R))
        csa_append_rows_multi(jobs)
        # 2. the groups completing in this chunk (pooled by token logits in a CSA layer: inside the index
        # call, whose first launch then also clears the selection's histograms)
        comp = ()
        if p.g_new > 0:
            L = p.g_new * self.m
            args = (self._ring_view(self.raw_ring, p.comp_lo, L), self._ring_view(self.logit_ring, p.comp_lo, L),
                    self.entries[:, p.g0:p.g0 + p.g_new])
            if self.mode == "csa" and self.pool != "channel" and q_idx.dtype == raw.dtype:
                comp = (args[0], args[1][..., 0], self.m, args[2])
            else:
                self._pool(*args)
        N = p.g0 + p.g_new
        raw_win = self._ring_view(self.raw_ring, p.win_lo, p.win_len)
        if out is None:
            out = torch.empty((B, n, self.H, self.d), dtype=torch.float32, device=raw.device)
        if lse is None:
            lse = torch.empty((B, n, self.H), dtype=torch.float32, device=raw.device)
        if self.mode == "csa":
            # 3. their index keys
            if p.g_new > 0 and self.index_keys == "pooled":
                L = p.g_new * self.m
                lg = self.kidx_logit_ring if self.pool == "channel" else self.logit_ring
                self._pool(self._ring_view(self.kidx_ring, p.comp_lo, L), self._ring_view(lg, p.comp_lo, L),
                           self.k_idx[:, p.g0:p.g0 + p.g_new])
            elif p.g_new > 0:
                if k_idx_new is None or k_idx_new.shape[1] != p.g_new:
                    raise ValueError(f"the chunk completes {p.g_new} groups: k_idx_new must hold {p.g_new} rows")
                if self.index_fmt == "mx4":
                    codes, scales = csa_mx4_quantize(k_idx_new.contiguous())
                    csa_append_rows_multi([(codes, self.k_codes, p.g0, 0), (scales, self.k_scales, p.g0, 0)])
                else:
                    csa_append_rows_multi([(k_idx_new, self.k_idx, p.g0, 0)])
            # 4. indexer + top-k
            if topk_idx is None:
                topk_idx = torch.empty((B, n, self.k), dtype=torch.int32, device=raw.device)
            if self.index_fmt == "mx4" and comp:
                csa_compress_index_topk_mx4(*comp, q_idx, w_idx, self.k_codes, self.k_scales, N, self.k, p.p0,
                                            topk_idx=topk_idx, workspace=self.idx_ws)
            elif self.index_fmt == "mx4":
                csa_index_topk_mx4(q_idx, w_idx, self.k_codes, self.k_scales, N, self.m, self.k, p.p0,
                                   topk_idx=topk_idx, workspace=self.idx_ws)
            elif comp:
                csa_compress_index_topk(*comp, q_idx, w_idx, self.k_idx, N, self.k, p.p0, topk_idx=topk_idx,
                                        workspace=self.idx_ws)
            else:
                csa_index_topk(q_idx, w_idx, self.k_idx, N, self.m, self.k, p.p0, topk_idx=topk_idx,
                               workspace=self.idx_ws)
            # 5. attention
            csa_sparse_mqa(q, self.entries, topk_idx, raw_win, N, self.m, self.W, p.p0, p.win_lo, scale=self.scale,
                           out=out, lse=lse, workspace=self.mqa_ws)
        else:
            hca_dense_mqa(q, self.entries, raw_win, N, self.m, self.W, p.p0, p.win_lo, scale=self.scale, out=out,
                          lse=lse, workspace=self.mqa_ws)
        self.pos, self.N = p.p0 + n, N
        return out, lse, topk_idx
