"""Ragged decode: one attention layer's cache for B sequences at different lengths.

DeepSeek-V4 overview page, section 2.2 (CSA) and 2.3 (HCA), in the serving
form: every sequence decodes one token per step, each at its own position.
The positions live in device memory (``pos``, int64 [B]: the position the
next token of each sequence takes) and every kernel of the step reads them,
so a whole decode step is one fixed sequence of launches: it can be captured
in a HIP graph once and replayed for every later token, the positions
advancing on the GPU.

A step (new token of sequence b at position t_b = pos[b]):
  1. one batched append: the raw row and logit into the mirrored rings at
     t_b mod R, and -- for the sequences whose token completes a group -- the
     group's index key into the key cache (given per token; only the
     completing token's key is kept, quantised first when the indexer runs
     on FP4);
  2. ragged compression: those sequences' groups pooled out of the rings;
  3. ragged index + top-k (CSA) over each sequence's visible entries (2 and
     3 in one call, the compression sharing a launch with the selection's
     histogram clear);
  4. ragged attention (selected or all visible entries, window from the ring);
  5. pos += 1.
Ring of R = max(W, m) positions: the window of the newest token and the
tokens of the group it completes.

Paged caches (page_rows = P, a power of two >= 16): the entries and index
keys of all sequences live in pools of P-row pages, sequence b's entry j in
row j mod P of page page_table[b, j // P]; one table serves both caches.
By default each sequence gets its pages from a shuffled free list up front
(assign_pages hands out other layouts).  A pool of fewer than B * max_pages
pages starts with an all-zero table: assign_pages must then give every
sequence its own pages before the layer is used.
"""
from __future__ import annotations

import torch

from . import (csa_append_rows, csa_append_rows_multi, csa_mx4_quantize, csa_positions_advance,
               csa_ragged_compress, csa_ragged_compress_index_topk, csa_ragged_compress_index_topk_mx4,
               csa_ragged_index_topk, csa_ragged_index_topk_mx4, csa_ragged_sparse_mqa, hca_ragged_dense_mqa,
               index_topk_workspace_bytes, mqa_workspace_bytes)


class RaggedLayer:
    def __init__(self, *, mode: str, B: int, H: int, d: int, m: int, W: int, capacity: int, dtype=torch.bfloat16,
                 k: int = 0, HI: int = 0, dI: int = 0, index_fmt: str = "elem", scale: float | None = None,
                 page_rows: int = 0, n_pages: int = 0, device="cuda", seed: int = 0):
        assert mode in ("csa", "hca") and index_fmt in ("elem", "mx4")
        if mode == "csa" and (k < 1 or HI < 1 or dI < 1):
            raise ValueError("CSA needs k, HI and dI")
        self.mode, self.B, self.H, self.d, self.m, self.W = mode, B, H, d, m, W
        self.k, self.HI, self.dI, self.index_fmt, self.dtype = k, HI, dI, index_fmt, dtype
        self.scale = (1.0 / d ** 0.5) if scale is None else scale
        self.R = max(W, m, 1)
        self.cap_e = max(1, capacity // m)
        self.pos = torch.zeros((B,), dtype=torch.int64, device=device)
        self.raw_ring = torch.zeros((B, 2 * self.R, d), dtype=dtype, device=device)
        self.logit_ring = torch.zeros((B, 2 * self.R, 1), dtype=torch.float32, device=device)
        self.page_rows = page_rows
        if page_rows:
            self.max_pages = -(-self.cap_e // page_rows)
            self.n_pages = n_pages or B * self.max_pages
            lead = (self.n_pages, page_rows)
            self.page_table = torch.zeros((B, self.max_pages), dtype=torch.int32, device=device)
            if self.n_pages >= B * self.max_pages:  # every sequence its own pages, interleaved in the pool
                g = torch.Generator().manual_seed(seed)
                perm = torch.randperm(self.n_pages, generator=g)[:B * self.max_pages].to(torch.int32)
                self.page_table.copy_(perm.reshape(B, self.max_pages))
            self.pages = (self.page_table, page_rows, self.n_pages)
        else:
            lead = (B, self.cap_e)
            self.pages = None
        self.entries = torch.zeros(lead + (d,), dtype=dtype, device=device)
        if mode == "csa":
            if index_fmt == "mx4":
                self.k_codes = torch.zeros(lead + (dI // 2,), dtype=torch.uint8, device=device)
                self.k_scales = torch.zeros(lead + (dI // 32,), dtype=torch.uint8, device=device)
                self._codes = torch.empty((B, 1, dI // 2), dtype=torch.uint8, device=device)
                self._scales = torch.empty((B, 1, dI // 32), dtype=torch.uint8, device=device)
            else:
                self.k_idx = torch.zeros(lead + (dI,), dtype=dtype, device=device)
            nb = index_topk_workspace_bytes(B, 1, self.cap_e, HI, k)
            # zero-filled once; the index calls (one shape) leave its top-k histograms zero
            self.idx_ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device=device)
            self.topk_idx = torch.empty((B, 1, k), dtype=torch.int32, device=device)
        rows_max = (k if mode == "csa" else self.cap_e) + W
        nb = mqa_workspace_bytes(B, 1, H, d, rows_max)
        self.mqa_ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=device)
        self.out = torch.empty((B, 1, H, d), dtype=torch.float32, device=device)
        self.lse = torch.empty((B, 1, H), dtype=torch.float32, device=device)

    def assign_pages(self, b: int, page_ids):
        """Give sequence b the listed pages of the pool (its entries 0 .. P-1 in the first, and so on)."""
        ids = torch.as_tensor(page_ids, dtype=torch.int32)
        self.page_table[b, :ids.numel()] = ids.to(self.page_table.device)

    def _cache_rows(self, t: torch.Tensor, b: int, n: int):
        """Sequence b's first n cache rows of t as a list of (view, lo, hi) pieces (one per page when paged)."""
        if not self.page_rows:
            return [(t[b, :n], 0, n)]
        P = self.page_rows
        ids = self.page_table[b].tolist()
        return [(t[ids[i // P], :min(P, n - i)], i, min(i + P, n)) for i in range(0, n, P)]

    def seed(self, b: int, pos_b: int, raw_tail: torch.Tensor, logits_tail: torch.Tensor,
             entries: torch.Tensor | None = None, k_idx: torch.Tensor | None = None):
        """Put sequence b's state in place: it has consumed positions 0 .. pos_b-1; raw_tail [L, d] and
        logits_tail [L] are its last L = min(R, pos_b) tokens; entries [pos_b//m, d] and (CSA) their index
        keys k_idx [pos_b//m, dI] are its cache."""
        L = min(self.R, pos_b)
        n_e = pos_b // self.m
        if raw_tail.shape[0] != L or logits_tail.shape[0] != L:
            raise ValueError(f"the ring holds the last {L} tokens")
        if n_e > self.cap_e:
            raise ValueError("entry capacity exceeded")
        if L:
            csa_append_rows(raw_tail[None], self.raw_ring[b:b + 1], pos_b - L, ring=self.R)
            csa_append_rows(logits_tail.reshape(1, L, 1), self.logit_ring[b:b + 1], pos_b - L, ring=self.R)
        if n_e:
            for view, lo, hi in self._cache_rows(self.entries, b, n_e):
                view.copy_(entries[lo:hi])
            if self.mode == "csa":
                if self.index_fmt == "mx4":
                    c, s = csa_mx4_quantize(k_idx.contiguous())
                    for view, lo, hi in self._cache_rows(self.k_codes, b, n_e):
                        view.copy_(c[lo:hi])
                    for view, lo, hi in self._cache_rows(self.k_scales, b, n_e):
                        view.copy_(s[lo:hi])
                else:
                    for view, lo, hi in self._cache_rows(self.k_idx, b, n_e):
                        view.copy_(k_idx[lo:hi])
        self.pos[b] = pos_b

    def step(self, raw: torch.Tensor, logits: torch.Tensor, q: torch.Tensor, k_idx_tok: torch.Tensor | None = None,
             q_idx: torch.Tensor | None = None, w_idx: torch.Tensor | None = None):
        """One token per sequence: raw [B, 1, d], logits [B, 1] f32, q [B, 1, H, d] (contiguous); CSA also
        k_idx_tok [B, 1, dI] (the index key of the group this token completes; read only for the sequences
        whose token completes one), q_idx [B, 1, HI, dI], w_idx [B, 1, HI].  Writes self.out, self.lse
        (and self.topk_idx) and advances self.pos.  Fixed launches: capturable in a HIP graph."""
        B = self.B
        jobs = [(raw, self.raw_ring, 0, self.R, self.pos), (logits.reshape(B, 1, 1), self.logit_ring, 0, self.R, self.pos)]
        if self.mode == "csa":
            pg = self.pages
            if self.index_fmt == "mx4":
                csa_mx4_quantize(k_idx_tok, codes=self._codes, scales=self._scales)
                jobs += [(self._codes, self.k_codes, 0, 0, self.pos, self.m, pg),
                         (self._scales, self.k_scales, 0, 0, self.pos, self.m, pg)]
            else:
                jobs.append((k_idx_tok, self.k_idx, 0, 0, self.pos, self.m, pg))
        csa_append_rows_multi(jobs)
        # the group the token completes (if any), pooled out of the rings: in one of the index call's launches
        # when the index operands share the rings' element type (CSA), else on its own
        comp = (self.raw_ring, self.logit_ring[..., 0], self.R, self.m, self.pos, self.entries)
        fuse = self.mode == "csa" and q_idx.dtype == self.raw_ring.dtype
        if not fuse:
            csa_ragged_compress(*comp, pages=self.pages)
        if self.mode == "csa":
            ix = dict(topk_idx=self.topk_idx, workspace=self.idx_ws, pages=self.pages)
            if self.index_fmt == "mx4":
                keys = (q_idx, w_idx, self.k_codes, self.k_scales, self.cap_e)
                if fuse:
                    csa_ragged_compress_index_topk_mx4(*comp, *keys, self.k, entry_pages=self.pages, hist_zero=True,
                                                       **ix)
                else:
                    csa_ragged_index_topk_mx4(*keys, self.m, self.k, self.pos, **ix)
            else:
                keys = (q_idx, w_idx, self.k_idx, self.cap_e)
                if fuse:
                    csa_ragged_compress_index_topk(*comp, *keys, self.k, entry_pages=self.pages, hist_zero=True, **ix)
                else:
                    csa_ragged_index_topk(*keys, self.m, self.k, self.pos, **ix)
            csa_ragged_sparse_mqa(q, self.entries, self.topk_idx, self.raw_ring, self.R, self.cap_e, self.m, self.W,
                                  self.pos, scale=self.scale, out=self.out, lse=self.lse, workspace=self.mqa_ws,
                                  pages=self.pages)
        else:
            hca_ragged_dense_mqa(q, self.entries, self.raw_ring, self.R, self.cap_e, self.m, self.W, self.pos,
                                 scale=self.scale, out=self.out, lse=self.lse, workspace=self.mqa_ws,
                                 pages=self.pages)
        csa_positions_advance(self.pos, 1)
        return self.out
