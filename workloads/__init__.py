"""Seeded synthetic workloads for compressed attention (CSA / HCA).

This module only describes shapes and draws random numbers.  It holds none of
the method's arithmetic, and both the HIP path and the CPU oracle take their
inputs from here.

Shapes follow the workloads the DeepSeek-V4 overview page describes (section
2.2: m=4 compression, top-1024 selection, million-token contexts; section 2.3:
m=128 dense attention) with the latent width of the MLA notes (512-d latent,
section "MLA" of the sealessland.top architecture notes).  No dataset is used:
every tensor is drawn from a seeded generator.

Seed of tensor ``name`` in a numbered workload ``c`` is ``1000*c + ordinal``
with ordinals raw=1, logits=2, entries=3, k_idx=4, q_idx=5, w_idx=6, q=7,
stress subset=8.  Values are drawn in float32 (``randn``/``rand``) and then
converted with round-to-nearest-even to bf16 where the workload is bf16.  The
same seed gives different numbers on a CPU generator and on a GPU generator;
each run is self-consistent because the oracle receives host copies of the
exact device tensors.
"""
from __future__ import annotations

import dataclasses
import math

import torch

ORD = dict(raw=1, logits=2, entries=3, k_idx=4, q_idx=5, w_idx=6, q=7, stress=8, k_idx_logits=9)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16": element type of raw, entries, q, q_idx, k_idx
    B: int              # batch (independent sequences)
    T: int              # context length including the new query tokens
    Tq: int             # number of new query tokens, positions T-Tq .. T-1
    m: int              # tokens per compressed entry
    d: int              # latent / entry / head width
    H: int              # query heads sharing the one KV
    W: int              # sliding window of raw tokens (includes the query position)
    k: int = 0          # top-k (CSA); 0 means dense HCA attention
    HI: int = 0         # index heads (CSA)
    dI: int = 0         # index width (CSA)
    stress_frac: float = 0.0   # fraction of entries whose row and index key are scaled by 8
    seed_base: int = 0  # 1000 * workload number
    index_fmt: str = "elem"    # indexer operands: "elem" (the element type) or "mx4" (MXFP4 codes + scales)

    # ---- derived shapes (bookkeeping only) ----
    @property
    def mode(self) -> str:
        return "csa" if self.k > 0 else "hca"

    @property
    def N(self) -> int:          # compressed entries that exist after this step
        return self.T // self.m

    @property
    def q_pos0(self) -> int:
        return self.T - self.Tq

    @property
    def g0(self) -> int:         # first group that contains a new token (compressed in the step)
        return min(self.q_pos0 // self.m, self.N)

    @property
    def G_new(self) -> int:      # groups compressed in the step
        return self.N - self.g0

    @property
    def raw_pos0(self) -> int:   # first raw position held in the raw buffer
        win0 = max(0, self.q_pos0 - self.W + 1) if self.W > 0 else self.q_pos0
        return min(self.g0 * self.m, win0)

    @property
    def raw_len(self) -> int:
        return self.T - self.raw_pos0

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The five workloads: a tiny fp32 CSA prefill, CSA decode at 128K, HCA decode at
# 1M, a CSA prefill chunk at 64K, and CSA decode at 1M with a stressed 1%.
CONFIGS = {
    "c1": Workload("csa_prefill_tiny_fp32_T2048", "f32", B=1, T=2048, Tq=2048, m=4, d=128, H=8, W=64,
                   k=64, HI=4, dI=32, seed_base=1000),
    "c2": Workload("csa_decode_bf16_B32_ctx128K", "bf16", B=32, T=131072, Tq=1, m=4, d=512, H=64, W=128,
                   k=1024, HI=64, dI=128, seed_base=2000),
    "c3": Workload("hca_decode_bf16_B16_ctx1M", "bf16", B=16, T=1048576, Tq=1, m=128, d=512, H=64, W=128,
                   seed_base=3000),
    "c4": Workload("csa_prefill_chunk_bf16_ctx64K_q4096", "bf16", B=1, T=65536, Tq=4096, m=4, d=512, H=64,
                   W=128, k=1024, HI=64, dI=128, seed_base=4000),
    "c5": Workload("csa_decode_bf16_B4_ctx1M_stress", "bf16", B=4, T=1048576, Tq=1, m=4, d=512, H=64, W=128,
                   k=1024, HI=64, dI=128, stress_frac=0.01, seed_base=5000),
}
# the 128K and 1M CSA decode steps with FP4 (MXFP4) index queries and keys:
# the same seeded inputs, the keys quantised once when the cache is prepared
CONFIGS["c2x"] = dataclasses.replace(CONFIGS["c2"], name="csa_decode_mx4idx_B32_ctx128K", index_fmt="mx4")
CONFIGS["c5x"] = dataclasses.replace(CONFIGS["c5"], name="csa_decode_mx4idx_B4_ctx1M_stress", index_fmt="mx4")
# the 64K prefill chunk with FP4 index operands
CONFIGS["c4x"] = dataclasses.replace(CONFIGS["c4"], name="csa_prefill_chunk_mx4idx_ctx64K_q4096", index_fmt="mx4")


def _gen(wl: Workload, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed_base + ORD[name])
    return g


def _randn(wl, name, shape, device, std=1.0):
    x = torch.randn(shape, generator=_gen(wl, name, device), device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def make_inputs(wl: Workload, device="cpu", entries_capacity: int | None = None) -> dict:
    """Draw every input of one step of ``wl`` on ``device``.

    Returns a dict of tensors:
      raw     [B, raw_len, d]   raw latents of positions raw_pos0 .. T-1 (window + new groups)
      logits  [B, G_new*m] f32  pooling logits of the tokens of the new groups
      entries [B, cap, d]       compressed cache; rows g0 .. N-1 are zero (the step writes them)
      q       [B, Tq, H, d]     attention queries
      and for CSA: k_idx [B, cap, dI], q_idx [B, Tq, HI, dI], w_idx [B, Tq, HI] f32.
    """
    dt = wl.torch_dtype
    cap = entries_capacity or wl.N
    assert cap >= wl.N
    out = {}
    out["raw"] = _randn(wl, "raw", (wl.B, wl.raw_len, wl.d), device).to(dt)
    out["logits"] = _randn(wl, "logits", (wl.B, wl.G_new * wl.m), device)
    ent = torch.zeros((wl.B, cap, wl.d), device=device, dtype=torch.float32)
    if wl.g0 > 0:
        ent[:, : wl.g0] = _randn(wl, "entries", (wl.B, wl.g0, wl.d), device)
    out["q"] = _randn(wl, "q", (wl.B, wl.Tq, wl.H, wl.d), device).to(dt)
    if wl.mode == "csa":
        s = 1.0 / math.sqrt(wl.dI)
        kI = torch.zeros((wl.B, cap, wl.dI), device=device, dtype=torch.float32)
        kI[:, : wl.N] = _randn(wl, "k_idx", (wl.B, wl.N, wl.dI), device, std=s)
        out["q_idx"] = _randn(wl, "q_idx", (wl.B, wl.Tq, wl.HI, wl.dI), device, std=s).to(dt)
        out["w_idx"] = torch.rand((wl.B, wl.Tq, wl.HI), generator=_gen(wl, "w_idx", device), device=device,
                                  dtype=torch.float32)
        if wl.stress_frac > 0:
            n_st = int(round(wl.stress_frac * wl.N))
            g = _gen(wl, "stress", device)
            for b in range(wl.B):
                sel = torch.randperm(wl.N, generator=g, device=device)[:n_st]
                ent[b, sel] *= 8.0
                kI[b, sel] *= 8.0
            out["stress_count"] = n_st
        out["k_idx"] = kI.to(dt)
    out["entries"] = ent.to(dt)
    return out


def scaled(wl: Workload, **changes) -> Workload:
    """A copy of ``wl`` with some fields replaced (used by tests for reduced shapes)."""
    return dataclasses.replace(wl, **changes)


# ---------------------------------------------------------------- sequences
@dataclasses.dataclass(frozen=True)
class Sequence:
    """A whole token stream for one layer, processed from position 0: prefill in
    the given chunks, then the rest of the T tokens decoded one at a time."""
    name: str
    dtype: str
    B: int
    T: int
    m: int
    d: int
    H: int
    W: int
    k: int = 0
    HI: int = 0
    dI: int = 0
    index_fmt: str = "elem"
    chunks: tuple = ()
    seed_base: int = 0
    pool: str = "token"         # pooling logits per token ("token") or per token and channel ("channel")
    index_keys: str = "given"   # one index key per group ("given") or per token, pooled ("pooled")

    @property
    def mode(self) -> str:
        return "csa" if self.k > 0 else "hca"

    @property
    def G(self) -> int:  # groups complete at the end of the stream
        return self.T // self.m

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def schedule(self) -> list:
        """Chunk lengths covering 0 .. T-1: the prefill chunks, then ones."""
        sizes = list(self.chunks)
        assert sum(sizes) <= self.T
        return sizes + [1] * (self.T - sum(sizes))


def make_sequence(sq: Sequence, device="cpu") -> dict:
    """Draw a whole stream on the CPU generator (then move it to ``device``):
      raw [B, T, d], logits [B, T] f32 ([B, T, d] with per-channel pooling),
      q [B, T, H, d]; for CSA the index keys -- one per group k_idx [B, G, dI],
      or one per token k_idx_tokens [B, T, dI] (pooled keys; with per-channel
      pooling also k_idx_logits [B, T, dI] f32) -- and q_idx [B, T, HI, dI],
      w_idx [B, T, HI] f32.  Distributions as make_inputs."""
    dt = sq.torch_dtype
    out = {}
    out["raw"] = _randn(sq, "raw", (sq.B, sq.T, sq.d), "cpu").to(dt)
    lshape = (sq.B, sq.T, sq.d) if sq.pool == "channel" else (sq.B, sq.T)
    out["logits"] = _randn(sq, "logits", lshape, "cpu")
    out["q"] = _randn(sq, "q", (sq.B, sq.T, sq.H, sq.d), "cpu").to(dt)
    if sq.mode == "csa":
        s = 1.0 / math.sqrt(sq.dI)
        if sq.index_keys == "pooled":
            out["k_idx_tokens"] = _randn(sq, "k_idx", (sq.B, sq.T, sq.dI), "cpu", std=s).to(dt)
            if sq.pool == "channel":
                out["k_idx_logits"] = _randn(sq, "k_idx_logits", (sq.B, sq.T, sq.dI), "cpu")
        else:
            out["k_idx"] = _randn(sq, "k_idx", (sq.B, sq.G, sq.dI), "cpu", std=s).to(dt)
        out["q_idx"] = _randn(sq, "q_idx", (sq.B, sq.T, sq.HI, sq.dI), "cpu", std=s).to(dt)
        out["w_idx"] = torch.rand((sq.B, sq.T, sq.HI), generator=_gen(sq, "w_idx", "cpu"), dtype=torch.float32)
    return {k: v.to(device) for k, v in out.items()}


# decode loops for the benchmark: the stream is resumed at position T (T // m
# entries and their index keys in the cache, the ring holding the last raw
# tokens) and decoded one token per sequence per step, a group emitted every
# m steps; two layers' states alternate step by step
LOOPS = {
    "l2": Sequence("csa_decode_loop_B32_ctx128K", "bf16", B=32, T=131072, m=4, d=512, H=64, W=128, k=1024, HI=64,
                   dI=128, seed_base=6000),
}
LOOPS["l2x"] = dataclasses.replace(LOOPS["l2"], name="csa_decode_loop_mx4idx_B32_ctx128K", index_fmt="mx4")
# the same loop with per-channel pooling logits and index keys pooled by the compressor from per-token keys
LOOPS["l2c"] = dataclasses.replace(LOOPS["l2"], name="csa_decode_loop_chpool_B32_ctx128K", pool="channel",
                                   index_keys="pooled")

# a whole prefill from position 0 through the streaming layer, in chunks
PREFILLS = {
    "p1": Sequence("csa_prefill_stream_B1_ctx64K_chunk4096", "bf16", B=1, T=65536, m=4, d=512, H=64, W=128,
                   k=1024, HI=64, dI=128, chunks=(4096,) * 16, seed_base=7000),
}


# ragged decode for the benchmark: B sequences at different lengths, every
# sequence one token per step through a stack of layers alternating CSA and HCA
@dataclasses.dataclass(frozen=True)
class RaggedStack:
    name: str
    B: int
    lengths: tuple            # each sequence's position when timing starts
    d: int
    H: int
    W: int
    csa: tuple = (("m", 4), ("k", 1024), ("HI", 64), ("dI", 128))
    hca: tuple = (("m", 128),)
    n_layers: int = 2
    dtype: str = "bf16"
    seed_base: int = 0

    def specs(self) -> list:
        return [dict(dict(self.csa), mode="csa") if i % 2 == 0 else dict(dict(self.hca), mode="hca")
                for i in range(self.n_layers)]


RAGGED = {
    # lengths 96K .. 158K in steps of 2K (mean ~127K), CSA then HCA
    "r2": RaggedStack("hybrid_decode_ragged_B32_ctx96K-158K", B=32, lengths=tuple(98304 + 2048 * b for b in range(32)),
                      d=512, H=64, W=128, seed_base=8000),
    # the same batch through one CSA layer
    "r1": RaggedStack("csa_decode_ragged_B32_ctx96K-158K", B=32, lengths=tuple(98304 + 2048 * b for b in range(32)),
                      d=512, H=64, W=128, n_layers=1, seed_base=8100),
    # the same batch and layer with paged caches: entries and index keys in pages of 64 rows, each
    # sequence's pages drawn from a shuffled pool
    "r1p": RaggedStack("csa_decode_ragged_paged64_B32_ctx96K-158K", B=32,
                       lengths=tuple(98304 + 2048 * b for b in range(32)), d=512, H=64, W=128, n_layers=1,
                       csa=(("m", 4), ("k", 1024), ("HI", 64), ("dI", 128), ("page_rows", 64)), seed_base=8200),
}
