"""A stack of attention layers alternating CSA and HCA, decoding ragged batches.

DeepSeek-V4 overview page, section 2.3: CSA (m = 4, top-k selection) and
HCA (m = 128, dense) layers are used alternately.  Each layer keeps its own
cache (RaggedLayer: rings, entries, index keys, per-sequence positions); one
stack step decodes one token of every sequence through every layer.  The
layers' inputs (raw latents, pooling logits, queries, index queries and head
weights, index keys) come from projections of the residual stream that are
outside this path, so they are given per layer; the stack only orders the
layers' calls.  The whole stack step is a fixed sequence of launches and can
be captured in one HIP graph and replayed for every token.
"""
from __future__ import annotations

import torch

from .ragged import RaggedLayer


def alternating(n_layers: int, csa: dict, hca: dict) -> list:
    """Layer specs CSA, HCA, CSA, ... (n_layers of them)."""
    return [dict(csa, mode="csa") if i % 2 == 0 else dict(hca, mode="hca") for i in range(n_layers)]


class HybridStack:
    def __init__(self, specs: list, *, B: int, H: int, d: int, W: int, capacity: int, dtype=torch.bfloat16,
                 device="cuda"):
        """specs: per layer a dict with mode ("csa"/"hca"), m, and for CSA k, HI, dI (optional index_fmt;
        optional page_rows for paged caches)."""
        self.B = B
        self.layers = [RaggedLayer(mode=s["mode"], B=B, H=H, d=d, m=s["m"], W=W, capacity=capacity, dtype=dtype,
                                   k=s.get("k", 0), HI=s.get("HI", 0), dI=s.get("dI", 0),
                                   index_fmt=s.get("index_fmt", "elem"), scale=s.get("scale"),
                                   page_rows=s.get("page_rows", 0), device=device, seed=i)
                       for i, s in enumerate(specs)]

    def step(self, inputs: list) -> list:
        """inputs[l]: the keyword arguments of layer l's RaggedLayer.step.  Returns each layer's out."""
        if len(inputs) != len(self.layers):
            raise ValueError("one input set per layer")
        return [layer.step(**x) for layer, x in zip(self.layers, inputs)]
