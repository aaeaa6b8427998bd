"""The oracle's view of one attention step (test infrastructure).

Runs the CPU oracle on host copies of a workload's generated inputs, taken
before any GPU work, so no oracle input comes from the HIP path.
"""
from __future__ import annotations

import numpy as np

import oracle as orc


def host_inputs(x: dict) -> dict:
    """Exact float32 host copies of every tensor input (bf16 widens exactly)."""
    out = {}
    for k, v in x.items():
        if hasattr(v, "detach"):
            v = v.detach().cpu()
            out[k] = v.numpy() if v.dtype.is_floating_point is False else v.float().numpy()
        else:
            out[k] = v
    return out


def oracle_step(wl, xh: dict, rows=None) -> dict:
    """Oracle results for workload ``wl`` on host inputs ``xh``.

    rows: query rows (0..Tq-1) to evaluate for the indexer / top-k /
    attention, as a list of row numbers or of (start, stop) ranges; None
    evaluates every row.  Compression is always complete.
    """
    N, m, g0 = wl.N, wl.m, wl.g0
    r0 = g0 * m - wl.raw_pos0
    e = orc.compress(xh["raw"][:, r0:r0 + wl.G_new * m], xh["logits"], m) if wl.G_new > 0 else None
    ent = np.array(xh["entries"][:, :N], dtype=np.float32, copy=True)
    if e is not None:
        ent[:, g0:N] = orc.round_bf16(e) if wl.dtype == "bf16" else e.astype(np.float32)
    res = {"e": e, "entries": ent}
    if rows is None:
        groups = [(0, wl.Tq)]
    else:
        groups = [tuple(r) if isinstance(r, (tuple, list)) else (r, r + 1) for r in rows]
    sel = [ti for a, b in groups for ti in range(a, b)]
    outs, lses, idxs, scs = [], [], [], []
    for a, b in groups:
        qp = wl.q_pos0 + a
        q = xh["q"][:, a:b]
        if wl.mode == "csa":
            qi, ki = xh["q_idx"][:, a:b], xh["k_idx"][:, :N]
            if getattr(wl, "index_fmt", "elem") == "mx4":  # the FP4 operands' exact values
                qi = orc.mx4_dequantize(*orc.mx4_quantize(qi))
                ki = orc.mx4_dequantize(*orc.mx4_quantize(ki))
            s = orc.index_scores(qi, xh["w_idx"][:, a:b], ki, m, qp)
            idx = orc.topk(s, wl.k, m, qp)
            o, l = orc.sparse_mqa(q, ent, idx, xh["raw"], wl.raw_pos0, wl.W, qp, wl.scale)
            scs.append(s)
            idxs.append(idx)
        else:
            o, l = orc.dense_mqa(q, ent, xh["raw"], wl.raw_pos0, m, wl.W, qp, wl.scale)
        outs.append(o)
        lses.append(l)
    res["rows"] = sel
    res["out"] = np.concatenate(outs, axis=1)
    res["lse"] = np.concatenate(lses, axis=1)
    if wl.mode == "csa":
        res["scores"] = np.concatenate(scs, axis=1)
        res["idx"] = np.concatenate(idxs, axis=1)
    return res


def oracle_sequence(sq, xh: dict) -> dict:
    """Oracle results for a whole stream processed from position 0 (host inputs of make_sequence)."""
    G, m = sq.G, sq.m
    pool = orc.compress_channels if sq.pool == "channel" else orc.compress
    store = (lambda v: orc.round_bf16(v)) if sq.dtype == "bf16" else (lambda v: v.astype(np.float32))
    e = pool(xh["raw"][:, :G * m], xh["logits"][:, :G * m], m) if G > 0 else None
    ent = np.zeros((sq.B, max(G, 1), sq.d), dtype=np.float32)
    if G > 0:
        ent[:, :G] = store(e)
    res = {"e": e, "entries": ent[:, :G]}
    if sq.mode == "csa":
        if sq.index_keys == "pooled":
            # the entries' index keys pooled by the same compressor, stored in the cache's type
            lg = xh["k_idx_logits"] if sq.pool == "channel" else xh["logits"]
            kp = pool(xh["k_idx_tokens"][:, :G * m], lg[:, :G * m], m)
            res["k_pooled"] = kp
            ki = store(kp)
        else:
            ki = xh["k_idx"]
        qi = xh["q_idx"]
        if sq.index_fmt == "mx4":
            qi = orc.mx4_dequantize(*orc.mx4_quantize(qi))
            ki = orc.mx4_dequantize(*orc.mx4_quantize(ki))
        s = orc.index_scores(qi, xh["w_idx"], ki, m, 0)
        idx = orc.topk(s, sq.k, m, 0)
        o, l = orc.sparse_mqa(xh["q"], ent[:, :G], idx, xh["raw"], 0, sq.W, 0, sq.scale)
        res.update(scores=s, idx=idx)
    else:
        o, l = orc.dense_mqa(xh["q"], ent[:, :G], xh["raw"], 0, m, sq.W, 0, sq.scale)
    res.update(out=o, lse=l)
    return res


def oracle_attention_on(q, entries, idx, raw, raw_pos0: int, W: int, q_pos0: int, scale: float):
    """The oracle's sparse attention evaluated on a given selection (e.g. the GPU's own top-k set, once it
    has passed the near-tie rule): the chain's output is compared with this on every row, so a legal swap
    is not counted as an attention error and no row goes unchecked."""
    return orc.sparse_mqa(q, entries, np.ascontiguousarray(idx, dtype=np.int32), raw, raw_pos0, W, q_pos0, scale)
