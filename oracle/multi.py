"""CPU oracle: one decoder layer over a batch with SEVERAL prefill chunks plus decodes.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import,
call or run anything in this package.  The product path never does, and nothing here comes from it.

What it computes.  A token-budget batch (junupark.xyz notes on Sarathi-Serve, "Stall Free Batching")
holds decodes, the remaining tokens of a partially prefilled prompt and the first tokens of new
prompts, each chunk from a different request.  As in the one-chunk hybrid batch (SARATHI: Efficient
LLM Inference by Piggybacking Decodes with Chunked Prefills, section 3, "Decode-Maximal Batching"),
the linear ops act row by row over all rows, and attention stays per request: chunk j's rows attend
causally to chunk j's cached prefix plus its own rows (the Figure 6 mask at chunk j's offset), each
decode to its own cache plus its new entry.  The row order is chunk 0, chunk 1, ..., then decodes.

Written with the same building blocks and in the same order as oracle.layer.layer_forward, so a
batch with one chunk gives exactly layer_forward's numbers.  float64 by default.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .layer import attend_rows, chunk_mask, gelu, layer_norm, rms_norm, rope_rotate, silu

__all__ = ["layer_forward_multi", "apply_multi_rows", "multi_positions"]


def multi_positions(chunks: Sequence[Dict], decode_len: Sequence[int]) -> np.ndarray:
    """Absolute position of every row: row t of chunk j is at chunks[j]['offset'] + t; decode i is at
    decode_len[i] (the slot its new token goes to)."""
    parts = [np.arange(int(c["offset"]), int(c["offset"]) + int(c["len"])) for c in chunks]
    parts.append(np.asarray(list(decode_len), dtype=np.int64))
    return np.concatenate(parts).astype(np.int64) if parts else np.zeros(0, np.int64)


def layer_forward_multi(shape, weights: Dict[str, Optional[np.ndarray]], batch: Dict,
                        dtype=np.float64) -> Dict[str, np.ndarray]:
    """Forward pass of one decoder layer over a batch of several chunks plus decodes.

    batch: x [T, H] (chunk rows in chunk order, then decode rows), chunks: list of dicts with len,
    offset, k, v ([nh, cap, d], slots 0..offset-1 valid), decode_len [B], decode_k / decode_v lists
    of [nh, cap_i, d].  Nothing is modified.  Returns what layer_forward returns (y, new_k, new_v,
    the intermediates, pos)."""
    f = lambda a: None if a is None else np.asarray(a, dtype=dtype)
    H, nh, d = shape.hidden, shape.n_heads, shape.head_dim
    A = nh * d
    gated = shape.arch == "llama"
    x = f(batch["x"])
    chunks = list(batch["chunks"])
    lens = [int(v) for v in batch["decode_len"]]
    C = sum(int(c["len"]) for c in chunks)
    B = len(lens)
    T = C + B
    assert x.shape == (T, H)
    pos = multi_positions(chunks, lens)

    if gated:
        n1 = rms_norm(x, f(weights["norm1_w"]), shape.norm_eps)
    else:
        n1 = layer_norm(x, f(weights["norm1_w"]), f(weights["norm1_b"]), shape.norm_eps)
    qkv = n1 @ f(weights["w_qkv"]).T
    q = qkv[:, 0:A].reshape(T, nh, d)
    k = qkv[:, A:2 * A].reshape(T, nh, d)
    v = qkv[:, 2 * A:3 * A].reshape(T, nh, d)
    if gated:
        q = rope_rotate(q, pos, shape.rope_base)
        k = rope_rotate(k, pos, shape.rope_base)

    # Attention per request: each chunk over its own cached prefix plus its own rows.
    attn = np.zeros((T, nh, d), dtype=dtype)
    r0 = 0
    for c in chunks:
        n, off = int(c["len"]), int(c["offset"])
        rows = slice(r0, r0 + n)
        keys = np.concatenate([f(c["k"][:, :off, :]), k[rows].transpose(1, 0, 2)], axis=1)
        vals = np.concatenate([f(c["v"][:, :off, :]), v[rows].transpose(1, 0, 2)], axis=1)
        attn[rows] = attend_rows(q[rows], keys, vals, chunk_mask(off, n))
        r0 += n
    for i, L in enumerate(lens):
        r = C + i
        keys = np.concatenate([f(batch["decode_k"][i][:, :L, :]), k[r][:, None, :]], axis=1)
        vals = np.concatenate([f(batch["decode_v"][i][:, :L, :]), v[r][:, None, :]], axis=1)
        attn[r:r + 1] = attend_rows(q[r:r + 1], keys, vals, np.ones((1, L + 1), dtype=bool))
    attn = attn.reshape(T, A)

    h1 = x + attn @ f(weights["w_o"]).T
    if gated:
        n2 = rms_norm(h1, f(weights["norm2_w"]), shape.norm_eps)
        act = silu(n2 @ f(weights["w_gate"]).T) * (n2 @ f(weights["w_up"]).T)
    else:
        n2 = layer_norm(h1, f(weights["norm2_w"]), f(weights["norm2_b"]), shape.norm_eps)
        act = gelu(n2 @ f(weights["w_up"]).T)
    y = h1 + act @ f(weights["w_down"]).T
    return {"y": y, "new_k": k, "new_v": v, "n1": n1, "qkv": qkv, "q_rot": q.reshape(T, A),
            "attn": attn, "h1": h1, "n2": n2, "act": act, "pos": pos}


def apply_multi_rows(batch: Dict, out: Dict) -> None:
    """Write a step's new K/V rows into the batch's cache arrays in place (row t of chunk j -> slot
    offset_j + t of chunk j's cache; decode i -> its slot decode_len[i])."""
    r0 = 0
    for c in batch["chunks"]:
        n, off = int(c["len"]), int(c["offset"])
        c["k"][:, off:off + n, :] = out["new_k"][r0:r0 + n].transpose(1, 0, 2)
        c["v"][:, off:off + n, :] = out["new_v"][r0:r0 + n].transpose(1, 0, 2)
        r0 += n
    for i, L in enumerate(batch["decode_len"]):
        batch["decode_k"][i][:, L, :] = out["new_k"][r0 + i]
        batch["decode_v"][i][:, L, :] = out["new_v"][r0 + i]
