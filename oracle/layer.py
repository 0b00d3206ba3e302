"""CPU oracle: one decoder layer's forward pass over a hybrid batch, written plainly.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import,
call or run anything in this package.  The product path (the HIP library and its binding) never does,
and this package imports nothing from it: it shares no kernels, helpers, tables or constants with it.

What it computes.  A hybrid batch is one prefill chunk of C tokens plus B single-token decodes, each
decode request holding its own KV cache (SARATHI: Efficient LLM Inference by Piggybacking Decodes with
Chunked Prefills, section 3, "Decode-Maximal Batching").  Batching them only groups work: the linear
ops of all C+B rows are one GEMM, but every row's result is that of its own request run alone, because
chunked attention with the progressively widening causal mask is mathematically the same as a full
prefill (same page, "Chunked-Prefills", Figure 6) and each decode attends only to its own cache (same
page, "Attention is NOT fused").  So this oracle computes each request's layer plainly and stacks the
rows: chunk rows first, then decodes in index order.

The layer itself (norms, RoPE, SwiGLU or GELU MLP) is not spelled out on the pages beyond the operation
list preproj / attention / postproj / FFN; the textbook LLaMA and GPT layer definitions are used, with
these readings (adjacent-pair RoPE, angles in float64, softmax
scale 1/sqrt(d), no biases, weights stored [out, in]).

Precision: float64 by default (dtype argument), inputs upcast once.  Loops are over requests and
heads; every contraction is a numpy matmul / einsum of the definition, with no blocking or fusion.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "rms_norm", "layer_norm", "rope_inv_freq", "rope_rotate", "chunk_mask", "attend_rows",
    "silu", "gelu", "layer_forward", "positions", "apply_new_rows", "stack_forward", "apply_stack_rows",
]


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gamma (LLaMA layer definition)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * gamma


def layer_norm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float) -> np.ndarray:
    """LayerNorm over the last axis with the biased variance: (x - mean) / sqrt(var + eps) * g + b."""
    mu = np.mean(x, axis=-1, keepdims=True)
    var = np.mean((x - mu) ** 2, axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * gamma + beta


def rope_inv_freq(head_dim: int, base: float) -> np.ndarray:
    """theta_j = base^(-2j/d) for j = 0..d/2-1 (rotary position embedding), in float64."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    return base ** (-2.0 * j / head_dim)


def rope_rotate(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate each adjacent pair (x[2j], x[2j+1]) of the last axis by the angle pos * theta_j.

    x is [..., n_rows, n_heads, d] with pos [n_rows]; the angle is formed in float64 before cos/sin
    (positions reach 8191 in the long-context workload)."""
    d = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[:, None] * rope_inv_freq(d, base)[None, :]   # [rows, d/2]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    xe = x[..., 0::2]
    xo = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * cos - xo * sin
    out[..., 1::2] = xe * sin + xo * cos
    return out


def chunk_mask(offset: int, chunk_len: int) -> np.ndarray:
    """Boolean [C, offset+C]: chunk query t (absolute position offset+t) may attend to key j iff
    j <= offset+t, i.e. the whole cached prefix plus the causal part of its own chunk
    (SARATHI page, "Chunked-Prefills", attention mask construction, Figure 6)."""
    t = np.arange(chunk_len)[:, None]
    j = np.arange(offset + chunk_len)[None, :]
    return j <= offset + t


def attend_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Masked softmax attention of one request, per head.

    q [R, nh, d]; k, v [nh, S, d] (the request's keys/values 0..S-1); mask bool [R, S].
    scores = q.k / sqrt(d); masked scores are -inf; softmax is max-subtracted; output = sum_j a_j v_j.
    Returns [R, nh, d]."""
    d = q.shape[-1]
    s = np.matmul(q.transpose(1, 0, 2), k.transpose(0, 2, 1)) / math.sqrt(d)   # [nh, R, S]
    s = np.where(mask[None, :, :], s, -np.inf)
    s = s - np.max(s, axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / np.sum(p, axis=-1, keepdims=True)
    return np.matmul(p, v).transpose(1, 0, 2)


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + e^-z)."""
    return z / (1.0 + np.exp(-z))


def gelu(z: np.ndarray) -> np.ndarray:
    """Exact GELU: z/2 * (1 + erf(z / sqrt(2)))."""
    from scipy.special import erf
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def positions(chunk_len: int, chunk_offset: int, decode_len: Sequence[int]) -> np.ndarray:
    """Absolute position of every row: chunk row t is at offset+t; decode i is at decode_len[i], the
    slot its new token is written to (its cache already holds decode_len[i] entries)."""
    return np.concatenate([np.arange(chunk_offset, chunk_offset + chunk_len),
                           np.asarray(list(decode_len), dtype=np.int64)]).astype(np.int64)


def layer_forward(shape, weights: Dict[str, Optional[np.ndarray]], batch: Dict,
                  dtype=np.float64) -> Dict[str, np.ndarray]:
    """Forward pass of one decoder layer over one hybrid batch.

    shape: the layer's LayerShape-like record (arch, hidden, n_heads, head_dim, ffn, norm_eps,
    rope_base).  weights: w_qkv [3A,H], w_o [H,A], w_gate [F,H] (gated only), w_up [F,H],
    w_down [H,F], norm1_w/norm2_w [H], norm1_b/norm2_b [H] (LayerNorm only).  batch: x [C+B,H] with
    chunk rows first, chunk_len C, chunk_offset, chunk_k/chunk_v [nh,cap,d] (slots 0..offset-1
    valid), decode_len [B], decode_k/decode_v lists of [nh,cap_i,d] (slots 0..len_i-1 valid).

    Nothing passed in is modified.  Returns y [C+B,H], the K/V rows the step writes (new_k/new_v
    [C+B,nh,d]: chunk row t goes to chunk slot offset+t, decode i to its slot decode_len[i]) and the
    intermediates n1, qkv, q_rot, attn [C+B,A], h1, n2, act [C+B,F]."""
    f = lambda a: None if a is None else np.asarray(a, dtype=dtype)
    H, nh, d, F = shape.hidden, shape.n_heads, shape.head_dim, shape.ffn
    A = nh * d
    gated = shape.arch == "llama"
    x = f(batch["x"])
    C = int(batch["chunk_len"])
    off = int(batch["chunk_offset"])
    lens = [int(v) for v in batch["decode_len"]]
    B = len(lens)
    T = C + B
    assert x.shape == (T, H)
    pos = positions(C, off, lens)

    # Norm 1 and the fused QKV projection over all C+B rows (preproj as one GEMM).
    if gated:
        n1 = rms_norm(x, f(weights["norm1_w"]), shape.norm_eps)
    else:
        n1 = layer_norm(x, f(weights["norm1_w"]), f(weights["norm1_b"]), shape.norm_eps)
    qkv = n1 @ f(weights["w_qkv"]).T                                   # [T, 3A]
    q = qkv[:, 0:A].reshape(T, nh, d)
    k = qkv[:, A:2 * A].reshape(T, nh, d)
    v = qkv[:, 2 * A:3 * A].reshape(T, nh, d)
    if gated:
        q = rope_rotate(q, pos, shape.rope_base)
        k = rope_rotate(k, pos, shape.rope_base)

    # Attention, split per request.  Each request's keys are its cached entries followed by the rows
    # this step appends (the append happens before the attention that reads it).
    attn = np.zeros((T, nh, d), dtype=dtype)
    if C:
        keys = np.concatenate([f(batch["chunk_k"][:, :off, :]), k[:C].transpose(1, 0, 2)], axis=1)
        vals = np.concatenate([f(batch["chunk_v"][:, :off, :]), v[:C].transpose(1, 0, 2)], axis=1)
        attn[:C] = attend_rows(q[:C], keys, vals, chunk_mask(off, C))
    for i, L in enumerate(lens):
        r = C + i
        # A decode's query attends to its L cached entries plus its own new entry: L+1 keys
        # (Sarathi-Serve Guide, "Attention Complexity Across Mixed Batches").
        keys = np.concatenate([f(batch["decode_k"][i][:, :L, :]), k[r][:, None, :]], axis=1)
        vals = np.concatenate([f(batch["decode_v"][i][:, :L, :]), v[r][:, None, :]], axis=1)
        attn[r:r + 1] = attend_rows(q[r:r + 1], keys, vals, np.ones((1, L + 1), dtype=bool))
    attn = attn.reshape(T, A)

    # Output projection with the residual, norm 2, FFN with the residual.
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


def apply_new_rows(batch: Dict, out: Dict) -> None:
    """Write a step's new K/V rows into the batch's cache arrays in place, the way the layer's
    append does (chunk row t -> chunk slot offset+t; decode i -> its slot decode_len[i]).  Used by
    callers that drive several steps (the chunk-by-chunk prompt); lengths are advanced by the caller."""
    C = int(batch["chunk_len"])
    off = int(batch["chunk_offset"])
    if C:
        batch["chunk_k"][:, off:off + C, :] = out["new_k"][:C].transpose(1, 0, 2)
        batch["chunk_v"][:, off:off + C, :] = out["new_v"][:C].transpose(1, 0, 2)
    for i, L in enumerate(batch["decode_len"]):
        batch["decode_k"][i][:, L, :] = out["new_k"][C + i]
        batch["decode_v"][i][:, L, :] = out["new_v"][C + i]


def stack_forward(shape, layer_weights: Sequence[Dict[str, Optional[np.ndarray]]], batch: Dict,
                  dtype=np.float64) -> Dict:
    """A stack of layers over one hybrid batch: layer l's input rows are layer l-1's output rows, and
    every layer attends over its own caches (SARATHI page, section 3: each chunk of a prompt passes
    through all layers, appending to each layer's KV cache).

    batch: x [C+B,H], chunk_len, chunk_offset, decode_len [B], and per layer l: chunk_k[l] /
    chunk_v[l] [nh,cap,d], decode_k[l] / decode_v[l] lists of [nh,cap_i,d].  Nothing is modified.
    Returns y (the last layer's output) and `layers`, each layer's layer_forward result."""
    x = batch["x"]
    outs = []
    for l, w in enumerate(layer_weights):
        bl = {"x": x, "chunk_len": batch["chunk_len"], "chunk_offset": batch["chunk_offset"],
              "decode_len": batch["decode_len"],
              "chunk_k": batch["chunk_k"][l] if batch["chunk_len"] else None,
              "chunk_v": batch["chunk_v"][l] if batch["chunk_len"] else None,
              "decode_k": batch["decode_k"][l], "decode_v": batch["decode_v"][l]}
        out = layer_forward(shape, w, bl, dtype)
        outs.append(out)
        x = out["y"]
    return {"y": x, "layers": outs}


def apply_stack_rows(batch: Dict, res: Dict) -> None:
    """apply_new_rows for every layer of a stack step (caches of layer l get layer l's new rows)."""
    for l, out in enumerate(res["layers"]):
        bl = {"chunk_len": batch["chunk_len"], "chunk_offset": batch["chunk_offset"],
              "decode_len": batch["decode_len"],
              "chunk_k": batch["chunk_k"][l] if batch["chunk_len"] else None,
              "chunk_v": batch["chunk_v"][l] if batch["chunk_len"] else None,
              "decode_k": batch["decode_k"][l], "decode_v": batch["decode_v"][l]}
        apply_new_rows(bl, out)
