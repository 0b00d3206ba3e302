"""Pins of the oracle's layer stack (CPU, float64).

A prompt prefilled chunk by chunk through a stack of layers, with decodes riding along in every step,
must give the same chunk outputs and leave the same KV caches in every layer as the prompt prefilled
in one chunk: chunked prefill is mathematically the same as a full prefill (SARATHI: Efficient LLM
Inference by Piggybacking Decodes with Chunked Prefills, section 3, "Chunked-Prefills"), layer by
layer, because a layer's output for token t depends only on its inputs for tokens <= t.  And every
decode row of a hybrid stack step equals the same decodes run alone (section 3, "Decode-Maximal
Batching": decodes share only the linear ops with the chunk)."""
import copy
import math

import numpy as np

import oracle
from chunked_prefill_hybrid_amd import workloads as wl


def rel(a, b):
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


def test_stack_chunked_prompt_equals_monolithic_and_decodes_are_independent():
    shape = wl.SHAPES["tiny"]
    n_layers, P, C = 3, 96, 32
    nh, d, H = shape.n_heads, shape.head_dim, shape.hidden
    rng = np.random.default_rng(11)
    W = [wl.make_weights(shape, rng) for _ in range(n_layers)]
    xp = rng.standard_normal((P, H))

    def zeros():
        return [np.zeros((nh, P, d)) for _ in range(n_layers)]

    mono = {"x": xp, "chunk_len": P, "chunk_offset": 0, "decode_len": [],
            "chunk_k": zeros(), "chunk_v": zeros(),
            "decode_k": [[] for _ in range(n_layers)], "decode_v": [[] for _ in range(n_layers)]}
    rm = oracle.stack_forward(shape, W, mono)
    oracle.apply_stack_rows(mono, rm)

    lens0 = [5, 20]
    steps = P // C
    st = {"chunk_k": zeros(), "chunk_v": zeros(),
          "decode_k": [[rng.standard_normal((nh, L + steps, d)) for L in lens0] for _ in range(n_layers)],
          "decode_v": [[rng.standard_normal((nh, L + steps, d)) for L in lens0] for _ in range(n_layers)]}
    ys = []
    for k in range(steps):
        xd = rng.standard_normal((len(lens0), H))
        lens = [L + k for L in lens0]
        b = dict(st, x=np.concatenate([xp[k * C:(k + 1) * C], xd]), chunk_len=C, chunk_offset=k * C,
                 decode_len=lens)
        alone = {"x": xd, "chunk_len": 0, "chunk_offset": 0, "decode_len": lens,
                 "chunk_k": None, "chunk_v": None,
                 "decode_k": copy.deepcopy(st["decode_k"]), "decode_v": copy.deepcopy(st["decode_v"])}
        r = oracle.stack_forward(shape, W, b)
        ra = oracle.stack_forward(shape, W, alone)
        assert rel(r["y"][C:], ra["y"]) < 1e-13, f"step {k}: decode rows depend on the chunk"
        oracle.apply_stack_rows(b, r)
        ys.append(r["y"][:C])
    assert rel(np.concatenate(ys), rm["y"]) < 1e-12
    for l in range(n_layers):
        assert rel(st["chunk_k"][l], mono["chunk_k"][l]) < 1e-12
        assert rel(st["chunk_v"][l], mono["chunk_v"][l]) < 1e-12


def test_stack_of_one_layer_is_the_layer():
    shape = wl.SHAPES["tiny"]
    rng = np.random.default_rng(3)
    w = wl.make_weights(shape, rng)
    spec = wl.BatchSpec(16, 8, 24, 2, decode_lens=(3, 9))
    b = wl.make_batch(shape, spec, rng)
    r1 = oracle.layer_forward(shape, w, b)
    sb = dict(b, chunk_k=[b["chunk_k"]], chunk_v=[b["chunk_v"]], decode_k=[b["decode_k"]],
              decode_v=[b["decode_v"]])
    rs = oracle.stack_forward(shape, [w], sb)
    assert np.array_equal(rs["y"], r1["y"])


# ------------------------------------------------------------------------------------------------
# Chaining closed form: every layer of the stack reduced to a map of its input rows that is written
# out here with Python loops (no call into the oracle), then composed layer after layer.
# ------------------------------------------------------------------------------------------------

SMALL = wl.LayerShape("small", "llama", 16, 2, 8, 24, "f32", 1e-6, 10000.0, None)


def _uniform_attention_layer(shape, gamma, s, c, ffn_rng):
    """W_q = W_k = 0, W_v = s I, W_o = c I, W_down = 0 (hidden = heads x head_dim), random gate/up.
    Every score is 0, so each row's attention is the plain mean of the V rows it may attend to."""
    H = shape.hidden
    w = wl.make_weights(shape, ffn_rng)
    w["norm1_w"] = np.asarray(gamma, dtype=np.float64)
    w["w_qkv"] = np.zeros((3 * H, H))
    w["w_qkv"][2 * H:] = s * np.eye(H)
    w["w_o"] = c * np.eye(H)
    w["w_down"] = np.zeros_like(w["w_down"])
    return w


def _closed_form_layer(x, gamma, s, c, eps, C, off, chunk_v, lens, dec_v, nh, d):
    """The layer above by hand: n1 = x / sqrt(mean(x^2) + eps) * gamma, new V row = s n1; chunk row t
    averages its request's cached V slots 0..off-1 and the chunk's new V rows 0..t; decode i averages
    its own cached slots 0..L_i-1 and its new V row; y = x + c * that mean.  Returns (y, new V rows)."""
    T, H = len(x), len(x[0])
    newv = []
    for r in range(T):
        ms = sum(float(v) ** 2 for v in x[r]) / H
        newv.append([s * float(x[r][col]) / math.sqrt(ms + eps) * float(gamma[col]) for col in range(H)])
    y = []
    for r in range(T):
        row = []
        for h in range(nh):
            for e in range(d):
                col = h * d + e
                if r < C:
                    vals = [chunk_v[h, j, e] for j in range(off)] + [newv[t][col] for t in range(r + 1)]
                else:
                    i = r - C
                    vals = [dec_v[i][h, j, e] for j in range(lens[i])] + [newv[r][col]]
                row.append(float(x[r][col]) + c * sum(float(v) for v in vals) / len(vals))
        y.append(row)
    return y, newv


def test_stack_chains_layers_in_order_closed_form():
    """Three layers with distinct gains, V and O scales and caches: the stack's output equals layer 3
    applied to layer 2's output applied to layer 1's output of x, each layer over its own caches, and
    each layer's new V rows are those of its own input.  Feeding every layer the stack input, running
    the layers in another order, or reading another layer's caches changes the result (the maps do
    not commute: the gains differ per column)."""
    shape = SMALL
    nh, d, H = shape.n_heads, shape.head_dim, shape.hidden
    rng = np.random.default_rng(29)
    params = [(rng.uniform(0.5, 1.5, H), 1.0, 1.0), (rng.uniform(0.5, 1.5, H), -0.7, 0.6),
              (rng.uniform(0.5, 1.5, H), 1.3, 1.7)]
    W = [_uniform_attention_layer(shape, g, s, c, rng) for g, s, c in params]
    C, off, lens = 3, 4, [2, 0, 5]
    n = len(params)
    chunk_k = [rng.standard_normal((nh, off + C, d)) for _ in range(n)]
    chunk_v = [rng.standard_normal((nh, off + C, d)) for _ in range(n)]
    dec_k = [[rng.standard_normal((nh, L + 1, d)) for L in lens] for _ in range(n)]
    dec_v = [[rng.standard_normal((nh, L + 1, d)) for L in lens] for _ in range(n)]
    x = rng.standard_normal((C + len(lens), H))
    b = {"x": x, "chunk_len": C, "chunk_offset": off, "decode_len": lens, "chunk_k": chunk_k,
         "chunk_v": chunk_v, "decode_k": dec_k, "decode_v": dec_v}
    res = oracle.stack_forward(shape, W, b)

    cur = [list(r) for r in x]
    for l, (g, s, c) in enumerate(params):
        y_ref, v_ref = _closed_form_layer(cur, g, s, c, shape.norm_eps, C, off, chunk_v[l], lens,
                                          dec_v[l], nh, d)
        out = res["layers"][l]
        assert np.max(np.abs(out["y"] - np.array(y_ref))) <= 1e-12, f"layer {l} output"
        assert np.max(np.abs(out["new_v"].reshape(len(cur), H) - np.array(v_ref))) <= 1e-12, f"layer {l} V rows"
        assert np.max(np.abs(out["new_k"])) == 0.0
        cur = y_ref
    assert np.max(np.abs(res["y"] - np.array(cur))) <= 1e-12
