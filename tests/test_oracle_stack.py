"""Pins of the oracle's layer stack (CPU, float64).

A prompt prefilled chunk by chunk through a stack of layers, with decodes riding along in every step,
must give the same chunk outputs and leave the same KV caches in every layer as the prompt prefilled
in one chunk: chunked prefill is mathematically the same as a full prefill (SARATHI: Efficient LLM
Inference by Piggybacking Decodes with Chunked Prefills, section 3, "Chunked-Prefills"), layer by
layer, because a layer's output for token t depends only on its inputs for tokens <= t.  And every
decode row of a hybrid stack step equals the same decodes run alone (section 3, "Decode-Maximal
Batching": decodes share only the linear ops with the chunk)."""
import copy

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
