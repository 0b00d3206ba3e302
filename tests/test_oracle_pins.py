"""Pins of the CPU oracle to facts fixed by the pages and by mathematics (no GPU).

Each test checks the oracle against something other than itself: the chunk masks the SARATHI page
spells out for Figure 6, the invariant that chunked prefill equals the monolithic prefill, the unified
block-diagonal hybrid mask of the Sarathi-Serve guide evaluated by brute force, closed forms, and
textbook special cases computed with Python's math module in explicit loops.
"""
import math

import numpy as np
import pytest

import oracle
from chunked_prefill_hybrid_amd import workloads as wl

SMALL = wl.LayerShape("small", "llama", 16, 2, 8, 24, "f32", 1e-6, 10000.0, None)
SMALL_GPT = wl.LayerShape("small-gpt", "gpt", 16, 2, 8, 24, "f32", 1e-5, 10000.0, None)


def _rand_layer(shape, seed=1, gamma_random=True):
    rng = np.random.default_rng(seed)
    w = wl.make_weights(shape, rng)
    if gamma_random:
        w["norm1_w"] = rng.uniform(0.5, 1.5, shape.hidden).astype(np.float32)
        w["norm2_w"] = rng.uniform(0.5, 1.5, shape.hidden).astype(np.float32)
        if shape.arch == "gpt":
            w["norm1_b"] = rng.normal(0, 0.1, shape.hidden).astype(np.float32)
            w["norm2_b"] = rng.normal(0, 0.1, shape.hidden).astype(np.float32)
    return w, rng


def _batch(shape, rng, C, off, lens, cap=None):
    spec = wl.BatchSpec(C, off, cap if cap is not None else off + C, len(lens), decode_lens=tuple(lens))
    return wl.make_batch(shape, spec, rng)


# ------------------------------------------------------------------------------------------------
# P2: the Figure 6 masks, as spelled out on the SARATHI page
# ------------------------------------------------------------------------------------------------

def _read_masks(path):
    masks, cur = [], None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("chunk"):
            _, off, n = line.split()
            cur = (int(off), int(n), [])
            masks.append(cur)
        else:
            cur[2].append([c == "1" for c in line])
    return [(o, n, np.array(rows, dtype=bool)) for o, n, rows in masks]


def test_fig6_chunk_masks(golden_dir):
    masks = _read_masks(f"{golden_dir}/fig6_chunk_masks.txt")
    assert len(masks) == 3
    for off, n, expect in masks:
        got = oracle.chunk_mask(off, n)
        assert got.shape == expect.shape
        assert np.array_equal(got, expect), (off, n)


# ------------------------------------------------------------------------------------------------
# P1: chunked prefill reproduces the monolithic prefill (the page's equivalence statement)
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [wl.SHAPES["tiny"], SMALL_GPT], ids=["llama", "gpt"])
def test_chunked_equals_monolithic(shape):
    rng = np.random.default_rng(3)
    w = wl.make_weights(shape, rng)
    P = 128 if shape.hidden == 256 else 24
    Cc = P // 4
    x = rng.standard_normal((P, shape.hidden)).astype(np.float32)
    nh, d = shape.n_heads, shape.head_dim

    def empty():
        return np.zeros((nh, P, d)), np.zeros((nh, P, d))

    k0, v0 = empty()
    mono = oracle.layer_forward(shape, w, {"x": x, "chunk_len": P, "chunk_offset": 0, "chunk_k": k0,
                                           "chunk_v": v0, "decode_len": [], "decode_k": [], "decode_v": []})
    kc, vc = empty()
    ys = []
    for c in range(4):
        b = {"x": x[c * Cc:(c + 1) * Cc], "chunk_len": Cc, "chunk_offset": c * Cc, "chunk_k": kc,
             "chunk_v": vc, "decode_len": [], "decode_k": [], "decode_v": []}
        out = oracle.layer_forward(shape, w, b)
        oracle.apply_new_rows(b, out)
        ys.append(out["y"])
    y = np.concatenate(ys)
    assert np.max(np.abs(y - mono["y"])) <= 1e-12 * np.max(np.abs(mono["y"]))
    assert np.max(np.abs(kc - mono["new_k"].transpose(1, 0, 2))) <= 1e-12
    assert np.max(np.abs(vc - mono["new_v"].transpose(1, 0, 2))) <= 1e-12


def test_chunked_equals_monolithic_fp32_mode():
    """The same invariant with the oracle evaluated in float32: agreement to 1e-5 relative."""
    shape = wl.SHAPES["tiny"]
    rng = np.random.default_rng(4)
    w = wl.make_weights(shape, rng)
    x = rng.standard_normal((128, 256)).astype(np.float32)
    z = lambda: np.zeros((4, 128, 64), np.float32)
    mono = oracle.layer_forward(shape, w, {"x": x, "chunk_len": 128, "chunk_offset": 0, "chunk_k": z(),
                                           "chunk_v": z(), "decode_len": [], "decode_k": [],
                                           "decode_v": []}, dtype=np.float32)
    kc, vc = z(), z()
    ys = []
    for c in range(4):
        b = {"x": x[32 * c:32 * c + 32], "chunk_len": 32, "chunk_offset": 32 * c, "chunk_k": kc,
             "chunk_v": vc, "decode_len": [], "decode_k": [], "decode_v": []}
        out = oracle.layer_forward(shape, w, b, dtype=np.float32)
        oracle.apply_new_rows(b, out)
        ys.append(out["y"])
    y = np.concatenate(ys)
    assert np.max(np.abs(y - mono["y"])) <= 1e-5 * np.max(np.abs(mono["y"]))


# ------------------------------------------------------------------------------------------------
# P3: brute force with the unified block-diagonal hybrid mask (Sarathi-Serve guide, Deep Dive)
# ------------------------------------------------------------------------------------------------

def test_unified_mask_bruteforce():
    """Dense attention over every key of the batch ([chunk prefix | chunk | each decode's history and
    own token]) with mask 0 where the key is the query's own request at a position not after it and
    -inf otherwise, evaluated with Python loops and math.exp, equals the oracle's per-request
    attention."""
    shape = SMALL
    w, rng = _rand_layer(shape, seed=5)
    C, off, lens = 3, 5, [0, 1, 6]
    b = _batch(shape, rng, C, off, lens)
    out = oracle.layer_forward(shape, w, b)
    nh, d = shape.n_heads, shape.head_dim
    q = out["q_rot"].reshape(C + len(lens), nh, d)
    # every key of the batch as (request, position, k[nh,d], v[nh,d])
    keys = []
    for j in range(off):
        keys.append((0, j, b["chunk_k"][:, j, :], b["chunk_v"][:, j, :]))
    for t in range(C):
        keys.append((0, off + t, out["new_k"][t], out["new_v"][t]))
    for i, L in enumerate(lens):
        for j in range(L):
            keys.append((1 + i, j, b["decode_k"][i][:, j, :], b["decode_v"][i][:, j, :]))
        keys.append((1 + i, L, out["new_k"][C + i], out["new_v"][C + i]))
    queries = [(0, off + t) for t in range(C)] + [(1 + i, L) for i, L in enumerate(lens)]
    brute = np.zeros((len(queries), nh, d))
    for r, (req, p) in enumerate(queries):
        for h in range(nh):
            scores = []
            for (kreq, kp, kk, _) in keys:
                m = 0.0 if (kreq == req and kp <= p) else -math.inf
                s = sum(float(q[r, h, e]) * float(kk[h, e]) for e in range(d))
                scores.append((s + m) / math.sqrt(d))
            mx = max(scores)
            ex = [math.exp(s - mx) if s != -math.inf else 0.0 for s in scores]
            tot = sum(ex)
            for e in range(d):
                brute[r, h, e] = sum(ex[j] / tot * float(keys[j][3][h, e]) for j in range(len(keys)))
    assert np.max(np.abs(brute.reshape(len(queries), -1) - out["attn"])) <= 1e-12


# ------------------------------------------------------------------------------------------------
# P4 / P5 / P11: attention closed forms
# ------------------------------------------------------------------------------------------------

def test_attention_mask_length_closed_form():
    """With W_q = 0 the softmax is uniform over the attended keys.  Cache slot j holds V = j and the
    step's new V rows are 0 (W_v = 0), so row p's output is sum_{j<first new slot} j / (#keys).  The
    chunk row t sees keys 0..off+t (prefix sum off(off-1)/2 over off+t+1 keys); decode i sees its L_i
    cached keys plus its own: L_i(L_i-1)/2 over L_i+1 keys."""
    shape = SMALL
    w, rng = _rand_layer(shape, seed=6)
    A, H = shape.attn_width, shape.hidden
    w["w_qkv"] = w["w_qkv"].copy()
    w["w_qkv"][0:A] = 0.0          # q = 0
    w["w_qkv"][2 * A:3 * A] = 0.0  # new v = 0
    C, off, lens = 4, 7, [0, 3, 9]
    b = _batch(shape, rng, C, off, lens)
    for j in range(b["chunk_v"].shape[1]):
        b["chunk_v"][:, j, :] = j
    for i, L in enumerate(lens):
        for j in range(b["decode_v"][i].shape[1]):
            b["decode_v"][i][:, j, :] = j
    out = oracle.layer_forward(shape, w, b)
    expect = [off * (off - 1) / 2 / (off + t + 1) for t in range(C)] + \
             [L * (L - 1) / 2 / (L + 1) for L in lens]
    for r, e in enumerate(expect):
        assert np.allclose(out["attn"][r], e, rtol=0, atol=1e-12), (r, out["attn"][r][:3], e)


def test_attention_one_hot():
    rng = np.random.default_rng(7)
    S, d = 9, 8
    k = rng.standard_normal((1, S, d))
    v = rng.standard_normal((1, S, d))
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 40.0
    k[0, :, 0] = 0.0
    k[0, 5, 0] = 10.0     # score of key 5 exceeds the others by 400/sqrt(8) > 140
    o = oracle.attend_rows(q, k, v, np.ones((1, S), bool))
    assert np.max(np.abs(o[0, 0] - v[0, 5])) <= 1e-6


def test_softmax_rows_sum_to_one_and_single_key():
    rng = np.random.default_rng(8)
    S = 6
    q = rng.standard_normal((3, 2, S))
    k = rng.standard_normal((2, S, S))
    v = np.broadcast_to(np.eye(S), (2, S, S)).copy()     # output = attention weights
    mask = oracle.chunk_mask(3, 3)
    o = oracle.attend_rows(q, k, v, mask)
    assert np.allclose(o.sum(-1), 1.0, atol=1e-14)
    assert np.all(o[~np.broadcast_to(mask[:, None, :], o.shape)] == 0)
    vv = rng.standard_normal((2, 1, S))
    one = oracle.attend_rows(q[:1], k[:, :1], vv, np.ones((1, 1), bool))
    assert np.allclose(one[0], vv[:, 0], atol=1e-15)


# ------------------------------------------------------------------------------------------------
# P6: row independence
# ------------------------------------------------------------------------------------------------

def test_rows_independent_of_batch_company():
    shape = SMALL
    w, rng = _rand_layer(shape, seed=9)
    C, off, lens = 5, 3, [2, 7, 4]
    b = _batch(shape, rng, C, off, lens)
    full = oracle.layer_forward(shape, w, b)
    for i, L in enumerate(lens):
        alone = {"x": b["x"][C + i:C + i + 1], "chunk_len": 0, "chunk_offset": 0,
                 "chunk_k": b["chunk_k"], "chunk_v": b["chunk_v"], "decode_len": [L],
                 "decode_k": [b["decode_k"][i]], "decode_v": [b["decode_v"][i]]}
        o = oracle.layer_forward(shape, w, alone)
        # equal up to BLAS rounding order (a 1-row product may take a different kernel)
        assert np.max(np.abs(o["y"][0] - full["y"][C + i])) <= 1e-13
    chunk_only = dict(b, x=b["x"][:C], decode_len=[], decode_k=[], decode_v=[])
    o = oracle.layer_forward(shape, w, chunk_only)
    assert np.max(np.abs(o["y"] - full["y"][:C])) <= 1e-13


# ------------------------------------------------------------------------------------------------
# P7: rotary embedding
# ------------------------------------------------------------------------------------------------

def test_rope_identity_norm_relative_and_textbook():
    rng = np.random.default_rng(10)
    d, base = 16, 10000.0
    x = rng.standard_normal((1, 3, d))
    assert np.array_equal(oracle.rope_rotate(x, np.array([0]), base), x)
    pos = np.array([8191])
    y = oracle.rope_rotate(x, pos, base)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)
    # relative property: <R_m q, R_n k> depends only on n - m
    q, k = rng.standard_normal((1, 1, d)), rng.standard_normal((1, 1, d))
    for m, n, s in [(3, 10, 5), (100, 37, 1000), (0, 8000, 191)]:
        a = np.sum(oracle.rope_rotate(q, np.array([m]), base) * oracle.rope_rotate(k, np.array([n]), base))
        b2 = np.sum(oracle.rope_rotate(q, np.array([m + s]), base) * oracle.rope_rotate(k, np.array([n + s]), base))
        assert abs(a - b2) <= 1e-10 * (1 + abs(a))
    # complex-number form, per element with Python math: (x0 + i x1) * exp(i * p * base^(-2j/d))
    for p in (1, 17, 4095, 8191):
        yy = oracle.rope_rotate(x, np.array([p]), base)
        for h in range(3):
            for j in range(d // 2):
                th = p * math.pow(base, -2.0 * j / d)
                z = complex(x[0, h, 2 * j], x[0, h, 2 * j + 1]) * complex(math.cos(th), math.sin(th))
                assert abs(yy[0, h, 2 * j] - z.real) <= 1e-12 and abs(yy[0, h, 2 * j + 1] - z.imag) <= 1e-12
    # d = 2: the textbook 2-D rotation by angle p (theta_0 = 1)
    v2 = np.array([[[0.3, -1.7]]])
    for p in (1, 2, 5):
        r = np.array([[math.cos(p), -math.sin(p)], [math.sin(p), math.cos(p)]])
        assert np.allclose(oracle.rope_rotate(v2, np.array([p]), base)[0, 0], r @ v2[0, 0], atol=1e-15)


# ------------------------------------------------------------------------------------------------
# P8 / P9: norms and activations
# ------------------------------------------------------------------------------------------------

def test_norm_closed_forms():
    eps = 1e-6
    g = np.linspace(0.5, 1.5, 8)
    for c in (-3.0, -1e-3, 0.0, 2.5):
        x = np.full((1, 8), c)
        expect = (math.copysign(1, c) * abs(c) / math.sqrt(c * c + eps)) * g if c != 0 else 0 * g
        assert np.allclose(oracle.rms_norm(x, g, eps)[0], expect, rtol=1e-14, atol=0)
        b = np.linspace(-1, 1, 8)
        assert np.allclose(oracle.layer_norm(x, g, b, 1e-5)[0], b, atol=1e-15)
    rng = np.random.default_rng(11)
    x = rng.standard_normal((4, 32)) * 3
    n = oracle.rms_norm(x, np.ones(32), eps)
    ms = np.array([sum(float(v) ** 2 for v in row) / 32 for row in x])
    assert np.allclose(np.sqrt(np.mean(n * n, -1)), np.sqrt(ms / (ms + eps)), rtol=1e-14)
    ln = oracle.layer_norm(x, np.ones(32), np.zeros(32), 0.0)
    assert np.allclose(ln.mean(-1), 0, atol=1e-14) and np.allclose(ln.std(-1), 1, rtol=1e-12)


def test_activations_vs_python_math():
    z = np.linspace(-12, 12, 97)
    s = oracle.silu(z)
    g = oracle.gelu(z)
    for i, v in enumerate(z):
        assert abs(s[i] - v / (1 + math.exp(-v))) <= 1e-15 * max(1, abs(v))
        assert abs(g[i] - 0.5 * v * (1 + math.erf(v / math.sqrt(2)))) <= 1e-15 * max(1, abs(v))
    assert oracle.silu(np.array([0.0]))[0] == 0 and oracle.gelu(np.array([0.0]))[0] == 0


# ------------------------------------------------------------------------------------------------
# P10: linear ops and the layer's data flow, by explicit loops on a tiny layer
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [SMALL, SMALL_GPT], ids=["llama", "gpt"])
def test_linear_ops_by_loops(shape):
    w, rng = _rand_layer(shape, seed=12)
    b = _batch(shape, rng, 2, 1, [3])
    out = oracle.layer_forward(shape, w, b)
    T, H, A, F = 3, shape.hidden, shape.attn_width, shape.ffn
    for t in range(T):
        for n in range(3 * A):
            ref = sum(float(out["n1"][t, k]) * float(w["w_qkv"][n, k]) for k in range(H))
            assert abs(out["qkv"][t, n] - ref) <= 1e-12
        for n in range(H):
            h1 = float(b["x"][t, n]) + sum(float(out["attn"][t, k]) * float(w["w_o"][n, k]) for k in range(A))
            assert abs(out["h1"][t, n] - h1) <= 1e-12
            y = h1 + sum(float(out["act"][t, k]) * float(w["w_down"][n, k]) for k in range(F))
            assert abs(out["y"][t, n] - y) <= 1e-12
        for j in range(F):
            u = sum(float(out["n2"][t, k]) * float(w["w_up"][j, k]) for k in range(H))
            if shape.arch == "llama":
                gg = sum(float(out["n2"][t, k]) * float(w["w_gate"][j, k]) for k in range(H))
                ref = gg / (1 + math.exp(-gg)) * u
            else:
                ref = 0.5 * u * (1 + math.erf(u / math.sqrt(2)))
            assert abs(out["act"][t, j] - ref) <= 1e-12
    # Q/K/V columns: Q is [0,A), K [A,2A), V [2A,3A); V is not rotated; K is rotated at its position
    v = out["qkv"][:, 2 * A:].reshape(T, shape.n_heads, shape.head_dim)
    assert np.array_equal(out["new_v"], v)
    if shape.arch == "gpt":
        assert np.array_equal(out["new_k"].reshape(T, A), out["qkv"][:, A:2 * A])


def test_whole_layer_identity_special_case():
    """W_q = W_k = 0, W_v = I, W_o = I, W_down = 0 (hidden = heads x head_dim): the layer reduces to
    y = x + mean over each row's attended keys of V, where the new rows' V is RMSNorm(x).  Computed
    independently with Python loops."""
    shape = SMALL
    H = shape.hidden
    w, rng = _rand_layer(shape, seed=13, gamma_random=False)
    w["w_qkv"] = np.zeros((3 * H, H), np.float32)
    w["w_qkv"][2 * H:] = np.eye(H)
    w["w_o"] = np.eye(H, dtype=np.float32)
    w["w_down"] = np.zeros_like(w["w_down"])
    C, off, lens = 3, 4, [2, 5]
    b = _batch(shape, rng, C, off, lens)
    out = oracle.layer_forward(shape, w, b)
    x = b["x"].astype(np.float64)

    def rms(row):
        ms = sum(float(v) ** 2 for v in row) / H
        return [float(v) / math.sqrt(ms + shape.norm_eps) for v in row]

    nh, d = shape.n_heads, shape.head_dim
    newv = [rms(x[r]) for r in range(C + len(lens))]
    for r in range(C + len(lens)):
        for h in range(nh):
            for e in range(d):
                col = h * d + e
                if r < C:
                    vals = [b["chunk_v"][h, j, e] for j in range(off)] + [newv[t][col] for t in range(r + 1)]
                else:
                    i = r - C
                    vals = [b["decode_v"][i][h, j, e] for j in range(lens[i])] + [newv[r][col]]
                ref = x[r, col] + sum(float(v) for v in vals) / len(vals)
                assert abs(out["y"][r, col] - ref) <= 1e-12


def test_gated_ffn_special_case():
    """W_qkv = 0 with zero value caches (attention output 0), W_gate = 2I, W_up = I, W_down = I
    (ffn = hidden): y = x + silu(2 n) * n with n = RMSNorm(x) * gamma2."""
    shape = wl.LayerShape("sq", "llama", 16, 2, 8, 16, "f32", 1e-6, 10000.0, None)
    w, rng = _rand_layer(shape, seed=14)
    H = 16
    w["w_qkv"] = np.zeros_like(w["w_qkv"])
    w["w_gate"] = 2 * np.eye(H, dtype=np.float32)
    w["w_up"] = np.eye(H, dtype=np.float32)
    w["w_down"] = np.eye(H, dtype=np.float32)
    b = _batch(shape, rng, 2, 3, [4])
    b["chunk_v"][:] = 0
    b["decode_v"][0][:] = 0
    out = oracle.layer_forward(shape, w, b)
    for r in range(3):
        row = [float(v) for v in b["x"][r]]
        ms = sum(v * v for v in row) / H
        for c in range(H):
            n = row[c] / math.sqrt(ms + 1e-6) * float(w["norm2_w"][c])
            ref = row[c] + (2 * n) / (1 + math.exp(-2 * n)) * n
            assert abs(out["y"][r, c] - ref) <= 1e-12
