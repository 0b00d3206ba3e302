"""GPU parity of the HIP path against the CPU oracle, through the C ABI (needs an MI355X).

Every case prints its name and shape before it touches the GPU.  Unused cache slots are filled with
NaN so that a read past a request's keys poisons the output and fails the comparison.
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_prefill_hybrid_amd import _abi
from chunked_prefill_hybrid_amd import layer as hl
from chunked_prefill_hybrid_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MID = wl.LayerShape("mid-llama", "llama", 512, 4, 128, 1408, "bf16", 1e-6, 10000.0, None)
MID_GPT = wl.LayerShape("mid-gpt", "gpt", 512, 4, 128, 1024, "bf16", 1e-5, 10000.0, None)
MID_F32 = wl.LayerShape("mid-llama-f32", "llama", 512, 4, 128, 1408, "f32", 1e-6, 10000.0, None)
# FFN products of more than 256 weight stripes: a fused main part and a split tail
MID_WIDE_FFN = wl.LayerShape("mid-llama-wide-ffn", "llama", 512, 4, 128, 17920, "bf16", 1e-6, 10000.0, None)
MID_GPT_WIDE_FFN = wl.LayerShape("mid-gpt-wide-ffn", "gpt", 512, 4, 128, 34816, "bf16", 1e-5, 10000.0, None)
# Five heads: with an odd number of (row, head) pairs per row, one merge wave holds pairs of two rows.
MID_F32_5H = wl.LayerShape("mid-llama-f32-5h", "llama", 640, 5, 128, 1408, "f32", 1e-6, 10000.0, None)
MID_D64 = wl.LayerShape("mid-llama-d64", "llama", 256, 4, 64, 704, "bf16", 1e-6, 10000.0, None)
# A llama-7b-sized layer: at 400+ rows every one of its GEMMs takes two row tiles of 256 columns per
# weight stripe
BIG = wl.LayerShape("big-llama", "llama", 4096, 32, 128, 11008, "bf16", 1e-6, 10000.0, None)


def pad_caches(b, extra):
    """Give every cache `extra` more slots filled with NaN."""
    def pad(c):
        nh, cap, d = c.shape
        out = np.full((nh, cap + extra, d), np.nan, np.float32)
        out[:, :cap] = c
        return out
    b["chunk_k"], b["chunk_v"] = pad(b["chunk_k"]), pad(b["chunk_v"])
    b["decode_k"] = [pad(c) for c in b["decode_k"]]
    b["decode_v"] = [pad(c) for c in b["decode_v"]]
    # slots past the valid entries of the prefix / history are unused: NaN them too
    off = b["chunk_offset"]
    b["chunk_k"][:, off:], b["chunk_v"][:, off:] = np.nan, np.nan
    for i, L in enumerate(b["decode_len"]):
        b["decode_k"][i][:, L:], b["decode_v"][i][:, L:] = np.nan, np.nan
    return b


def case(shape, C, off, lens, seed=0, extra=5):
    rng = np.random.default_rng(seed)
    w = wl.make_weights(shape, rng)
    spec = wl.BatchSpec(C, off, off + C, len(lens), decode_lens=tuple(lens))
    b = pad_caches(wl.make_batch(shape, spec, rng), extra)
    return w, b


def run_case(shape, C, off, lens, seed=0, label=None, max_pos=None):
    label = label or f"{shape.name} C={C} off={off} B={len(lens)}"
    gu.say(f"case {label}")
    w, b = case(shape, C, off, lens, seed)
    ref = oracle.layer_forward(shape, w, b)
    T = C + len(lens)
    mp = max_pos or max([off + C] + [L + 1 for L in lens]) + 8
    layer = hl.HybridLayer(shape, gu.upload_weights(shape, w), max_tokens=T, max_pos=mp)
    db = gu.upload_batch(shape, b)
    dd = gu.run(layer, db)
    errs = gu.compare(shape, b, ref, db, dd, label=label)
    layer.close()
    return errs


# ------------------------------------------------------------------------------------------------
# GEMM alone
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("m,n,k", [(1, 128, 64), (17, 384, 320), (36, 768, 256), (105, 1536, 512),
                                   (274, 640, 5120), (289, 192, 1408), (560, 256, 640),
                                   # enough columns for one round of two-row-tile stripes of 256 columns
                                   (300, 30720, 256), (560, 30720, 512),
                                   # more than 576 rows: four 192-row tiles of 256 columns per stripe
                                   (700, 768, 512)])
def test_gemm_bf16(m, n, k):
    gu.say(f"gemm bf16 m={m} n={n} k={k}")
    rng = np.random.default_rng(m * 7 + n)
    a = wl.bf16_round(rng.standard_normal((m, k), dtype=np.float32))
    w = wl.bf16_round(rng.standard_normal((n, k), dtype=np.float32) * 0.02)
    out = hl.gemm(gu.dev(a, torch.bfloat16), gu.dev(w, torch.bfloat16))
    torch.cuda.synchronize()
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    err = gu.rel(out.float().cpu().numpy(), ref)
    gu.say(f"  rel={err:.2e}")
    assert err <= 8e-3   # output rounded to bf16 (2^-9 relative) with float32 accumulation


@pytest.mark.parametrize("m,n,k", [(1, 64, 16), (36, 688, 256), (70, 256, 688), (130, 100, 33)])
def test_gemm_f32(m, n, k):
    gu.say(f"gemm f32 m={m} n={n} k={k}")
    rng = np.random.default_rng(m + n + k)
    a = rng.standard_normal((m, k), dtype=np.float32)
    w = rng.standard_normal((n, k), dtype=np.float32)
    out = hl.gemm(gu.dev(a, torch.float32), gu.dev(w, torch.float32))
    torch.cuda.synchronize()
    ref = a.astype(np.float64) @ w.astype(np.float64).T
    assert gu.rel(out.cpu().numpy(), ref) <= 1e-5


# ------------------------------------------------------------------------------------------------
# The tiny fp32 workload: a 128-token prompt in 4 chunks of 32 with 4 decodes riding along
# ------------------------------------------------------------------------------------------------

def test_tiny_fp32_schedule():
    shape, w, px, dx, dk, dv, lens = wl.tiny_schedule(fill_rest=np.nan)
    nh, d = shape.n_heads, shape.head_dim
    host_ck = np.full((nh, 128, d), np.nan, np.float32)
    host_cv = host_ck.copy()
    layer = hl.HybridLayer(shape, gu.upload_weights(shape, w), max_tokens=36, max_pos=256)
    dck, dcv = gu.dev(host_ck, torch.float32), gu.dev(host_cv, torch.float32)
    ddk = [gu.dev(k, torch.float32) for k in dk]
    ddv = [gu.dev(v, torch.float32) for v in dv]
    for step in range(4):
        gu.say(f"case tiny fp32 step {step}")
        cur = [L + step for L in lens]
        b = {"x": np.concatenate([px[32 * step:32 * step + 32], dx[step]]), "chunk_len": 32,
             "chunk_offset": 32 * step, "chunk_k": host_ck, "chunk_v": host_cv, "decode_len": cur,
             "decode_k": dk, "decode_v": dv}
        ref = oracle.layer_forward(shape, w, b)
        db = {"x": gu.dev(b["x"], torch.float32), "chunk_len": 32, "chunk_offset": 32 * step,
              "chunk_kv": (dck, dcv), "decode_kv": list(zip(ddk, ddv)), "decode_len": cur}
        db["y"] = torch.empty_like(db["x"])
        dd = gu.run(layer, db)
        gu.compare(shape, b, ref, db, dd, label=f"tiny step {step}")
        oracle.apply_new_rows(b, ref)   # the host caches advance like the device ones
    layer.close()


def test_gpu_chunked_equals_monolithic_fp32():
    """The HIP path run as 4 chunks of 32 reproduces its own 1x128 prefill (and the caches agree)."""
    shape = wl.SHAPES["tiny"]
    gu.say("case gpu chunked vs monolithic fp32")
    rng = np.random.default_rng(21)
    w = wl.make_weights(shape, rng)
    x = rng.standard_normal((128, 256), dtype=np.float32)
    layer = hl.HybridLayer(shape, gu.upload_weights(shape, w), max_tokens=128, max_pos=128)
    outs = {}
    for n_chunks in (1, 4):
        C = 128 // n_chunks
        k = torch.zeros((4, 128, 64), device="cuda")
        v = torch.zeros_like(k)
        ys = []
        for c in range(n_chunks):
            xd = gu.dev(x[c * C:(c + 1) * C], torch.float32)
            y = torch.empty_like(xd)
            layer.forward(xd, y, C, c * C, (k, v), [], [])
            ys.append(y)
        torch.cuda.synchronize()
        outs[n_chunks] = (torch.cat(ys).cpu().numpy(), k.cpu().numpy(), v.cpu().numpy())
    for a, b in zip(outs[1], outs[4]):
        assert gu.rel(b, a) <= 1e-5
    layer.close()


# ------------------------------------------------------------------------------------------------
# bf16 layers spanning several tiles with ragged tails
# ------------------------------------------------------------------------------------------------

def test_mid_bf16_llama():
    run_case(MID, 100, 37, [0, 1, 63, 64, 300])


def test_mid_bf16_gpt():
    run_case(MID_GPT, 100, 37, [0, 1, 63, 64, 300])


def test_mid_fp32_llama():
    run_case(MID_F32, 100, 37, [0, 1, 63, 64, 300])


@pytest.mark.parametrize("shape", [MID_WIDE_FFN, MID_GPT_WIDE_FFN], ids=["swiglu", "gelu"])
def test_mid_bf16_wide_ffn(shape):
    run_case(shape, 100, 37, [0, 1, 300])


def test_mid_bf16_head_dim_64():
    run_case(MID_D64, 65, 200, [5, 511, 512, 1000])


@pytest.mark.parametrize("C,off,lens", [
    (0, 0, [7, 300, 1]),            # decode-only batch
    (77, 11, []),                   # chunk-only batch
    (1, 0, []),                     # a single token
    (0, 0, [0]),                    # a decode with an empty history attends only to itself
    (257, 0, [3, 9]),               # ragged chunk just past a tile multiple
    (3, 5, list(range(1, 141, 2))), # 70 decodes: more than one launch group of 64
    (200, 901, [5, 700]),           # chunk offset off the 64-key tile grid
    (64, 2051, [5]),                # one query block, long prefix: its keys split in two
    (0, 0, [2046, 2047, 2048, 3000]),  # decodes at the 256/1024-key split threshold
    (5, 2, [6001]),                 # a long decode: 1024-key splits, the last one ragged
    (650, 40, [3, 0, 90, 257, 1]),  # 655 rows, past 576: four row tiles of 256 columns per stripe
])
def test_edge_batches(C, off, lens):
    run_case(MID, C, off, lens, seed=C + len(lens))


# ------------------------------------------------------------------------------------------------
# Invariants on the GPU
# ------------------------------------------------------------------------------------------------

@pytest.mark.parametrize("shape,C,lens", [(MID, 60, [4, 250, 31]), (MID_F32, 60, [4, 250, 31]),
                                           (BIG, 400, [4, 250, 31]), (MID_WIDE_FFN, 300, [4, 250, 31]),
                                           (MID, 60, [2500, 4, 6001]), (MID_F32_5H, 7, [600, 4, 1100])],
                         ids=["bf16", "f32", "bf16-tall-tiles", "bf16-ffn-tail", "bf16-long-splits",
                              "f32-odd-heads"])
def test_decode_row_alone_equals_in_batch(shape, C, lens):
    """A decode row run alone (one GEMM row: a 32-row tile of 128 columns) equals the same decode
    inside a batch, bit for bit; with C = 400 the batch's GEMMs take two row tiles of 256 columns,
    whose k-sums must be cut at the same points and accumulated in the same order.  Alone, a decode's attention runs
    in the split-KV kernel's pipelined key walk; in a batch with a short chunk, in the fused kernel's
    walk (two steps of loads at a time); the long rows take 1024-key splits of four passes.  With
    five heads and a 7-row float32 chunk (whose rows take the general merge), the merge wave of the
    last chunk row's last head also holds decode 0's first head, which it then merges with a whole
    wave; alone, that pair is merged by a lane group of a wave: both must give the same bits."""
    gu.say(f"case decode alone vs in batch {shape.name} C={C} lens={lens}")
    w, b = case(shape, C, 9, lens, seed=3)
    layer = hl.HybridLayer(shape, gu.upload_weights(shape, w), max_tokens=C + 3,
                           max_pos=max(512, max(lens) + 1))
    db = gu.upload_batch(shape, b)
    gu.run(layer, db, dump=False)
    y_full = db["y"].clone()
    for i, L in enumerate(b["decode_len"]):
        db2 = gu.upload_batch(shape, {**b, "x": b["x"][C + i:C + i + 1], "chunk_len": 0,
                                      "decode_len": [L], "decode_k": [b["decode_k"][i]],
                                      "decode_v": [b["decode_v"][i]]})
        gu.run(layer, db2, dump=False)
        assert torch.equal(db2["y"][0], y_full[C + i]), f"decode {i} differs alone vs in batch"
    layer.close()


def test_run_twice_bitwise():
    gu.say("case determinism")
    w, b = case(MID, 50, 20, [10, 200], seed=4)
    layer = hl.HybridLayer(MID, gu.upload_weights(MID, w), max_tokens=52, max_pos=512)
    db = gu.upload_batch(MID, b)
    gu.run(layer, db, dump=False)
    y1 = db["y"].clone()
    gu.run(layer, db, dump=False)   # same lengths: overwrites the same cache slots
    assert torch.equal(y1, db["y"])
    layer.close()


@pytest.mark.parametrize("shape", [MID, MID_GPT], ids=lambda s: s.name)
def test_projection_weights_copied_at_create(shape):
    """A bf16 layer packs its projection weights at create and never reads the caller's projection
    buffers again: overwriting them with NaN after create leaves the forward's output unchanged
    (bit for bit) and still equal to the oracle's."""
    gu.say(f"case weights copied at create {shape.name}")
    w, b = case(shape, 40, 24, [7, 90], seed=9)
    ref = oracle.layer_forward(shape, w, b)
    wd = gu.upload_weights(shape, w)
    layer = hl.HybridLayer(shape, wd, max_tokens=42, max_pos=512)
    db = gu.upload_batch(shape, b)
    gu.run(layer, db, dump=False)
    y1 = db["y"].clone()
    for name in ("w_qkv", "w_o", "w_gate", "w_up", "w_down"):
        if wd.get(name) is not None:
            wd[name].fill_(float("nan"))
    torch.cuda.synchronize()
    db = gu.upload_batch(shape, b)   # fresh caches: the first forward appended its rows
    dd = gu.run(layer, db)
    assert torch.equal(y1, db["y"])
    gu.compare(shape, b, ref, db, dd, label=f"{shape.name} weights copied")
    layer.close()


def test_capacity_error_writes_nothing():
    gu.say("case capacity error")
    w, b = case(MID, 8, 0, [5], seed=5, extra=0)
    layer = hl.HybridLayer(MID, gu.upload_weights(MID, w), max_tokens=9, max_pos=64)
    db = gu.upload_batch(MID, b)
    db["y"].fill_(7.0)
    k_before = db["decode_kv"][0][0].clone()
    with pytest.raises(_abi.SarathiError) as e:
        # decode 0 claims 6 cached entries: slot 6 does not fit its capacity of 6
        layer.forward(db["x"], db["y"], 8, 0, db["chunk_kv"], db["decode_kv"], [6])
    assert e.value.status == _abi.SARATHI_ERR_CAPACITY
    torch.cuda.synchronize()
    assert torch.all(db["y"] == 7.0)
    assert torch.equal(k_before.view(torch.int16), db["decode_kv"][0][0].view(torch.int16))  # bitwise (NaN slots)
    layer.close()


@pytest.mark.parametrize("shape", [MID, MID_F32], ids=["bf16", "f32"])
def test_attention_mask_length_closed_form(shape):
    """Attention stage alone with q = 0 and V[:, j] = j: row at position p averages 0..p, i.e. p/2
    (the chunk row t sees keys 0..off+t; decode i sees its L_i cached keys plus its own slot L_i)."""
    gu.say(f"case attention closed form {shape.name}")
    nh, d = shape.n_heads, shape.head_dim
    dt = gu.tdtype(shape)
    C, off, lens = 40, 100, [0, 5, 130, 255]
    T = C + len(lens)

    def cache(n):
        k = torch.randn((nh, n, d), device="cuda").to(dt)
        v = torch.arange(n, device="cuda", dtype=torch.float32).view(1, n, 1).expand(nh, n, d)
        return k, v.to(dt).contiguous()

    ck = cache(off + C)
    dks = [cache(L + 1) for L in lens]
    q = torch.zeros((T, nh * d), device="cuda", dtype=dt)
    out = torch.full((T, nh * d), float("nan"), device="cuda", dtype=dt)
    hl.attention(shape, q, out, C, off, ck, dks, lens, max_pos=512)
    torch.cuda.synchronize()
    expect = np.array([(off + t) / 2 for t in range(C)] + [L / 2 for L in lens])
    got = out.float().cpu().numpy()
    err = np.max(np.abs(got - expect[:, None]) / np.maximum(expect[:, None], 1))
    gu.say(f"  max rel err {err:.2e}")
    assert err <= (4e-3 if shape.dtype == "bf16" else 1e-5)
