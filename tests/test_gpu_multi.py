"""GPU parity of batches with several prefill chunks (sarathi_multi_forward) against the oracle,
through the C ABI (needs an MI355X).

Token-budget batches put the remaining tokens of partly prefilled prompts and the first tokens of new
prompts next to the decodes (junupark.xyz notes on Sarathi-Serve, "Stall Free Batching").  Unused
cache slots are NaN, so a chunk reading another request's keys, or past its own, fails.
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_prefill_hybrid_amd import layer as hl
from chunked_prefill_hybrid_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MID = wl.LayerShape("mid-llama", "llama", 512, 4, 128, 1408, "bf16", 1e-6, 10000.0, None)
MID_GPT = wl.LayerShape("mid-gpt", "gpt", 512, 4, 128, 1024, "bf16", 1e-5, 10000.0, None)
MID_D64 = wl.LayerShape("mid-llama-d64", "llama", 256, 4, 64, 704, "bf16", 1e-6, 10000.0, None)
# 20 heads: enough chunk work items that the planner runs a long chunk with two 16-query blocks per
# wave (pinned in test_abi_cpu.py)
WIDE = wl.LayerShape("wide-llama", "llama", 2560, 20, 128, 1024, "bf16", 1e-6, 10000.0, None)
WIDE_D64 = wl.LayerShape("wide-llama-d64", "llama", 1280, 20, 64, 1024, "bf16", 1e-6, 10000.0, None)


def make(shape, chunk_specs, dec_lens, seed, extra=3):
    """Seeded weights and a batch: chunks [(len, offset)], decode lengths; NaN past valid slots."""
    rng = np.random.default_rng(seed)
    nh, d, H = shape.n_heads, shape.head_dim, shape.hidden
    rnd = (lambda a: wl.bf16_round(a.astype(np.float32))) if shape.dtype == "bf16" else \
        (lambda a: a.astype(np.float32))
    w = wl.make_weights(shape, rng)

    def cache(filled, cap):
        c = np.full((nh, cap, d), np.nan, np.float32)
        c[:, :filled] = rnd(rng.standard_normal((nh, filled, d)))
        return c
    chunks = [{"len": n, "offset": o, "k": cache(o, o + n + extra), "v": cache(o, o + n + extra)}
              for n, o in chunk_specs]
    T = sum(n for n, _ in chunk_specs) + len(dec_lens)
    b = {"x": rnd(rng.standard_normal((T, H))), "chunks": chunks, "decode_len": list(dec_lens),
         "decode_k": [cache(L, L + 1 + extra) for L in dec_lens],
         "decode_v": [cache(L, L + 1 + extra) for L in dec_lens]}
    return w, b


def run_case(shape, chunk_specs, dec_lens, seed=0, label=None):
    label = label or f"{shape.name} chunks={chunk_specs} B={len(dec_lens)}"
    gu.say(f"case {label}")
    w, b = make(shape, chunk_specs, dec_lens, seed)
    ref = oracle.layer_forward_multi(shape, w, b)
    T = b["x"].shape[0]
    mp = max([o + n for n, o in chunk_specs] + [L + 1 for L in dec_lens]) + 8
    layer = hl.HybridLayer(shape, gu.upload_weights(shape, w), max_tokens=T, max_pos=mp)
    db = gu.upload_multi(shape, b)
    dd = gu.run_multi(layer, db)
    errs = gu.compare_multi(shape, b, ref, db, dd, label=label)
    layer.close()
    return errs


@pytest.mark.parametrize("shape,chunks,lens", [
    (MID, [(40, 70), (64, 0), (1, 5), (130, 200)], [5, 700, 64]),
    (MID, [(94, 930), (300, 0), (100, 0)], [1024] * 3),          # the budget workload's composition
    (MID_GPT, [(33, 0), (65, 128)], [17]),
    (MID_D64, [(17, 3), (80, 100)], []),
    (MID, [(64, 2100), (40, 2500)], [30]),                         # long prefixes: split key ranges
    (MID, [(64, 2100), (100, 0), (30, 50)], []),                   # per-chunk splits 3, 1, 1
    (MID, [(64, 2100), (100, 0), (30, 50)], [40, 900]),            # the same in the fused launch
    (MID, [(n, 7 * n) for n in range(1, 17)], [3]),                # sixteen chunks of 1..16 rows
    (MID, [], [9, 300]),                                           # no chunk at all
    (WIDE, [(1024, 2000)], [30]),                                  # 128-query blocks, 3 key splits
    (WIDE, [(1000, 2000), (37, 100)], []),                         # the same, ragged, splits 3 and 1
    (WIDE_D64, [(1000, 2000), (37, 100)], [30]),                   # d = 64
    (WIDE, [(300, 50), (200, 0)], [40, 500]),                      # fused launch, two blocks per wave
    (WIDE_D64, [(300, 50), (200, 0)], [40, 500]),                  # the same, d = 64
])
def test_multi_bf16(shape, chunks, lens):
    run_case(shape, chunks, lens)


def test_multi_fp32_tiny():
    run_case(wl.SHAPES["tiny"], [(10, 20), (32, 0), (5, 90)], [3, 90])


def test_one_chunk_multi_is_bitwise_the_single_entry_point():
    shape = MID
    gu.say("case multi(1 chunk) vs single entry point, bitwise")
    w, b = make(shape, [(77, 150)], [12, 400], seed=3)
    layer = hl.HybridLayer(shape, gu.upload_weights(shape, w), max_tokens=79, max_pos=512)
    db = gu.upload_multi(shape, b)
    gu.run_multi(layer, db, dump=False)
    c = b["chunks"][0]
    single = {"x": b["x"], "chunk_len": 77, "chunk_offset": 150, "chunk_k": c["k"], "chunk_v": c["v"],
              "decode_len": b["decode_len"], "decode_k": b["decode_k"], "decode_v": b["decode_v"]}
    ds = gu.upload_batch(shape, single)
    gu.run(layer, ds, dump=False)
    assert torch.equal(db["y"], ds["y"])
    n, off, (k, v) = db["chunks"][0]
    # slots past off + n stay NaN in both (NaN != NaN), so compare the written ones
    assert torch.equal(k[:, :off + n], ds["chunk_kv"][0][:, :off + n])
    assert torch.equal(v[:, :off + n], ds["chunk_kv"][1][:, :off + n])
    layer.close()


def test_rows_bitwise_independent_of_the_other_requests():
    """Each request's rows in a token-budget batch equal, bit for bit, the same request run in a batch
    of its own (linear ops are batch-invariant per row; no chunk here splits its key range)."""
    shape = MID
    gu.say("case multi rows vs each request alone, bitwise")
    specs = [(30, 100), (64, 0), (9, 40)]
    lens = [50, 333]
    w, b = make(shape, specs, lens, seed=4)
    layer = hl.HybridLayer(shape, gu.upload_weights(shape, w), max_tokens=110, max_pos=512)
    db = gu.upload_multi(shape, b)
    gu.run_multi(layer, db, dump=False)
    y_all = db["y"].clone()
    r0 = 0
    dt = gu.tdtype(shape)
    for j, (n, off) in enumerate(specs):
        c = b["chunks"][j]
        sub = {"x": b["x"][r0:r0 + n], "chunks": [c], "decode_len": [], "decode_k": [], "decode_v": []}
        ds = gu.upload_multi(shape, sub)
        gu.run_multi(layer, ds, dump=False)
        assert torch.equal(ds["y"], y_all[r0:r0 + n]), f"chunk {j}"
        r0 += n
    for i, L in enumerate(lens):
        sub = {"x": b["x"][r0 + i:r0 + i + 1], "chunks": [], "decode_len": [L],
               "decode_k": [b["decode_k"][i]], "decode_v": [b["decode_v"][i]]}
        ds = gu.upload_multi(shape, sub)
        gu.run_multi(layer, ds, dump=False)
        assert torch.equal(ds["y"], y_all[r0 + i:r0 + i + 1]), f"decode {i}"
    layer.close()


def test_two_prompts_in_budget_steps_on_gpu():
    """Two prompts prefilled side by side in token-budget steps (budget 96, two decodes riding along),
    GPU caches and outputs against the oracle driving the same steps with its own caches."""
    shape = MID
    rng = np.random.default_rng(8)
    nh, d, H = shape.n_heads, shape.head_dim, shape.hidden
    rnd = lambda a: wl.bf16_round(a.astype(np.float32))
    w = wl.make_weights(shape, rng)
    P = [150, 70]
    xs = [rnd(rng.standard_normal((p, H))) for p in P]
    host = [(np.full((nh, p, d), np.nan, np.float32), np.full((nh, p, d), np.nan, np.float32)) for p in P]
    dlen = [20, 260]
    dk = [np.full((nh, L + 8, d), np.nan, np.float32) for L in dlen]
    dv = [np.full((nh, L + 8, d), np.nan, np.float32) for L in dlen]
    for c, L in zip(dk + dv, dlen + dlen):
        c[:, :L] = rnd(rng.standard_normal((nh, L, d)))
    dev = lambda a: gu.dev(a, torch.bfloat16)
    g_ck = [(dev(k), dev(v)) for k, v in host]
    g_dk = [(dev(k), dev(v)) for k, v in zip(dk, dv)]
    layer = hl.HybridLayer(shape, gu.upload_weights(shape, w), max_tokens=96, max_pos=512)
    done, step = [0, 0], 0
    while done != P:
        n_dec, picked = wl.budget_batch(96, 2, [(P[i], done[i]) for i in range(2)])
        lens = [L + step for L in dlen]
        x = np.concatenate([xs[i][off:off + n] for i, n, off in picked] + [rnd(rng.standard_normal((n_dec, H)))])
        gu.say(f"case budget step {step}: chunks {[(n, off) for _, n, off in picked]} decodes {lens}")
        b = {"x": x, "chunks": [{"len": n, "offset": off, "k": host[i][0], "v": host[i][1]} for i, n, off in picked],
             "decode_len": lens, "decode_k": dk, "decode_v": dv}
        ref = oracle.layer_forward_multi(shape, w, b)
        db = {"x": dev(x), "chunks": [(n, off, g_ck[i]) for i, n, off in picked], "decode_kv": g_dk,
              "decode_len": lens}
        db["y"] = torch.empty_like(db["x"])
        gu.run_multi(layer, db, dump=False)
        gu.compare_multi(shape, b, ref, db, None, label=f"budget step {step}")
        oracle.apply_multi_rows(b, ref)
        for i, n, off in picked:
            done[i] += n
        step += 1
    layer.close()


def test_workspace_contents_on_entry_do_not_matter():
    """The workspace is filled with NaN before the forward: decodes with fewer key splits than the
    batch's largest, and split chunk rows, must never read an unwritten partial into the result."""
    shape = MID
    gu.say("case NaN-filled workspace, multi and single entry points")
    specs, lens = [(64, 2100), (40, 2500)], [3, 40, 900]
    w, b = make(shape, specs, lens, seed=11)
    ref = oracle.layer_forward_multi(shape, w, b)
    layer = hl.HybridLayer(shape, gu.upload_weights(shape, w), max_tokens=107, max_pos=2600)
    db = gu.upload_multi(shape, b)
    bb, keep = layer.multi_batch(db["x"], db["y"], db["chunks"], db["decode_kv"], db["decode_len"])
    need = layer.workspace_size(bb)
    ws = torch.full(((need + 3) // 4,), float("nan"), device="cuda").view(torch.uint8)
    gu.run_multi(layer, db, dump=False, workspace=ws)
    gu.compare_multi(shape, b, ref, db, None, label="nan workspace multi")
    # the single entry point: a decode-only batch with lengths of 1..4 key splits
    w2, b2 = make(shape, [], [3, 300, 700, 1000], seed=12)
    ref2 = oracle.layer_forward_multi(shape, w2, b2)
    layer2 = hl.HybridLayer(shape, gu.upload_weights(shape, w2), max_tokens=4, max_pos=1100)
    single = {"x": b2["x"], "chunk_len": 0, "chunk_offset": 0, "chunk_k": None, "chunk_v": None,
              "decode_len": b2["decode_len"], "decode_k": b2["decode_k"], "decode_v": b2["decode_v"]}
    ds = {"x": gu.dev(single["x"], torch.bfloat16), "chunk_len": 0, "chunk_offset": 0, "chunk_kv": None,
          "decode_len": single["decode_len"],
          "decode_kv": [(gu.dev(k, torch.bfloat16), gu.dev(v, torch.bfloat16))
                        for k, v in zip(b2["decode_k"], b2["decode_v"])]}
    ds["y"] = torch.empty_like(ds["x"])
    ws2 = torch.full((1 << 22,), float("nan"), device="cuda").view(torch.uint8)
    gu.run(layer2, ds, dump=False, workspace=ws2)
    nk, nv = gu.new_rows_from_caches(ds, 0, 0, single["decode_len"])
    gu.compare_rows(shape, b2["x"], ref2, ds["y"], nk, nv, None, label="nan workspace single")
    layer.close()
    layer2.close()
