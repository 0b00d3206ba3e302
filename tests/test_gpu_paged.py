"""GPU parity of the paged-KV path (sarathi_paged_forward) through the C ABI (needs an MI355X).

Each case lays the same request caches out twice: contiguous (one buffer per request) and in a
shuffled page pool.  The paged forward must give bitwise the contiguous forward's outputs (only the
addressing differs) and write its new K/V rows into the pool slots of their positions; it is also
compared with the paged oracle.  Unused slots and pages hold NaN.
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_prefill_hybrid_amd import layer as hl
from chunked_prefill_hybrid_amd import workloads as wl
from tests import gpu_util as gu
from tests.test_gpu_multi import MID, MID_D64, MID_GPT, make

pytestmark = pytest.mark.gpu


def to_pool(shape, b, page, seed=1):
    """Pool + tables holding the batch's caches (capacity of each request rounded up to pages)."""
    caches = [(c["k"], c["v"]) for c in b["chunks"]] + list(zip(b["decode_k"], b["decode_v"]))
    return wl.paginate(caches, page, seed=seed, extra_pages=3, fill=np.nan)


def run_paged_case(shape, chunk_specs, dec_lens, page, seed=0, label=None, full_compare=True):
    label = label or f"{shape.name} page={page} chunks={chunk_specs} B={len(dec_lens)}"
    gu.say(f"case {label}")
    w, b = make(shape, chunk_specs, dec_lens, seed)
    kp, vp, tables = to_pool(shape, b, page, seed + 1)
    dt = gu.tdtype(shape)
    T = b["x"].shape[0]
    mp = max([o + n for n, o in chunk_specs] + [L + 1 for L in dec_lens]) + 8
    layer = hl.HybridLayer(shape, gu.upload_weights(shape, w), max_tokens=T, max_pos=mp)
    # contiguous reference run on the GPU
    db = gu.upload_multi(shape, b)
    gu.run_multi(layer, db, dump=False)
    # paged run
    x = gu.dev(b["x"], dt)
    y = torch.full_like(x, float("nan"))
    pool = (gu.dev(kp, dt), gu.dev(vp, dt))
    gt = [torch.from_numpy(t).to("cuda") for t in tables]
    nc = len(chunk_specs)
    layer.forward_paged(x, y, pool, [(n, o, gt[j]) for j, (n, o) in enumerate(chunk_specs)], gt[nc:], dec_lens)
    torch.cuda.synchronize()
    assert torch.equal(y, db["y"]), f"{label}: paged output differs from contiguous"
    # new rows: read back from the pool at each row's slot
    kph, vph = pool[0].float().cpu().numpy(), pool[1].float().cpu().numpy()
    nk, nv = gu.new_rows_multi(db)
    r = 0
    slots = [(tables[j], o + t) for j, (n, o) in enumerate(chunk_specs) for t in range(n)]
    slots += [(tables[nc + i], L) for i, L in enumerate(dec_lens)]
    for tbl, pos in slots:
        pg, row = oracle.paged_slot(tbl, pos, page)
        assert np.array_equal(kph[pg, :, row, :], nk[r]) and np.array_equal(vph[pg, :, row, :], nv[r]), \
            f"{label}: row {r} written to the wrong pool slot"
        r += 1
    if full_compare:
        pb = {"x": b["x"], "k_pool": kp, "v_pool": vp, "page_size": page,
              "chunks": [{"len": n, "offset": o, "table": tables[j]} for j, (n, o) in enumerate(chunk_specs)],
              "decode_len": dec_lens, "decode_tables": tables[nc:]}
        ref = oracle.layer_forward_paged(shape, w, pb)
        gu.compare_rows(shape, b["x"], ref, y, nk, nv, None, label=label + " vs oracle")
    layer.close()


@pytest.mark.parametrize("page", [8, 16, 32, 64, 256])
def test_paged_bf16_page_sizes(page):
    run_paged_case(MID, [(70, 130), (33, 0)], [5, 300, 64], page)


@pytest.mark.parametrize("shape,chunks,lens,page", [
    (MID_GPT, [(65, 128)], [17], 16),
    (MID_D64, [(17, 3), (80, 100)], [9], 32),
    (MID, [(64, 2100), (40, 2500)], [30], 16),      # split key ranges of the chunk kernel
    (MID, [(64, 2100), (100, 0), (30, 50)], [], 8), # per-chunk split counts 3, 1, 1
    (MID, [], [1, 40, 1023], 16),                   # decodes only
    (MID, [(200, 0)], [], 1),                       # one-token pages
    (MID, [], [2049, 4500], 1),                     # long decodes (1024-key splits), one-token pages
    (MID, [(30, 10)], [2100, 3333], 16),            # long decodes beside a chunk
])
def test_paged_cases(shape, chunks, lens, page):
    run_paged_case(shape, chunks, lens, page)


def test_paged_fp32_tiny():
    run_paged_case(wl.SHAPES["tiny"], [(10, 20), (32, 0)], [3, 90], 16)


def test_shared_prefix_pages():
    """Two decodes share their first pages (a common prefix, read only) and own their last pages;
    the paged forward matches the oracle and leaves the shared pages untouched."""
    shape, page = MID, 16
    gu.say("case shared prefix pages")
    rng = np.random.default_rng(21)
    nh, d, H = shape.n_heads, shape.head_dim, shape.hidden
    w = wl.make_weights(shape, rng)
    rnd = lambda a: wl.bf16_round(a.astype(np.float32))
    n_pages = 12
    kp = np.full((n_pages, nh, page, d), np.nan, np.float32)
    vp = kp.copy()
    prefix = 40                                     # tokens 0..39: pages 0, 1 and part of 2
    L = [prefix + 5, prefix + 9]                    # each decode has a private tail
    kp[:3] = rnd(rng.standard_normal((3, nh, page, d)))
    vp[:3] = rnd(rng.standard_normal((3, nh, page, d)))
    # decode i: shared pages 0, 1; private copy of page 2 content for its own tail -> pages 3+i*2.
    tables = []
    for i in range(2):
        own = [3 + 2 * i, 4 + 2 * i]
        kp[own[0]] = kp[2]
        vp[own[0]] = vp[2]
        kp[own[0], :, prefix - 32:, :] = rnd(rng.standard_normal((nh, page - (prefix - 32), d)))
        vp[own[0], :, prefix - 32:, :] = rnd(rng.standard_normal((nh, page - (prefix - 32), d)))
        kp[own[1]] = rnd(rng.standard_normal((nh, page, d)))
        vp[own[1]] = rnd(rng.standard_normal((nh, page, d)))
        tables.append(np.array([0, 1] + own, np.int32))
    shared_before = (kp[:2].copy(), vp[:2].copy())
    x = rnd(rng.standard_normal((2, H)))
    pb = {"x": x, "k_pool": kp.copy(), "v_pool": vp.copy(), "page_size": page, "chunks": [],
          "decode_len": L, "decode_tables": tables}
    ref = oracle.layer_forward_paged(shape, w, pb)
    layer = hl.HybridLayer(shape, gu.upload_weights(shape, w), max_tokens=2, max_pos=128)
    pool = (gu.dev(kp, torch.bfloat16), gu.dev(vp, torch.bfloat16))
    gx = gu.dev(x, torch.bfloat16)
    gy = torch.empty_like(gx)
    gt = [torch.from_numpy(t).to("cuda") for t in tables]
    layer.forward_paged(gx, gy, pool, [], gt, L)
    torch.cuda.synchronize()
    kph = pool[0].float().cpu().numpy()
    assert np.array_equal(kph[:2], shared_before[0], equal_nan=True), "shared pages were written"
    nk = np.stack([kph[oracle.paged_slot(tables[i], L[i], page)[0], :, oracle.paged_slot(tables[i], L[i], page)[1], :]
                   for i in range(2)])
    vph = pool[1].float().cpu().numpy()
    nv = np.stack([vph[oracle.paged_slot(tables[i], L[i], page)[0], :, oracle.paged_slot(tables[i], L[i], page)[1], :]
                   for i in range(2)])
    gu.compare_rows(shape, x, ref, gy, nk, nv, None, label="shared prefix")
    layer.close()


def test_full_size_paged_equals_contiguous():
    """The llama13b workload (C = 256 at offset 768 + 18 decodes of 1024) with its caches in a shuffled
    pool of 16-token pages: bitwise the contiguous forward's output."""
    wk = wl.workload("llama13b")
    gu.say("case full-size llama13b paged (16-token pages) vs contiguous, bitwise")
    w, b = wl.generate(wk)
    shape = wk.shape
    dt = torch.bfloat16
    T = b["x"].shape[0]
    layer = hl.HybridLayer(shape, gu.upload_weights(shape, w), max_tokens=T, max_pos=1025)
    db = gu.upload_batch(shape, b)
    gu.run(layer, db, dump=False)
    caches = [(b["chunk_k"], b["chunk_v"])] + list(zip(b["decode_k"], b["decode_v"]))
    kp, vp, tables = wl.paginate(caches, 16, seed=7, extra_pages=10)
    pool = (gu.dev(kp, dt), gu.dev(vp, dt))
    del kp, vp
    gt = [torch.from_numpy(t).to("cuda") for t in tables]
    x = gu.dev(b["x"], dt)
    y = torch.empty_like(x)
    layer.forward_paged(x, y, pool, [(b["chunk_len"], b["chunk_offset"], gt[0])], gt[1:], b["decode_len"])
    torch.cuda.synchronize()
    assert torch.equal(y, db["y"])
    layer.close()
