"""Pins of the paged-KV oracle (CPU, float64).

- A hand-built pool: token t of a request is row t % page_size of pool page table[t // page_size];
  gather_cache returns exactly the rows written there, and paged_slot names them.
- Paged == contiguous: a several-chunk batch whose caches are laid out in a shuffled page pool
  (workloads.paginate) gives bitwise the outputs of the same batch with contiguous caches, and the
  rows the step writes land in the pool slots that hold the same logical positions.
- A block-table mistake planted in a copy of gather_cache (an off-by-one page) fails the first pin.
"""
import numpy as np

import oracle
from chunked_prefill_hybrid_amd import workloads as wl


def test_hand_built_pool():
    P, nh, d = 2, 1, 1
    pool = np.zeros((4, nh, P, d))
    # request with table [3, 0, 2]: tokens 0,1 in page 3; 2,3 in page 0; 4 in page 2 (row 0)
    for t, (page, row) in enumerate([(3, 0), (3, 1), (0, 0), (0, 1), (2, 0)]):
        pool[page, 0, row, 0] = 100 + t
    table = np.array([3, 0, 2], np.int32)
    got = oracle.gather_cache(pool, table, 5, P)
    assert got[0, :, 0].tolist() == [100, 101, 102, 103, 104]
    assert oracle.paged_slot(table, 4, P) == (2, 0) and oracle.paged_slot(table, 3, P) == (0, 1)


def test_planted_table_mistake_fails():
    P = 2
    pool = np.arange(4 * P, dtype=float).reshape(4, 1, P, 1)
    table = np.array([1, 3], np.int32)

    def gather_off_by_one(pool, table, n, P):
        return np.stack([pool[table[min(t // P + 1, len(table) - 1)], :, t % P, :] for t in range(n)], axis=1)

    good = oracle.gather_cache(pool, table, 4, P)
    assert good[0, :, 0].tolist() == [2, 3, 6, 7]
    assert not np.array_equal(gather_off_by_one(pool, table, 4, P), good)


def test_paged_equals_contiguous():
    shape = wl.SHAPES["tiny"]
    rng = np.random.default_rng(5)
    nh, d, H = shape.n_heads, shape.head_dim, shape.hidden
    w = wl.make_weights(shape, rng)
    specs, lens = [(9, 21), (16, 0)], [4, 37]
    P = 8
    caches = [(rng.standard_normal((nh, o + n + 3, d)), rng.standard_normal((nh, o + n + 3, d))) for n, o in specs]
    caches += [(rng.standard_normal((nh, L + 2, d)), rng.standard_normal((nh, L + 2, d))) for L in lens]
    x = rng.standard_normal((sum(n for n, _ in specs) + len(lens), H))
    mb = {"x": x, "chunks": [{"len": n, "offset": o, "k": caches[j][0].copy(), "v": caches[j][1].copy()}
                             for j, (n, o) in enumerate(specs)],
          "decode_len": lens, "decode_k": [caches[2 + i][0].copy() for i in range(2)],
          "decode_v": [caches[2 + i][1].copy() for i in range(2)]}
    kp, vp, tables = wl.paginate([(k.astype(np.float32), v.astype(np.float32)) for k, v in caches], P,
                                 seed=3, extra_pages=5)
    kp, vp = kp.astype(np.float64), vp.astype(np.float64)
    # exact float32 copies on both sides
    for j in range(2):
        mb["chunks"][j]["k"] = caches[j][0].astype(np.float32).astype(np.float64)
        mb["chunks"][j]["v"] = caches[j][1].astype(np.float32).astype(np.float64)
    for i in range(2):
        mb["decode_k"][i] = caches[2 + i][0].astype(np.float32).astype(np.float64)
        mb["decode_v"][i] = caches[2 + i][1].astype(np.float32).astype(np.float64)
    ref = oracle.layer_forward_multi(shape, w, mb)
    pb = {"x": x, "k_pool": kp, "v_pool": vp, "page_size": P,
          "chunks": [{"len": n, "offset": o, "table": tables[j]} for j, (n, o) in enumerate(specs)],
          "decode_len": lens, "decode_tables": tables[2:]}
    got = oracle.layer_forward_paged(shape, w, pb)
    for key in ("y", "new_k", "new_v", "attn"):
        assert np.array_equal(got[key], ref[key]), key
    oracle.apply_paged_rows(pb, got)
    oracle.apply_multi_rows(mb, ref)
    for j, (n, o) in enumerate(specs):
        assert np.array_equal(oracle.gather_cache(kp, tables[j], o + n, P), mb["chunks"][j]["k"][:, :o + n])
    for i, L in enumerate(lens):
        assert np.array_equal(oracle.gather_cache(vp, tables[2 + i], L + 1, P), mb["decode_v"][i][:, :L + 1])
