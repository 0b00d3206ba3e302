"""CPU oracle: the layer over a batch whose KV caches live in a page pool (paged KV cache).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import,
call or run anything in this package.  The product path never does, and nothing here comes from it.

What it computes.  Paged storage changes where a request's K/V rows sit, not what attention computes:
token t of a request is row t % page_size of pool page table[t // page_size] (per head), and the
request's logical cache is the sequence of those rows.  (Dynamic, non-contiguous KV allocation is the
memory-management technique the SARATHI page lists as complementary: SARATHI: Efficient LLM Inference
by Piggybacking Decodes with Chunked Prefills, "System Optimizations from Prior Work".)  So the oracle
gathers each request's logical cache out of the pools, runs layer_forward_multi on it, and writes the
step's new rows back to the pool slots they belong to.

Pool layout: k_pool and v_pool are [n_pages, n_heads, page_size, head_dim].
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .multi import layer_forward_multi

__all__ = ["gather_cache", "layer_forward_paged", "apply_paged_rows", "paged_slot"]


def paged_slot(table, t: int, page_size: int):
    """(pool page, row within the page) of token t of a request with block table `table`."""
    return int(table[t // page_size]), t % page_size


def gather_cache(pool: np.ndarray, table, n_tokens: int, page_size: int) -> np.ndarray:
    """The request's logical cache [n_heads, n_tokens, d]: entry t is pool[page, :, row, :] with
    (page, row) = paged_slot(table, t)."""
    nh, d = pool.shape[1], pool.shape[3]
    out = np.empty((nh, n_tokens, d), dtype=pool.dtype)
    for t in range(n_tokens):
        page, row = paged_slot(table, t, page_size)
        out[:, t, :] = pool[page, :, row, :]
    return out


def layer_forward_paged(shape, weights, batch: Dict, dtype=np.float64) -> Dict[str, np.ndarray]:
    """batch: x, k_pool, v_pool, page_size, chunks (list of dicts len, offset, table), decode_len,
    decode_tables.  Nothing is modified.  Returns layer_forward_multi's result."""
    P = int(batch["page_size"])
    kp, vp = batch["k_pool"], batch["v_pool"]
    chunks = []
    for c in batch["chunks"]:
        n = int(c["offset"]) + int(c["len"])
        chunks.append({"len": c["len"], "offset": c["offset"],
                       "k": gather_cache(kp, c["table"], n, P), "v": gather_cache(vp, c["table"], n, P)})
    lens = [int(L) for L in batch["decode_len"]]
    dk = [gather_cache(kp, t, L + 1, P) for t, L in zip(batch["decode_tables"], lens)]
    dv = [gather_cache(vp, t, L + 1, P) for t, L in zip(batch["decode_tables"], lens)]
    mb = {"x": batch["x"], "chunks": chunks, "decode_len": lens, "decode_k": dk, "decode_v": dv}
    return layer_forward_multi(shape, weights, mb, dtype)


def apply_paged_rows(batch: Dict, out: Dict) -> None:
    """Write the step's new K/V rows into the pools in place (row t of chunk j -> its request's slot
    offset_j + t; decode i -> slot decode_len[i])."""
    P = int(batch["page_size"])
    r = 0
    for c in batch["chunks"]:
        for t in range(int(c["len"])):
            page, row = paged_slot(c["table"], int(c["offset"]) + t, P)
            batch["k_pool"][page, :, row, :] = out["new_k"][r]
            batch["v_pool"][page, :, row, :] = out["new_v"][r]
            r += 1
    for tbl, L in zip(batch["decode_tables"], batch["decode_len"]):
        page, row = paged_slot(tbl, int(L), P)
        batch["k_pool"][page, :, row, :] = out["new_k"][r]
        batch["v_pool"][page, :, row, :] = out["new_v"][r]
        r += 1
