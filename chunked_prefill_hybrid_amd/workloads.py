"""Seeded synthetic workloads for the hybrid-batch decoder layer.

A hybrid batch is one prefill chunk of C tokens plus B single-token decodes, each decode with its own
KV cache ("decode-maximal batching", SARATHI: Efficient LLM Inference by Piggybacking Decodes with
Chunked Prefills, section 3 "Decode-Maximal Batching").  This module holds the five layer shapes and
batch compositions the library is measured and checked on, and a seeded generator of host arrays:
weights, hidden states, KV caches and lengths.

None of the layer's arithmetic lives here.  The HIP path and the CPU oracle both consume these arrays
as they are; the only numeric step is rounding the drawn values to bfloat16 (round to nearest even)
for the bf16 workloads, so that both sides see identical, exactly representable inputs.

Seeding.  A workload's root numpy SeedSequence(seed) spawns one child stream per drawn tensor, in a
fixed order (so every sweep point of one shape shares its weights): W_qkv, W_o, W_gate (gated shapes
only), W_up, W_down, then X, then the chunk request's prefix cache (K then V), then the decode
lengths, then each decode cache in request order (K then V).  A tensor's values are drawn in fixed
blocks of 2^22 elements, block i from PCG64 seeded by the i-th child of the tensor's stream, so the
result does not depend on how many threads fill the blocks.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "LayerShape", "BatchSpec", "Workload", "SHAPES", "bf16_round", "bf16_bits",
    "make_weights", "make_batch", "workload", "sweep", "tiny_schedule", "WORKLOADS",
    "MultiSpec", "budget_batch", "make_multi_batch", "chunks_of", "paginate",
]


@dataclass(frozen=True)
class LayerShape:
    """One decoder layer's shape.  arch 'llama': RMSNorm, RoPE, SwiGLU FFN.  arch 'gpt': LayerNorm,
    no RoPE, GELU MLP.  w_std is the standard deviation of the weight draws; None means
    1/sqrt(fan_in) per matrix (fan_in = the matrix's input width)."""
    name: str
    arch: str
    hidden: int
    n_heads: int
    head_dim: int
    ffn: int
    dtype: str               # 'f32' or 'bf16': storage type of weights, activations and caches
    norm_eps: float
    rope_base: float
    w_std: Optional[float]

    @property
    def attn_width(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def gated(self) -> bool:
        return self.arch == "llama"

    def n_params(self) -> int:
        h, a, f = self.hidden, self.attn_width, self.ffn
        return 3 * a * h + h * a + (2 if self.gated else 1) * f * h + h * f


@dataclass(frozen=True)
class BatchSpec:
    """Composition of one hybrid batch.  Rows 0..C-1 are the chunk at positions offset..offset+C-1 of
    a prompt of prompt_len tokens; row C+i is decode i at position decode_len[i] (its cache already
    holds decode_len[i] entries).  decode_lens fixes the lengths; otherwise they are drawn uniformly
    from the closed range decode_len_range."""
    chunk_len: int
    chunk_offset: int
    prompt_len: int
    n_decodes: int
    decode_lens: Optional[Tuple[int, ...]] = None
    decode_len_range: Optional[Tuple[int, int]] = None


@dataclass(frozen=True)
class MultiSpec:
    """Composition of one token-budget batch: `budget` tokens go to the decodes first, then to prefill
    chunks cut from `prompts` in order (each (prompt_len, tokens already prefilled); a partially
    prefilled prompt is listed first), the stall-free step composition of the Sarathi-Serve notes.
    Decode lengths as in BatchSpec."""
    budget: int
    prompts: Tuple[Tuple[int, int], ...]
    n_decodes: int
    decode_lens: Optional[Tuple[int, ...]] = None
    decode_len_range: Optional[Tuple[int, int]] = None


def budget_batch(budget: int, n_decodes: int, prompts: Sequence[Tuple[int, int]]):
    """One step of token-budget batching (junupark.xyz notes on Sarathi-Serve, "Stall Free Batching"):
    the decodes are taken first, one token each; then each prompt in order gets
    min(remaining budget, its remaining tokens), until the budget is spent.  Returns (decodes taken,
    [(prompt index, chunk length, chunk offset)])."""
    n_dec = min(n_decodes, budget)
    left = budget - n_dec
    chunks = []
    for i, (plen, done) in enumerate(prompts):
        if left <= 0:
            break
        n = min(left, plen - done)
        if n > 0:
            chunks.append((i, n, done))
            left -= n
    return n_dec, chunks


SHAPES = {
    "tiny": LayerShape("tiny-llama", "llama", 256, 4, 64, 688, "f32", 1e-6, 10000.0, None),
    "llama13b": LayerShape("llama-13b", "llama", 5120, 40, 128, 13824, "bf16", 1e-6, 10000.0, 0.02),
    "llama33b": LayerShape("llama-33b", "llama", 6656, 52, 128, 17920, "bf16", 1e-6, 10000.0, 0.02),
    "gpt3tp8": LayerShape("gpt3-175b-tp8-shard", "gpt", 12288, 12, 128, 6144, "bf16", 1e-5, 10000.0, 0.02),
}


@dataclass(frozen=True)
class Workload:
    key: str
    shape: LayerShape
    batch: BatchSpec
    seed: int = 0
    note: str = ""
    page_size: Optional[int] = None   # caches laid out in a page pool of this many tokens per page


WORKLOADS = {
    # Tiny fp32 layer; the 128-token prompt runs as 4 chunks of 32 (see tiny_schedule); this entry is
    # the first of those steps.
    "tiny": Workload("tiny", SHAPES["tiny"], BatchSpec(32, 0, 128, 4, decode_lens=(17, 33, 64, 100))),
    "llama13b": Workload("llama13b", SHAPES["llama13b"],
                         BatchSpec(256, 768, 1024, 18, decode_lens=(1024,) * 18)),
    "llama33b": Workload("llama33b", SHAPES["llama33b"],
                         BatchSpec(512, 0, 512, 32, decode_len_range=(256, 2048))),
    "gpt3tp8": Workload("gpt3tp8", SHAPES["gpt3tp8"],
                        BatchSpec(256, 0, 256, 64, decode_lens=(2048,) * 64)),
    "llama13b_long": Workload("llama13b_long", SHAPES["llama13b"],
                              BatchSpec(512, 7680, 8192, 48, decode_len_range=(2048, 8192))),
    # The llama13b batch with every cache in one pool of 16-token pages (shuffled page order).
    "llama13b_paged": Workload("llama13b_paged", SHAPES["llama13b"],
                               BatchSpec(256, 768, 1024, 18, decode_lens=(1024,) * 18), page_size=16),
    # Token-budget batch: 512 tokens = 18 decodes + the last 94 tokens of a 1024-token prompt + a whole
    # 300-token prompt + the first 100 tokens of a new 1024-token prompt.
    "llama13b_budget": Workload("llama13b_budget", SHAPES["llama13b"],
                                MultiSpec(512, ((1024, 930), (300, 0), (1024, 0)), 18,
                                          decode_lens=(1024,) * 18)),
}


def chunks_of(batch: dict):
    """The prefill chunks of a generated batch as a list of dicts (len, offset, k, v), whichever kind
    of batch it is (one chunk: chunk_len / chunk_offset / chunk_k / chunk_v; several: chunks)."""
    if "chunks" in batch:
        return list(batch["chunks"])
    if batch["chunk_len"]:
        return [{"len": batch["chunk_len"], "offset": batch["chunk_offset"], "k": batch["chunk_k"],
                 "v": batch["chunk_v"]}]
    return []


def paginate(caches, page_size: int, seed: int = 0, extra_pages: int = 0, fill: float = 0.0):
    """Lay requests' caches out in a page pool (input preparation for the paged-KV path).

    caches: list of (K, V) arrays [nh, cap_i, d].  Request i gets ceil(cap_i / page_size) pages, at
    pool positions drawn from a seeded random permutation (so logically adjacent pages are scattered);
    extra_pages unused pages are added to the pool.  Slots past cap_i in a request's last page, and
    unused pages, hold `fill`.  Returns (k_pool, v_pool, tables): pools [n_pages, nh, page_size, d],
    tables a list of int32 arrays (request i's logical page -> pool page)."""
    nh, d = caches[0][0].shape[0], caches[0][0].shape[2]
    counts = [-(-k.shape[1] // page_size) for k, _ in caches]
    n_pages = sum(counts) + extra_pages
    perm = np.random.default_rng(seed).permutation(n_pages).astype(np.int32)
    kp = np.full((n_pages, nh, page_size, d), fill, np.float32)
    vp = np.full((n_pages, nh, page_size, d), fill, np.float32)
    tables, start = [], 0
    for (k, v), n in zip(caches, counts):
        t = perm[start:start + n]
        start += n
        for i, page in enumerate(t):
            rows = slice(i * page_size, min((i + 1) * page_size, k.shape[1]))
            m = rows.stop - rows.start
            kp[page, :, :m, :] = k[:, rows, :]
            vp[page, :, :m, :] = v[:, rows, :]
        tables.append(t.copy())
    return kp, vp, tables


def workload(key: str, **batch_changes) -> Workload:
    """A named workload, optionally with fields of its BatchSpec replaced (sweep points)."""
    w = WORKLOADS[key]
    if batch_changes:
        w = dataclasses.replace(w, batch=dataclasses.replace(w.batch, **batch_changes))
    return w


def sweep_changes(key: str) -> List[dict]:
    """The C or B sweep a workload is measured on, as BatchSpec field changes: chunk length C for
    llama33b (tile quantization: with its 32 decodes C = 257 is one row into a new 32-row step, C = 544
    fills the 576 rows of one round of GEMM workgroups and C = 545 is one row past it), the number of piggybacked decodes B for
    gpt3tp8 (the P:D sweep) and llama13b."""
    b = WORKLOADS[key].batch
    if key == "llama33b":
        return [dict(chunk_len=c, prompt_len=max(c, b.chunk_offset + c)) for c in (128, 256, 257, 512, 544, 545)]
    if key == "gpt3tp8":
        return [dict(n_decodes=n, decode_lens=(2048,) * n) for n in (1, 2, 4, 8, 16, 32, 64)]
    if key == "llama13b":
        return [dict(n_decodes=n, decode_lens=(1024,) * n) for n in (1, 4, 8, 18, 32, 64)]
    return []


def sweep(key: str) -> List[Workload]:
    """Sweep points of a workload: the hybrid batch, its chunk-only (B=0) and decode-only (C=0) parts,
    and the C or B sweep the workload is measured on."""
    w = WORKLOADS[key]
    b = w.batch
    pts: List[Workload] = [w, workload(key, n_decodes=0, decode_lens=() if b.decode_lens else None),
                           workload(key, chunk_len=0)]
    pts += [workload(key, **ch) for ch in sweep_changes(key)]
    return pts


# ----------------------------------------------------------------------------------------------
# bfloat16 rounding of the drawn values (input preparation only)
# ----------------------------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit patterns (uint16) of x rounded to bfloat16 with round-to-nearest-even.  x must be finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """x rounded to the nearest bfloat16 (ties to even), returned as float32."""
    b = bf16_bits(x).astype(np.uint32) << 16
    return b.view(np.float32).reshape(np.shape(x))


_BLOCK = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))


class Draws:
    """The ordered child streams of one workload seed."""

    def __init__(self, seed: int):
        self._root = np.random.SeedSequence(seed)

    def next(self) -> np.random.SeedSequence:
        return self._root.spawn(1)[0]

    def generator(self) -> np.random.Generator:
        return np.random.Generator(np.random.PCG64(self.next()))


def as_draws(rng) -> Draws:
    """A Draws from a Draws, an int seed, or a numpy Generator (which supplies the seed)."""
    if isinstance(rng, Draws):
        return rng
    if isinstance(rng, np.random.Generator):
        return Draws(int(rng.integers(0, 2 ** 63 - 1)))
    return Draws(int(rng))


# Where _normal draws: None = host numpy arrays (PCG64 blocks, as described above); a torch device
# string = tensors drawn on that device (see generate(..., device=...)).
_DEVICE = None


def _normal_device(seq: np.random.SeedSequence, shape, std: float, dtype: str):
    """N(0, std^2) values drawn on _DEVICE by torch's generator, seeded from the tensor's stream; stored
    as bfloat16 (round to nearest even) for the bf16 workloads, else float32."""
    import torch
    g = torch.Generator(device=_DEVICE)
    g.manual_seed(int(seq.generate_state(1, np.uint64)[0] >> np.uint64(1)))
    t = torch.randn(tuple(int(v) for v in shape), generator=g, device=_DEVICE, dtype=torch.float32)
    if std != 1.0:
        t *= std
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _normal(draws: Draws, shape, std: float, dtype: str) -> np.ndarray:
    """float32 N(0, std^2) values of the given shape from the next stream, bf16-rounded if asked."""
    if _DEVICE is not None:
        return _normal_device(draws.next(), shape, std, dtype)
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    seeds = draws.next().spawn(max(1, -(-n // _BLOCK)))

    def fill(i):
        seg = out[i * _BLOCK:(i + 1) * _BLOCK]
        np.random.Generator(np.random.PCG64(seeds[i])).standard_normal(out=seg, dtype=np.float32)
        if std != 1.0:
            seg *= np.float32(std)
        if dtype == "bf16":
            seg[:] = bf16_round(seg)

    if len(seeds) == 1:
        fill(0)
    else:
        with _cf.ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(len(seeds))))
    return out.reshape(shape)


def make_weights(shape: LayerShape, rng) -> dict:
    """Layer weights, each stored [out_features, in_features] (y = x @ W.T).  W_qkv's rows are
    [Q | K | V], each block head-major.  Norm gains are 1 and biases 0 (none are drawn).
    rng: a Draws (or a seed)."""
    rng = as_draws(rng)
    h, a, f = shape.hidden, shape.attn_width, shape.ffn

    def std(fan_in):
        return shape.w_std if shape.w_std is not None else 1.0 / np.sqrt(fan_in)

    w = {}
    w["w_qkv"] = _normal(rng, (3 * a, h), std(h), shape.dtype)
    w["w_o"] = _normal(rng, (h, a), std(a), shape.dtype)
    w["w_gate"] = _normal(rng, (f, h), std(h), shape.dtype) if shape.gated else None
    w["w_up"] = _normal(rng, (f, h), std(h), shape.dtype)
    w["w_down"] = _normal(rng, (h, f), std(f), shape.dtype)
    w["norm1_w"] = np.ones(h, np.float32)
    w["norm2_w"] = np.ones(h, np.float32)
    w["norm1_b"] = np.zeros(h, np.float32) if shape.arch == "gpt" else None
    w["norm2_b"] = np.zeros(h, np.float32) if shape.arch == "gpt" else None
    return w


def _cache(draws: Draws, shape: LayerShape, cap: int, filled: int, fill_rest: float):
    """One request's K and V caches, each [n_heads, cap, head_dim]; slots 0..filled-1 hold N(0,1)
    draws (K from one stream, then V from the next), the remaining slots hold fill_rest."""
    nh, d = shape.n_heads, shape.head_dim
    out = []
    for _ in range(2):
        vals = _normal(draws, (nh, filled, d), 1.0, shape.dtype) if filled else None
        if filled == cap:
            c = vals
        elif _DEVICE is not None:
            import torch
            c = torch.full((nh, cap, d), fill_rest, device=_DEVICE,
                           dtype=torch.bfloat16 if shape.dtype == "bf16" else torch.float32)
            if filled:
                c[:, :filled, :] = vals
        else:
            c = np.empty((nh, cap, d), np.float32)
            c[:, filled:, :] = fill_rest
            if filled:
                c[:, :filled, :] = vals
        out.append(c)
    return out[0], out[1]


def make_batch(shape: LayerShape, spec: BatchSpec, rng, fill_rest: float = 0.0) -> dict:
    """Hidden states and caches of one hybrid batch (drawn after the weights from the same rng).

    The chunk request's cache has capacity prompt_len (at least offset+C) and holds N(0,1) entries in
    its prefix slots 0..offset-1.  Decode i's cache has capacity decode_len[i]+1 and holds N(0,1)
    entries in slots 0..decode_len[i]-1.  Unwritten slots hold fill_rest (tests use NaN there to
    catch reads past a request's keys).  rng: the Draws the weights came from (or a seed)."""
    rng = as_draws(rng)
    C, B = spec.chunk_len, spec.n_decodes
    x = _normal(rng, (C + B, shape.hidden), 1.0, shape.dtype)
    cap = max(spec.prompt_len, spec.chunk_offset + C, 1)
    ck, cv = _cache(rng, shape, cap, spec.chunk_offset, fill_rest)
    lens = _decode_lens(spec, rng, B)
    dk, dv = [], []
    for L in lens:
        k, v = _cache(rng, shape, L + 1, L, fill_rest)
        dk.append(k)
        dv.append(v)
    return {"x": x, "chunk_len": C, "chunk_offset": spec.chunk_offset, "chunk_k": ck, "chunk_v": cv,
            "decode_len": lens, "decode_k": dk, "decode_v": dv}


def _decode_lens(spec, rng: Draws, B: int) -> List[int]:
    if spec.decode_lens is not None:
        lens = list(spec.decode_lens)[:B]
        assert len(lens) == B, "decode_lens must list one length per decode"
        return lens
    if B:
        lo, hi = spec.decode_len_range
        return [int(v) for v in rng.generator().integers(lo, hi, size=B, endpoint=True)]
    return []


def make_multi_batch(shape: LayerShape, spec: MultiSpec, rng, fill_rest: float = 0.0) -> dict:
    """Hidden states and caches of one token-budget batch (drawn after the weights).  The chunks come
    from budget_batch; chunk j's request has a cache of capacity prompt_len holding N(0,1) entries in
    its already-prefilled slots; decodes as in make_batch.  Draw order: X, each chunk's cache (K then
    V) in chunk order, the decode lengths, each decode cache."""
    rng = as_draws(rng)
    B, picked = budget_batch(spec.budget, spec.n_decodes, spec.prompts)
    C = sum(n for _, n, _ in picked)
    x = _normal(rng, (C + B, shape.hidden), 1.0, shape.dtype)
    chunks = []
    for i, n, off in picked:
        k, v = _cache(rng, shape, spec.prompts[i][0], off, fill_rest)
        chunks.append({"len": n, "offset": off, "k": k, "v": v})
    lens = _decode_lens(spec, rng, B)
    dk, dv = [], []
    for L in lens:
        k, v = _cache(rng, shape, L + 1, L, fill_rest)
        dk.append(k)
        dv.append(v)
    return {"x": x, "chunks": chunks, "decode_len": lens, "decode_k": dk, "decode_v": dv}


def generate(w: Workload, fill_rest: float = 0.0, device: Optional[str] = None) -> Tuple[dict, dict]:
    """(weights, batch) of a workload, drawn from its seed in the fixed order.

    device=None: host numpy float32 arrays (bf16-rounded values for the bf16 workloads), the inputs
    of the parity tests.  device='cuda' (throughput runs): the same streams in the same order, but
    every normal tensor is drawn on the GPU by torch's generator seeded from its stream and kept in
    the storage type (bfloat16 or float32); lengths and compositions are the same as on the host,
    the values are not.  Norm gains and biases stay host arrays in both cases."""
    global _DEVICE
    rng = Draws(w.seed)
    _DEVICE = device
    try:
        weights = make_weights(w.shape, rng)
        if isinstance(w.batch, MultiSpec):
            batch = make_multi_batch(w.shape, w.batch, rng, fill_rest)
        else:
            batch = make_batch(w.shape, w.batch, rng, fill_rest)
    finally:
        _DEVICE = None
    return weights, batch


def tiny_schedule(seed: int = 0, n_chunks: int = 4, chunk: int = 32,
                  decode_lens: Sequence[int] = (17, 33, 64, 100), fill_rest: float = 0.0):
    """The tiny fp32 workload as a sequence of hybrid steps over one 128-token prompt.

    Step k holds prompt rows k*chunk..k*chunk+chunk-1 (chunk offset k*chunk) plus the same decodes at
    lengths decode_lens[i]+k, each with a fresh N(0,1) hidden row per step.  The prompt cache starts
    empty (the layer fills it chunk by chunk); decode caches start with decode_lens[i] N(0,1)
    entries and capacity decode_lens[i]+n_chunks.

    Returns (shape, weights, prompt_x [n_chunks*chunk, H], decode_x [n_chunks, B, H],
    decode_k, decode_v, decode_lens)."""
    shape = SHAPES["tiny"]
    rng = Draws(seed)
    weights = make_weights(shape, rng)
    prompt_x = _normal(rng, (n_chunks * chunk, shape.hidden), 1.0, shape.dtype)
    dk, dv = [], []
    for L in decode_lens:
        k, v = _cache(rng, shape, L + n_chunks, L, fill_rest)
        dk.append(k)
        dv.append(v)
    decode_x = _normal(rng, (n_chunks, len(decode_lens), shape.hidden), 1.0, shape.dtype)
    return shape, weights, prompt_x, decode_x, dk, dv, list(decode_lens)
