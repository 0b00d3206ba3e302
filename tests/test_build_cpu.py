"""Build-level checks on the CPU: every gfx950 kernel compiles without per-lane scratch memory.

A register spill would put scratch loads into the LDS-DMA loops of the GEMM and chunk-attention
kernels, and every scratch access makes the wave wait for all of its outstanding global loads, which
drains the load pipeline those loops rely on.  The per-kernel figures come from the compiler's
resource-usage remarks, recorded by the build in _build/kernel_resources.json."""
import json
import os

from chunked_prefill_hybrid_amd import build


def _resources():
    srcs = build.sources()
    stale = (not os.path.exists(build.RESOURCES) or
             os.path.getmtime(build.RESOURCES) < max(os.path.getmtime(s) for s in srcs))
    if stale:
        build.build()
    with open(build.RESOURCES) as f:
        return json.load(f)


def test_no_kernel_uses_scratch():
    res = _resources()
    assert len(res) > 20, "resource remarks missing"
    spilled = {k: v for k, v in res.items() if v.get("ScratchSize", 0) != 0}
    assert not spilled, f"kernels with scratch: {spilled}"


def test_hot_kernels_fit_their_occupancy_targets():
    """The GEMM runs 8 waves (2 per SIMD) per workgroup, the chunk attention two 4-wave workgroups
    per CU and the split-KV decode attention four: their register budgets must allow that."""
    res = _resources()
    gemm = {k: v for k, v in res.items() if "gemm_bf16_rows" in k}
    chunk = {k: v for k, v in res.items() if "attn_chunk_mfma" in k}
    split = {k: v for k, v in res.items() if "attn_rows_split" in k}
    assert gemm and chunk and split
    assert all(v["Occupancy"] >= 4 for v in split.values()), split
    assert all(v["Occupancy"] >= 2 for v in gemm.values()), gemm
    assert len(chunk) == 6, chunk   # d in {64, 128} x (contiguous: one or two query blocks; paged: one)
    assert all(v["Occupancy"] >= 2 for v in chunk.values()), chunk
