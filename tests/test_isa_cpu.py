"""ISA-level checks of the gfx950 kernels on the CPU (compiles every kernel source to assembly).

- No flat memory instructions: every device pointer the kernels touch is a global-memory pointer,
  and flat accesses would also tie the LDS wait counter to global memory traffic (the LDS-DMA loops
  wait on that counter).
- No writes through the scalar data cache (scalar stores, scalar atomics, scalar cache write-back):
  all stores are vector stores.
- No register spills or scratch memory in any kernel, and the attention kernels within the register
  budgets of the occupancy they are tuned for.
"""
import os
import re
import subprocess
import tempfile

import pytest

from chunked_prefill_hybrid_amd import build

CLANG = "/opt/rocm/lib/llvm/bin/clang++"
FORBIDDEN_SCALAR = re.compile(r"^\s*s_(store|buffer_store|atomic|buffer_atomic|dcache_wb|scratch_store)", re.M)
FLAT = re.compile(r"^\s*flat_(load|store|atomic)", re.M)


def _asm(src):
    with tempfile.TemporaryDirectory() as td:
        out = os.path.join(td, "k.s")
        cmd = [CLANG, *build.COMMON, "--cuda-device-only", "-x", "hip", "-S", src, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


@pytest.fixture(scope="module")
def listings():
    if not os.path.exists(CLANG):
        pytest.skip("no ROCm compiler")
    return {os.path.basename(s): _asm(s) for s in build.sources() if s.endswith(".hip")}


def test_no_flat_memory_instructions(listings):
    bad = {k: len(FLAT.findall(v)) for k, v in listings.items() if FLAT.search(v)}
    assert not bad, f"flat memory instructions in {bad}"


def test_no_scalar_cache_writes(listings):
    bad = {k: FORBIDDEN_SCALAR.findall(v)[:3] for k, v in listings.items() if FORBIDDEN_SCALAR.search(v)}
    assert not bad, f"scalar-cache writes in {bad}"


def _kernels(listing):
    """(name, metadata dict) of every kernel in an assembly listing's amdhsa.kernels block."""
    md = listing[listing.index("amdhsa.kernels:"):]
    out = []
    for blk in md.split("\n  - ")[1:]:
        name = re.search(r"\.name:\s+(\S+)", blk)
        if not name or not re.search(r"\.vgpr_count:", blk):
            continue
        field = lambda k: int(re.search(r"\.%s:\s+(\d+)" % k, blk).group(1))
        out.append((name.group(1), {k: field(k) for k in ("vgpr_count", "agpr_count", "vgpr_spill_count",
                                                          "private_segment_fixed_size")}))
    return out


def test_no_register_spills(listings):
    bad = [(src, n[:80]) for src, v in listings.items() for n, m in _kernels(v)
           if m["vgpr_spill_count"] or m["private_segment_fixed_size"]]
    assert not bad, f"kernels with spills or scratch memory: {bad}"


def test_attention_register_budgets(listings):
    """The occupancy the attention kernels are tuned for: the split-KV kernel at four 256-thread
    workgroups per compute unit (at most 128 registers per lane), the chunk kernel at two (256)."""
    split = [(n, m) for n, m in _kernels(listings["attn_rows.hip"]) if "attn_rows_split" in n]
    chunk = [(n, m) for n, m in _kernels(listings["attn_chunk.hip"]) if "attn_chunk_mfma" in n]
    assert split and chunk
    for n, m in split:
        assert m["vgpr_count"] + m["agpr_count"] <= 128, (n, m)
    for n, m in chunk:
        assert m["vgpr_count"] + m["agpr_count"] <= 256, (n, m)
