"""ISA-level checks of the gfx950 kernels on the CPU (compiles every kernel source to assembly).

- No flat memory instructions: every device pointer the kernels touch is a global-memory pointer,
  and flat accesses would also tie the LDS wait counter to global memory traffic (the LDS-DMA loops
  wait on that counter).
- No writes through the scalar data cache (scalar stores, scalar atomics, scalar cache write-back):
  all stores are vector stores.
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

