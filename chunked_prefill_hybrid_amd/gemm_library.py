"""The ROCm BLAS library's GEMM on the layer's four projection shapes, as a reference point.

Times torch.matmul (bf16 in, bf16 out, float32 accumulation; on ROCm it dispatches to hipBLASLt) for
the QKV, O, gate|up and down products of a workload's layer at its batch row count T, with three
weight replicas rotated so that the 256 MB last-level cache cannot hold a product's weights, as in
bench.py.  The library computes the plain product only: the layer's own gate/up stage also applies
SiLU * up, and its split-K stages write float32 partials that the next kernel sums.

    python -m chunked_prefill_hybrid_amd.gemm_library --workload llama13b
"""
from __future__ import annotations

import argparse
import json
import sys


def shapes(shape):
    """(name, N, K) of the layer's products; the gated FFN's gate and up weights as one product."""
    H, A, F = shape.hidden, shape.attn_width, shape.ffn
    up_n = 2 * F if shape.arch == "llama" else F
    return [("qkv", 3 * A, H), ("o", H, A), ("ffn_up", up_n, H), ("ffn_down", H, F)]


def batch_rows(work) -> int:
    """C + B of a workload's batch (a token-budget batch: its budget, decodes first)."""
    b = work.batch
    if hasattr(b, "budget"):
        return b.budget
    return b.chunk_len + b.n_decodes


def main(argv=None) -> int:
    import torch

    from . import workloads as wl

    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama13b")
    ap.add_argument("--reps", type=int, default=60)
    ap.add_argument("--replicas", type=int, default=3)
    ap.add_argument("--json", default=None)
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        raise SystemExit("gemm_library needs a GPU")
    work = wl.workload(args.workload)
    shape = work.shape
    if shape.dtype != "bf16":
        raise SystemExit("gemm_library compares bf16 products only")
    T = batch_rows(work)
    torch.manual_seed(0)
    out = {"workload": args.workload, "rows": T, "gemms": {}}
    print(f"torch.matmul (hipBLASLt), {args.workload}: T = {T} rows, {args.replicas} weight replicas")
    for name, N, K in shapes(shape):
        a = torch.randn(T, K, device="cuda", dtype=torch.bfloat16)
        ws = [torch.randn(N, K, device="cuda", dtype=torch.bfloat16) for _ in range(args.replicas)]
        for i in range(10):
            a @ ws[i % args.replicas].t()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.reps):
            a @ ws[i % args.replicas].t()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.reps
        flops = 2.0 * T * N * K
        tflops = flops / us / 1e6
        out["gemms"][name] = {"n": N, "k": K, "avg_us": round(us, 2), "tflops": round(tflops, 1)}
        print(f"  {name:8s} N={N:6d} K={K:6d}  {us:7.1f} us  {tflops:6.0f} TFLOP/s "
              f"({100 * tflops / 2500:4.1f}% of dense bf16 peak)", flush=True)
        del ws, a
    if args.json:
        with open(args.json, "w") as f:
            json.dump(out, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
