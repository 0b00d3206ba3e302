"""Tile/wave-quantization sweep of the layer's GEMMs on MI355X.

The SARATHI page ("Identifying the Ideal Chunk Size", Figure 7) shows the linear ops' time jumping when
the number of batch rows crosses a multiple of the GPU's GEMM tile (128 on A100), and derives the rule
that the chunk size plus the decodes should fill whole tiles.  This module measures the same curve for
this library's kernels: it runs the layer on batches of T rows (a chunk of T tokens at offset 0, no
decodes) for T = t0..t1 and records the per-stage times of the four GEMMs (QKV, O, gate/up, down)
with the library's stage timer, in their layer configuration (split-K partials, fused SwiGLU).

    python -m chunked_prefill_hybrid_amd.tile_sweep --workload llama13b --t0 1 --t1 1024 \\
        --csv tile_sweep.csv

Prints one CSV line per T (stage averages in microseconds) and, at the end, the steps: the values of T
at which a stage's time rises by more than --step-frac over its time at T - 1.
"""
from __future__ import annotations

import argparse
import sys

GEMM_STAGES = ("qkv", "o", "ffn_up", "ffn_down")


def main(argv=None) -> int:
    import numpy as np
    import torch

    from . import _abi
    from . import layer as hl
    from . import workloads as wl

    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama13b", help="layer shape taken from this workload")
    ap.add_argument("--t0", type=int, default=1)
    ap.add_argument("--t1", type=int, default=1024)
    ap.add_argument("--stride", type=int, default=1)
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--step-frac", type=float, default=0.04)
    ap.add_argument("--csv", default=None)
    args = ap.parse_args(argv)
    torch.cuda.set_device(0)
    shape = wl.workload(args.workload).shape
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    rng = np.random.default_rng(0)
    w = wl.make_weights(shape, rng)
    wdev = {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda").to(torch.float32 if k.startswith("norm") else dt)
            for k, v in w.items() if v is not None}
    tmax = args.t1
    layer = hl.HybridLayer(shape, wdev, max_tokens=tmax, max_pos=tmax + 1)
    H, A = shape.hidden, shape.attn_width
    x = (torch.randn(tmax, H, device="cuda") ).to(dt)
    y = torch.empty_like(x)
    ck = torch.zeros(shape.n_heads, tmax, shape.head_dim, device="cuda", dtype=dt)
    cv = torch.zeros_like(ck)
    stream = torch.cuda.current_stream().cuda_stream
    mask = _abi.stage_mask(*GEMM_STAGES)
    ws = None
    rows = []
    out = open(args.csv, "w") if args.csv else None
    header = "T," + ",".join(GEMM_STAGES)
    print(header, flush=True)
    if out:
        out.write(header + "\n")
    for T in range(args.t0, args.t1 + 1, args.stride):
        b, keep = layer.batch(x[:T], y[:T], T, 0, (ck, cv), [], [])
        need = layer.workspace_size(b)
        if ws is None or ws.numel() < need:
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        for _ in range(args.warmup):
            _abi.sarathi_layer_forward(layer.handle, b, ws.data_ptr(), ws.numel(), stream)
        timer = _abi.sarathi_timer_create(args.reps, mask)
        for _ in range(args.reps):
            _abi.sarathi_layer_forward_timed(layer.handle, b, ws.data_ptr(), ws.numel(), stream, timer)
        st = _abi.sarathi_timer_read(timer)
        _abi.sarathi_timer_destroy(timer)
        vals = [st[s][0] / max(1, st[s][1]) * 1e3 for s in GEMM_STAGES]
        rows.append((T, vals))
        line = f"{T}," + ",".join(f"{v:.2f}" for v in vals)
        print(line, flush=True)
        if out:
            out.write(line + "\n")
    if out:
        out.close()
    print("steps (T at which a stage's time rises by more than "
          f"{100 * args.step_frac:.0f}% over T - {args.stride}):", flush=True)
    for i, s in enumerate(GEMM_STAGES):
        jumps = [f"{rows[k][0]} ({rows[k - 1][1][i]:.1f}->{rows[k][1][i]:.1f} us)"
                 for k in range(1, len(rows)) if rows[k][1][i] > rows[k - 1][1][i] * (1 + args.step_frac)]
        print(f"  {s}: " + (", ".join(jumps) if jumps else "none"), flush=True)
    layer.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
