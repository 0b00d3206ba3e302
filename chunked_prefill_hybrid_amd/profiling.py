"""Driver for hardware-counter runs of the layer forward (use under rocprofv3 --pmc).

Runs a workload's hybrid-batch forward `--steps` times (after a short warmup), then one device-to-
device copy of `--copy-mib` MiB.  The copy reads and writes a known number of bytes, so the FETCH_SIZE
and WRITE_SIZE counts of its dispatch calibrate the byte counters of the layer's kernels.

    rocprofv3 --pmc FETCH_SIZE -d <dir> -o run --output-format csv -- \\
        python -m chunked_prefill_hybrid_amd.profiling --workload llama13b --steps 20
"""
from __future__ import annotations

import argparse
import sys

import numpy as np
import torch

from . import _abi
from . import layer as hl
from . import workloads as wl


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama13b")
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--copy-mib", type=int, default=512)
    args = ap.parse_args(argv)
    torch.cuda.set_device(0)
    wk = wl.workload(args.workload)
    shape = wk.shape
    weights, batch = wl.generate(wk)
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32

    def dev(a, t=dt):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(t)

    wdev = {k: dev(v, torch.float32 if k.startswith("norm") else dt) for k, v in weights.items() if v is not None}
    C, off, lens = batch["chunk_len"], batch["chunk_offset"], list(batch["decode_len"])
    layer = hl.HybridLayer(shape, wdev, max_tokens=C + len(lens),
                           max_pos=max([off + C] + [L + 1 for L in lens]))
    x = dev(batch["x"])
    y = torch.empty_like(x)
    ckv = (dev(batch["chunk_k"]), dev(batch["chunk_v"])) if C else None
    dkv = [(dev(k), dev(v)) for k, v in zip(batch["decode_k"], batch["decode_v"])]
    b, keep = layer.batch(x, y, C, off, ckv, dkv, lens)
    ws = torch.empty(layer.workspace_size(b), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(args.warmup + args.steps):
        _abi.sarathi_layer_forward(layer.handle, b, ws.data_ptr(), ws.numel(), stream)
    torch.cuda.synchronize()
    n = args.copy_mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"profiling run done: {args.workload}, {args.warmup}+{args.steps} forwards, "
          f"copy of {args.copy_mib} MiB", flush=True)
    layer.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
