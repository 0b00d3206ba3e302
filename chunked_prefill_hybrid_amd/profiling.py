"""Hardware-counter runs of the layer forward, and their summary.

Run mode (under rocprofv3 --pmc): runs a workload's hybrid-batch forward `--steps` times after a short
warmup, then one device-to-device copy of `--copy-mib` MiB.  The copy reads and writes a known number
of bytes, so the FETCH_SIZE and WRITE_SIZE counts of its dispatch calibrate the byte counters of the
layer's kernels.

    rocprofv3 --pmc FETCH_SIZE -d <dir> -o run --output-format csv -- \\
        python -m chunked_prefill_hybrid_amd.profiling --workload llama13b --steps 20

Summary mode (CPU only): reads the two counter CSVs, scales each kernel's average per-dispatch count
by the copy's calibration factor, prints a markdown table, and records the bytes per launch of one
stage's kernel in a JSON file keyed "<workload>:<stage>" together with a hash of the sources that
kernel is compiled from, so that a reader can tell when the figure no longer describes the code.

    python -m chunked_prefill_hybrid_amd.profiling summarize --fetch <fetch.csv> --write <write.csv> \\
        --workload llama13b --stage ffn_up --kernel 'gemm_bf16_rows<4, 9, 2>' --json profiles/traffic.json
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def kernel_source_hash(files=None) -> str:
    """SHA-1 (12 hex digits) over the HIP/C++ sources (all of them, or the named ones), in file-name
    order."""
    h = hashlib.sha1()
    paths = sorted(glob.glob(os.path.join(CSRC, "*"))) if files is None else \
        sorted(os.path.join(CSRC, f) for f in files)
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:12]


# The sources each stage's kernels are compiled from: a stage's traffic record stays valid while
# these files are unchanged.
_GEMM_SOURCES = ("common.h", "gemm.hip", "kernels.h")
STAGE_SOURCES = {
    "qkv": _GEMM_SOURCES, "o": _GEMM_SOURCES, "ffn_up": _GEMM_SOURCES, "ffn_down": _GEMM_SOURCES,
    "attn_decode": ("attn_chunk_body.h", "attn_rows.hip", "common.h", "kernels.h"),
    "attn_chunk": ("attn_chunk.hip", "attn_chunk_body.h", "common.h", "kernels.h"),
}


def stage_source_hash(stage) -> str:
    """Hash of the sources of one stage's kernels (all sources for a stage not listed)."""
    return kernel_source_hash(STAGE_SOURCES.get(stage))


def run(argv) -> int:
    import numpy as np
    import torch

    from . import _abi
    from . import layer as hl
    from . import workloads as wl

    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama13b")
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--copy-mib", type=int, default=512)
    args = ap.parse_args(argv)
    torch.cuda.set_device(0)
    wk = wl.workload(args.workload)
    shape = wk.shape
    weights, batch = wl.generate(wk, device="cuda")
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32

    def dev(a, t=dt):
        if isinstance(a, torch.Tensor):
            return a.to(t)
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(t)

    wdev = {k: dev(v, torch.float32 if k.startswith("norm") else dt) for k, v in weights.items() if v is not None}
    chunks = wl.chunks_of(batch)
    lens = list(batch["decode_len"])
    T = sum(c["len"] for c in chunks) + len(lens)
    layer = hl.HybridLayer(shape, wdev, max_tokens=T,
                           max_pos=max([c["offset"] + c["len"] for c in chunks] + [L + 1 for L in lens]))
    x = dev(batch["x"])
    y = torch.empty_like(x)
    ckv = [(dev(c["k"]), dev(c["v"])) for c in chunks]
    dkv = [(dev(k), dev(v)) for k, v in zip(batch["decode_k"], batch["decode_v"])]
    if "chunks" in batch:
        b, keep = layer.multi_batch(x, y, [(c["len"], c["offset"], kv) for c, kv in zip(chunks, ckv)], dkv, lens)
        fwd = _abi.sarathi_multi_forward
    else:
        b, keep = layer.batch(x, y, batch["chunk_len"], batch["chunk_offset"], ckv[0] if ckv else None, dkv, lens)
        fwd = _abi.sarathi_layer_forward
    ws = torch.empty(layer.workspace_size(b), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(args.warmup + args.steps):
        fwd(layer.handle, b, ws.data_ptr(), ws.numel(), stream)
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


def _short(name: str) -> str:
    name = re.sub(r"^void ", "", name)
    name = name.replace("sarathi::(anonymous namespace)::", "")
    return re.sub(r"\(.*", "", name)


def _per_kernel(path: str, counter: str):
    """{short kernel name: [per-dispatch values]} for one counter of a rocprofv3 counter CSV."""
    out = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return out


def summarize(argv) -> int:
    ap = argparse.ArgumentParser(prog="profiling summarize")
    ap.add_argument("--fetch", required=True, help="counter CSV of the FETCH_SIZE run")
    ap.add_argument("--write", required=True, help="counter CSV of the WRITE_SIZE run")
    ap.add_argument("--copy-mib", type=int, default=512)
    ap.add_argument("--workload", default="llama13b")
    ap.add_argument("--stage", default=None)
    ap.add_argument("--kernel", default=None, help="short kernel name of --stage")
    ap.add_argument("--json", default=None, help="traffic record file to update")
    args = ap.parse_args(argv)
    fetch = _per_kernel(args.fetch, "FETCH_SIZE")
    write = _per_kernel(args.write, "WRITE_SIZE")
    copy_bytes = float(args.copy_mib << 20)

    def calib(table, name):
        copies = [v for k, vs in table.items() if "copyBuffer" in k or "copy" in k.lower() for v in vs]
        if not copies:
            raise SystemExit(f"no copy dispatch found in the {name} CSV")
        return copy_bytes / (max(copies) * 1024.0)

    f_fetch, f_write = calib(fetch, "FETCH_SIZE"), calib(write, "WRITE_SIZE")
    print(f"calibration: {args.copy_mib} MiB copy -> FETCH_SIZE factor {f_fetch:.3f}, "
          f"WRITE_SIZE factor {f_write:.3f}\n")
    print("| kernel | dispatches | fetch MB/launch | write MB/launch |\n|---|---|---|---|")
    rec = None
    for k in sorted(set(fetch) | set(write), key=lambda k: -(sum(fetch.get(k, [0])) / max(1, len(fetch.get(k, [1]))))):
        fv, wv = fetch.get(k, []), write.get(k, [])
        fb = sum(fv) / len(fv) * 1024.0 * f_fetch if fv else 0.0
        wb = sum(wv) / len(wv) * 1024.0 * f_write if wv else 0.0
        print(f"| `{k}` | {len(fv)} | {fb / 1e6:.1f} | {wb / 1e6:.1f} |")
        if args.kernel and k == args.kernel:
            rec = {"kernel": k, "bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb),
                   "write_bytes": round(wb), "fetch_factor": round(f_fetch, 4),
                   "write_factor": round(f_write, 4), "source_hash": stage_source_hash(args.stage),
                   "sources": list(STAGE_SOURCES.get(args.stage, ["*"]))}
    if args.json and args.stage:
        if rec is None:
            raise SystemExit(f"kernel {args.kernel!r} not in the CSVs")
        data = {}
        if os.path.exists(args.json):
            with open(args.json) as f:
                data = json.load(f)
        data[f"{args.workload}:{args.stage}"] = rec
        with open(args.json, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
            f.write("\n")
        print(f"\nrecorded {args.workload}:{args.stage} -> {rec['bytes_per_launch'] / 1e6:.1f} MB/launch")
    return 0


def main(argv=None) -> int:
    argv = list(sys.argv[1:] if argv is None else argv)
    if argv and argv[0] == "summarize":
        return summarize(argv[1:])
    return run(argv)


if __name__ == "__main__":
    sys.exit(main())
