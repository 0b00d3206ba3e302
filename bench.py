"""Throughput of the hybrid-batch decoder-layer forward on one MI355X.

One step = one forward of one decoder layer over one hybrid batch: a prefill chunk plus piggybacked
decodes (SARATHI: Efficient LLM Inference by Piggybacking Decodes with Chunked Prefills, section 3,
"Decode-Maximal Batching").  Default workload: LLaMA-13B layer shape in bf16, chunk C=256 at offset
768 of a 1024-token prompt plus B=18 decodes with 1024 cached entries each.  Inputs are seeded and
synthetic and already resident in HBM when timing starts.  Three replicas of the weights, caches and
activations are rotated step by step so that the 256 MB last-level cache cannot hold a step's data.

Passes: W warmup steps; a breakdown pass in which the library records HIP events around every stage
(this perturbs the step time, so it is not the timed region); then exactly K timed steps in which
events are recorded on the launch stream only around the dominant kernel's stage, giving that
kernel's live average duration for the roofline.  Prints ONE JSON line: tokens/s over the K timed
steps, the roofline of the dominant kernel, the per-stage breakdown, the layer's roofline fraction,
the piggybacking comparison (the same rows run as a chunk-only and a decode-only batch, giving the
marginal cost of a decode that rides with the chunk), and the CPU oracle's throughput on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "hybrid-batch layer tokens/s (chunk+decodes); % bf16 MFMA and HBM roofline"


from chunked_prefill_hybrid_amd.profiling import kernel_source_hash, stage_source_hash  # noqa: E402


def stage_work(shape, chunks, lens):
    """Algorithmic work of each stage: (flops, bytes).  chunks: [(len, offset)] of the batch's prefill
    chunks.  GEMM flops use the unpadded row count."""
    C = sum(n for n, _ in chunks)
    T = C + len(lens)
    H, A, F = shape.hidden, shape.attn_width, shape.ffn
    el = 2 if shape.dtype == "bf16" else 4
    up_n = 2 * F if shape.gated else F
    w = {
        "qkv": (2.0 * T * H * 3 * A, el * (3 * A * H + T * H + T * 3 * A)),
        "o": (2.0 * T * A * H, el * (H * A + T * A + T * H) + 4 * T * H),
        "ffn_up": (2.0 * T * H * up_n, el * (up_n * H + T * H + T * F)),
        "ffn_down": (2.0 * T * F * H, el * (H * F + T * F + T * H) + 4 * T * H),
        # decode attention streams each decode's K and V over its L_i + 1 keys, plus its query
        "attn_decode": (4.0 * A * sum(L + 1 for L in lens), el * sum(2 * A * (L + 1) + A for L in lens)),
        # each chunk reads its request's K/V over offset + len keys once, plus its q and output rows
        "attn_chunk": (sum(4.0 * A * (n * o + n * (n + 1) / 2) for n, o in chunks),
                       el * sum(2 * A * (o + n) + 2 * n * A for n, o in chunks)),
        "norm1": (0.0, el * 2 * T * H),
        "norm2": (0.0, (4 + el) * T * H),
        "rope_append": (0.0, el * 2 * T * 3 * A),
        "attn_merge": (0.0, 0.0),
    }
    return w


BOUND = {"qkv": "mfma", "o": "mfma", "ffn_up": "mfma", "ffn_down": "mfma", "attn_chunk": "mfma",
         "attn_decode": "hbm", "norm1": "hbm", "norm2": "hbm", "rope_append": "hbm", "attn_merge": "hbm"}


def roofline_entry(stage, avg_ms, flops, nbytes, dtype):
    bound = BOUND[stage]
    if bound == "mfma":
        achieved = flops / (avg_ms * 1e-3) / 1e12
        peak = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_F32_TFLOPS
        unit = "TFLOP/s"
    else:
        achieved = nbytes / (avg_ms * 1e-3) / 1e9
        peak = PEAK_HBM_GBS
        unit = "GB/s"
    e = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4)}
    if bound == "mfma" and nbytes > 0:
        # A contraction whose arithmetic intensity lies below the ridge point (peak flops / peak HBM
        # bandwidth, 312 FLOP/B for bf16) has the HBM line as its roofline ceiling: its algorithmic
        # bytes over the duration, against 8 TB/s, are reported beside the MFMA fraction.
        e["intensity"] = round(flops / nbytes, 1)
        e["hbm_frac"] = round(nbytes / (avg_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    return e


def load_traffic(stage, workload_key):
    """HBM bytes per launch measured by rocprofv3 counters for this kernel source, if recorded."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{workload_key}:{stage}")
    except Exception:
        return None
    if not rec or rec.get("source_hash") != stage_source_hash(stage):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(wk, weights, batch, budget_s=25.0, target_s=10.0):
    """The CPU oracle (as it is, float64 NumPy) on the full batch, repeated until about target_s of
    CPU work (at least 3 runs) while it stays within the time budget; BLAS threads capped at 16 (one
    GPU's share of host cores)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    cores = min(16, os.cpu_count() or 1)
    times = []
    with threadpool_limits(limits=cores, user_api="blas"):
        used = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            if "chunks" in batch:
                oracle.layer_forward_multi(wk.shape, weights, batch)
            else:
                oracle.layer_forward(wk.shape, weights, batch)
            times.append(time.perf_counter() - t0)
            spent = time.perf_counter() - t_start
            if spent + times[-1] > budget_s or (len(times) >= 3 and spent >= target_s):
                break
    T = batch["x"].shape[0]
    t = statistics.median(times)
    return {"value": round(T / t, 2), "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "sample": f"full batch ({T} rows, one layer, float64 NumPy), {len(times)} run(s), median {t:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama13b")
    ap.add_argument("--replicas", type=int, default=3)
    ap.add_argument("--page-size", type=int, default=None,
                    help="lay the caches out in a page pool with this many tokens per page "
                         "(overrides the workload's own layout; 0 = contiguous caches)")
    ap.add_argument("--batch", default=None,
                    help="replace fields of the workload's batch composition, a JSON object such as "
                         "'{\"n_decodes\": 4, \"decode_lens\": [2048, 2048, 2048, 2048]}' (sweep points)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the chunk-only / decode-only runs behind the decode-cost comparison")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build measures a single MI355X "
              f"(got --gpus {args.gpus}); multi-GPU sharding is described in the design notes.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from chunked_prefill_hybrid_amd import _abi
    from chunked_prefill_hybrid_amd import layer as hl
    from chunked_prefill_hybrid_amd import workloads as wl

    torch.cuda.set_device(0)
    changes = {k: tuple(v) if isinstance(v, list) else v for k, v in json.loads(args.batch or "{}").items()}
    wk = wl.workload(args.workload, **changes)
    if args.page_size is not None:
        wk = dataclasses.replace(wk, page_size=args.page_size or None)
    shape = wk.shape
    weights, batch = wl.generate(wk)
    chunks = wl.chunks_of(batch)            # [{len, offset, k, v}]: one chunk, several, or none
    multi = "chunks" in batch               # token-budget workloads use the several-chunk entry point
    lens = list(batch["decode_len"])
    C = sum(c["len"] for c in chunks)
    T = C + len(lens)
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32

    def dev(a, t=dt):
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(t)

    wdev = {k: dev(v, torch.float32 if k.startswith("norm") else dt) for k, v in weights.items() if v is not None}
    paged = wk.page_size is not None
    if paged:
        # every request's cache in one pool of fixed-size pages, in a shuffled page order
        caches = [(c["k"], c["v"]) for c in chunks] + list(zip(batch["decode_k"], batch["decode_v"]))
        kp, vp, tables = wl.paginate(caches, wk.page_size, seed=wk.seed + 1)
        base = {"x": dev(batch["x"]), "pool": (dev(kp), dev(vp)),
                "tables": [torch.from_numpy(t).to("cuda") for t in tables]}
        del kp, vp, caches
    else:
        base = {"x": dev(batch["x"]), "ck": [(dev(c["k"]), dev(c["v"])) for c in chunks],
                "dk": [dev(k) for k in batch["decode_k"]], "dv": [dev(v) for v in batch["decode_v"]]}
    max_pos = max([c["offset"] + c["len"] for c in chunks] + [L + 1 for L in lens])
    reps = []
    for r in range(args.replicas):
        cl = (lambda t: t) if r == 0 else (lambda t: t.clone())
        wr = {k: cl(v) for k, v in wdev.items()}
        layer = hl.HybridLayer(shape, wr, max_tokens=T, max_pos=max_pos)
        x = cl(base["x"])
        y = torch.empty_like(x)
        if paged:
            pool = (cl(base["pool"][0]), cl(base["pool"][1]))
            tbs = [cl(t) for t in base["tables"]]
            nc = len(chunks)
            spec = [(c["len"], c["offset"], t) for c, t in zip(chunks, tbs)]
            b, keep = layer.paged_batch(x, y, pool, spec, tbs[nc:], lens)
            ws = torch.empty(layer.workspace_size(b), dtype=torch.uint8, device="cuda")
            sub = {}
            if C > 0 and lens:
                sub["chunk_only"] = layer.paged_batch(x[:C], y[:C], pool, spec, [], [])
                sub["decode_only"] = layer.paged_batch(x[C:], y[C:], pool, [], tbs[nc:], lens)
            reps.append(dict(layer=layer, b=b, keep=keep, ws=ws, sub=sub, bufs=(x, y, pool, tbs, wr)))
            continue
        ckv = [(cl(k), cl(v)) for k, v in base["ck"]]
        dkv = [(cl(k), cl(v)) for k, v in zip(base["dk"], base["dv"])]
        if multi:
            spec = [(c["len"], c["offset"], kv) for c, kv in zip(chunks, ckv)]
            b, keep = layer.multi_batch(x, y, spec, dkv, lens)
        else:
            spec = None
            b, keep = layer.batch(x, y, C, chunks[0]["offset"] if chunks else 0, ckv[0] if ckv else None,
                                  dkv, lens)
        ws = torch.empty(layer.workspace_size(b), dtype=torch.uint8, device="cuda")
        sub = {}
        if C > 0 and lens:
            # the same rows split into a chunk-only and a decode-only batch (same caches, same slots)
            if multi:
                sub["chunk_only"] = layer.multi_batch(x[:C], y[:C], spec, [], [])
                sub["decode_only"] = layer.multi_batch(x[C:], y[C:], [], dkv, lens)
            else:
                sub["chunk_only"] = layer.batch(x[:C], y[:C], C, chunks[0]["offset"], ckv[0], [], [])
                sub["decode_only"] = layer.batch(x[C:], y[C:], 0, 0, None, dkv, lens)
            for name, (sb, _) in sub.items():
                assert layer.workspace_size(sb) <= ws.numel(), name
        reps.append(dict(layer=layer, b=b, keep=keep, ws=ws, sub=sub, bufs=(x, y, ckv, dkv, wr)))
    stream = torch.cuda.current_stream().cuda_stream
    if paged:
        fwd, fwd_timed = _abi.sarathi_paged_forward, _abi.sarathi_paged_forward_timed
    elif multi:
        fwd, fwd_timed = _abi.sarathi_multi_forward, _abi.sarathi_multi_forward_timed
    else:
        fwd, fwd_timed = _abi.sarathi_layer_forward, _abi.sarathi_layer_forward_timed

    def step(i, timer=None):
        r = reps[i % len(reps)]
        nb = r["ws"].numel()
        if timer:
            fwd_timed(r["layer"].handle, r["b"], r["ws"].data_ptr(), nb, stream, timer)
        else:
            fwd(r["layer"].handle, r["b"], r["ws"].data_ptr(), nb, stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Per-stage breakdown (outside the timed region: every stage boundary carries two HIP events,
    # which themselves cost a few microseconds).
    n_break = max(10, min(args.steps, 50))
    timer = _abi.sarathi_timer_create(n_break, _abi.ALL_STAGES)
    for i in range(n_break):
        step(i, timer)
    stages = _abi.sarathi_timer_read(timer)
    _abi.sarathi_timer_destroy(timer)
    work = stage_work(shape, [(c["len"], c["offset"]) for c in chunks], lens)
    if chunks and lens and stages["attn_chunk"][1] == 0:
        # chunk and decode attention ran as one launch, recorded as the decode stage
        work["attn_decode"] = tuple(a + b for a, b in zip(work["attn_decode"], work["attn_chunk"]))
    breakdown = {}
    for name, (tot, cnt) in stages.items():
        if cnt == 0:
            continue
        avg = tot / cnt
        fl, by = work[name]
        e = roofline_entry(name, avg, fl, by, shape.dtype)
        breakdown[name] = {"avg_us": round(avg * 1e3, 2), "frac": e["frac"], "bound": e["bound"],
                           "achieved": e["achieved"], "unit": e["unit"]}
    dominant = max(breakdown, key=lambda n: breakdown[n]["avg_us"])

    # Timed region: exactly K steps; HIP events on the launch stream only around the dominant
    # kernel's stage give its live average duration.
    timer = _abi.sarathi_timer_create(args.steps, _abi.stage_mask(dominant))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, timer)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    live = _abi.sarathi_timer_read(timer)
    _abi.sarathi_timer_destroy(timer)
    tot, cnt = live[dominant]
    dom_avg_ms = tot / cnt
    roof = roofline_entry(dominant, dom_avg_ms, *work[dominant], shape.dtype)
    roof["traffic"] = load_traffic(dominant, wk.key)
    roof["kernel"] = dominant
    roof["avg_us"] = round(dom_avg_ms * 1e3, 2)
    gemm_ms = sum(breakdown[n]["avg_us"] for n in ("qkv", "o", "ffn_up", "ffn_down")) / 1e3
    gemm_flops = sum(work[n][0] for n in ("qkv", "o", "ffn_up", "ffn_down"))
    summary = {
        "gemm_mfma_frac": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "decode_attn_hbm_frac": breakdown.get("attn_decode", {}).get("frac"),
        "sum_of_stages_us": round(sum(v["avg_us"] for v in breakdown.values()), 2),
        "breakdown_note": "per-stage times from a separate pass with events around every stage",
    }

    ms_per_step = elapsed / args.steps * 1e3
    # Layer roofline fraction: sum over stages of the time each would take at its own bound, over the
    # measured step time.
    peak_c = PEAK_BF16_TFLOPS if shape.dtype == "bf16" else PEAK_F32_TFLOPS
    floor_us = sum(max(fl / (peak_c * 1e12), by / (PEAK_HBM_GBS * 1e9)) for fl, by in work.values()) * 1e6
    summary["layer_floor_us"] = round(floor_us, 2)
    summary["layer_roofline_frac"] = round(floor_us / (ms_per_step * 1e3), 4)

    # Piggybacking comparison (SARATHI page, "Experiments", decode speedup): the marginal cost of a
    # decode riding with the chunk, (t(C,B) - t(C,0)) / B, against a decode in a decode-only batch,
    # t(0,B) / B.
    sweep = None
    if not args.no_sweep and reps[0]["sub"]:
        n_sw = max(20, min(args.steps, 100))

        def time_batch(name):
            for i in range(5):
                r = reps[i % len(reps)]
                fwd(r["layer"].handle, r["sub"][name][0], r["ws"].data_ptr(), r["ws"].numel(), stream)
            torch.cuda.synchronize()
            t_0 = time.perf_counter()
            for i in range(n_sw):
                r = reps[i % len(reps)]
                fwd(r["layer"].handle, r["sub"][name][0], r["ws"].data_ptr(), r["ws"].numel(), stream)
            torch.cuda.synchronize()
            return (time.perf_counter() - t_0) / n_sw * 1e6

        t_c, t_d = time_batch("chunk_only"), time_batch("decode_only")
        t_h = ms_per_step * 1e3
        B = len(lens)
        marginal = (t_h - t_c) / B
        alone = t_d / B
        sweep = {"steps": n_sw, "t_hybrid_us": round(t_h, 2), "t_chunk_only_us": round(t_c, 2),
                 "t_decode_only_us": round(t_d, 2), "marginal_decode_us": round(marginal, 3),
                 "decode_only_per_decode_us": round(alone, 3),
                 "decode_speedup": round(alone / marginal, 2) if marginal > 0 else None}
    value = T * args.steps / elapsed
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": shape.dtype,
        "data": "synthetic",
        "config": {"workload": f"{shape.name} layer, "
                               + (" + ".join(f"chunk {c['len']} at offset {c['offset']}" for c in chunks)
                                  or "no chunk")
                               + f" + {len(lens)} decodes "
                               f"(KV lengths {min(lens) if lens else 0}..{max(lens) if lens else 0})"
                               + (f", paged KV ({wk.page_size}-token pages)" if paged else ""),
                   "hidden": shape.hidden, "heads": shape.n_heads, "head_dim": shape.head_dim,
                   "ffn": shape.ffn, "chunk": C,
                   "chunk_offset": chunks[0]["offset"] if len(chunks) == 1 else None,
                   "chunks": [[c["len"], c["offset"]] for c in chunks],
                   "decodes": len(lens), "rows": T, "replicas": args.replicas,
                   "kv_page_size": wk.page_size},
        "roofline": roof,
        "stages": breakdown,
        "summary": summary,
        "piggyback": sweep,
        "kernel_source": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wk, weights, batch)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    for r in reps:
        r["layer"].close()


if __name__ == "__main__":
    main()
