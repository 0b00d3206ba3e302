"""Throughput of the hybrid-batch decoder-layer forward on one MI355X.

One step = one forward of one decoder layer over one hybrid batch: a prefill chunk plus piggybacked
decodes (SARATHI: Efficient LLM Inference by Piggybacking Decodes with Chunked Prefills, section 3,
"Decode-Maximal Batching").  Default workload: the largest single-GPU batch of the measured set, the
LLaMA-13B layer shape in bf16 with a chunk C=512 at offset 7680 of an 8192-token prompt plus B=48
decodes whose KV lengths are uniform in [2048, 8192] (560 rows, about 5 GB of KV per step; the
attention-dominated regime that section 6 of the same page, "Limitations and Trade-offs", points to).
The C=256 + 18-decode LLaMA-13B batch is measured in the same run and reported under `secondary`.

Inputs are seeded and synthetic, drawn on the GPU (workloads.generate(..., device="cuda")) and
already resident in HBM when timing starts.  Three replicas of the weights, caches and activations
are rotated step by step so that the 256 MB last-level cache cannot hold a step's data.

Passes per workload: W warmup steps; a breakdown pass in which the library records HIP events around
every stage (this perturbs the step time, so it is not the timed region); then exactly K timed steps
in which events are recorded on the launch stream only around the dominant kernel's stage, giving
that kernel's live average duration for the roofline, and two one-thread kernels around them sample
the shader clock counter, giving the average GPU clock over the timed steps.  Prints ONE JSON line:
tokens/s over the K timed steps, the roofline of the dominant kernel, the per-stage breakdown, the layer's roofline fraction, the piggybacking comparison (the same
rows run as a chunk-only and a decode-only batch, giving the marginal cost of a decode that rides
with the chunk), the GPU clock during the timed steps, and the CPU oracle's throughput on the same
inputs (float32, on the host cores given to this process, plus a one-thread run).
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
DEFAULT_WORKLOAD = "llama13b_long"
DEFAULT_SECONDARY = "llama13b"


from chunked_prefill_hybrid_amd.profiling import kernel_source_hash, stage_source_hash  # noqa: E402


def _split_count(n_keys):
    """Key splits of a decode row's split-KV attention: 256 keys each, 1024 for rows of more than 2048
    keys (the library's rule; a CPU test checks the two agree through sarathi_plan_describe)."""
    per = 1024 if n_keys > 2048 else 256
    return (n_keys + per - 1) // per


def stage_work(shape, chunks, lens, chunk_splits=None):
    """Algorithmic work of each stage: (flops, bytes).  chunks: [(len, offset)] of the batch's prefill
    chunks; chunk_splits: key splits of each chunk (the merge reads the partials of split chunks).
    GEMM flops use the unpadded row count."""
    C = sum(n for n, _ in chunks)
    T = C + len(lens)
    H, A, F = shape.hidden, shape.attn_width, shape.ffn
    nh, d = shape.n_heads, shape.head_dim
    el = 2 if shape.dtype == "bf16" else 4
    up_n = 2 * F if shape.gated else F
    splits = chunk_splits or [1] * len(chunks)
    # the merge reads each split partial (d floats of o plus m and l) of the rows that have several,
    # and writes those rows' attention output
    merge_rows = [(n, s) for (n, _), s in zip(chunks, splits) if s > 1] + \
                 [(1, _split_count(L + 1)) for L in lens]
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
        "attn_merge": (0.0, sum(n * (nh * s * (d + 2) * 4 + A * el) for n, s in merge_rows)),
    }
    return w


BOUND = {"qkv": "mfma", "o": "mfma", "ffn_up": "mfma", "ffn_down": "mfma", "attn_chunk": "mfma",
         "attn_decode": "hbm", "norm1": "hbm", "norm2": "hbm", "rope_append": "hbm", "attn_merge": "hbm"}
# Stages whose work is the method's own (the floor of the layer); the merge of split partials is a
# cost of this design's key splits, reported but not counted in the floor.
FLOOR_STAGES = ("qkv", "o", "ffn_up", "ffn_down", "attn_decode", "attn_chunk", "norm1", "norm2",
                "rope_append")


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


class DeviceClock:
    """Average shader clock over enqueued work: a kernel before and one after it each sample, on every
    compute unit it reaches, that unit's shader-clock timestamp counter (s_memtime) and the 100 MHz
    real-time counter (s_memrealtime).  Per unit the clock is 100 MHz x (timestamp delta) / (real-time
    delta); the figure is the median over the units sampled both times (each unit counts on its
    own, so samples of two different units are never paired)."""

    SLOTS = 2048

    def __init__(self, stream):
        import torch

        from chunked_prefill_hybrid_amd import _abi
        self._abi = _abi
        self.stream = stream
        self.buf = torch.zeros(4 * self.SLOTS, dtype=torch.int64, device="cuda")

    def start(self):
        self._abi.sarathi_clock_sample(self.buf.data_ptr(), self.stream)

    def stop(self):
        self._abi.sarathi_clock_sample(self.buf.data_ptr() + 16 * self.SLOTS, self.stream)

    def per_unit(self):
        return unit_clocks([int(x) for x in self.buf.cpu().tolist()], self.SLOTS)

    def summary(self):
        return clock_summary(self.per_unit())


def unit_clocks(values, slots):
    """(MHz, interval ms) per compute unit from two clock samples: values holds the first sample's
    `slots` (s_memtime, s_memrealtime) pairs, then the second's.  A unit counts only if the first
    sample wrote its slot (nonzero real time) and its real-time counter advanced."""
    before, after = values[:2 * slots], values[2 * slots:4 * slots]
    out = []
    for u in range(slots):
        t0, r0, t1, r1 = before[2 * u], before[2 * u + 1], after[2 * u], after[2 * u + 1]
        if r0 and r1 > r0:
            out.append((100.0 * (t1 - t0) / (r1 - r0), (r1 - r0) / 1e5))
    return out


def clock_summary(units):
    """The bench line's gpu_clock: the median over the units, their 10th and 90th percentiles."""
    if not units:
        return {"source": "s_memtime / s_memrealtime per compute unit", "error": "no real-time interval"}
    mhz = sorted(m for m, _ in units)
    return {"source": "s_memtime / s_memrealtime per compute unit around the timed steps",
            "gfx_mhz_avg": round(statistics.median(mhz), 1),
            "gfx_mhz_p10_p90": [round(mhz[len(mhz) // 10], 1), round(mhz[(9 * len(mhz)) // 10], 1)],
            "units": len(mhz), "interval_ms": round(max(s for _, s in units), 3)}


def host_cpu():
    """CPU model and the host threads this process may use (its affinity, capped by OMP_NUM_THREADS)."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS")
    threads = min(avail, int(cap)) if cap and cap.isdigit() and int(cap) > 0 else avail
    return model, threads, os.cpu_count()


def cpu_baseline(wk, weights, batch):
    """The CPU oracle as it is (plain NumPy, float32 arithmetic) on one full step of the same inputs
    the GPU ran: once with BLAS on the host threads given to this process, once on one thread."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle

    def host(a):
        if a is None or isinstance(a, (int, float, list, tuple, dict)) or isinstance(a, np.ndarray):
            return a
        return a.float().cpu().numpy()

    hw = {k: host(v) for k, v in weights.items()}
    hb = {k: (host(v) if not isinstance(v, list) else [host(t) for t in v]) for k, v in batch.items()}
    if "chunks" in hb:
        hb["chunks"] = [{kk: host(vv) for kk, vv in c.items()} for c in batch["chunks"]]
    fwd = oracle.layer_forward_multi if "chunks" in hb else oracle.layer_forward
    model, threads, ncpu = host_cpu()
    blas = [{"api": i.get("internal_api"), "version": i.get("version"), "threads": i.get("num_threads")}
            for i in threadpool_info() if i.get("user_api") == "blas"]
    T = hb["x"].shape[0]

    def timed(n_threads):
        with threadpool_limits(limits=n_threads, user_api="blas"):
            used = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
            t0 = time.perf_counter()
            fwd(wk.shape, hw, hb, dtype=np.float32)
            return time.perf_counter() - t0, used

    t_all, used = timed(threads)
    t_one, _ = timed(1)
    return {"value": round(T / t_all, 2), "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "sample": f"one full step ({T} rows, one layer), float32 NumPy on the inputs the GPU ran",
            "seconds": round(t_all, 2),
            "one_thread": {"value": round(T / t_one, 2), "unit": "tokens/s", "seconds": round(t_one, 2)},
            "cpu_model": model, "host_cpus": ncpu, "blas": blas}


def measure(key, args, changes=None, page_size=None, sweep=True):
    """Runs one workload: warmup, stage breakdown, exactly args.steps timed steps, the piggyback
    comparison.  Returns (report dict, workload, device weights, device batch)."""
    import torch

    from chunked_prefill_hybrid_amd import _abi
    from chunked_prefill_hybrid_amd import layer as hl
    from chunked_prefill_hybrid_amd import workloads as wl

    wk = wl.workload(key, **(changes or {}))
    if page_size is not None:
        wk = dataclasses.replace(wk, page_size=page_size or None)
    shape = wk.shape
    weights, batch = wl.generate(wk, device="cuda")
    chunks = wl.chunks_of(batch)            # [{len, offset, k, v}]: one chunk, several, or none
    multi = "chunks" in batch               # token-budget workloads use the several-chunk entry point
    lens = list(batch["decode_len"])
    C = sum(c["len"] for c in chunks)
    T = C + len(lens)
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32

    def dev(a, t=dt):
        if isinstance(a, torch.Tensor):
            return a.to(t)
        import numpy as np
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(t)

    wdev = {k: dev(v, torch.float32 if k.startswith("norm") else dt) for k, v in weights.items() if v is not None}
    paged = wk.page_size is not None
    if paged:
        # every request's cache in one pool of fixed-size pages, in a shuffled page order
        caches = [(c["k"].float().cpu().numpy(), c["v"].float().cpu().numpy()) for c in chunks] + \
                 [(k.float().cpu().numpy(), v.float().cpu().numpy())
                  for k, v in zip(batch["decode_k"], batch["decode_v"])]
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
            sub = {}
            if C > 0 and lens:
                sub["chunk_only"] = layer.paged_batch(x[:C], y[:C], pool, spec, [], [])
                sub["decode_only"] = layer.paged_batch(x[C:], y[C:], pool, [], tbs[nc:], lens)
            need = max([layer.workspace_size(b)] + [layer.workspace_size(sb) for sb, _ in sub.values()])
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
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
        sub = {}
        if C > 0 and lens:
            # the same rows split into a chunk-only and a decode-only batch (same caches, same slots)
            if multi:
                sub["chunk_only"] = layer.multi_batch(x[:C], y[:C], spec, [], [])
                sub["decode_only"] = layer.multi_batch(x[C:], y[C:], [], dkv, lens)
            else:
                sub["chunk_only"] = layer.batch(x[:C], y[:C], C, chunks[0]["offset"], ckv[0], [], [])
                sub["decode_only"] = layer.batch(x[C:], y[C:], 0, 0, None, dkv, lens)
        # one workspace serves the batch and its chunk-only and decode-only parts (a part's plan can
        # need more: a chunk alone may split its key ranges where the hybrid batch's fused launch
        # does not)
        need = max([layer.workspace_size(b)] + [layer.workspace_size(sb) for sb, _ in sub.values()])
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        reps.append(dict(layer=layer, b=b, keep=keep, ws=ws, sub=sub, bufs=(x, y, ckv, dkv, wr)))
    info = _abi.plan_describe(reps[0]["layer"].desc, reps[0]["b"])
    chunk_splits = [int(info.chunk_splits[j]) for j in range(len(chunks))]
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
    work = stage_work(shape, [(c["len"], c["offset"]) for c in chunks], lens, chunk_splits)
    fused = chunks and lens and stages["attn_chunk"][1] == 0
    if fused:
        # chunk and decode attention ran as one launch, recorded as the decode stage
        work["attn_decode"] = tuple(a + b for a, b in zip(work["attn_decode"], work["attn_chunk"]))
        work["attn_chunk"] = (0.0, 0.0)
    breakdown = {}
    for name, (tot, cnt) in stages.items():
        if cnt == 0:
            continue
        avg = tot / cnt
        fl, by = work[name]
        e = roofline_entry(name, avg, fl, by, shape.dtype)
        breakdown[name] = {"avg_us": round(avg * 1e3, 2), "frac": e["frac"], "bound": e["bound"],
                           "achieved": e["achieved"], "unit": e["unit"]}
        if "hbm_frac" in e:
            breakdown[name]["hbm_frac"] = e["hbm_frac"]
    dominant = max(breakdown, key=lambda n: breakdown[n]["avg_us"])

    # Timed region: exactly K steps; HIP events on the launch stream only around the dominant
    # kernel's stage give its live average duration; a host thread samples the GPU clock.
    timer = _abi.sarathi_timer_create(args.steps, _abi.stage_mask(dominant))
    clocks = DeviceClock(stream)
    torch.cuda.synchronize()
    clocks.start()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, timer)
    clocks.stop()
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
    gemms = [n for n in ("qkv", "o", "ffn_up", "ffn_down") if n in breakdown]
    gemm_ms = sum(breakdown[n]["avg_us"] for n in gemms) / 1e3
    gemm_flops = sum(work[n][0] for n in gemms)
    peak_c = PEAK_BF16_TFLOPS if shape.dtype == "bf16" else PEAK_F32_TFLOPS
    summary = {
        "gemm_mfma_frac": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / peak_c, 4) if gemm_ms else None,
        "decode_attn_hbm_frac": breakdown.get("attn_decode", {}).get("frac"),
        "decode_attn_includes_chunk": bool(fused),
        "sum_of_stages_us": round(sum(v["avg_us"] for v in breakdown.values()), 2),
        "breakdown_note": "per-stage times from a separate pass with events around every stage",
    }
    ms_per_step = elapsed / args.steps * 1e3
    # Layer roofline fraction: sum over the method's stages of the time each would take at its own
    # bound, over the measured step time.
    floor_us = sum(max(work[n][0] / (peak_c * 1e12), work[n][1] / (PEAK_HBM_GBS * 1e9))
                   for n in FLOOR_STAGES) * 1e6
    summary["layer_floor_us"] = round(floor_us, 2)
    summary["layer_roofline_frac"] = round(floor_us / (ms_per_step * 1e3), 4)

    # Piggybacking comparison (SARATHI page, "Experiments", decode speedup): the marginal cost of a
    # decode riding with the chunk, (t(C,B) - t(C,0)) / B, against a decode in a decode-only batch,
    # t(0,B) / B.
    pig = None
    if sweep and reps[0]["sub"]:
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
        pig = {"steps": n_sw, "t_hybrid_us": round(t_h, 2), "t_chunk_only_us": round(t_c, 2),
               "t_decode_only_us": round(t_d, 2), "marginal_decode_us": round(marginal, 3),
               "decode_only_per_decode_us": round(alone, 3),
               "decode_speedup": round(alone / marginal, 2) if marginal > 0 else None}
    config = {"workload": f"{shape.name} layer, "
                          + (" + ".join(f"chunk {c['len']} at offset {c['offset']}" for c in chunks)
                             or "no chunk")
                          + f" + {len(lens)} decodes "
                          f"(KV lengths {min(lens) if lens else 0}..{max(lens) if lens else 0})"
                          + (f", paged KV ({wk.page_size}-token pages)" if paged else ""),
              "key": wk.key, "hidden": shape.hidden, "heads": shape.n_heads, "head_dim": shape.head_dim,
              "ffn": shape.ffn, "chunk": C,
              "chunk_offset": chunks[0]["offset"] if len(chunks) == 1 else None,
              "chunks": [[c["len"], c["offset"]] for c in chunks],
              "decodes": len(lens), "rows": T, "replicas": args.replicas, "kv_page_size": wk.page_size,
              "kv_bytes": int(sum(2 * shape.attn_width * (2 if shape.dtype == "bf16" else 4) * (L + 1)
                                  for L in lens))}
    report = {"value": round(T * args.steps / elapsed, 1), "ms_per_step": round(ms_per_step, 4),
              "dtype": shape.dtype, "config": config, "roofline": roof, "stages": breakdown,
              "summary": summary, "piggyback": pig, "gpu_clock": clocks.summary(),
              "plan": {"chunk_splits": chunk_splits, "fused_attention": int(info.fused_attention),
                       "workspace_bytes": int(info.workspace_bytes)}}
    for r in reps:
        r["layer"].close()
    reps.clear()
    del base
    return report, wk, weights, batch


def note(msg):
    """Progress on stderr (the JSON line is the only stdout output)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--secondary", default=None,
                    help="comma-separated workloads measured after the headline and reported under "
                         f"`secondary` (default: {DEFAULT_SECONDARY} when the headline is the default "
                         "workload and its batch is unchanged; '' for none)")
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

    import torch

    torch.cuda.set_device(0)
    changes = {k: tuple(v) if isinstance(v, list) else v for k, v in json.loads(args.batch or "{}").items()}
    if args.secondary is None:
        plain = args.workload == DEFAULT_WORKLOAD and not changes and args.page_size is None
        secondary = [DEFAULT_SECONDARY] if plain else []
    else:
        secondary = [s for s in args.secondary.split(",") if s]

    rep, wk, weights, batch = measure(args.workload, args, changes, args.page_size, sweep=not args.no_sweep)
    note(f"{args.workload}: {rep['value']:.0f} tokens/s, {rep['ms_per_step']:.4f} ms/step")
    torch.cuda.empty_cache()
    extra = {}
    for key in secondary:
        r2, *_ = measure(key, args, sweep=not args.no_sweep)
        note(f"{key}: {r2['value']:.0f} tokens/s, {r2['ms_per_step']:.4f} ms/step")
        torch.cuda.empty_cache()
        extra[key] = r2
    out = {
        "metric": METRIC, "value": rep["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": rep["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": rep["dtype"],
        "data": "synthetic (seeded, drawn on the GPU; random-init weights of the layer shape)",
        "config": rep["config"],
        "roofline": rep["roofline"],
        "stages": rep["stages"],
        "summary": rep["summary"],
        "piggyback": rep["piggyback"],
        "gpu_clock": rep["gpu_clock"],
        "plan": rep["plan"],
        "secondary": extra or None,
        "kernel_source": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        note("CPU oracle baseline")
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(wk, weights, batch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
