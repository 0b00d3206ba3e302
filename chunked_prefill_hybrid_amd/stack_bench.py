"""Whole-model measurements of chunked prefills and decode-maximal batching on one MI355X.

A stack of n_layers decoder layers of one workload's shape (LLaMA-13B: 40 layers) runs whole prompts
chunk by chunk through the library's stack entry point, with decodes riding along, and reports the
two comparisons the SARATHI page builds its case on (SARATHI: Efficient LLM Inference by
Piggybacking Decodes with Chunked Prefills):

* Table 2 analog (section 3, "Decode-Maximal Batching", Table 2): per-token time of a prefill-only
  batch (one 1024-token prompt), of a decode-only batch (4 decodes at 1024 cached tokens) and of a
  decode-maximal batch (a 1021-token chunk plus 3 decodes), with the stage split of the page's table
  (pre-projection = norm + QKV + RoPE/append, attention, post-projection = O, FFN = norm + up + down)
  and the marginal time of a piggybacked decode: (t(1021 + 3 decodes) - t(1021 alone)) / 3, from
  alternating runs of the two batches (median of the paired differences).
* Figure 8 analog (section 5, decode speedup vs batch size): for prompt and decode lengths
  L in {1K, 2K, 3K} and batch size B (1 prompt + B - 1 decodes), the whole L-token prompt runs in
  chunks of 256 with B - 1 decodes riding in every step, and again alone.  The marginal decode time
  is the difference of the two passes divided by the decode tokens produced (chunks x (B - 1)); the
  baseline is a decode-only batch of B decodes at length L (time / B).  Speedup = baseline /
  marginal.  B is capped where the decodes' caches would exceed --kv-gib, as the page's batch size
  is capped by memory.  Two more passes per point run the prompt with chunk sizes that make chunk
  plus decodes a multiple of the GEMMs' 32-row time step (section 4.4's tile rule for these kernels).

Weights and caches are drawn on the GPU from a seeded generator (values do not change timing: every
kernel's work is fixed by the shapes).  Every time is a median over --reps repetitions of the whole
stack, measured with HIP events on the launch stream.

    python -m chunked_prefill_hybrid_amd.stack_bench --workload llama13b --layers 40 \\
        --json stack_llama13b.json
"""
from __future__ import annotations

import argparse
import json
import statistics
import sys
import time

PREPROJ = ("norm1", "qkv", "rope_append")
ATTN = ("attn_chunk", "attn_decode", "attn_merge")
POSTPROJ = ("o",)
FFN = ("norm2", "ffn_up", "ffn_down")


def say(*a):
    print(*a, flush=True)


class Model:
    """n_layers layers of one shape with seeded device weights, and a stack over them."""

    def __init__(self, shape, n_layers: int, max_tokens: int, max_pos: int, seed: int):
        import torch

        from . import layer as hl
        self.torch = torch
        self.shape = shape
        self.n_layers = n_layers
        self.dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        H, A, F = shape.hidden, shape.attn_width, shape.ffn

        def w(n, k):
            std = shape.w_std if shape.w_std is not None else k ** -0.5
            t = torch.randn((n, k), generator=g, device="cuda", dtype=torch.float32)
            return t.mul_(std).to(self.dt)

        self.weights = []
        for _ in range(n_layers):
            d = {"w_qkv": w(3 * A, H), "w_o": w(H, A), "w_up": w(F, H), "w_down": w(H, F),
                 "norm1_w": torch.ones(H, device="cuda"), "norm2_w": torch.ones(H, device="cuda")}
            if shape.gated:
                d["w_gate"] = w(F, H)
            if shape.arch == "gpt":
                d["norm1_b"] = torch.zeros(H, device="cuda")
                d["norm2_b"] = torch.zeros(H, device="cuda")
            self.weights.append(d)
        self.layers = [hl.HybridLayer(shape, d, max_tokens=max_tokens, max_pos=max_pos) for d in self.weights]
        self.stack = hl.HybridStack(self.layers)
        self.gen = g
        self.x = torch.randn((max_tokens, H), generator=g, device="cuda").to(self.dt)
        self.y = torch.empty_like(self.x)
        self._ws = None

    def caches(self, n_req: int, cap: int):
        """Caches for n_req requests in every layer: a [n_layers, n_req, 2, nh, cap, d] tensor and its
        per-layer lists of (K, V) views."""
        t = self.torch.empty((self.n_layers, n_req, 2, self.shape.n_heads, cap, self.shape.head_dim),
                             device="cuda", dtype=self.dt)
        t.normal_(generator=self.gen)
        kv = [[(t[l, i, 0], t[l, i, 1]) for i in range(n_req)] for l in range(self.n_layers)]
        return t, kv

    def prepare(self, C, off, chunk_kv, decode_kv, lens):
        """A call that enqueues one stack step with its batch struct built in advance, so that the
        timed region holds the launches only."""
        from . import _abi
        T = C + len(lens)
        b, keep = self.stack.batch(self.x[:T], self.y[:T], C, off, chunk_kv if C else None,
                                   decode_kv if lens else [], lens)
        need = self.stack.workspace_size(b)
        if need == 0:
            raise RuntimeError(f"stack batch rejected: C={C} off={off} B={len(lens)}")
        if self._ws is None or self._ws.numel() < need:
            self._ws = self.torch.empty(need, dtype=self.torch.uint8, device="cuda")
        ws = self._ws
        handles = [l.handle for l in self.layers]
        stream = self.torch.cuda.current_stream().cuda_stream

        def call():
            _abi.sarathi_stack_forward(handles, b, ws.data_ptr(), ws.numel(), stream)
        call.keep = (b, keep, ws)
        return call

    def close(self):
        self.stack.close()


def timed(model, fn, reps: int, warmup: int = 1) -> float:
    """Median milliseconds of fn() over reps runs, HIP events on the current stream."""
    torch = model.torch
    for _ in range(warmup):
        fn()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    return statistics.median(times)


def timed_pair(model, fa, fb, reps: int):
    """Times fa and fb alternately, reps times each; returns (median ms of fa, median ms of fb, median
    of the per-repetition differences fb - fa).  Pairing the runs cancels slow drifts of the clock,
    which matters when the difference is small next to the times."""
    torch = model.torch
    fa()
    fb()
    ta, tb = [], []
    for _ in range(reps):
        for f, out in ((fa, ta), (fb, tb)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            f()
            b.record()
            b.synchronize()
            out.append(a.elapsed_time(b))
    return statistics.median(ta), statistics.median(tb), statistics.median([y - x for x, y in zip(ta, tb)])


def stage_split(model, C, off, chunk_kv0, decode_kv0, lens, reps: int):
    """Per-stage milliseconds of one stack step, from layer 0's stage timer times n_layers (all layers
    have the same shape and work)."""
    from . import _abi
    torch = model.torch
    layer = model.layers[0]
    T = C + len(lens)
    b, keep = layer.batch(model.x[:T], model.y[:T], C, off, chunk_kv0 if C else None, decode_kv0, lens)
    ws = torch.empty(layer.workspace_size(b), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    _abi.sarathi_layer_forward(layer.handle, b, ws.data_ptr(), ws.numel(), stream)
    timer = _abi.sarathi_timer_create(reps)
    for _ in range(reps):
        _abi.sarathi_layer_forward_timed(layer.handle, b, ws.data_ptr(), ws.numel(), stream, timer)
    st = _abi.sarathi_timer_read(timer)
    _abi.sarathi_timer_destroy(timer)
    del keep

    def grp(names):
        return model.n_layers * sum(st[n][0] / max(1, st[n][1]) for n in names)
    return {"preproj": grp(PREPROJ), "attn": grp(ATTN), "postproj": grp(POSTPROJ), "ffn": grp(FFN)}


def table2(model, reps: int):
    """Prefill-only, decode-only and decode-maximal batches (page's Table 2 compositions)."""
    P, B = 1024, 4
    pf_cache, pf_kv = model.caches(1, P)
    dec_cache, dec_kv = model.caches(B, P + 1)
    chunk = [pf_kv[l][0] for l in range(model.n_layers)]
    rows = {}

    def run(name, C, nd, n_tokens):
        lens = [P] * nd
        dkv = [row[:nd] for row in dec_kv]
        t = timed(model, model.prepare(C, 0, chunk, dkv, lens), reps)
        split = stage_split(model, C, 0, chunk[0], dkv[0], lens, reps)
        rows[name] = {"chunk": C, "decodes": nd, "ms": t, "ms_per_token": t / n_tokens, **split}
        say(f"  {name:15s} C={C:4d} B={nd}: {t:8.3f} ms, {t / n_tokens * 1e3:8.2f} us/token  " +
            " ".join(f"{k}={v:.3f}" for k, v in split.items()))

    run("prefill_only", P, 0, P)
    run("decode_only", 0, B, B)
    run("decode_maximal", P - 3, 3, P)
    run("chunk_1021_alone", P - 3, 0, P - 3)
    # the marginal decode time is a small difference of two ~35 ms runs: time them alternately
    dkv3 = [row[:3] for row in dec_kv]
    _, _, diff = timed_pair(model, model.prepare(P - 3, 0, chunk, [], []),
                            model.prepare(P - 3, 0, chunk, dkv3, [P] * 3), max(reps, 15))
    marg = diff / 3
    rows["marginal_decode_ms"] = marg
    rows["decode_speedup"] = rows["decode_only"]["ms_per_token"] / marg if marg > 0 else None
    say(f"  marginal decode: {marg * 1e3:.2f} us/token; decode-only {rows['decode_only']['ms_per_token'] * 1e3:.2f}"
        f" us/token -> {rows['decode_speedup']:.1f}x")
    del pf_cache, dec_cache
    return rows


ROW_STEP = 32      # the layer GEMMs' time rises every 32 batch rows (measured by tile_sweep)
ROW_TILE = 576     # ... and steps up further past 576 rows (a second round of GEMM workgroups)


def aligned_chunks(chunk: int, nd: int):
    """Chunk sizes that make chunk + nd decodes fill whole 32-row steps: `down` trims the chunk to the
    step below (the page's rule: C + B a multiple of the tile), `up` gives the chunk the rows the last
    step pads anyway (kept within one row tile when chunk + nd fits in one)."""
    rows = chunk + nd
    down = (rows // ROW_STEP) * ROW_STEP - nd
    up_rows = -(-rows // ROW_STEP) * ROW_STEP
    if rows <= ROW_TILE:
        up_rows = min(up_rows, ROW_TILE)
    return max(1, down), up_rows - nd


def fig8(model, Ls, Bs, chunk: int, kv_gib: float, reps: int):
    """Decode speedup vs batch size for each length (page's Figure 8 setup), plus the same prompt run
    with chunk sizes that make chunk + decodes fill whole 32-row GEMM steps (page's section 4.4 rule
    restated for these kernels)."""
    sh = model.shape
    el = 2 if sh.dtype == "bf16" else 4
    out = []
    for L in Ls:
        n_chunks = (L + chunk - 1) // chunk
        b_all = [B for B in Bs if B - 1 < chunk]
        max_steps = max((L + c - 1) // c for B in b_all for c in aligned_chunks(chunk, B - 1))
        cap = L + max(max_steps, n_chunks) + 1
        per_req = model.n_layers * 2 * sh.n_heads * cap * sh.head_dim * el
        b_fit = [B for B in b_all if B * per_req <= kv_gib * 2**30]
        if not b_fit:
            continue
        pf_cache, pf_kv = model.caches(1, L)
        chunk_kv = [pf_kv[l][0] for l in range(model.n_layers)]
        dec_cache, dec_kv = model.caches(max(b_fit), cap)
        torch = model.torch

        def prompt_pass(nd, ch):
            dkv = [row[:nd] for row in dec_kv]
            n = (L + ch - 1) // ch
            calls = [model.prepare(min(ch, L - s * ch), s * ch, chunk_kv, dkv, [L + s] * nd)
                     for s in range(n)]

            def run():
                for c in calls:
                    c()
            return run, n

        t_alone = timed(model, prompt_pass(0, chunk)[0], reps)
        say(f"  L={L}: prompt alone in {n_chunks} chunks of {chunk}: {t_alone:.2f} ms")
        for B in b_fit:
            nd = B - 1
            dkv = [row[:B] for row in dec_kv]
            t_dec = timed(model, model.prepare(0, 0, None, dkv, [L] * B), reps)
            base = t_dec / B
            rec = {"L": L, "B": B, "decode_only_ms": t_dec, "baseline_ms_per_token": base,
                   "prompt_alone_ms": t_alone, "prompt_with_decodes_ms": None, "marginal_ms_per_token": None,
                   "speedup": None}
            if nd:
                t_hyb = timed(model, prompt_pass(nd, chunk)[0], reps)
                marg = (t_hyb - t_alone) / (n_chunks * nd)
                rec.update(prompt_with_decodes_ms=t_hyb, marginal_ms_per_token=marg,
                           speedup=base / marg if marg > 0 else None)
                for tag, c_a in zip(("down", "up"), aligned_chunks(chunk, nd)):
                    run_a, n_a = prompt_pass(nd, c_a)
                    t_a = timed(model, run_a, reps)
                    t_a0 = timed(model, prompt_pass(0, c_a)[0], reps)
                    m_a = (t_a - t_a0) / (n_a * nd)
                    rec[f"{tag}_chunk"] = c_a
                    rec[f"{tag}_alone_ms"] = t_a0
                    rec[f"{tag}_ms"] = t_a
                    rec[f"{tag}_marginal_ms_per_token"] = m_a
                    rec[f"{tag}_speedup"] = base / m_a if m_a > 0 else None
            out.append(rec)
            msg = (f"    B={B:3d}: decode-only {base * 1e3:8.2f} us/token, piggybacked "
                   f"{(rec['marginal_ms_per_token'] or 0) * 1e3:8.2f} us/token (x{rec['speedup'] or 0:.2f})")
            for tag in ("down", "up"):
                if f"{tag}_chunk" in rec:
                    msg += (f", {tag} C={rec[tag + '_chunk']}: {rec[tag + '_marginal_ms_per_token'] * 1e3:8.2f}"
                            f" us/token (x{rec[tag + '_speedup'] or 0:.2f}; prompt alone "
                            f"{rec[tag + '_alone_ms']:.2f} ms)")
            say(msg)
        del pf_cache, dec_cache, chunk_kv
        torch.cuda.empty_cache()
    return out


def markdown(res, command: str) -> str:
    """The results as the markdown summary kept with the profiles."""
    t2, f8 = res["table2"], res["fig8"]
    out = [f"# Whole-model chunked prefills and decode-maximal batching: {res['layers']} x {res['shape']}", "",
           "Command (repository root, one MI355X):", "", "```", command, "```", "",
           f"Median of {res['reps']} runs of the whole {res['layers']}-layer stack per point (HIP events "
           "on the launch stream); stage split from layer 0's stage timer times the layer count.", "",
           "## Table 2 compositions (ms for the whole stack)", "",
           "| batch | chunk | decodes | preproj | attn | postproj | FFN | total | per token |",
           "|---|---|---|---|---|---|---|---|---|"]
    for name in ("prefill_only", "decode_only", "decode_maximal", "chunk_1021_alone"):
        r = t2[name]
        out.append(f"| {name} | {r['chunk']} | {r['decodes']} | {r['preproj']:.2f} | {r['attn']:.2f} | "
                   f"{r['postproj']:.2f} | {r['ffn']:.2f} | {r['ms']:.2f} | {r['ms_per_token']:.4f} |")
    sp = t2["decode_speedup"]
    out += ["", f"Marginal time of a piggybacked decode: {t2['marginal_decode_ms']:.4f} ms/token "
            f"(decode-only: {t2['decode_only']['ms_per_token']:.4f} ms/token; "
            f"{'n/a' if sp is None else f'{sp:.1f}x'}).", "",
            f"## Decode speedup vs batch size (chunk {res['chunk']})", "",
            "B = 1 prompt + (B - 1) decodes; baseline = B decodes alone.  The marginal time is the "
            "extra time of the whole prompt pass with the decodes riding along over the prompt pass "
            f"alone in chunks of {res['chunk']}, per decode token.  `down` / `up` run the prompt in "
            "chunks that make chunk + decodes a multiple of 32 rows (the layer GEMMs' time step): "
            "`down` trims the chunk, `up` gives it the rows the last step pads anyway.  Their marginal "
            "time is taken against the prompt alone in chunks of the same size, whose time is listed "
            "(the prompt's own cost of the chunk choice).", "",
            "| L | B | decode-only ms/token | piggybacked ms/token | speedup | down C | prompt alone ms | "
            "down ms/token | down speedup | up C | prompt alone ms | up ms/token | up speedup |",
            "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]

    def f(v, spec):
        return "-" if v is None else format(v, spec)
    for r in f8:
        out.append(f"| {r['L']} | {r['B']} | {f(r['baseline_ms_per_token'], '.4f')} | "
                   f"{f(r['marginal_ms_per_token'], '.4f')} | {f(r['speedup'], '.2f')} | "
                   f"{f(r.get('down_chunk'), 'd')} | {f(r.get('down_alone_ms'), '.2f')} | "
                   f"{f(r.get('down_marginal_ms_per_token'), '.4f')} | "
                   f"{f(r.get('down_speedup'), '.2f')} | {f(r.get('up_chunk'), 'd')} | {f(r.get('up_alone_ms'), '.2f')} | "
                   f"{f(r.get('up_marginal_ms_per_token'), '.4f')} | {f(r.get('up_speedup'), '.2f')} |")
    return "\n".join(out) + "\n"


def main(argv=None) -> int:
    import torch

    from . import workloads as wl
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama13b")
    ap.add_argument("--layers", type=int, default=40)
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--chunk", type=int, default=256)
    ap.add_argument("--lengths", default="1024,2048,3072")
    ap.add_argument("--batches", default="2,4,8,12,18,32,64")
    ap.add_argument("--kv-gib", type=float, default=120.0,
                    help="memory allowed for the decodes' caches in the Figure 8 sweep")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--json", default=None)
    ap.add_argument("--md", default=None, help="also write the markdown summary here")
    args = ap.parse_args(argv)
    torch.cuda.set_device(0)
    shape = wl.workload(args.workload).shape
    Ls = [int(v) for v in args.lengths.split(",")]
    Bs = [int(v) for v in args.batches.split(",")]
    max_tokens = max(1024, args.chunk + max(Bs))
    max_pos = max(Ls + [1024]) + max(Ls) // args.chunk + 8
    t0 = time.time()
    model = Model(shape, args.layers, max_tokens, max_pos, args.seed)
    say(f"stack: {args.layers} x {shape.name} layers, {sum(p.numel() * p.element_size() for d in model.weights for p in d.values()) / 2**30:.1f} GiB of weights")
    say("Table 2 compositions:")
    t2 = table2(model, args.reps)
    say(f"Figure 8 sweep (chunk {args.chunk}):")
    f8 = fig8(model, Ls, Bs, args.chunk, args.kv_gib, args.reps)
    res = {"workload": args.workload, "shape": shape.name, "layers": args.layers, "chunk": args.chunk,
           "reps": args.reps, "table2": t2, "fig8": f8, "seconds": round(time.time() - t0, 1)}
    if args.json:
        with open(args.json, "w") as f:
            json.dump(res, f, indent=1)
    if args.md:
        cmd = "python -m chunked_prefill_hybrid_amd.stack_bench " + " ".join(sys.argv[1:] if argv is None else argv)
        with open(args.md, "w") as f:
            f.write(markdown(res, cmd))
    model.close()
    say(f"done in {res['seconds']} s")
    return 0


if __name__ == "__main__":
    sys.exit(main())
