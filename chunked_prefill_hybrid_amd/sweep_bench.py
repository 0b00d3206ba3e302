"""Batch-composition sweeps of one workload, each point measured by bench.py.

For every point of `workloads.sweep_changes(key)` (the number of piggybacked decodes B for llama13b and
gpt3tp8, the chunk length C for llama33b) this runs `bench.py --workload key --batch {...}` in a child
process and collects its line: tokens/s, time per forward, and, for batches with both a chunk and
decodes, the decode-cost comparison of the SARATHI page's "Decode-Maximal Batching" section (the
marginal cost of a decode riding with the chunk, (t(C, B) - t(C, 0)) / B, against t(0, B) / B in a
decode-only batch).

    python -m chunked_prefill_hybrid_amd.sweep_bench --workload gpt3tp8 --md sweep.md --json sweep.json
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_point(key, changes, steps, warmup):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", key, "--batch", json.dumps(changes),
           "--steps", str(steps), "--warmup", str(warmup), "--no-cpu-baseline"]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT)
    if r.returncode != 0:
        raise SystemExit(f"bench.py failed for {changes} (exit {r.returncode}):\n{r.stderr[-2000:]}")
    return json.loads(r.stdout.strip().splitlines()[-1])


def table(key, rows):
    out = [f"| C | B | rows | tokens/s | ms per forward | gate/up % MFMA | decode attention % HBM | "
           f"marginal decode us | decode-only us per decode | ratio |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for ch, line in rows:
        cfg, st, pg = line["config"], line["stages"], line.get("piggyback") or {}
        C = sum(c[0] for c in cfg["chunks"])
        dec = st.get("attn_decode", {})
        dec_frac = f"{100 * dec['frac']:.1f}" if dec.get("frac") else "-"
        out.append(f"| {C} | {cfg['decodes']} | {cfg['rows']} | {line['value']:.0f} | {line['ms_per_step']} | "
                   f"{100 * st['ffn_up']['frac']:.1f} | {dec_frac} | "
                   f"{pg.get('marginal_decode_us', '-')} | {pg.get('decode_only_per_decode_us', '-')} | "
                   f"{pg.get('decode_speedup', '-')} |")
    return out


def main(argv=None) -> int:
    from . import workloads as wl

    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="gpt3tp8")
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--md", default=None)
    ap.add_argument("--json", default=None)
    args = ap.parse_args(argv)
    points = wl.sweep_changes(args.workload)
    if not points:
        raise SystemExit(f"no sweep defined for {args.workload}")
    rows = []
    for ch in points:
        line = run_point(args.workload, ch, args.steps, args.warmup)
        rows.append((ch, line))
        pg = line.get("piggyback") or {}
        print(f"{args.workload} {json.dumps({k: v for k, v in ch.items() if k != 'decode_lens'})}: "
              f"{line['value']:.0f} tokens/s, {line['ms_per_step']} ms, marginal decode "
              f"{pg.get('marginal_decode_us')} us vs {pg.get('decode_only_per_decode_us')} us", flush=True)
    lines = table(args.workload, rows)
    print("\n".join(lines))
    if args.md:
        with open(args.md, "w") as f:
            f.write("\n".join(lines) + "\n")
    if args.json:
        with open(args.json, "w") as f:
            json.dump([{"changes": ch, "line": line} for ch, line in rows], f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
