"""Helpers of the GPU parity tests: upload seeded workloads, run the layer through the C ABI, and
compare with the oracle.

Error metric (per tensor): rel = max|gpu - ref| / max|ref|; any NaN/Inf fails.  Tolerances: 1e-4 in
float32 mode, 2e-2 in bf16 mode (bf16 inputs, float32 accumulation).  Besides y the checks cover
dY = y - x (the residual would otherwise hide attention errors), the attention output, the rotated
queries and the K/V rows written into the caches.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from chunked_prefill_hybrid_amd import layer as hl

TOL = {"f32": 1e-4, "bf16": 2e-2}
DEV = "cuda"
# Every comparison of a session: (label, tolerance, {tensor: rel error}); the test session's summary
# prints them as a table (and writes it to $SARATHI_PARITY_TABLE when set).
RECORDS = []


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tdtype(shape):
    return torch.float32 if shape.dtype == "f32" else torch.bfloat16


def dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dtype)


def upload_weights(shape, w):
    dt = tdtype(shape)
    out = {}
    for k, v in w.items():
        if v is None:
            continue
        out[k] = dev(v, torch.float32 if k.startswith("norm") else dt)
    return out


def upload_batch(shape, b):
    dt = tdtype(shape)
    d = {"x": dev(b["x"], dt), "chunk_len": b["chunk_len"], "chunk_offset": b["chunk_offset"],
         "decode_len": list(b["decode_len"])}
    d["chunk_kv"] = (dev(b["chunk_k"], dt), dev(b["chunk_v"], dt)) if b["chunk_len"] else None
    d["decode_kv"] = [(dev(k, dt), dev(v, dt)) for k, v in zip(b["decode_k"], b["decode_v"])]
    d["y"] = torch.empty_like(d["x"])
    return d


def run(layer, db, dump=True, workspace=None):
    shape = layer.shape
    T = db["x"].shape[0]
    A = shape.attn_width
    widths = {"n1": shape.hidden, "qkv": 3 * A, "q_rot": A, "attn": A, "h1": shape.hidden,
              "n2": shape.hidden, "act": shape.ffn}
    dd = {k: torch.full((T, w), float("nan"), device=DEV) for k, w in widths.items()} if dump else None
    layer.forward(db["x"], db["y"], db["chunk_len"], db["chunk_offset"], db["chunk_kv"],
                  db["decode_kv"], db["decode_len"], workspace=workspace, dump=dd)
    torch.cuda.synchronize()
    return dd


def rel(g, r):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if not np.all(np.isfinite(g)):
        return float("inf")
    den = np.max(np.abs(r))
    return float(np.max(np.abs(g - r)) / (den if den > 0 else 1.0))


def new_rows_from_caches(db, C, off, lens):
    """The K/V rows the step wrote, read back from the device caches: [C+B, nh, d] each."""
    ks, vs = [], []
    if C:
        k, v = db["chunk_kv"]
        ks.append(k[:, off:off + C, :].permute(1, 0, 2).float().cpu().numpy())
        vs.append(v[:, off:off + C, :].permute(1, 0, 2).float().cpu().numpy())
    for (k, v), L in zip(db["decode_kv"], lens):
        ks.append(k[:, L:L + 1, :].permute(1, 0, 2).float().cpu().numpy())
        vs.append(v[:, L:L + 1, :].permute(1, 0, 2).float().cpu().numpy())
    return np.concatenate(ks), np.concatenate(vs)


def compare(shape, b, ref, db, dd, tol=None, label=""):
    """Errors of every checked tensor; asserts each is within tolerance."""
    C, off, lens = b["chunk_len"], b["chunk_offset"], list(b["decode_len"])
    nk, nv = new_rows_from_caches(db, C, off, lens)
    return compare_rows(shape, b["x"], ref, db["y"], nk, nv, dd, tol, label)


def compare_rows(shape, x, ref, y_dev, nk, nv, dd, tol=None, label=""):
    tol = tol if tol is not None else TOL[shape.dtype]
    y = y_dev.float().cpu().numpy()
    x = np.asarray(x, dtype=np.float64)
    errs = {"y": rel(y, ref["y"]), "dy": rel(y - x, ref["y"] - x), "new_k": rel(nk, ref["new_k"]),
            "new_v": rel(nv, ref["new_v"])}
    if dd is not None:
        for k in ("n1", "qkv", "q_rot", "attn", "h1", "n2", "act"):
            errs[k] = rel(dd[k].cpu().numpy(), ref[k])
    say(f"[{label}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    RECORDS.append((label, tol, dict(errs)))
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    assert not bad, f"{label}: over tolerance {tol}: {bad}"
    return errs


# ---- batches with several prefill chunks ----------------------------------------------------------

def upload_multi(shape, b):
    dt = tdtype(shape)
    d = {"x": dev(b["x"], dt), "decode_len": list(b["decode_len"]),
         "chunks": [(c["len"], c["offset"], (dev(c["k"], dt), dev(c["v"], dt))) for c in b["chunks"]],
         "decode_kv": [(dev(k, dt), dev(v, dt)) for k, v in zip(b["decode_k"], b["decode_v"])]}
    d["y"] = torch.empty_like(d["x"])
    return d


def run_multi(layer, db, dump=True, workspace=None):
    shape = layer.shape
    T = db["x"].shape[0]
    A = shape.attn_width
    widths = {"n1": shape.hidden, "qkv": 3 * A, "q_rot": A, "attn": A, "h1": shape.hidden,
              "n2": shape.hidden, "act": shape.ffn}
    dd = {k: torch.full((T, w), float("nan"), device=DEV) for k, w in widths.items()} if dump else None
    layer.forward_multi(db["x"], db["y"], db["chunks"], db["decode_kv"], db["decode_len"],
                        workspace=workspace, dump=dd)
    torch.cuda.synchronize()
    return dd


def new_rows_multi(db):
    """The K/V rows the step wrote, read back from the device caches: [T, nh, d] each."""
    ks, vs = [], []
    for n, off, (k, v) in db["chunks"]:
        ks.append(k[:, off:off + n, :].permute(1, 0, 2).float().cpu().numpy())
        vs.append(v[:, off:off + n, :].permute(1, 0, 2).float().cpu().numpy())
    for (k, v), L in zip(db["decode_kv"], db["decode_len"]):
        ks.append(k[:, L:L + 1, :].permute(1, 0, 2).float().cpu().numpy())
        vs.append(v[:, L:L + 1, :].permute(1, 0, 2).float().cpu().numpy())
    return np.concatenate(ks), np.concatenate(vs)


def compare_multi(shape, b, ref, db, dd, tol=None, label=""):
    nk, nv = new_rows_multi(db)
    return compare_rows(shape, b["x"], ref, db["y"], nk, nv, dd, tol, label)


def oracle_ref(shape, w, b):
    return oracle.layer_forward(shape, w, b)


PARITY_COLUMNS = ("y", "dy", "attn", "q_rot", "new_k", "new_v", "n1", "h1", "n2", "act")


def parity_table(records=None):
    """Markdown table of recorded comparisons: per tensor, rel = max|gpu - ref| / max|ref|, and the
    margin (tolerance / worst error)."""
    records = RECORDS if records is None else records
    head = "| case | tol | " + " | ".join(PARITY_COLUMNS) + " | worst / tol |"
    lines = [head, "|" + "---|" * (len(PARITY_COLUMNS) + 3)]
    for label, tol, errs in records:
        worst = max(errs.values()) if errs else 0.0
        cells = [f"{errs[c]:.2e}" if c in errs else "" for c in PARITY_COLUMNS]
        lines.append(f"| {label} | {tol:g} | " + " | ".join(cells) + f" | {worst / tol:.3f} |")
    return "\n".join(lines)
