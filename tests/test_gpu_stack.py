"""GPU parity of the layer stack (sarathi_stack_forward) against the oracle's stack, through the C ABI.

A prompt is prefilled chunk by chunk through a stack of layers while decodes ride along in every step
(SARATHI: Efficient LLM Inference by Piggybacking Decodes with Chunked Prefills, section 3): the GPU
and the oracle each run the whole schedule from the same seeded inputs and keep their own caches, so
a wrong cache row in any layer shows up in later steps.  Unused cache slots are NaN.
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_prefill_hybrid_amd import layer as hl
from chunked_prefill_hybrid_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MID = wl.LayerShape("mid-llama", "llama", 512, 4, 128, 1408, "bf16", 1e-6, 10000.0, None)
MID_GPT = wl.LayerShape("mid-gpt", "gpt", 512, 4, 128, 1024, "bf16", 1e-5, 10000.0, None)


def schedule(shape, n_layers, P, C, lens0, seed):
    """Seeded weights per layer, prompt rows, per-step decode rows and per-layer caches (host)."""
    rng = np.random.default_rng(seed)
    nh, d, H = shape.n_heads, shape.head_dim, shape.hidden
    rnd = (lambda a: wl.bf16_round(a.astype(np.float32))) if shape.dtype == "bf16" else \
        (lambda a: a.astype(np.float32))
    W = [wl.make_weights(shape, rng) for _ in range(n_layers)]
    steps = (P + C - 1) // C
    xp = rnd(rng.standard_normal((P, H)))
    xd = rnd(rng.standard_normal((steps, len(lens0), H)))
    ck = [np.full((nh, P + 3, d), np.nan, np.float32) for _ in range(n_layers)]
    cv = [np.full((nh, P + 3, d), np.nan, np.float32) for _ in range(n_layers)]

    def dcache(L):
        c = np.full((nh, L + steps + 2, d), np.nan, np.float32)
        c[:, :L] = rnd(rng.standard_normal((nh, L, d)))
        return c
    dk = [[dcache(L) for L in lens0] for _ in range(n_layers)]
    dv = [[dcache(L) for L in lens0] for _ in range(n_layers)]
    return W, xp, xd, ck, cv, dk, dv


def run_schedule(shape, n_layers, P, C, lens0, seed, label):
    W, xp, xd, ck, cv, dk, dv = schedule(shape, n_layers, P, C, lens0, seed)
    dt = gu.tdtype(shape)
    steps = (P + C - 1) // C
    T = C + len(lens0)
    layers = [hl.HybridLayer(shape, gu.upload_weights(shape, w), max_tokens=T,
                             max_pos=max([P] + [L + steps for L in lens0]) + 4) for w in W]
    stack = hl.HybridStack(layers)
    gck = [gu.dev(c, dt) for c in ck]
    gcv = [gu.dev(c, dt) for c in cv]
    gdk = [[gu.dev(c, dt) for c in row] for row in dk]
    gdv = [[gu.dev(c, dt) for c in row] for row in dv]
    host = {"chunk_k": ck, "chunk_v": cv, "decode_k": dk, "decode_v": dv}
    tol = gu.TOL[shape.dtype]
    for s in range(steps):
        c = min(C, P - s * C)
        lens = [L + s for L in lens0]
        gu.say(f"case {label} step {s}: chunk {c} at {s * C}, decodes {lens}")
        x = np.concatenate([xp[s * C:s * C + c], xd[s]])
        b = dict(host, x=x, chunk_len=c, chunk_offset=s * C, decode_len=lens)
        ref = oracle.stack_forward(shape, W, b)
        gx = gu.dev(x, dt)
        gy = torch.full_like(gx, float("nan"))
        stack.forward(gx, gy, c, s * C, list(zip(gck, gcv)),
                      [list(zip(gdk[l], gdv[l])) for l in range(n_layers)], lens)
        torch.cuda.synchronize()
        y = gy.float().cpu().numpy()
        # dY of the last layer against the oracle's input to it (reported; earlier layers' errors
        # reach it through the residual, so only y and the cache rows are held to the tolerance)
        last_x = ref["layers"][-2]["y"] if n_layers > 1 else x
        info = {"dy_last": gu.rel(y - last_x, ref["y"] - last_x)}
        errs = {"y": gu.rel(y, ref["y"])}
        for l in range(n_layers):
            nk = np.concatenate([gck[l][:, s * C:s * C + c].permute(1, 0, 2).float().cpu().numpy()] +
                                [gdk[l][i][:, L:L + 1].permute(1, 0, 2).float().cpu().numpy()
                                 for i, L in enumerate(lens)])
            nv = np.concatenate([gcv[l][:, s * C:s * C + c].permute(1, 0, 2).float().cpu().numpy()] +
                                [gdv[l][i][:, L:L + 1].permute(1, 0, 2).float().cpu().numpy()
                                 for i, L in enumerate(lens)])
            errs[f"k{l}"] = gu.rel(nk, ref["layers"][l]["new_k"])
            errs[f"v{l}"] = gu.rel(nv, ref["layers"][l]["new_v"])
        gu.say(f"[{label} step {s}] " + " ".join(f"{k}={v:.2e}" for k, v in {**errs, **info}.items()))
        bad = {k: v for k, v in errs.items() if not (v <= tol)}
        assert not bad, f"{label} step {s}: over tolerance {tol}: {bad}"
        oracle.apply_stack_rows(b, ref)
    stack.close()


def test_stack_tiny_fp32_prompt_in_chunks_with_decodes():
    run_schedule(wl.SHAPES["tiny"], 3, 96, 32, [17, 40], seed=5, label="tiny f32 3 layers")


def test_stack_mid_bf16_prompt_in_chunks_with_decodes():
    run_schedule(MID, 2, 300, 128, [60, 200, 333], seed=6, label="mid bf16 2 layers")


def test_stack_mid_gpt_bf16():
    run_schedule(MID_GPT, 2, 160, 96, [7, 150], seed=7, label="mid gpt bf16 2 layers")


def test_stack_chunked_equals_monolithic_on_gpu():
    """The same 96-token prompt through a 2-layer fp32 stack as 3 chunks of 32 and as one chunk of
    96: outputs and every layer's cache agree to float32 tolerance."""
    shape = wl.SHAPES["tiny"]
    gu.say("case stack chunked vs monolithic, tiny f32 2 layers, P=96")
    rng = np.random.default_rng(9)
    nh, d, H = shape.n_heads, shape.head_dim, shape.hidden
    W = [wl.make_weights(shape, rng) for _ in range(2)]
    xp = gu.dev(rng.standard_normal((96, H)).astype(np.float32), torch.float32)
    stacks, caches, ys = [], [], []
    for chunk in (32, 96):
        layers = [hl.HybridLayer(shape, gu.upload_weights(shape, w), max_tokens=96, max_pos=128) for w in W]
        st = hl.HybridStack(layers)
        kv = [(torch.full((nh, 96, d), float("nan"), device="cuda"),
               torch.full((nh, 96, d), float("nan"), device="cuda")) for _ in range(2)]
        y = torch.full((96, H), float("nan"), device="cuda")
        for s in range(96 // chunk):
            st.forward(xp[s * chunk:(s + 1) * chunk].contiguous(), y[s * chunk:(s + 1) * chunk],
                       chunk, s * chunk, kv, [], [])
        torch.cuda.synchronize()
        stacks.append(st)
        caches.append(kv)
        ys.append(y.cpu().numpy())
    errs = {"y": gu.rel(ys[0], ys[1])}
    for l in range(2):
        errs[f"k{l}"] = gu.rel(caches[0][l][0].cpu().numpy(), caches[1][l][0].cpu().numpy())
        errs[f"v{l}"] = gu.rel(caches[0][l][1].cpu().numpy(), caches[1][l][1].cpu().numpy())
    gu.say(" ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= 1e-4 for v in errs.values()), errs
    for st in stacks:
        st.close()


@pytest.mark.parametrize("shape", [MID, MID_GPT, wl.SHAPES["tiny"]], ids=["llama-bf16", "gpt-bf16", "tiny-f32"])
def test_stack_equals_layers_run_one_by_one(shape):
    """A 3-layer stack, whose layers end with the next layer's norm 1 fused into their output sum,
    gives bit for bit what the three single-layer forwards give when chained by hand (each with its
    own norm 1), output and caches."""
    gu.say(f"case stack vs chained layers {shape.name}")
    rng = np.random.default_rng(31)
    nh, d, H = shape.n_heads, shape.head_dim, shape.hidden
    dt = gu.tdtype(shape)
    n_layers, C, off, lens = 3, 70, 40, [5, 90]
    W = [wl.make_weights(shape, rng) for _ in range(n_layers)]
    layers = [hl.HybridLayer(shape, gu.upload_weights(shape, w), max_tokens=C + len(lens), max_pos=256)
              for w in W]

    def caches():
        g = torch.Generator(device="cpu").manual_seed(3)
        mk = lambda n: torch.randn((nh, n, d), generator=g).to(dt).to("cuda")
        return [(mk(off + C), mk(off + C)) for _ in range(n_layers)], \
               [[(mk(L + 1), mk(L + 1)) for L in lens] for _ in range(n_layers)]
    x = gu.dev(rng.standard_normal((C + len(lens), H)).astype(np.float32), dt)
    ck1, dk1 = caches()
    ck2, dk2 = caches()
    y_stack = torch.full_like(x, float("nan"))
    stack = hl.HybridStack(layers)
    stack.forward(x, y_stack, C, off, ck1, dk1, lens)
    cur = x
    for l in range(n_layers):
        y = torch.full_like(x, float("nan"))
        layers[l].forward(cur, y, C, off, ck2[l], dk2[l], lens)
        cur = y
    torch.cuda.synchronize()
    assert torch.equal(y_stack, cur), "stack output differs from the chained layers"
    for l in range(n_layers):
        assert torch.equal(ck1[l][0], ck2[l][0]) and torch.equal(ck1[l][1], ck2[l][1]), f"layer {l} chunk cache"
        for i in range(len(lens)):
            assert torch.equal(dk1[l][i][0], dk2[l][i][0]) and torch.equal(dk1[l][i][1], dk2[l][i][1]), \
                f"layer {l} decode {i} cache"
    stack.close()
