"""The layer forward inside a HIP graph: the C ABI's forward enqueues kernels only (no allocation,
copy, memset or synchronisation), so a caller can capture it.  Each test captures one forward,
replays it several times with eager work and synchronisations in between, and checks every replay
bit for bit against the eager forward (a forward writes the same cache slots with the same values,
so replays are idempotent)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from chunked_prefill_hybrid_amd import layer as hl
from chunked_prefill_hybrid_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MID = wl.LayerShape("mid-llama", "llama", 512, 4, 128, 1408, "bf16", 1e-6, 10000.0, None)


@pytest.mark.parametrize("C,off,lens", [
    (70, 30, [5, 300, 64]),     # one launch of chunk and decode attention
    (64, 2100, []),             # a chunk whose key range is split, merged by a second kernel
])
def test_forward_replays_from_a_graph(C, off, lens):
    gu.say(f"case graph C={C} off={off} B={len(lens)}")
    rng = np.random.default_rng(C + off)
    w = wl.make_weights(MID, rng)
    b = wl.make_batch(MID, wl.BatchSpec(C, off, off + C, len(lens), decode_lens=tuple(lens)), rng)
    layer = hl.HybridLayer(MID, gu.upload_weights(MID, w), max_tokens=C + len(lens),
                           max_pos=max([off + C] + [L + 1 for L in lens]) + 8)
    db = gu.upload_batch(MID, b)
    ws = torch.empty(layer.workspace_size(layer.batch(db["x"], db["y"], C, off, db["chunk_kv"],
                                                      db["decode_kv"], db["decode_len"])[0]),
                     dtype=torch.uint8, device="cuda")

    def fwd():
        layer.forward(db["x"], db["y"], C, off, db["chunk_kv"], db["decode_kv"], db["decode_len"],
                      workspace=ws)

    fwd()
    torch.cuda.synchronize()
    y_eager = db["y"].clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()   # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    torch.cuda.synchronize()

    noise = torch.randn(512, 512, device="cuda")
    for rep in range(3):
        db["y"].fill_(float("nan"))
        for _ in range(4):
            noise = torch.tanh(noise @ noise.t() / 512.0)   # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(db["y"], y_eager), f"replay {rep}"
    del g
    layer.close()
