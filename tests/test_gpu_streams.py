"""The binding on a caller's side stream: when the wrapper allocates the workspace itself (on the
current stream) and enqueues the layer on another stream, the caching allocator must not hand that
memory to an allocation on the current stream while the layer still uses it."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from chunked_prefill_hybrid_amd import layer as hl
from chunked_prefill_hybrid_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MID = wl.LayerShape("mid-llama", "llama", 512, 4, 128, 1408, "bf16", 1e-6, 10000.0, None)


def test_forward_on_side_stream_with_own_workspace():
    C, off, lens = 70, 30, [5, 300, 64]
    gu.say(f"case side-stream C={C} off={off} B={len(lens)}")
    rng = np.random.default_rng(5)
    w = wl.make_weights(MID, rng)
    b = wl.make_batch(MID, wl.BatchSpec(C, off, off + C, len(lens), decode_lens=tuple(lens)), rng)
    layer = hl.HybridLayer(MID, gu.upload_weights(MID, w), max_tokens=C + len(lens),
                           max_pos=max([off + C] + [L + 1 for L in lens]) + 8)
    db = gu.upload_batch(MID, b)
    need = layer.workspace_size(layer.batch(db["x"], db["y"], C, off, db["chunk_kv"], db["decode_kv"],
                                            db["decode_len"])[0])

    def fwd(stream=None):
        layer.forward(db["x"], db["y"], C, off, db["chunk_kv"], db["decode_kv"], db["decode_len"],
                      stream=stream)

    fwd()
    torch.cuda.synchronize()
    y_ref = db["y"].clone()

    side = torch.cuda.Stream()
    for rep in range(3):
        db["y"].fill_(float("nan"))
        side.wait_stream(torch.cuda.current_stream())
        fwd(stream=side)   # workspace allocated by the wrapper on the current stream, used on `side`
        # new allocations of the workspace's size on the current stream, written while the layer runs
        junk = [torch.empty(need, dtype=torch.uint8, device="cuda") for _ in range(4)]
        for _ in range(8):
            for j in junk:
                j.fill_(0xFF)
        del junk
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        assert torch.equal(db["y"], y_ref), f"replay {rep}: y differs on the side stream"
    layer.close()
