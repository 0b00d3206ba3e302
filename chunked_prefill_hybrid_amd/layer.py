"""Torch-facing wrapper of the C ABI: marshals device tensors into the library's structs.

PyTorch supplies device memory and streams only; every step of the layer runs in libsarathi.so.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import torch

from . import _abi

_DT = {"f32": (_abi.SARATHI_F32, torch.float32), "bf16": (_abi.SARATHI_BF16, torch.bfloat16)}


def _ptr(t: Optional[torch.Tensor], dtype=None) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _hold_for(t: torch.Tensor, stream) -> None:
    """Tell torch's caching allocator that `t` (a workspace this module allocated on the current
    stream) is in use by the work just enqueued on `stream`, so its memory is not handed to another
    allocation before that work ends.  Nothing to do when the work runs on the current stream."""
    if stream is None:
        return
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(_stream(stream))
    if s.cuda_stream != torch.cuda.current_stream().cuda_stream:
        t.record_stream(s)


def make_desc(shape, max_tokens: int, max_pos: int) -> _abi.sarathi_layer_desc:
    return _abi.sarathi_layer_desc(
        shape.hidden, shape.n_heads, shape.head_dim, shape.ffn,
        _abi.SARATHI_ARCH_LLAMA if shape.arch == "llama" else _abi.SARATHI_ARCH_GPT,
        _DT[shape.dtype][0], float(shape.norm_eps), float(shape.rope_base), int(max_tokens), int(max_pos))


KV = Tuple[torch.Tensor, torch.Tensor]   # (K, V), each [n_heads, capacity, head_dim]


class HybridLayer:
    """One decoder layer bound to caller-owned device weights.

    weights: dict with w_qkv [3A,H], w_o [H,A], w_gate [F,H] (llama), w_up [F,H], w_down [H,F] in the
    storage dtype, and float32 norm1_w, norm2_w (+ norm1_b, norm2_b for gpt).  A bf16 layer copies
    the five projection weights into its own packed layout at create; the norm weights (and every
    weight of a float32 layer) must stay alive and unchanged while the layer exists (the wrapper
    keeps references to all of them)."""

    def __init__(self, shape, weights: dict, max_tokens: int, max_pos: int):
        self.shape = shape
        self.dtype = _DT[shape.dtype][1]
        self.desc = make_desc(shape, max_tokens, max_pos)
        self._weights = dict(weights)
        dt = self.dtype
        w = _abi.sarathi_weights(
            _ptr(weights["w_qkv"], dt), _ptr(weights["w_o"], dt), _ptr(weights.get("w_gate"), dt),
            _ptr(weights["w_up"], dt), _ptr(weights["w_down"], dt),
            _ptr(weights["norm1_w"], torch.float32), _ptr(weights.get("norm1_b"), torch.float32),
            _ptr(weights["norm2_w"], torch.float32), _ptr(weights.get("norm2_b"), torch.float32))
        self.handle = _abi.sarathi_layer_create(self.desc, w)

    def close(self) -> None:
        if self.handle:
            _abi.sarathi_layer_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def batch(self, x: Optional[torch.Tensor], y: Optional[torch.Tensor], chunk_len: int,
              chunk_offset: int, chunk_kv: Optional[KV], decode_kv: Sequence[KV],
              decode_len: Sequence[int]):
        """(sarathi_batch, keepalive) for the given tensors."""
        dt = self.dtype
        ck = None
        if chunk_kv is not None and chunk_len > 0:
            ck = (_ptr(chunk_kv[0], dt), _ptr(chunk_kv[1], dt), chunk_kv[0].shape[1])
        dkv = [(_ptr(k, dt), _ptr(v, dt), k.shape[1]) for k, v in decode_kv]
        return _abi.make_batch(chunk_len, chunk_offset, ck, dkv, list(decode_len),
                               _ptr(x, dt), _ptr(y, dt))

    def workspace_size(self, batch) -> int:
        if isinstance(batch, _abi.sarathi_paged_batch):
            return _abi.sarathi_paged_workspace_size(self.desc, batch)
        if isinstance(batch, _abi.sarathi_multi_batch):
            return _abi.sarathi_multi_workspace_size(self.desc, batch)
        return _abi.sarathi_workspace_size(self.desc, batch)

    def multi_batch(self, x: Optional[torch.Tensor], y: Optional[torch.Tensor],
                    chunks: Sequence[Tuple[int, int, KV]], decode_kv: Sequence[KV],
                    decode_len: Sequence[int]):
        """(sarathi_multi_batch, keepalive).  chunks: list of (len, offset, (K, V)), rows in list
        order, then the decodes."""
        dt = self.dtype
        ch = [(ln, off, _ptr(kv[0], dt), _ptr(kv[1], dt), kv[0].shape[1]) for ln, off, kv in chunks]
        dkv = [(_ptr(k, dt), _ptr(v, dt), k.shape[1]) for k, v in decode_kv]
        return _abi.make_multi_batch(ch, dkv, list(decode_len), _ptr(x, dt), _ptr(y, dt))

    def paged_batch(self, x: Optional[torch.Tensor], y: Optional[torch.Tensor], pool: Tuple[torch.Tensor, torch.Tensor],
                    chunks: Sequence[Tuple[int, int, torch.Tensor]], decode_tables: Sequence[torch.Tensor],
                    decode_len: Sequence[int]):
        """(sarathi_paged_batch, keepalive).  pool: (K pool, V pool), each [n_pages, nh, page_size, d];
        chunks: list of (len, offset, block table); decode_tables: one block table per decode.  Block
        tables are int32 device tensors."""
        dt = self.dtype
        kp, vp = pool
        n_pages, page = kp.shape[0], kp.shape[2]
        ch = [(ln, off, _ptr(t, torch.int32), t.numel()) for ln, off, t in chunks]
        tb = [(_ptr(t, torch.int32), t.numel()) for t in decode_tables]
        return _abi.make_paged_batch((_ptr(kp, dt), _ptr(vp, dt), n_pages, page), ch, tb, list(decode_len),
                                     _ptr(x, dt), _ptr(y, dt))

    def forward_paged(self, x, y, pool, chunks, decode_tables, decode_len,
                      workspace: Optional[torch.Tensor] = None, stream=None, dump: Optional[dict] = None):
        """Enqueue the layer over a batch whose caches live in a page pool (see paged_batch)."""
        b, keep = self.paged_batch(x, y, pool, chunks, decode_tables, decode_len)
        need = _abi.sarathi_paged_workspace_size(self.desc, b)
        if need == 0:
            st = _abi.sarathi_paged_batch_check(self.desc, b)
            raise _abi.SarathiError(st, "paged batch", _abi.sarathi_last_error())
        own_ws = workspace is None
        if own_ws:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        ws_ptr = _ptr(workspace)
        nbytes = workspace.numel() * workspace.element_size()
        if dump:
            d = _abi.sarathi_debug_dump(*[_ptr(dump.get(n), torch.float32) for n in
                                          ("n1", "qkv", "q_rot", "attn", "h1", "n2", "act")])
            _abi.sarathi_paged_forward_debug(self.handle, b, ws_ptr, nbytes, _stream(stream), d)
        else:
            _abi.sarathi_paged_forward(self.handle, b, ws_ptr, nbytes, _stream(stream))
        if own_ws:
            _hold_for(workspace, stream)
        del keep
        return y

    def forward_multi(self, x, y, chunks, decode_kv, decode_len, workspace: Optional[torch.Tensor] = None,
                      stream=None, dump: Optional[dict] = None):
        """Enqueue the layer over a batch with several prefill chunks (see multi_batch); y and the
        caches are written in place.  dump as in forward."""
        b, keep = self.multi_batch(x, y, chunks, decode_kv, decode_len)
        need = _abi.sarathi_multi_workspace_size(self.desc, b)
        if need == 0:
            st = _abi.sarathi_multi_batch_check(self.desc, b)
            raise _abi.SarathiError(st, "multi batch", _abi.sarathi_last_error())
        own_ws = workspace is None
        if own_ws:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        ws_ptr = _ptr(workspace)
        nbytes = workspace.numel() * workspace.element_size()
        if dump:
            d = _abi.sarathi_debug_dump(*[_ptr(dump.get(n), torch.float32) for n in
                                          ("n1", "qkv", "q_rot", "attn", "h1", "n2", "act")])
            _abi.sarathi_multi_forward_debug(self.handle, b, ws_ptr, nbytes, _stream(stream), d)
        else:
            _abi.sarathi_multi_forward(self.handle, b, ws_ptr, nbytes, _stream(stream))
        if own_ws:
            _hold_for(workspace, stream)
        del keep
        return y

    def forward(self, x, y, chunk_len, chunk_offset, chunk_kv, decode_kv, decode_len,
                workspace: Optional[torch.Tensor] = None, stream=None, dump: Optional[dict] = None):
        """Enqueue the layer over one hybrid batch (y and the caches are written in place).
        dump: optional dict name -> float32 [C+B, width] tensor for the intermediates n1, qkv, q_rot,
        attn, h1, n2, act."""
        b, keep = self.batch(x, y, chunk_len, chunk_offset, chunk_kv, decode_kv, decode_len)
        need = self.workspace_size(b)
        if need == 0:
            st = _abi.sarathi_batch_check(self.desc, b)
            raise _abi.SarathiError(st, "batch", _abi.sarathi_last_error())
        own_ws = workspace is None
        if own_ws:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        ws_ptr = _ptr(workspace)
        nbytes = workspace.numel() * workspace.element_size()
        if dump:
            d = _abi.sarathi_debug_dump(*[_ptr(dump.get(n), torch.float32) for n in
                                          ("n1", "qkv", "q_rot", "attn", "h1", "n2", "act")])
            _abi.sarathi_layer_forward_debug(self.handle, b, ws_ptr, nbytes, _stream(stream), d)
        else:
            _abi.sarathi_layer_forward(self.handle, b, ws_ptr, nbytes, _stream(stream))
        if own_ws:
            _hold_for(workspace, stream)
        del keep
        return y


def gemm(a: torch.Tensor, w: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None):
    """out[M,N] = a[M,K] w[N,K]^T with the library's GEMM kernel."""
    m, k = a.shape
    n = w.shape[0]
    dt = _abi.SARATHI_BF16 if a.dtype == torch.bfloat16 else _abi.SARATHI_F32
    if out is None:
        out = torch.empty((m, n), dtype=a.dtype, device=a.device)
    _abi.sarathi_gemm(dt, m, n, k, _ptr(a, a.dtype), _ptr(w, a.dtype), _ptr(out, a.dtype), _stream(stream))
    return out


def attention(shape, q: torch.Tensor, out: torch.Tensor, chunk_len: int, chunk_offset: int,
              chunk_kv: Optional[KV], decode_kv: Sequence[KV], decode_len: Sequence[int],
              max_pos: int, stream=None):
    """The split attention alone over caches that already hold this step's K/V rows."""
    desc = make_desc(shape, q.shape[0], max_pos)
    dt = _DT[shape.dtype][1]
    ck = None
    if chunk_kv is not None and chunk_len > 0:
        ck = (_ptr(chunk_kv[0], dt), _ptr(chunk_kv[1], dt), chunk_kv[0].shape[1])
    dkv = [(_ptr(k, dt), _ptr(v, dt), k.shape[1]) for k, v in decode_kv]
    b, keep = _abi.make_batch(chunk_len, chunk_offset, ck, dkv, list(decode_len), 0, 0)
    need = _abi.sarathi_workspace_size(desc, b)
    if need == 0:
        raise _abi.SarathiError(_abi.sarathi_batch_check(desc, b), "batch", _abi.sarathi_last_error())
    ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    _abi.sarathi_attention(desc, b, _ptr(q, dt), _ptr(out, dt), _ptr(ws), need, _stream(stream))
    _hold_for(ws, stream)
    del keep
    return out


class HybridStack:
    """A stack of decoder layers run over one hybrid batch per call: every layer sees the same chunk
    and decodes, with its own KV caches; layer l's output rows are layer l+1's input rows (chained in
    the workspace, so only x and y are caller tensors).

    layers: HybridLayer objects of one hidden size and storage type (the stack keeps references)."""

    def __init__(self, layers: Sequence[HybridLayer]):
        if not layers:
            raise ValueError("a stack needs at least one layer")
        self.layers = list(layers)
        self.dtype = self.layers[0].dtype
        self._ws: Optional[torch.Tensor] = None

    def batch(self, x, y, chunk_len: int, chunk_offset: int, chunk_kv: Optional[Sequence[KV]],
              decode_kv: Sequence[Sequence[KV]], decode_len: Sequence[int]):
        """(sarathi_stack_batch, keepalive).  chunk_kv: per layer (K, V) or None; decode_kv: per
        layer, a list over decodes of (K, V)."""
        dt = self.dtype
        n = len(self.layers)
        ck = None
        if chunk_kv is not None and chunk_len > 0:
            if len(chunk_kv) != n:
                raise ValueError(f"chunk_kv has {len(chunk_kv)} layers, stack has {n}")
            ck = [(_ptr(k, dt), _ptr(v, dt), k.shape[1]) for k, v in chunk_kv]
        B = len(decode_len)
        dkv = []
        if B:
            if len(decode_kv) != n or any(len(row) != B for row in decode_kv):
                raise ValueError("decode_kv must hold one (K, V) per decode for every layer")
            dkv = [[(_ptr(k, dt), _ptr(v, dt), k.shape[1]) for k, v in row] for row in decode_kv]
        return _abi.make_stack_batch(chunk_len, chunk_offset, ck, dkv if B else None, list(decode_len),
                                     _ptr(x, dt), _ptr(y, dt))

    def workspace_size(self, batch) -> int:
        return _abi.sarathi_stack_workspace_size([l.handle for l in self.layers], batch)

    def forward(self, x, y, chunk_len, chunk_offset, chunk_kv, decode_kv, decode_len,
                workspace: Optional[torch.Tensor] = None, stream=None):
        """Enqueue all layers over one hybrid batch; y and every layer's caches are written in place.
        Without `workspace` the stack keeps one that grows to the largest batch seen."""
        b, keep = self.batch(x, y, chunk_len, chunk_offset, chunk_kv, decode_kv, decode_len)
        handles = [l.handle for l in self.layers]
        need = _abi.sarathi_stack_workspace_size(handles, b)
        if need == 0:
            # Re-run with reporting so the error names the offending layer and field.
            _abi.sarathi_stack_forward(handles, b, 0, 0, _stream(stream))
            raise RuntimeError("stack batch rejected")
        own_ws = workspace is None
        if own_ws:
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.empty(need, dtype=torch.uint8, device=x.device)
            workspace = self._ws
        _abi.sarathi_stack_forward(handles, b, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream))
        if own_ws:
            _hold_for(workspace, stream)
        del keep
        return y

    def close(self) -> None:
        for l in self.layers:
            l.close()
