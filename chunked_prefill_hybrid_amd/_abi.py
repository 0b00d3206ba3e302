"""ctypes binding of libsarathi.so (the C ABI of include/sarathi.h).

Argument marshalling only: every step of the layer runs in the library's HIP kernels.  Functions keep
the C names (sarathi_layer_create, sarathi_layer_forward, ...).  Loading fails loudly when the
library has not been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_float, c_int32, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsarathi.so")

SARATHI_OK = 0
SARATHI_ERR_INVALID = -1
SARATHI_ERR_UNSUPPORTED = -2
SARATHI_ERR_CAPACITY = -3
SARATHI_ERR_HIP = -4
SARATHI_ERR_NOMEM = -5
SARATHI_ERR_WORKSPACE = -6
SARATHI_ERR_INTERNAL = -7

SARATHI_F32 = 0
SARATHI_BF16 = 1
SARATHI_ARCH_LLAMA = 0
SARATHI_ARCH_GPT = 1

EXPORTED = [
    "sarathi_layer_create", "sarathi_layer_destroy", "sarathi_batch_check", "sarathi_workspace_size",
    "sarathi_layer_forward", "sarathi_layer_forward_debug", "sarathi_layer_forward_noalloc",
    "sarathi_gemm", "sarathi_attention", "sarathi_clock_sample",
    "sarathi_status_str", "sarathi_last_error", "sarathi_timer_create", "sarathi_timer_destroy",
    "sarathi_layer_forward_timed", "sarathi_timer_read", "sarathi_stack_workspace_size",
    "sarathi_stack_forward", "sarathi_multi_batch_check", "sarathi_multi_workspace_size",
    "sarathi_multi_forward", "sarathi_multi_forward_debug", "sarathi_multi_forward_timed",
    "sarathi_paged_batch_check", "sarathi_paged_workspace_size", "sarathi_paged_forward",
    "sarathi_paged_forward_debug", "sarathi_paged_forward_timed",
    "sarathi_plan_describe", "sarathi_multi_plan_describe", "sarathi_paged_plan_describe",
]

SARATHI_MAX_CHUNKS = 16

STAGES = ["norm1", "qkv", "rope_append", "attn_chunk", "attn_decode", "attn_merge", "o", "norm2",
          "ffn_up", "ffn_down"]
N_STAGES = len(STAGES)


class sarathi_layer_desc(ctypes.Structure):
    _fields_ = [("hidden", c_int32), ("n_heads", c_int32), ("head_dim", c_int32), ("ffn", c_int32),
                ("arch", c_int32), ("dtype", c_int32), ("norm_eps", c_float), ("rope_base", c_float),
                ("max_tokens", c_int32), ("max_pos", c_int32)]


class sarathi_weights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("w_qkv", "w_o", "w_gate", "w_up", "w_down",
                                        "norm1_w", "norm1_b", "norm2_w", "norm2_b")]


class sarathi_kv(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("capacity", c_int32), ("reserved", c_int32)]


class sarathi_batch(ctypes.Structure):
    _fields_ = [("chunk_len", c_int32), ("chunk_offset", c_int32), ("chunk_kv", sarathi_kv),
                ("n_decodes", c_int32), ("reserved", c_int32),
                ("decode_kv", POINTER(sarathi_kv)), ("decode_len", POINTER(c_int32)),
                ("x", c_void_p), ("y", c_void_p)]


class sarathi_stack_batch(ctypes.Structure):
    _fields_ = [("chunk_len", c_int32), ("chunk_offset", c_int32), ("chunk_kv", POINTER(sarathi_kv)),
                ("n_decodes", c_int32), ("reserved", c_int32), ("decode_kv", POINTER(sarathi_kv)),
                ("decode_len", POINTER(c_int32)), ("x", c_void_p), ("y", c_void_p)]


class sarathi_chunk(ctypes.Structure):
    _fields_ = [("len", c_int32), ("offset", c_int32), ("kv", sarathi_kv)]


class sarathi_multi_batch(ctypes.Structure):
    _fields_ = [("n_chunks", c_int32), ("reserved", c_int32), ("chunks", POINTER(sarathi_chunk)),
                ("n_decodes", c_int32), ("reserved2", c_int32), ("decode_kv", POINTER(sarathi_kv)),
                ("decode_len", POINTER(c_int32)), ("x", c_void_p), ("y", c_void_p)]


class sarathi_page_pool(ctypes.Structure):
    _fields_ = [("k_pool", c_void_p), ("v_pool", c_void_p), ("n_pages", c_int32), ("page_size", c_int32)]


class sarathi_page_table(ctypes.Structure):
    _fields_ = [("pages", c_void_p), ("n_entries", c_int32), ("reserved", c_int32)]


class sarathi_paged_chunk(ctypes.Structure):
    _fields_ = [("len", c_int32), ("offset", c_int32), ("table", sarathi_page_table)]


class sarathi_paged_batch(ctypes.Structure):
    _fields_ = [("pool", sarathi_page_pool), ("n_chunks", c_int32), ("reserved", c_int32),
                ("chunks", POINTER(sarathi_paged_chunk)), ("n_decodes", c_int32), ("reserved2", c_int32),
                ("decode_tables", POINTER(sarathi_page_table)), ("decode_len", POINTER(c_int32)),
                ("x", c_void_p), ("y", c_void_p)]


class sarathi_gemm_plan(ctypes.Structure):
    _fields_ = [("epilogue", c_int32), ("row_tiles", c_int32), ("col_tiles", c_int32), ("k_splits", c_int32),
                ("tile_cols", c_int32)]


class sarathi_plan_info(ctypes.Structure):
    _fields_ = [("rows", c_int32), ("rows_alloc", c_int32), ("n_chunks", c_int32),
                ("fused_attention", c_int32), ("chunk_splits", c_int32 * SARATHI_MAX_CHUNKS),
                ("max_key_splits", c_int32), ("chunk_query_blocks", c_int32),
                ("qkv", sarathi_gemm_plan), ("o", sarathi_gemm_plan), ("up", sarathi_gemm_plan),
                ("down", sarathi_gemm_plan), ("up_tail", sarathi_gemm_plan),
                ("workspace_bytes", ctypes.c_uint64)]


class sarathi_debug_dump(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("n1", "qkv", "q_rot", "attn", "h1", "n2", "act")]


class SarathiError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: status {status} ({sarathi_status_str(status)}): {message}")
        self.status = status


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m chunked_prefill_hybrid_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.sarathi_layer_create.argtypes = [POINTER(sarathi_layer_desc), POINTER(sarathi_weights),
                                           POINTER(c_void_p)]
        L.sarathi_layer_create.restype = c_int32
        L.sarathi_layer_destroy.argtypes = [c_void_p]
        L.sarathi_layer_destroy.restype = None
        L.sarathi_batch_check.argtypes = [POINTER(sarathi_layer_desc), POINTER(sarathi_batch)]
        L.sarathi_batch_check.restype = c_int32
        L.sarathi_workspace_size.argtypes = [POINTER(sarathi_layer_desc), POINTER(sarathi_batch)]
        L.sarathi_workspace_size.restype = c_size_t
        L.sarathi_layer_forward.argtypes = [c_void_p, POINTER(sarathi_batch), c_void_p, c_size_t, c_void_p]
        L.sarathi_layer_forward.restype = c_int32
        L.sarathi_layer_forward_noalloc.argtypes = [c_void_p, POINTER(sarathi_batch), c_void_p]
        L.sarathi_layer_forward_noalloc.restype = c_int32
        L.sarathi_layer_forward_debug.argtypes = [c_void_p, POINTER(sarathi_batch), c_void_p, c_size_t,
                                                  c_void_p, POINTER(sarathi_debug_dump)]
        L.sarathi_layer_forward_debug.restype = c_int32
        L.sarathi_gemm.argtypes = [c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]
        L.sarathi_gemm.restype = c_int32
        L.sarathi_attention.argtypes = [POINTER(sarathi_layer_desc), POINTER(sarathi_batch), c_void_p,
                                        c_void_p, c_void_p, c_size_t, c_void_p]
        L.sarathi_attention.restype = c_int32
        L.sarathi_timer_create.argtypes = [c_int32, ctypes.c_uint32, POINTER(c_void_p)]
        L.sarathi_timer_create.restype = c_int32
        L.sarathi_timer_destroy.argtypes = [c_void_p]
        L.sarathi_timer_destroy.restype = None
        L.sarathi_layer_forward_timed.argtypes = [c_void_p, POINTER(sarathi_batch), c_void_p, c_size_t,
                                                  c_void_p, c_void_p]
        L.sarathi_layer_forward_timed.restype = c_int32
        L.sarathi_timer_read.argtypes = [c_void_p, POINTER(ctypes.c_double), POINTER(c_int32)]
        L.sarathi_timer_read.restype = c_int32
        L.sarathi_stack_workspace_size.argtypes = [POINTER(c_void_p), c_int32, POINTER(sarathi_stack_batch)]
        L.sarathi_stack_workspace_size.restype = c_size_t
        L.sarathi_stack_forward.argtypes = [POINTER(c_void_p), c_int32, POINTER(sarathi_stack_batch),
                                            c_void_p, c_size_t, c_void_p]
        L.sarathi_stack_forward.restype = c_int32
        MB = POINTER(sarathi_multi_batch)
        L.sarathi_multi_batch_check.argtypes = [POINTER(sarathi_layer_desc), MB]
        L.sarathi_multi_batch_check.restype = c_int32
        L.sarathi_multi_workspace_size.argtypes = [POINTER(sarathi_layer_desc), MB]
        L.sarathi_multi_workspace_size.restype = c_size_t
        L.sarathi_multi_forward.argtypes = [c_void_p, MB, c_void_p, c_size_t, c_void_p]
        L.sarathi_multi_forward.restype = c_int32
        L.sarathi_multi_forward_debug.argtypes = [c_void_p, MB, c_void_p, c_size_t, c_void_p,
                                                  POINTER(sarathi_debug_dump)]
        L.sarathi_multi_forward_debug.restype = c_int32
        L.sarathi_multi_forward_timed.argtypes = [c_void_p, MB, c_void_p, c_size_t, c_void_p, c_void_p]
        L.sarathi_multi_forward_timed.restype = c_int32
        PB = POINTER(sarathi_paged_batch)
        L.sarathi_paged_batch_check.argtypes = [POINTER(sarathi_layer_desc), PB]
        L.sarathi_paged_batch_check.restype = c_int32
        L.sarathi_paged_workspace_size.argtypes = [POINTER(sarathi_layer_desc), PB]
        L.sarathi_paged_workspace_size.restype = c_size_t
        L.sarathi_paged_forward.argtypes = [c_void_p, PB, c_void_p, c_size_t, c_void_p]
        L.sarathi_paged_forward.restype = c_int32
        L.sarathi_paged_forward_debug.argtypes = [c_void_p, PB, c_void_p, c_size_t, c_void_p,
                                                  POINTER(sarathi_debug_dump)]
        L.sarathi_paged_forward_debug.restype = c_int32
        L.sarathi_paged_forward_timed.argtypes = [c_void_p, PB, c_void_p, c_size_t, c_void_p, c_void_p]
        L.sarathi_paged_forward_timed.restype = c_int32
        PI = POINTER(sarathi_plan_info)
        L.sarathi_plan_describe.argtypes = [POINTER(sarathi_layer_desc), POINTER(sarathi_batch), PI]
        L.sarathi_plan_describe.restype = c_int32
        L.sarathi_multi_plan_describe.argtypes = [POINTER(sarathi_layer_desc), MB, PI]
        L.sarathi_multi_plan_describe.restype = c_int32
        L.sarathi_paged_plan_describe.argtypes = [POINTER(sarathi_layer_desc), PB, PI]
        L.sarathi_paged_plan_describe.restype = c_int32
        L.sarathi_clock_sample.argtypes = [c_void_p, c_void_p]
        L.sarathi_clock_sample.restype = c_int32
        L.sarathi_status_str.argtypes = [c_int32]
        L.sarathi_status_str.restype = c_char_p
        L.sarathi_last_error.argtypes = []
        L.sarathi_last_error.restype = c_char_p
        _lib = L
    return _lib


def sarathi_clock_sample(out: int, stream: int) -> None:
    """Enqueue a sample of (shader-clock timestamp, 100 MHz real-time counter) into device uint64[2]."""
    _check(lib().sarathi_clock_sample(out, stream), "sarathi_clock_sample")


def sarathi_status_str(status: int) -> str:
    return lib().sarathi_status_str(status).decode()


def sarathi_last_error() -> str:
    return lib().sarathi_last_error().decode()


def _check(status: int, where: str) -> None:
    if status != SARATHI_OK:
        raise SarathiError(status, where, sarathi_last_error())


def sarathi_layer_create(desc: sarathi_layer_desc, weights: sarathi_weights) -> int:
    h = c_void_p()
    _check(lib().sarathi_layer_create(byref(desc), byref(weights), byref(h)), "sarathi_layer_create")
    return h.value


def sarathi_layer_destroy(handle: int) -> None:
    lib().sarathi_layer_destroy(handle)


def sarathi_batch_check(desc: sarathi_layer_desc, batch: sarathi_batch) -> int:
    return lib().sarathi_batch_check(byref(desc), byref(batch))


def sarathi_workspace_size(desc: sarathi_layer_desc, batch: sarathi_batch) -> int:
    return lib().sarathi_workspace_size(byref(desc), byref(batch))


def sarathi_layer_forward(handle: int, batch: sarathi_batch, ws: int, ws_bytes: int, stream: int) -> None:
    _check(lib().sarathi_layer_forward(handle, byref(batch), ws, ws_bytes, stream), "sarathi_layer_forward")


def sarathi_layer_forward_noalloc(handle: int, batch: sarathi_batch, stream: int) -> None:
    """The layer forward on the library's fixed 128 MiB device scratch (no workspace argument)."""
    _check(lib().sarathi_layer_forward_noalloc(handle, byref(batch), stream), "sarathi_layer_forward_noalloc")


NOALLOC_SCRATCH_BYTES = 128 << 20


def sarathi_layer_forward_debug(handle: int, batch: sarathi_batch, ws: int, ws_bytes: int, stream: int,
                                dump: sarathi_debug_dump) -> None:
    _check(lib().sarathi_layer_forward_debug(handle, byref(batch), ws, ws_bytes, stream, byref(dump)),
           "sarathi_layer_forward_debug")


def sarathi_gemm(dtype: int, m: int, n: int, k: int, a: int, w: int, out: int, stream: int) -> None:
    _check(lib().sarathi_gemm(dtype, m, n, k, a, w, out, stream), "sarathi_gemm")


def sarathi_attention(desc: sarathi_layer_desc, batch: sarathi_batch, q: int, out: int, ws: int,
                      ws_bytes: int, stream: int) -> None:
    _check(lib().sarathi_attention(byref(desc), byref(batch), q, out, ws, ws_bytes, stream),
           "sarathi_attention")


ALL_STAGES = (1 << N_STAGES) - 1


def stage_mask(*names) -> int:
    return sum(1 << STAGES.index(n) for n in names)


def sarathi_timer_create(capacity: int, mask: int = ALL_STAGES) -> int:
    h = c_void_p()
    _check(lib().sarathi_timer_create(capacity, mask, byref(h)), "sarathi_timer_create")
    return h.value


def sarathi_timer_destroy(timer: int) -> None:
    lib().sarathi_timer_destroy(timer)


def sarathi_layer_forward_timed(handle: int, batch: sarathi_batch, ws: int, ws_bytes: int, stream: int,
                                timer: int) -> None:
    _check(lib().sarathi_layer_forward_timed(handle, byref(batch), ws, ws_bytes, stream, timer),
           "sarathi_layer_forward_timed")


def sarathi_timer_read(timer: int):
    """{stage name: (total_ms, count)} over the forwards recorded since the last read."""
    tot = (ctypes.c_double * N_STAGES)()
    cnt = (c_int32 * N_STAGES)()
    _check(lib().sarathi_timer_read(timer, tot, cnt), "sarathi_timer_read")
    return {STAGES[i]: (tot[i], cnt[i]) for i in range(N_STAGES)}


def _handles(handles):
    arr = (c_void_p * max(len(handles), 1))(*[h or 0 for h in handles])
    return arr, len(handles)


def sarathi_stack_workspace_size(handles, batch: sarathi_stack_batch) -> int:
    arr, n = _handles(handles)
    return lib().sarathi_stack_workspace_size(ctypes.cast(arr, POINTER(c_void_p)), n, byref(batch))


def sarathi_stack_forward(handles, batch: sarathi_stack_batch, ws: int, ws_bytes: int, stream: int) -> None:
    arr, n = _handles(handles)
    _check(lib().sarathi_stack_forward(ctypes.cast(arr, POINTER(c_void_p)), n, byref(batch), ws,
                                       ws_bytes, stream), "sarathi_stack_forward")


def make_stack_batch(chunk_len: int, chunk_offset: int, chunk_kv, decode_kv, decode_len, x: int, y: int):
    """Build a sarathi_stack_batch.  chunk_kv: list over layers of (k_ptr, v_ptr, capacity), or None;
    decode_kv: list over layers of lists over decodes of (k_ptr, v_ptr, capacity); decode_len: list
    of ints.  Returns (batch, keepalive) as make_batch."""
    B = len(decode_len)
    n_layers = len(decode_kv) if decode_kv else (len(chunk_kv) if chunk_kv else 0)
    ck_arr = (sarathi_kv * max(n_layers, 1))()
    if chunk_kv:
        for l, (k, v, cap) in enumerate(chunk_kv):
            ck_arr[l] = sarathi_kv(k, v, int(cap), 0)
    dk_arr = (sarathi_kv * max(n_layers * B, 1))()
    for l in range(n_layers if B else 0):
        for i, (k, v, cap) in enumerate(decode_kv[l]):
            dk_arr[l * B + i] = sarathi_kv(k, v, int(cap), 0)
    len_arr = (c_int32 * max(B, 1))(*[int(L) for L in decode_len])
    b = sarathi_stack_batch(int(chunk_len), int(chunk_offset),
                            ctypes.cast(ck_arr, POINTER(sarathi_kv)) if chunk_kv else None, B, 0,
                            ctypes.cast(dk_arr, POINTER(sarathi_kv)) if B else None,
                            ctypes.cast(len_arr, POINTER(c_int32)), x or 0, y or 0)
    return b, (ck_arr, dk_arr, len_arr)


def make_batch(chunk_len: int, chunk_offset: int, chunk_kv, decode_kv, decode_len, x: int, y: int):
    """Build a sarathi_batch.  chunk_kv: (k_ptr, v_ptr, capacity) or None; decode_kv: list of
    (k_ptr, v_ptr, capacity); decode_len: list of ints.  Returns (batch, keepalive) — keep the second
    value alive while the batch is used (it owns the host arrays the batch points to)."""
    B = len(decode_len)
    kv_arr = (sarathi_kv * max(B, 1))()
    len_arr = (c_int32 * max(B, 1))()
    for i, ((k, v, cap), L) in enumerate(zip(decode_kv, decode_len)):
        kv_arr[i] = sarathi_kv(k, v, int(cap), 0)
        len_arr[i] = int(L)
    ck = sarathi_kv(0, 0, 0, 0) if chunk_kv is None else sarathi_kv(chunk_kv[0], chunk_kv[1], int(chunk_kv[2]), 0)
    b = sarathi_batch(int(chunk_len), int(chunk_offset), ck, B, 0,
                      ctypes.cast(kv_arr, POINTER(sarathi_kv)), ctypes.cast(len_arr, POINTER(c_int32)),
                      x or 0, y or 0)
    return b, (kv_arr, len_arr)


def sarathi_multi_batch_check(desc: sarathi_layer_desc, batch: sarathi_multi_batch) -> int:
    return lib().sarathi_multi_batch_check(byref(desc), byref(batch))


def sarathi_multi_workspace_size(desc: sarathi_layer_desc, batch: sarathi_multi_batch) -> int:
    return lib().sarathi_multi_workspace_size(byref(desc), byref(batch))


def sarathi_multi_forward(handle: int, batch: sarathi_multi_batch, ws: int, ws_bytes: int, stream: int) -> None:
    _check(lib().sarathi_multi_forward(handle, byref(batch), ws, ws_bytes, stream), "sarathi_multi_forward")


def sarathi_multi_forward_debug(handle: int, batch: sarathi_multi_batch, ws: int, ws_bytes: int, stream: int,
                                dump: sarathi_debug_dump) -> None:
    _check(lib().sarathi_multi_forward_debug(handle, byref(batch), ws, ws_bytes, stream, byref(dump)),
           "sarathi_multi_forward_debug")


def sarathi_multi_forward_timed(handle: int, batch: sarathi_multi_batch, ws: int, ws_bytes: int, stream: int,
                                timer: int) -> None:
    _check(lib().sarathi_multi_forward_timed(handle, byref(batch), ws, ws_bytes, stream, timer),
           "sarathi_multi_forward_timed")


def make_multi_batch(chunks, decode_kv, decode_len, x: int, y: int):
    """Build a sarathi_multi_batch.  chunks: list of (len, offset, k_ptr, v_ptr, capacity);
    decode_kv: list of (k_ptr, v_ptr, capacity); decode_len: list of ints.  Returns (batch, keepalive)
    as make_batch."""
    n = len(chunks)
    ch_arr = (sarathi_chunk * max(n, 1))()
    for j, (ln, off, k, v, cap) in enumerate(chunks):
        ch_arr[j] = sarathi_chunk(int(ln), int(off), sarathi_kv(k, v, int(cap), 0))
    B = len(decode_len)
    kv_arr = (sarathi_kv * max(B, 1))()
    len_arr = (c_int32 * max(B, 1))()
    for i, ((k, v, cap), L) in enumerate(zip(decode_kv, decode_len)):
        kv_arr[i] = sarathi_kv(k, v, int(cap), 0)
        len_arr[i] = int(L)
    b = sarathi_multi_batch(n, 0, ctypes.cast(ch_arr, POINTER(sarathi_chunk)) if n else None, B, 0,
                            ctypes.cast(kv_arr, POINTER(sarathi_kv)) if B else None,
                            ctypes.cast(len_arr, POINTER(c_int32)), x or 0, y or 0)
    return b, (ch_arr, kv_arr, len_arr)


def sarathi_paged_batch_check(desc: sarathi_layer_desc, batch: sarathi_paged_batch) -> int:
    return lib().sarathi_paged_batch_check(byref(desc), byref(batch))


def sarathi_paged_workspace_size(desc: sarathi_layer_desc, batch: sarathi_paged_batch) -> int:
    return lib().sarathi_paged_workspace_size(byref(desc), byref(batch))


def sarathi_paged_forward(handle: int, batch: sarathi_paged_batch, ws: int, ws_bytes: int, stream: int) -> None:
    _check(lib().sarathi_paged_forward(handle, byref(batch), ws, ws_bytes, stream), "sarathi_paged_forward")


def sarathi_paged_forward_debug(handle: int, batch: sarathi_paged_batch, ws: int, ws_bytes: int, stream: int,
                                dump: sarathi_debug_dump) -> None:
    _check(lib().sarathi_paged_forward_debug(handle, byref(batch), ws, ws_bytes, stream, byref(dump)),
           "sarathi_paged_forward_debug")


def sarathi_paged_forward_timed(handle: int, batch: sarathi_paged_batch, ws: int, ws_bytes: int, stream: int,
                                timer: int) -> None:
    _check(lib().sarathi_paged_forward_timed(handle, byref(batch), ws, ws_bytes, stream, timer),
           "sarathi_paged_forward_timed")


def make_paged_batch(pool, chunks, decode_tables, decode_len, x: int, y: int):
    """Build a sarathi_paged_batch.  pool: (k_pool_ptr, v_pool_ptr, n_pages, page_size); chunks: list
    of (len, offset, table_ptr, n_entries); decode_tables: list of (table_ptr, n_entries); decode_len:
    list of ints.  Returns (batch, keepalive) as make_batch."""
    n = len(chunks)
    ch_arr = (sarathi_paged_chunk * max(n, 1))()
    for j, (ln, off, tp, ne) in enumerate(chunks):
        ch_arr[j] = sarathi_paged_chunk(int(ln), int(off), sarathi_page_table(tp, int(ne), 0))
    B = len(decode_len)
    tb_arr = (sarathi_page_table * max(B, 1))()
    len_arr = (c_int32 * max(B, 1))()
    for i, ((tp, ne), L) in enumerate(zip(decode_tables, decode_len)):
        tb_arr[i] = sarathi_page_table(tp, int(ne), 0)
        len_arr[i] = int(L)
    b = sarathi_paged_batch(sarathi_page_pool(pool[0], pool[1], int(pool[2]), int(pool[3])), n, 0,
                            ctypes.cast(ch_arr, POINTER(sarathi_paged_chunk)) if n else None, B, 0,
                            ctypes.cast(tb_arr, POINTER(sarathi_page_table)) if B else None,
                            ctypes.cast(len_arr, POINTER(c_int32)), x or 0, y or 0)
    return b, (ch_arr, tb_arr, len_arr)


def plan_describe(desc: sarathi_layer_desc, batch) -> sarathi_plan_info:
    """The launch plan of a forward over a single-chunk, multi-chunk or paged batch (host only)."""
    info = sarathi_plan_info()
    if isinstance(batch, sarathi_multi_batch):
        st = lib().sarathi_multi_plan_describe(byref(desc), byref(batch), byref(info))
    elif isinstance(batch, sarathi_paged_batch):
        st = lib().sarathi_paged_plan_describe(byref(desc), byref(batch), byref(info))
    else:
        st = lib().sarathi_plan_describe(byref(desc), byref(batch), byref(info))
    _check(st, "plan_describe")
    return info
