"""Host logic of the library GEMM comparison: the products it times are the layer's four, at the
batch's row count (CPU only; the timing itself needs a GPU)."""
from chunked_prefill_hybrid_amd import gemm_library as gl
from chunked_prefill_hybrid_amd import workloads as wl


def test_products_match_the_layer():
    sh = wl.workload("llama13b").shape
    got = dict((n, (N, K)) for n, N, K in gl.shapes(sh))
    H, A, F = sh.hidden, sh.attn_width, sh.ffn
    assert got == {"qkv": (3 * A, H), "o": (H, A), "ffn_up": (2 * F, H), "ffn_down": (H, F)}
    gpt = wl.workload("gpt3tp8").shape
    assert dict((n, (N, K)) for n, N, K in gl.shapes(gpt))["ffn_up"] == (gpt.ffn, gpt.hidden)


def test_batch_rows():
    assert gl.batch_rows(wl.workload("llama13b")) == 256 + 18
    assert gl.batch_rows(wl.workload("llama13b_budget")) == 512
    assert gl.batch_rows(wl.workload("llama33b")) == 544
