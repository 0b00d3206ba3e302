"""Host-side checks of the batch-composition sweeps (no GPU): every sweep point is a valid batch of its
workload, and the sweep table renders a benchmark line."""
from chunked_prefill_hybrid_amd import sweep_bench
from chunked_prefill_hybrid_amd import workloads as wl


def test_sweep_points_are_valid_batches():
    for key, field, values in (("gpt3tp8", "n_decodes", [1, 2, 4, 8, 16, 32, 64]),
                               ("llama13b", "n_decodes", [1, 4, 8, 18, 32, 64]),
                               ("llama33b", "chunk_len", [128, 256, 257, 512, 544, 545])):
        pts = wl.sweep_changes(key)
        assert [p[field] for p in pts] == values
        for ch in pts:
            b = wl.workload(key, **ch).batch
            assert b.chunk_offset + b.chunk_len <= b.prompt_len
            assert b.decode_lens is None or len(b.decode_lens) == b.n_decodes
    assert wl.sweep_changes("tiny") == []


def test_sweep_table_renders_a_line():
    line = {"value": 1000.0, "ms_per_step": 0.5,
            "config": {"chunks": [[256, 0]], "decodes": 4, "rows": 260},
            "stages": {"ffn_up": {"frac": 0.25}, "attn_decode": {"frac": 0.5}},
            "piggyback": {"marginal_decode_us": 6.0, "decode_only_per_decode_us": 30.0, "decode_speedup": 5.0}}
    rows = sweep_bench.table("gpt3tp8", [({"n_decodes": 4}, line)])
    assert rows[2] == "| 256 | 4 | 260 | 1000 | 0.5 | 25.0 | 50.0 | 6.0 | 30.0 | 5.0 |"
