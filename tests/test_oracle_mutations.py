"""The oracle's pins catch plausible mistakes: each case plants one mistake in the oracle (on the CPU,
by replacing one of its functions for the duration of the test) and checks that at least one pin
then fails."""
import math

import numpy as np
import pytest

import oracle.layer as L
import tests.test_oracle_pins as pins


def _mask_ignores_prefix(offset, chunk_len):
    t = np.arange(chunk_len)[:, None]
    j = np.arange(offset + chunk_len)[None, :]
    return (j <= t) | (j < 0)


def _mask_excludes_self(offset, chunk_len):
    t = np.arange(chunk_len)[:, None]
    j = np.arange(offset + chunk_len)[None, :]
    return (j < offset + t) | (j == 0)


def _rope_wrong_sign(x, pos, base):
    return L.__dict__["_orig_rope"](x, -np.asarray(pos), base)


def _rope_rotate_half(x, pos, base):
    d = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[:, None] * L.rope_inv_freq(d, base)[None, :]
    cos, sin = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)


def _rms_no_eps(x, gamma, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) * gamma


def _rms_mean_abs(x, gamma, eps):
    return x / (np.mean(np.abs(x), axis=-1, keepdims=True) + eps) * gamma


def _attend_no_scale(q, k, v, mask):
    return L.__dict__["_orig_attend"](q * math.sqrt(q.shape[-1]), k, v, mask)


def _silu_wrong(z):
    return z / (1.0 + np.exp(z))


MUTATIONS = {
    "mask_ignores_prefix": ("chunk_mask", _mask_ignores_prefix),
    "mask_excludes_self": ("chunk_mask", _mask_excludes_self),
    "rope_wrong_sign": ("rope_rotate", _rope_wrong_sign),
    "rope_rotate_half_pairing": ("rope_rotate", _rope_rotate_half),
    "rms_without_eps": ("rms_norm", _rms_no_eps),
    "rms_mean_abs": ("rms_norm", _rms_mean_abs),
    "attention_without_scale": ("attend_rows", _attend_no_scale),
    "silu_wrong_sign": ("silu", _silu_wrong),
}

PINS = [
    lambda gd: pins.test_fig6_chunk_masks(gd),
    lambda gd: pins.test_chunked_equals_monolithic(pins.wl.SHAPES["tiny"]),
    lambda gd: pins.test_unified_mask_bruteforce(),
    lambda gd: pins.test_attention_mask_length_closed_form(),
    lambda gd: pins.test_attention_one_hot(),
    lambda gd: pins.test_rope_identity_norm_relative_and_textbook(),
    lambda gd: pins.test_norm_closed_forms(),
    lambda gd: pins.test_activations_vs_python_math(),
    lambda gd: pins.test_linear_ops_by_loops(pins.SMALL),
    lambda gd: pins.test_whole_layer_identity_special_case(),
    lambda gd: pins.test_gated_ffn_special_case(),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch, golden_dir):
    attr, fn = MUTATIONS[name]
    monkeypatch.setitem(L.__dict__, "_orig_rope", L.rope_rotate)
    monkeypatch.setitem(L.__dict__, "_orig_attend", L.attend_rows)
    monkeypatch.setattr(L, attr, fn)
    # the pins call the oracle through the package namespace as well
    import oracle
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    failed = 0
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(golden_dir)
            except (AssertionError, FloatingPointError, ValueError):
                failed += 1
    assert failed >= 1, f"no pin caught the planted mistake {name}"


# ------------------------------------------------------------------------------------------------
# Planted mistakes in the layer stack's chaining.
# ------------------------------------------------------------------------------------------------

def _stack_layer_batch(batch, l, x):
    return {"x": x, "chunk_len": batch["chunk_len"], "chunk_offset": batch["chunk_offset"],
            "decode_len": batch["decode_len"],
            "chunk_k": batch["chunk_k"][l] if batch["chunk_len"] else None,
            "chunk_v": batch["chunk_v"][l] if batch["chunk_len"] else None,
            "decode_k": batch["decode_k"][l], "decode_v": batch["decode_v"][l]}


def _stack_input_to_every_layer(shape, layer_weights, batch, dtype=np.float64):
    outs = [L.layer_forward(shape, w, _stack_layer_batch(batch, l, batch["x"]), dtype)
            for l, w in enumerate(layer_weights)]
    return {"y": outs[-1]["y"], "layers": outs}


def _stack_weights_reversed(shape, layer_weights, batch, dtype=np.float64):
    x, outs = batch["x"], []
    for l, w in enumerate(reversed(list(layer_weights))):
        outs.append(L.layer_forward(shape, w, _stack_layer_batch(batch, l, x), dtype))
        x = outs[-1]["y"]
    return {"y": x, "layers": outs}


def _stack_first_layer_caches(shape, layer_weights, batch, dtype=np.float64):
    x, outs = batch["x"], []
    for w in layer_weights:
        outs.append(L.layer_forward(shape, w, _stack_layer_batch(batch, 0, x), dtype))
        x = outs[-1]["y"]
    return {"y": x, "layers": outs}


STACK_MUTATIONS = {
    "stack_input_to_every_layer": _stack_input_to_every_layer,
    "stack_weights_reversed": _stack_weights_reversed,
    "stack_first_layer_caches": _stack_first_layer_caches,
}


@pytest.mark.parametrize("name", sorted(STACK_MUTATIONS))
def test_planted_stack_mistake_is_caught(name, monkeypatch):
    import oracle
    import tests.test_oracle_stack as stack_pins
    monkeypatch.setattr(L, "stack_forward", STACK_MUTATIONS[name])
    monkeypatch.setattr(oracle, "stack_forward", STACK_MUTATIONS[name])
    failed = 0
    for pin in (stack_pins.test_stack_chunked_prompt_equals_monolithic_and_decodes_are_independent,
                stack_pins.test_stack_of_one_layer_is_the_layer,
                stack_pins.test_stack_chains_layers_in_order_closed_form):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin caught the planted mistake {name}"
