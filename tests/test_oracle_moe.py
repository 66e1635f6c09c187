"""Pins of the MoE oracle: the pure-Python brute force, and special cases that reduce to a dense
SwiGLU MLP or to the biases alone."""

import numpy as np
import pytest

from mixed_precision_moe_amd import synth
from oracle import moe as M
from oracle import quant as Q


def quantize_experts(masters):
    qs, ss = zip(*[Q.quantize_ref(m) for m in masters])
    return np.stack(qs), np.stack(ss)


def build(cfg):
    x, logits = synth.moe_activations(cfg)
    ms = [synth.moe_master_expert(cfg, e) for e in range(cfg.E)]
    w13_q, w13_s = quantize_experts([m[0] for m in ms])
    w2_q, w2_s = quantize_experts([m[1] for m in ms])
    b13, b2 = synth.moe_biases(cfg)
    return x, logits, w13_q, w13_s, w2_q, w2_s, b13, b2


@pytest.mark.parametrize("ren", [True, False])
def test_vectorized_matches_bruteforce_small(ren):
    cfg = synth.custom_moe_config("t", T=6, E=4, k=2, H=64, I=32, bias=True, renormalize=ren)
    args = build(cfg)
    y, _, _ = M.moe_ref(*args[:2], cfg.k, *args[2:], renormalize=ren)
    yb = M.moe_bruteforce(*args[:2], cfg.k, *args[2:], renormalize=ren)
    np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-15)


def test_vectorized_matches_bruteforce_tiny_config():
    cfg = synth.MOE_CONFIGS["tiny"]
    args = build(cfg)
    y, _, _ = M.moe_ref(*args[:2], cfg.k, *args[2:])
    yb = M.moe_bruteforce(*args[:2], cfg.k, *args[2:])
    np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-15)


def test_single_expert_is_dense_swiglu_mlp():
    """E = 1, k = 1, no biases: y = W2 (silu(W1 x) * (W3 x)) with W1, W3 the two halves of w13."""
    cfg = synth.custom_moe_config("d", T=5, E=1, k=1, H=96, I=64, bias=False)
    x, logits, w13_q, w13_s, w2_q, w2_s, _, _ = build(cfg)
    y, _, w = M.moe_ref(x, logits, 1, w13_q, w13_s, w2_q, w2_s)
    assert np.all(w == 1.0)
    W13 = Q.dequant_ref(w13_q[0], w13_s[0])
    W1, W3 = W13[: cfg.I], W13[cfg.I:]
    W2 = Q.dequant_ref(w2_q[0], w2_s[0])
    X = Q.bf16_to_f64(x)
    g = X @ W1.T
    want = ((g * 0.5 * (1 + np.tanh(g / 2))) * (X @ W3.T)) @ W2.T  # silu via tanh identity
    np.testing.assert_allclose(y, want, rtol=1e-11, atol=1e-14)


def test_zero_input_and_zero_down_projection():
    cfg = synth.custom_moe_config("z", T=8, E=3, k=2, H=64, I=32, bias=True)
    x, logits, w13_q, w13_s, w2_q, w2_s, b13, b2 = build(cfg)
    from oracle.route import route_ref
    ids, w = route_ref(logits, 2)
    B13 = Q.bf16_to_f64(b13)
    B2 = Q.bf16_to_f64(b2)
    W2 = np.stack([Q.dequant_ref(w2_q[e], w2_s[e]) for e in range(cfg.E)])
    # x = 0: every expert sees h = b13, so y = sum_j w_j (W2 (silu(b1) * b3) + b2)
    y, _, _ = M.moe_ref(np.zeros_like(x), logits, 2, w13_q, w13_s, w2_q, w2_s, b13, b2)
    g, u = B13[:, : cfg.I], B13[:, cfg.I:]
    per_e = np.einsum("ehi,ei->eh", W2, g / (1 + np.exp(-g)) * u) + B2
    want = np.einsum("tj,tjh->th", w, per_e[ids])
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-15)
    # W2 = 0: y = sum_j w_j b2
    y, _, _ = M.moe_ref(x, logits, 2, w13_q, w13_s, np.zeros_like(w2_q), w2_s, b13, b2)
    np.testing.assert_allclose(y, np.einsum("tj,tjh->th", w, B2[ids]), rtol=1e-13, atol=1e-16)


def test_token_subset_equals_full_rows():
    cfg = synth.custom_moe_config("s", T=12, E=5, k=3, H=64, I=32, bias=False)
    args = build(cfg)
    y, _, _ = M.moe_ref(*args[:2], cfg.k, *args[2:])
    sub = np.array([1, 7, 11])
    ys, _, _ = M.moe_ref(*args[:2], cfg.k, *args[2:], tokens=sub)
    np.testing.assert_allclose(ys[sub], y[sub], rtol=1e-12, atol=1e-15)
    assert np.all(ys[np.setdiff1d(np.arange(12), sub)] == 0)


def test_expert_partition_sums_to_the_whole_layer():
    """y is a sum of per-expert terms: the results over a partition of the experts add up to the
    result over all of them (how the full-size GPU parity tests spread the oracle over threads)."""
    cfg = synth.custom_moe_config("p", T=20, E=6, k=3, H=64, I=32, bias=True)
    args = build(cfg)
    y, _, _ = M.moe_ref(*args[:2], cfg.k, *args[2:])
    parts = [M.moe_ref(*args[:2], cfg.k, *args[2:], experts=ex)[0] for ex in ([0, 3], [1, 5], [2, 4])]
    np.testing.assert_allclose(parts[0] + parts[1] + parts[2], y, rtol=1e-12, atol=1e-15)
    assert not np.allclose(parts[0], y)  # each part alone is not the layer


@pytest.mark.parametrize("act", ["mxfp8", "mxfp4"])
def test_quantized_activation_variants_match_bruteforce(act):
    """The quantized-activation variants, vectorized, against the scalar brute force (its own block
    quantizer from math.frexp and a linear nearest-magnitude search)."""
    cfg = synth.custom_moe_config("q", T=6, E=4, k=2, H=64, I=64, bias=True)
    args = build(cfg)
    y, _, _ = M.moe_ref(*args[:2], cfg.k, *args[2:], act=act)
    yb = M.moe_bruteforce(*args[:2], cfg.k, *args[2:], act=act)
    np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-15)
    # a different result than the bf16 layer (the quantization is not a no-op), within a few percent
    y16, _, _ = M.moe_ref(*args[:2], cfg.k, *args[2:])
    rel = np.sqrt(np.mean((y - y16) ** 2) / np.mean(y16 ** 2))
    assert 1e-4 < rel < (0.05 if act == "mxfp8" else 0.25)


@pytest.mark.parametrize("act", ["mxfp8", "mxfp4"])
def test_quantized_activation_variants_special_cases(act):
    cfg = synth.custom_moe_config("z", T=8, E=3, k=2, H=64, I=32, bias=True)
    x, logits, w13_q, w13_s, w2_q, w2_s, b13, b2 = build(cfg)
    from oracle.route import route_ref
    ids, w = route_ref(logits, 2)
    B2 = Q.bf16_to_f64(b2)
    # W2 = 0: y = sum_j w_j b2, whatever the activations were
    y, _, _ = M.moe_ref(x, logits, 2, w13_q, w13_s, np.zeros_like(w2_q), w2_s, b13, b2, act=act)
    np.testing.assert_allclose(y, np.einsum("tj,tjh->th", w, B2[ids]), rtol=1e-13, atol=1e-16)
    # x = 0 quantizes to 0: h = b13 for every expert, as in the bf16 layer, and the SwiGLU output is
    # quantized once
    B13 = Q.bf16_to_f64(b13)
    g, u = B13[:, : cfg.I], B13[:, cfg.I:]
    aq = M.quantize_activation((g / (1 + np.exp(-g)) * u).astype(np.float32), act)
    W2 = np.stack([Q.dequant_ref(w2_q[e], w2_s[e]) for e in range(cfg.E)])
    per_e = np.einsum("ehi,ei->eh", W2, aq) + B2
    y, _, _ = M.moe_ref(np.zeros_like(x), logits, 2, w13_q, w13_s, w2_q, w2_s, b13, b2, act=act)
    np.testing.assert_allclose(y, np.einsum("tj,tjh->th", w, per_e[ids]), rtol=1e-12, atol=1e-15)


def test_ambiguity_window_marks_only_near_ties():
    """Values on a quantization grid point (far from every midpoint) give no ambiguity; a value on a
    rounding midpoint and a block maximum on the scale's round-up threshold do."""
    blk = np.zeros((3, 32), np.float32)
    blk[:, 0] = 4.0                    # scale 2**0 for E2M1 (4 -> e = 127), grid points 0.5, 1, ...
    blk[0, 1:9] = [0.5, 1.0, 1.5, 2.0, 3.0, -4.0, 0.0, -1.0]
    blk[1, 1] = 1.25                   # midpoint between 1.0 and 1.5
    blk[2, 0] = 7.0                    # 1.75 * 2**2: the round-up threshold of the scale
    amb = M.activation_ambiguity(blk, "mxfp4")
    assert np.all(amb[0] == 0)
    assert amb[1, 1] > 0 and np.all(amb[1, 2:] == 0)
    assert amb[2, 0] > 0
