"""Pins of the dense-linear oracle: a per-scalar brute force, weights that dequantize to a scaled
identity, zero weights, and the relation to a one-expert MoE's first product."""

import numpy as np

from mixed_precision_moe_amd import synth
from oracle import linear as L
from oracle import moe as M
from oracle import quant as Q


def test_matches_bruteforce():
    g = np.random.default_rng(1)
    x = synth.to_bf16_bits(g.standard_normal((5, 64)))
    wq, ws = Q.quantize_ref(synth.to_bf16_bits(g.standard_normal((6, 64)) * 0.1))
    b = synth.to_bf16_bits(g.standard_normal(6) * 0.01)
    np.testing.assert_allclose(L.linear_ref(x, wq, ws, b), L.linear_bruteforce(x, wq, ws, b), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(L.linear_ref(x, wq, ws), L.linear_bruteforce(x, wq, ws), rtol=1e-12, atol=1e-15)


def test_scaled_identity_and_zero_weights():
    """W = 2 * identity (code 4 = 2.0 under scale 2^0 on the diagonal) gives y = 2 x exactly; W = 0
    gives y = b."""
    K = 64
    codes = np.zeros((K, K), np.uint8)
    codes[np.arange(K), np.arange(K)] = 4
    wq = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    ws = np.full((K, K // 32), 127, np.uint8)
    g = np.random.default_rng(2)
    x = synth.to_bf16_bits(g.standard_normal((7, K)))
    np.testing.assert_array_equal(L.linear_ref(x, wq, ws), 2 * Q.bf16_to_f64(x))
    b = synth.to_bf16_bits(g.standard_normal(K))
    np.testing.assert_array_equal(L.linear_ref(x, np.zeros_like(wq), ws, b), np.broadcast_to(Q.bf16_to_f64(b), (7, K)))


def test_equals_the_moe_layers_first_product():
    """With one expert and top-1 the MoE layer is a dense SwiGLU MLP: its first product is the linear
    layer with the fused w13 as weights, so the MoE oracle equals silu(g) * u of that product, pushed
    through w2."""
    cfg = synth.custom_moe_config("l", T=5, E=1, k=1, H=64, I=32, bias=False)
    x, logits = synth.moe_activations(cfg)
    m13, m2 = synth.moe_master_expert(cfg, 0)
    w13q, w13s = Q.quantize_ref(m13)
    w2q, w2s = Q.quantize_ref(m2)
    y, _, _ = M.moe_ref(x, logits, 1, w13q[None], w13s[None], w2q[None], w2s[None])
    h = L.linear_ref(x, w13q, w13s)
    g, u = h[:, :32], h[:, 32:]
    a = g / (1 + np.exp(-g)) * u
    want = a @ Q.dequant_ref(w2q, w2s).T
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-15)
