"""GPU parity of the dense MXFP4-weight linear layer (mxfp4_linear_pack / mxfp4_linear_forward)
against the float64 oracle: |y - y_ref| <= 2e-2 * rms(y_ref) + 1e-3 on every output element, on small,
ragged, strided and full-size shapes; repeated calls are bit-identical."""

import numpy as np
import pytest
import torch

import mixed_precision_moe_amd as mx
from mixed_precision_moe_amd import synth
from oracle import linear as L
from oracle import quant as Q
from tests.gpu_common import assert_moe_close, bf16_dev, bf16_host_f64

pytestmark = pytest.mark.gpu


def run_case(M, N, K, bias, ldx_pad=0, seed=0):
    print(f"linear M={M} N={N} K={K} bias={bias} ldx_pad={ldx_pad}", flush=True)
    g = synth.rng(180, seed, M, N, K)
    w_bits = synth.to_bf16_bits(g.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    x_bits = synth.to_bf16_bits(g.standard_normal((M, K), dtype=np.float32))
    b_bits = synth.to_bf16_bits(g.normal(0.0, 0.01, size=N)) if bias else None
    wq, ws, _ = mx.quantize(bf16_dev(w_bits), flat=True, tiled=False)
    layer = mx.Linear(wq, ws, bf16_dev(b_bits) if bias else None)
    if ldx_pad:
        buf = np.zeros((M, K + ldx_pad), np.uint16)
        buf[:, :K] = x_bits
        xd = bf16_dev(buf)[:, :K]
    else:
        xd = bf16_dev(x_bits)
    y = bf16_host_f64(layer(xd))
    np.testing.assert_array_equal(bf16_host_f64(layer(xd)), y)
    wq_ref, ws_ref = Q.quantize_ref(w_bits)
    y_ref = L.linear_ref(x_bits, wq_ref, ws_ref, b_bits)
    ratio, bad = assert_moe_close(y, y_ref, None, f"linear {M}x{N}x{K}")
    print(f"  max|err|/rms = {ratio:.3e}, elements outside tolerance: {bad} of {y_ref.size}", flush=True)


@pytest.mark.parametrize("M,N,K,bias", [(1, 32, 32, False), (37, 96, 96, True), (70, 160, 288, True),
                                        (300, 2048, 2048, False), (129, 7168, 2048, True), (33, 512, 7168, False)])
def test_shapes(M, N, K, bias):
    run_case(M, N, K, bias)


def test_strided_activations():
    run_case(50, 128, 192, True, ldx_pad=24)


def test_full_size_8192_tokens():
    """8192 tokens through a 2048 x 2048 layer (the prefill workload's hidden size), every output."""
    run_case(8192, 2048, 2048, False)
