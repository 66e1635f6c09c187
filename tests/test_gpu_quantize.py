"""GPU parity of mxfp4_quantize against the oracle: bit-exact nibbles, flat and tiled scales."""

import numpy as np
import pytest
import torch

import mixed_precision_moe_amd as mx
from mixed_precision_moe_amd import synth
from oracle import quant as Q
from tests.exhaustive import exhaustive_matrix
from tests.gpu_common import bf16_dev

pytestmark = pytest.mark.gpu


def run_gpu(bits, ldx=None):
    M, K = bits.shape
    if ldx is not None and ldx != K:
        buf = np.zeros((M, ldx), np.uint16)
        buf[:, :K] = bits
        xd = bf16_dev(buf)[:, :K]
    else:
        xd = bf16_dev(bits)
    q, sf, st = mx.quantize(xd)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sf.cpu().numpy(), st.cpu().numpy()


def check_full(bits, ldx=None):
    q, sf, st = run_gpu(bits, ldx)
    qr, sr = Q.quantize_ref(bits)
    np.testing.assert_array_equal(sf, sr)
    np.testing.assert_array_equal(q, qr)
    np.testing.assert_array_equal(st, Q.tile_scales(sr))


def test_exhaustive_every_pattern_every_exponent():
    x, ee = exhaustive_matrix()
    print(f"exhaustive matrix {x.shape}", flush=True)
    q, sf, st = run_gpu(x)
    assert np.array_equal(sf[:, 0], ee)
    qr, sr = Q.quantize_ref(x)
    np.testing.assert_array_equal(sf, sr)
    np.testing.assert_array_equal(q, qr)
    np.testing.assert_array_equal(Q.untile_scales(st, x.shape[0], 32), sf)


@pytest.mark.parametrize("M,K,ldx", [(1, 32, 32), (3, 64, 72), (127, 160, 160), (129, 96, 104), (300, 4128, 4136),
                                     (128, 128, 128), (257, 1056, 1056), (64, 7168, 7168)])
def test_ragged_and_strided_shapes(M, K, ldx):
    print(f"quantize M={M} K={K} ldx={ldx}", flush=True)
    bits = synth.random_bits_matrix(M, K, seed=M * 7 + K)
    check_full(bits, ldx)
    # realistic values too
    check_full(synth.quant_matrix(M, K, cid=200 + M), ldx)


def test_full_size_quantize_config_every_row():
    """The 8192 x 7168 workload, every nibble and both scale layouts compared with the oracle."""
    cfg = synth.QUANT_CONFIG
    M, K = cfg["M"], cfg["K"]
    bits = synth.quant_matrix(M, K, cid=cfg["cid"])
    print(f"quantize {M}x{K}", flush=True)
    q, sf, st = run_gpu(bits)
    qr, sr = Q.quantize_ref(bits)
    np.testing.assert_array_equal(sf, sr)
    np.testing.assert_array_equal(q, qr)
    np.testing.assert_array_equal(st, Q.tile_scales(sr))
    # zero blocks of the input give scale 0
    zb = np.all(bits.reshape(M, K // 32, 32) == 0, axis=2)
    assert np.count_nonzero(zb) >= 18350
    assert np.all(sf[zb] == 0)
    # saturated fraction: blocks whose largest scaled magnitude exceeds 6 (significand in (1.5, 1.75))
    sig = Q.bf16_to_f64(bits.reshape(M, K // 32, 32) & np.uint16(0x7FFF)).max(axis=2)
    m, _ = np.frexp(sig[sig > 0])
    frac = float(np.mean((2 * m > 1.5) & (2 * m < 1.75)))
    print(f"  saturating blocks: {frac:.4f}", flush=True)


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_flat_scales_at_any_byte_offset(offset):
    """The flat scale output may start at any byte: K/32 = 8 would take dword stores from an aligned
    pointer, an offset pointer takes byte stores; nothing outside [M, K/32] is written."""
    M, K = 130, 256
    bits = synth.quant_matrix(M, K, cid=400 + offset)
    xd = bf16_dev(bits)
    q = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    buf = torch.full((M * (K // 32) + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    L = mx._lib.lib()
    st = L.mxfp4_quantize(xd.data_ptr(), M, K, K, q.data_ptr(), buf.data_ptr() + offset, None, None)
    assert st == 0
    torch.cuda.synchronize()
    qr, sr = Q.quantize_ref(bits)
    got = buf.cpu().numpy()
    np.testing.assert_array_equal(got[offset: offset + M * (K // 32)].reshape(M, K // 32), sr)
    assert np.all(got[:offset] == 0xA5) and np.all(got[offset + M * (K // 32):] == 0xA5)
    np.testing.assert_array_equal(q.cpu().numpy(), qr)


def test_empty_matrix_is_noop_and_bad_shapes_rejected():
    L = mx._lib.lib()
    assert L.mxfp4_quantize(None, 0, 64, 64, None, None, None, None) == 0
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((4, 32), dtype=torch.uint8, device="cuda")
    assert L.mxfp4_quantize(x.data_ptr(), 4, 48, 64, q.data_ptr(), None, None, None) == 2  # K % 32
    assert L.mxfp4_quantize(x.data_ptr(), 4, 64, 60, q.data_ptr(), None, None, None) == 2  # ldx < K
    assert L.mxfp4_quantize(x.data_ptr() + 2, 4, 64, 64, q.data_ptr(), None, None, None) == 3  # misaligned


def test_deterministic_across_runs():
    bits = synth.quant_matrix(512, 2048, cid=300)
    a = run_gpu(bits)
    b = run_gpu(bits)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
