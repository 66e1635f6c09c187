"""moe_mxfp4_forward_noalloc (the forward pass on the library's device scratch array) against
moe_mxfp4_forward (the same kernels on a caller workspace): bit-identical outputs, on two calls in a
row with the second on a smaller input, and the documented rejection of shapes beyond the array."""

import ctypes

import numpy as np
import pytest
import torch

import mixed_precision_moe_amd as mx
from mixed_precision_moe_amd import synth
from mixed_precision_moe_amd._lib import MoeDims, lib
from tests.gpu_common import bf16_dev, gpu_standard_weights

pytestmark = pytest.mark.gpu


def call_noalloc(layer, x, logits, y, ids, tw):
    d = MoeDims(layer.E, layer.H, layer.I, 1 if layer.has_bias else 0)
    T = x.shape[0]
    st = lib().moe_mxfp4_forward_noalloc(ctypes.byref(d), ctypes.c_void_p(layer.packed.data_ptr()),
                                         ctypes.c_void_p(x.data_ptr()), T, x.stride(0),
                                         ctypes.c_void_p(logits.data_ptr()), layer.top_k, 1,
                                         ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(ids.data_ptr()),
                                         ctypes.c_void_p(tw.data_ptr()),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_matches_workspace_forward_on_two_calls():
    cfg = synth.MOE_CONFIGS["decode"]  # E = 128, H = 2048, I = 768, top-8, biases
    print(f"noalloc decode shape, T = {cfg.T} then 23", flush=True)
    x_bits, logits = synth.moe_activations(cfg)
    layer = mx.MoE(*gpu_standard_weights(cfg), top_k=cfg.k)
    xd, ld = bf16_dev(x_bits), torch.from_numpy(logits).cuda()
    for T in (cfg.T, 23):  # the second call smaller than the first
        x, lg = xd[:T], ld[:T].contiguous()
        ids_ref = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
        w_ref = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
        y_ref = layer(x, lg, topk_ids=ids_ref, topk_w=w_ref)
        y = torch.full((T, cfg.H), float("nan"), dtype=torch.bfloat16, device="cuda")
        ids = torch.full((T, cfg.k), -1, dtype=torch.int32, device="cuda")
        tw = torch.full((T, cfg.k), -1.0, dtype=torch.float32, device="cuda")
        assert call_noalloc(layer, x, lg, y, ids, tw) == 0
        torch.cuda.synchronize()
        assert torch.equal(ids.cpu(), ids_ref.cpu())
        assert torch.equal(tw.cpu(), w_ref.cpu())
        np.testing.assert_array_equal(y.view(torch.int16).cpu().numpy(), y_ref.view(torch.int16).cpu().numpy())


def test_noalloc_rejects_shapes_beyond_the_array():
    d = MoeDims(128, 2048, 768, 1)
    T = 4096
    need = lib().moe_mxfp4_workspace_bytes(ctypes.byref(d), T, 8)
    assert need > mx.NOALLOC_SCRATCH_BYTES
    # rejected during validation, before any launch: the pointers are never used
    fake = 1 << 20
    st = lib().moe_mxfp4_forward_noalloc(ctypes.byref(d), fake, fake, T, 2048, fake, 8, 1, fake, None, None, None)
    assert st == 4
    # argument errors keep their own status; no tokens is a no-op
    assert lib().moe_mxfp4_forward_noalloc(ctypes.byref(d), fake, fake, 16, 2000, fake, 8, 1, fake, None, None,
                                           None) == 2
    assert lib().moe_mxfp4_forward_noalloc(ctypes.byref(d), fake, fake, 0, 2048, fake, 8, 1, fake, None, None,
                                           None) == 0
