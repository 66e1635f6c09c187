"""GPU parity of moe_mxfp4_route: bit-exact expert ids, offsets and stable pair order; weights within
fp32 rounding of the float64 oracle."""

import numpy as np
import pytest
import torch

import mixed_precision_moe_amd as mx
from mixed_precision_moe_amd import synth
from oracle import route as R

pytestmark = pytest.mark.gpu


def check(logits, k, ren):
    ld = torch.from_numpy(logits).cuda()
    ids, w, offs, sp = mx.route(ld, k, ren)
    torch.cuda.synchronize()
    ri, rw = R.route_ref(logits, k, ren)
    ro, rs = R.sort_pairs_ref(ri, logits.shape[1])
    np.testing.assert_array_equal(ids.cpu().numpy(), ri)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=2e-6, atol=1e-7)
    np.testing.assert_array_equal(offs.cpu().numpy(), ro)
    np.testing.assert_array_equal(sp.cpu().numpy(), rs)


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "large"])
def test_route_configs(name):
    cfg = synth.MOE_CONFIGS[name]
    _, logits = synth.moe_activations(cfg)
    print(f"route {name} T={cfg.T} E={cfg.E} k={cfg.k}", flush=True)
    check(logits, cfg.k, True)


@pytest.mark.parametrize("T,E,k,ren", [(1, 1, 1, True), (5, 3, 3, False), (33, 64, 8, False), (100, 1024, 32, True),
                                       (64, 1024, 32, True), (64, 300, 8, False), (65, 128, 8, True),
                                       (70, 200, 7, True), (513, 130, 5, True)])
def test_route_shapes(T, E, k, ren):
    g = np.random.default_rng(T * 1000 + E)
    logits = g.standard_normal((T, E)).astype(np.float32)
    check(logits, k, ren)


def test_route_ties_and_signed_zero():
    g = np.random.default_rng(3)
    logits = np.round(g.standard_normal((300, 40)) * 2).astype(np.float32) / 2  # many exact ties
    logits[:, 7] = -0.0
    logits[:, 9] = 0.0
    check(logits, 8, True)
    check(logits, 32, False)


def test_route_empty():
    logits = np.zeros((0, 8), np.float32)
    ld = torch.from_numpy(logits).cuda()
    ids, w, offs, sp = mx.route(ld, 2, True)
    torch.cuda.synchronize()
    assert offs.cpu().numpy().tolist() == [0] * 9
