"""GPU checks of the weight conversion: the execution layout round-trips exactly, and the checked
conversions reproduce the pages' layouts as computed by the oracle (swap, tiled scales, bf16 bias)."""

import numpy as np
import pytest
import torch

import mixed_precision_moe_amd as mx
from oracle import convert as C
from oracle import quant as Q

pytestmark = pytest.mark.gpu


def random_weights(E, H, I, bias, seed, fp32_bias=True):
    g = np.random.default_rng(seed)
    w13_q = g.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)
    w13_s = g.integers(0, 256, (E, 2 * I, H // 32), dtype=np.uint8)
    w2_q = g.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    w2_s = g.integers(0, 256, (E, H, I // 32), dtype=np.uint8)
    b13 = b2 = None
    if bias:
        b13 = g.standard_normal((E, 2 * I)).astype(np.float32)
        b2 = g.standard_normal((E, H)).astype(np.float32)
    return w13_q, w13_s, w2_q, w2_s, b13, b2


def dev(a, bf16=False):
    if a is None:
        return None
    t = torch.from_numpy(a).cuda()
    return t


@pytest.mark.parametrize("E,H,I,bias", [(4, 256, 128, True), (3, 96, 96, True), (2, 32, 32, False),
                                        (5, 160, 224, True), (128, 2048, 768, False)])
def test_execution_layout_round_trip(E, H, I, bias):
    print(f"repack round trip E={E} H={H} I={I} bias={bias}", flush=True)
    w = random_weights(E, H, I, bias, seed=E * H + I)
    tw = [dev(a) for a in w]
    packed = mx.repack_weights(*tw)
    assert mx.check_packed(packed, E, H, I, bias) == 0
    assert mx.check_packed(packed, E, H, I + 32, bias) == 5
    back = mx.unpack_weights(packed, E, H, I, bias)
    torch.cuda.synchronize()
    for a, b in zip(w[:4], back[:4]):
        np.testing.assert_array_equal(b.cpu().numpy(), a)
    if bias:
        np.testing.assert_array_equal(back[4].view(torch.int16).cpu().numpy().view(np.uint16),
                                      C.f32_to_bf16_bits(w[4]))
        np.testing.assert_array_equal(back[5].view(torch.int16).cpu().numpy().view(np.uint16),
                                      C.f32_to_bf16_bits(w[5]))


@pytest.mark.parametrize("layout", [mx.LAYOUT_STD_W31, mx.LAYOUT_SCALE_TILED, mx.LAYOUT_STD_W31 | mx.LAYOUT_SCALE_TILED])
@pytest.mark.parametrize("E,H,I", [(4, 256, 128), (3, 96, 96), (2, 288, 160)])
def test_checked_conversions_match_oracle(layout, E, H, I):
    w = random_weights(E, H, I, True, seed=layout * 100 + E)
    out = mx.repack_weights(*[dev(a) for a in w], layout=layout)
    torch.cuda.synchronize()
    swap = bool(layout & mx.LAYOUT_STD_W31)
    tiled = bool(layout & mx.LAYOUT_SCALE_TILED)
    w13_q, w13_s, w2_q, w2_s, b13, b2 = w
    e13q = C.swap_w13_w31(w13_q) if swap else w13_q
    e13s = C.swap_w13_w31(w13_s) if swap else w13_s
    if tiled:
        e13s = C.tile_expert_scales(e13s)
        e2s = C.tile_expert_scales(w2_s)
    else:
        e2s = w2_s
    eb13 = C.f32_to_bf16_bits(C.swap_b13_b31(b13) if swap else b13)
    eb2 = C.f32_to_bf16_bits(b2)
    got = [t.cpu() for t in out]  # the page's order: w13, w2, w13 scale, w2 scale, b13, b2
    np.testing.assert_array_equal(got[0].numpy(), e13q)
    np.testing.assert_array_equal(got[1].numpy(), w2_q)
    np.testing.assert_array_equal(got[2].numpy(), e13s)
    np.testing.assert_array_equal(got[3].numpy(), e2s)
    np.testing.assert_array_equal(got[4].view(torch.int16).numpy().view(np.uint16), eb13)
    np.testing.assert_array_equal(got[5].view(torch.int16).numpy().view(np.uint16), eb2)


def test_page_swap_probe_through_the_library():
    """The page's arange probe tensors, at the smallest shape the library accepts (32-multiples):
    rows of w13 and its scales swap halves, w2 is unchanged, b13 halves swap, biases become bf16."""
    E, H, I = 1, 32, 32
    w13_q = np.arange(E * 2 * I * H // 2, dtype=np.uint32).astype(np.uint8).reshape(E, 2 * I, H // 2)
    w13_s = np.arange(E * 2 * I, dtype=np.uint8).reshape(E, 2 * I, 1)
    w2_q = np.arange(E * H * I // 2, dtype=np.uint32).astype(np.uint8).reshape(E, H, I // 2)
    w2_s = np.arange(E * H, dtype=np.uint8).reshape(E, H, 1)
    b13 = np.arange(2 * I, dtype=np.float32).reshape(E, 2 * I)
    b2 = np.arange(H, dtype=np.float32).reshape(E, H)
    converted = mx.repack_weights(*[dev(a) for a in (w13_q, w13_s, w2_q, w2_s, b13, b2)], layout=mx.LAYOUT_STD_W31)
    torch.cuda.synchronize()
    # indexed as the page's test indexes the conversion result: 0 w13, 1 w2, 2 w13 scale, 3 w2 scale,
    # 4 w13 bias, 5 w2 bias
    out = converted
    np.testing.assert_array_equal(out[0].cpu().numpy(), np.concatenate([w13_q[:, I:], w13_q[:, :I]], axis=1))
    np.testing.assert_array_equal(out[1].cpu().numpy(), w2_q)
    np.testing.assert_array_equal(out[2].cpu().numpy(), np.concatenate([w13_s[:, I:], w13_s[:, :I]], axis=1))
    np.testing.assert_array_equal(out[3].cpu().numpy(), w2_s)
    np.testing.assert_array_equal(out[4].float().cpu().numpy(), np.concatenate([b13[:, I:], b13[:, :I]], axis=1))
    np.testing.assert_array_equal(out[5].float().cpu().numpy(), b2)


def test_bf16_bias_input_passes_through():
    E, H, I = 2, 64, 64
    w = list(random_weights(E, H, I, True, seed=9))
    b13 = torch.from_numpy(w[4]).to(torch.bfloat16)
    b2 = torch.from_numpy(w[5]).to(torch.bfloat16)
    packed = mx.repack_weights(*[dev(a) for a in w[:4]], b13.cuda(), b2.cuda())
    back = mx.unpack_weights(packed, E, H, I, True)
    torch.cuda.synchronize()
    assert torch.equal(back[4].cpu(), b13)
    assert torch.equal(back[5].cpu(), b2)
