"""The C-ABI library loads and exports every function the public header declares; argument validation
returns the documented status codes before any device work (so these run without a GPU)."""

import ctypes
import os
import re

import pytest

from mixed_precision_moe_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mxfp4moe.h")

OK, NULL, SHAPE, ALIGN, WS, LAYOUT = 0, 1, 2, 3, 4, 5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", text)) - {"if", "sizeof"})


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmxfp4moe.so is not built; run __graft_entry__.build()")
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.EXPORTED)


def test_status_strings(L):
    for s in range(7):
        assert len(L.mxfp4_status_str(s)) > 1
    assert L.mxfp4_status_str(99) == b"unknown status"
    assert L.mxfp4_version() >> 16 == 1


def dims(E, H, I, b=0):
    return ctypes.byref(_lib.MoeDims(E, H, I, b))


# A 256-byte aligned address that is never dereferenced: every call below fails validation (or has
# nothing to do) before any device work, so these tests are also safe on a machine with a GPU.
FAKE = 1 << 20


def test_quantize_validation(L):
    assert L.mxfp4_quantize(FAKE, 4, 48, 64, FAKE, None, None, None) == SHAPE   # K % 32
    assert L.mxfp4_quantize(FAKE, 4, 0, 64, FAKE, None, None, None) == SHAPE
    assert L.mxfp4_quantize(FAKE, 4, 64, 32, FAKE, None, None, None) == SHAPE   # ldx < K
    assert L.mxfp4_quantize(FAKE, 4, 64, 68, FAKE, None, None, None) == SHAPE   # ldx % 8
    assert L.mxfp4_quantize(FAKE, -1, 64, 64, FAKE, None, None, None) == SHAPE
    assert L.mxfp4_quantize(None, 4, 64, 64, FAKE, None, None, None) == NULL
    assert L.mxfp4_quantize(FAKE, 4, 64, 64, None, None, None, None) == NULL
    assert L.mxfp4_quantize(FAKE + 8, 4, 64, 64, FAKE, None, None, None) == ALIGN
    assert L.mxfp4_quantize(FAKE, 4, 64, 64, FAKE + 2, None, None, None) == ALIGN
    assert L.mxfp4_quantize(FAKE, 4, 64, 64, FAKE, None, FAKE + 4, None) == ALIGN  # tiled scales: 16 bytes
    assert L.mxfp4_quantize(None, 0, 64, 64, None, None, None, None) == OK  # empty: no-op
    assert L.mxfp4_tiled_scale_bytes(8192, 7168) == 64 * 56 * 512
    assert L.mxfp4_tiled_scale_bytes(129, 160) == 2 * 2 * 512
    assert L.mxfp4_tiled_scale_bytes(1, 40) == 0


def test_repack_validation(L):
    assert L.mxfp4_repack_bytes(dims(4, 256, 128), 0) > 0
    assert L.mxfp4_repack_bytes(dims(4, 250, 128), 0) == 0
    assert L.mxfp4_repack_bytes(dims(4, 256, 128), 8) == 0
    assert L.mxfp4_repack_bytes(None, 0) == 0
    n = L.mxfp4_repack_bytes(dims(4, 256, 128, 1), 0)
    f = L.mxfp4_repack_weights
    assert f(None, FAKE, FAKE, FAKE, FAKE, None, None, 0, 0, FAKE, n, None) == NULL
    assert f(dims(0, 256, 128), FAKE, FAKE, FAKE, FAKE, None, None, 0, 0, FAKE, n, None) == SHAPE
    assert f(dims(4, 256, 100), FAKE, FAKE, FAKE, FAKE, None, None, 0, 0, FAKE, n, None) == SHAPE
    assert f(dims(4, 256, 128, 2), FAKE, FAKE, FAKE, FAKE, None, None, 0, 0, FAKE, n, None) == SHAPE
    assert f(dims(4, 256, 128, 1), FAKE, FAKE, FAKE, FAKE, None, None, 0, 0, FAKE, n, None) == NULL  # bias missing
    assert f(dims(4, 256, 128), FAKE, FAKE, None, FAKE, None, None, 0, 0, FAKE, n, None) == NULL
    assert f(dims(4, 256, 128), FAKE, FAKE, FAKE, FAKE, None, None, 0, 7, FAKE, n, None) == LAYOUT
    assert f(dims(4, 256, 128), FAKE + 8, FAKE, FAKE, FAKE, None, None, 0, 0, FAKE, n, None) == ALIGN
    assert f(dims(4, 256, 128), FAKE, FAKE, FAKE, FAKE, None, None, 0, 0, FAKE + 16, n, None) == ALIGN
    assert f(dims(4, 256, 128), FAKE, FAKE, FAKE, FAKE, None, None, 0, 0, FAKE, 100, None) == WS
    offs = (ctypes.c_size_t * 6)()
    assert L.mxfp4_repack_offsets(dims(4, 256, 128, 1), 1, offs) == OK
    assert list(offs)[0] == 0 and all(o % 256 == 0 for o in offs) and list(offs) == sorted(offs)
    assert L.mxfp4_repack_offsets(dims(4, 256, 128, 1), 0, offs) == LAYOUT


def test_route_and_forward_validation(L):
    assert L.moe_mxfp4_route_workspace_bytes(64, 128, 8) > 0
    assert L.moe_mxfp4_route_workspace_bytes(64, 128, 0) == 0
    assert L.moe_mxfp4_route_workspace_bytes(64, 4, 5) == 0        # k > E
    assert L.moe_mxfp4_route_workspace_bytes(64, 2048, 8) == 0     # E > 1024
    assert L.moe_mxfp4_route_workspace_bytes(64, 128, 33) == 0     # k > 32
    r = L.moe_mxfp4_route
    n = L.moe_mxfp4_route_workspace_bytes(64, 128, 8)
    assert r(FAKE, 64, 128, 8, 1, FAKE, FAKE, FAKE, FAKE, FAKE, n - 1, None) == WS
    assert r(FAKE, 64, 128, 8, 1, None, FAKE, FAKE, FAKE, FAKE, n, None) == NULL
    assert r(FAKE, 64, 128, 8, 1, FAKE, FAKE, FAKE, FAKE, FAKE + 64, n, None) == ALIGN
    d = dims(128, 2048, 768)
    nws = L.moe_mxfp4_workspace_bytes(d, 64, 8)
    assert nws > 0
    fw = L.moe_mxfp4_forward
    args = [d, FAKE, FAKE, 64, 2048, FAKE, 8, 1, FAKE, None, None, FAKE, nws, None]
    bad = list(args); bad[11] = None
    assert fw(*bad) == NULL
    bad = list(args); bad[12] = nws - 1
    assert fw(*bad) == WS
    bad = list(args); bad[4] = 2000
    assert fw(*bad) == SHAPE  # ldx < H
    bad = list(args); bad[6] = 0
    assert fw(*bad) == SHAPE
    bad = list(args); bad[1] = FAKE + 16
    assert fw(*bad) == ALIGN
    bad = list(args); bad[2] = FAKE + 2
    assert fw(*bad) == ALIGN
    bad = list(args); bad[3] = 0
    assert fw(*bad) == OK  # no tokens: nothing to do


def test_forward_rejects_activation_buffers_past_32_bit_offsets(L):
    """The GEMMs address the split activations with 32-bit byte offsets: the first GEMM's records
    take T * H / 64 * 144 bytes, the second GEMM's operand about 2 bytes per padded row and I
    element.  Shapes whose buffers reach 4 GiB are rejected before any launch (and before the
    workspace size is looked at)."""
    fw = L.moe_mxfp4_forward
    d = dims(8, 7168, 2048)
    limit = (1 << 32) // (7168 // 64 * 144)  # tokens at which the first GEMM's records reach 4 GiB
    assert fw(d, FAKE, FAKE, limit + 1, 7168, FAKE, 1, 1, FAKE, None, None, FAKE, 1 << 62, None) == SHAPE
    # just below: the size check passes and the (too small) workspace is what fails
    assert fw(d, FAKE, FAKE, limit - 1, 7168, FAKE, 1, 1, FAKE, None, None, FAKE, 256, None) == WS
    # the second GEMM's operand: 100000 tokens x top-16 pairs, I = 2048 -> about 4.9e9 bytes
    d2 = dims(64, 256, 2048)
    assert fw(d2, FAKE, FAKE, 100000, 256, FAKE, 16, 1, FAKE, None, None, FAKE, 1 << 62, None) == SHAPE
