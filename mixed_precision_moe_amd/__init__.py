"""MXFP4 block quantization and the MXFP4-weight x BF16-activation MoE layer on MI355X (gfx950).

Thin torch binding of the C ABI in include/mxfp4moe.h: it checks dtypes, shapes and devices,
allocates outputs and workspaces with torch, and passes raw device pointers plus the current HIP
stream.  Every step of the computation runs in the library's HIP kernels.
"""

import ctypes

import torch

from . import _lib
from ._lib import MoeDims, Mxfp4Error, check

LAYOUT_GFX950 = 0
LAYOUT_STD_W31 = 1
LAYOUT_SCALE_TILED = 2

ACT_BF16 = 0   # bf16 activations (three-term split inside the kernels)
ACT_MXFP8 = 1  # both GEMM inputs quantized to MXFP8 (E4M3 + E8M0 per 32)
ACT_MXFP4 = 2  # both GEMM inputs quantized to MXFP4 (E2M1 + E8M0 per 32)

__all__ = ["quantize", "tiled_scale_shape", "nvfp4_quantize", "nvfp4_tiled_scale_shape", "repack_weights", "unpack_weights", "check_packed", "route",
           "moe_forward", "moe_forward_noalloc", "NOALLOC_SCRATCH_BYTES", "MoE", "Linear", "MoeDims", "Mxfp4Error",
           "LAYOUT_GFX950", "LAYOUT_STD_W31", "LAYOUT_SCALE_TILED", "ACT_BF16", "ACT_MXFP8", "ACT_MXFP4"]


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _cuda(t, name):
    _need(t.is_cuda, f"{name} must be a GPU tensor")


def tiled_scale_shape(M, K):
    return ((M + 127) // 128, (K // 32 + 3) // 4, 32, 4, 4)


def quantize(x, flat=True, tiled=True):
    """x: bf16 [M, K] on the GPU (rows may be strided; the last dim must be contiguous).
    Returns (q uint8 [M, K/2], flat scales uint8 [M, K/32] or None, tiled scales uint8
    [ceil(M/128), ceil(K/128), 32, 4, 4] or None)."""
    _cuda(x, "x")
    _need(x.dtype == torch.bfloat16 and x.dim() == 2, "x must be a 2-D bfloat16 tensor")
    _need(x.stride(1) == 1, "x's last dimension must be contiguous")
    M, K = x.shape
    q = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    sf = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device) if flat else None
    st = torch.empty(tiled_scale_shape(M, K), dtype=torch.uint8, device=x.device) if tiled else None
    check("mxfp4_quantize", _lib.lib().mxfp4_quantize(_ptr(x), M, K, x.stride(0), _ptr(q), _ptr(sf), _ptr(st), _stream()))
    return q, sf, st


def nvfp4_tiled_scale_shape(M, K):
    return ((M + 127) // 128, (K // 16 + 3) // 4, 32, 4, 4)


def nvfp4_quantize(x, global_scale, flat=True, tiled=True):
    """NVFP4: x bf16 [M, K] on the GPU (K % 16 == 0; rows may be strided), global_scale a positive float.
    Returns (q uint8 [M, K/2], E4M3 scales uint8 [M, K/16] or None, tiled scales uint8
    [ceil(M/128), ceil(K/64), 32, 4, 4] or None)."""
    _cuda(x, "x")
    _need(x.dtype == torch.bfloat16 and x.dim() == 2, "x must be a 2-D bfloat16 tensor")
    _need(x.stride(1) == 1, "x's last dimension must be contiguous")
    M, K = x.shape
    q = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    sf = torch.empty((M, K // 16), dtype=torch.uint8, device=x.device) if flat else None
    st = torch.empty(nvfp4_tiled_scale_shape(M, K), dtype=torch.uint8, device=x.device) if tiled else None
    check("nvfp4_quantize", _lib.lib().nvfp4_quantize(_ptr(x), M, K, x.stride(0), float(global_scale), _ptr(q), _ptr(sf),
                                                      _ptr(st), _stream()))
    return q, sf, st


def _dims(E, H, I, has_bias):
    return MoeDims(E, H, I, 1 if has_bias else 0)


def repack_weights(w13_q, w13_s, w2_q, w2_s, b13=None, b2=None, layout=LAYOUT_GFX950):
    """Standard checkpoint tensors (w13 rows [w1; w3]) -> execution blob (layout GFX950), or the six
    standard tensors of a checked conversion (other layouts), returned as a tuple in the order
    (w13_q, w2_q, w13_s, w2_s, b13, b2)."""
    for n, t in (("w13_q", w13_q), ("w13_s", w13_s), ("w2_q", w2_q), ("w2_s", w2_s)):
        _cuda(t, n)
        _need(t.dtype == torch.uint8 and t.is_contiguous() and t.dim() == 3, f"{n} must be contiguous uint8 3-D")
    E, I2, Hh = w13_q.shape
    H, I = Hh * 2, I2 // 2
    _need(w13_s.shape == (E, 2 * I, H // 32) and w2_q.shape == (E, H, I // 2) and w2_s.shape == (E, H, I // 32),
          "inconsistent weight shapes")
    has_bias = b13 is not None
    _need((b13 is None) == (b2 is None), "give both biases or neither")
    is_fp32 = 0
    if has_bias:
        _need(b13.dtype == b2.dtype and b13.dtype in (torch.float32, torch.bfloat16), "biases must be fp32 or bf16")
        _need(b13.shape == (E, 2 * I) and b2.shape == (E, H) and b13.is_contiguous() and b2.is_contiguous(),
              "bias shapes")
        is_fp32 = 1 if b13.dtype == torch.float32 else 0
    d = _dims(E, H, I, has_bias)
    L = _lib.lib()
    nbytes = L.mxfp4_repack_bytes(ctypes.byref(d), layout)
    _need(nbytes > 0, "invalid dimensions or layout")
    out = torch.empty(nbytes, dtype=torch.uint8, device=w13_q.device)
    check("mxfp4_repack_weights",
          L.mxfp4_repack_weights(ctypes.byref(d), _ptr(w13_q), _ptr(w13_s), _ptr(w2_q), _ptr(w2_s), _ptr(b13), _ptr(b2),
                                 is_fp32, layout, _ptr(out), nbytes, _stream()))
    if layout == LAYOUT_GFX950:
        return out
    offs = (ctypes.c_size_t * 6)()
    check("mxfp4_repack_offsets", L.mxfp4_repack_offsets(ctypes.byref(d), layout, offs))
    tiled = bool(layout & LAYOUT_SCALE_TILED)
    # the order of the pages' conversion result: w13, w2, w13 scales, w2 scales, b13, b2
    shapes = [(E, 2 * I, H // 2),
              (E, H, I // 2),
              (E,) + tiled_scale_shape(2 * I, H) if tiled else (E, 2 * I, H // 32),
              (E,) + tiled_scale_shape(H, I) if tiled else (E, H, I // 32),
              (E, 2 * I), (E, H)]
    res = []
    for i, shp in enumerate(shapes):
        if i >= 4:
            if not has_bias:
                res.append(None)
                continue
            n = 1
            for s in shp:
                n *= s
            res.append(out[offs[i]: offs[i] + 2 * n].view(torch.bfloat16).view(shp))
        else:
            n = 1
            for s in shp:
                n *= s
            res.append(out[offs[i]: offs[i] + n].view(shp))
    return tuple(res)


def unpack_weights(packed, E, H, I, has_bias):
    """Execution blob -> (w13_q, w13_s, w2_q, w2_s, b13 bf16 or None, b2 bf16 or None)."""
    _cuda(packed, "packed")
    dev = packed.device
    w13_q = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=dev)
    w13_s = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=dev)
    w2_q = torch.empty((E, H, I // 2), dtype=torch.uint8, device=dev)
    w2_s = torch.empty((E, H, I // 32), dtype=torch.uint8, device=dev)
    b13 = torch.empty((E, 2 * I), dtype=torch.bfloat16, device=dev) if has_bias else None
    b2 = torch.empty((E, H), dtype=torch.bfloat16, device=dev) if has_bias else None
    d = _dims(E, H, I, has_bias)
    check("mxfp4_unpack_weights",
          _lib.lib().mxfp4_unpack_weights(ctypes.byref(d), _ptr(packed), _ptr(w13_q), _ptr(w13_s), _ptr(w2_q),
                                          _ptr(w2_s), _ptr(b13), _ptr(b2), _stream()))
    return w13_q, w13_s, w2_q, w2_s, b13, b2


def check_packed(packed, E, H, I, has_bias):
    d = _dims(E, H, I, has_bias)
    return _lib.lib().mxfp4_check_packed(ctypes.byref(d), _ptr(packed), _stream())


def route(logits, top_k, renormalize=True):
    """logits fp32 [T, E] -> (topk_ids int32 [T, k], topk_w fp32 [T, k], expert_offsets int32 [E+1],
    sorted_pairs int32 [T*k])."""
    _cuda(logits, "logits")
    _need(logits.dtype == torch.float32 and logits.dim() == 2 and logits.is_contiguous(), "logits: contiguous fp32 2-D")
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sp = torch.empty(T * top_k, dtype=torch.int32, device=dev)
    L = _lib.lib()
    nws = L.moe_mxfp4_route_workspace_bytes(T, E, top_k)
    _need(nws > 0, "invalid routing arguments")
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    check("moe_mxfp4_route", L.moe_mxfp4_route(_ptr(logits), T, E, top_k, 1 if renormalize else 0, _ptr(ids), _ptr(w),
                                              _ptr(offs), _ptr(sp), _ptr(ws), nws, _stream()))
    return ids, w, offs, sp


def workspace_bytes(E, H, I, has_bias, T, top_k):
    d = _dims(E, H, I, has_bias)
    return _lib.lib().moe_mxfp4_workspace_bytes(ctypes.byref(d), T, top_k)


def moe_forward(packed, E, H, I, has_bias, x, logits, top_k, renormalize=True, workspace=None, y=None,
                topk_ids=None, topk_w=None, act_format=ACT_BF16):
    """One MoE layer.  x bf16 [T, H] (rows may be strided), logits fp32 [T, E]; returns y bf16 [T, H].
    act_format: ACT_BF16, or ACT_MXFP8 / ACT_MXFP4 for the quantized-activation variants."""
    _cuda(x, "x")
    _cuda(logits, "logits")
    _need(x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1 and x.shape[1] == H, "x: bf16 [T, H]")
    T = x.shape[0]
    _need(logits.dtype == torch.float32 and logits.shape == (T, E) and logits.is_contiguous(), "logits: fp32 [T, E]")
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    d = _dims(E, H, I, has_bias)
    L = _lib.lib()
    nws = L.moe_mxfp4_workspace_bytes(ctypes.byref(d), T, top_k)
    _need(nws > 0, "invalid MoE arguments")
    if workspace is None:
        workspace = torch.empty(nws, dtype=torch.uint8, device=x.device)
    check("moe_mxfp4_forward_act",
          L.moe_mxfp4_forward_act(ctypes.byref(d), act_format, _ptr(packed), _ptr(x), T, x.stride(0), _ptr(logits),
                                  top_k, 1 if renormalize else 0, _ptr(y), _ptr(topk_ids), _ptr(topk_w),
                                  _ptr(workspace), workspace.numel(), _stream()))
    return y


NOALLOC_SCRATCH_BYTES = 32 << 20  # MXFP4_NOALLOC_SCRATCH_BYTES


def moe_forward_noalloc(packed, E, H, I, has_bias, x, logits, top_k, y, renormalize=True, topk_ids=None,
                        topk_w=None):
    """moe_forward on the library's own device scratch array (no workspace, nothing allocated by the
    library; y is the caller's).  Fails with status 4 when the shape needs more workspace than the
    array holds (NOALLOC_SCRATCH_BYTES)."""
    _cuda(x, "x")
    _cuda(logits, "logits")
    _need(x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1 and x.shape[1] == H, "x: bf16 [T, H]")
    T = x.shape[0]
    _need(logits.dtype == torch.float32 and logits.shape == (T, E) and logits.is_contiguous(), "logits: fp32 [T, E]")
    _need(y.dtype == torch.bfloat16 and y.shape == (T, H) and y.is_contiguous(), "y: bf16 [T, H]")
    d = _dims(E, H, I, has_bias)
    check("moe_mxfp4_forward_noalloc",
          _lib.lib().moe_mxfp4_forward_noalloc(ctypes.byref(d), _ptr(packed), _ptr(x), T, x.stride(0), _ptr(logits),
                                               top_k, 1 if renormalize else 0, _ptr(y), _ptr(topk_ids),
                                               _ptr(topk_w), _stream()))
    return y


class Linear:
    """A dense MXFP4-weight linear layer y = x W^T + b (W4A16): packed weights and a reusable workspace.
    w_q uint8 [N, K/2], w_s uint8 [N, K/32] (device), bias fp32 / bf16 [N] or None."""

    def __init__(self, w_q, w_s, bias=None):
        for n, t in (("w_q", w_q), ("w_s", w_s)):
            _cuda(t, n)
            _need(t.dtype == torch.uint8 and t.is_contiguous() and t.dim() == 2, f"{n} must be contiguous uint8 2-D")
        self.N, Kh = w_q.shape
        self.K = 2 * Kh
        _need(w_s.shape == (self.N, self.K // 32), "w_s shape")
        self.has_bias = bias is not None
        is_fp32 = 0
        if bias is not None:
            _need(bias.dtype in (torch.float32, torch.bfloat16) and bias.shape == (self.N,) and bias.is_contiguous(),
                  "bias: contiguous fp32 or bf16 [N]")
            is_fp32 = 1 if bias.dtype == torch.float32 else 0
        L = _lib.lib()
        n = L.mxfp4_linear_pack_bytes(self.N, self.K, 1 if self.has_bias else 0)
        _need(n > 0, "invalid linear dimensions")
        self.packed = torch.empty(n, dtype=torch.uint8, device=w_q.device)
        check("mxfp4_linear_pack", L.mxfp4_linear_pack(self.N, self.K, _ptr(w_q), _ptr(w_s), _ptr(bias), is_fp32,
                                                        _ptr(self.packed), n, _stream()))
        self._ws = None

    def __call__(self, x, y=None):
        _cuda(x, "x")
        _need(x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1 and x.shape[1] == self.K,
              "x: bf16 [M, K]")
        M = x.shape[0]
        if y is None:
            y = torch.empty((M, self.N), dtype=torch.bfloat16, device=x.device)
        L = _lib.lib()
        n = L.mxfp4_linear_workspace_bytes(M, self.N, self.K)
        _need(n > 0, "invalid linear arguments")
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(n, dtype=torch.uint8, device=x.device)
        check("mxfp4_linear_forward",
              L.mxfp4_linear_forward(_ptr(self.packed), self.N, self.K, 1 if self.has_bias else 0, _ptr(x), M,
                                     x.stride(0), _ptr(y), _ptr(self._ws), self._ws.numel(), _stream()))
        return y


class MoE:
    """An MXFP4 MoE layer: packed weights and a reusable workspace."""

    def __init__(self, w13_q, w13_s, w2_q, w2_s, b13=None, b2=None, top_k=8, renormalize=True, act_format=ACT_BF16):
        self.E, I2, Hh = w13_q.shape
        self.H, self.I = Hh * 2, I2 // 2
        self.has_bias = b13 is not None
        self.top_k, self.renormalize, self.act_format = top_k, renormalize, act_format
        self.packed = repack_weights(w13_q, w13_s, w2_q, w2_s, b13, b2, LAYOUT_GFX950)
        self._ws = None

    def workspace(self, T):
        n = workspace_bytes(self.E, self.H, self.I, self.has_bias, T, self.top_k)
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(n, dtype=torch.uint8, device=self.packed.device)
        return self._ws

    def __call__(self, x, logits, y=None, topk_ids=None, topk_w=None):
        return moe_forward(self.packed, self.E, self.H, self.I, self.has_bias, x, logits, self.top_k, self.renormalize,
                           self.workspace(x.shape[0]), y, topk_ids, topk_w, self.act_format)
