"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and rounds them to the storage types (bf16 via torch's
round-to-nearest-even cast, float32).  It holds none of the quantization or MoE arithmetic: both
the HIP path and the CPU oracle receive the same draws and do their own work on them.

Every tensor has its own seed, ``SeedSequence([20261202, config_id, tensor_id(, expert)])`` on an
SFC64 generator (fast enough for the 16.9 G weights of the largest configuration), so a tensor (or one
expert's weights) can be regenerated alone and in any order.
"""

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

ROOT_SEED = 20261202

# tensor ids
_X, _LOGITS, _OFFSETS, _W13, _W2, _B13, _B2, _QMAT, _ZERO = range(9)


@dataclass(frozen=True)
class MoEConfig:
    name: str
    cid: int
    T: int
    E: int
    k: int
    H: int
    I: int
    bias: bool
    w_sigma: float
    logits: str  # "normal" | "offset" | "zipf"
    renormalize: bool = True


MOE_CONFIGS = {
    # 16 tokens, 4 experts, top-2, hidden 256, intermediate 128, biases N(0, 0.01)
    "tiny": MoEConfig("tiny", 0, 16, 4, 2, 256, 128, True, 0.02, "normal"),
    # decode shape: 64 tokens, 128 experts, top-8, hidden 2048, intermediate 768, biases present
    "decode": MoEConfig("decode", 2, 64, 128, 8, 2048, 768, True, 0.02, "normal"),
    # prefill shape: 8192 tokens, same experts; per-expert logit offsets N(0, 1.5); no biases
    "prefill": MoEConfig("prefill", 3, 8192, 128, 8, 2048, 768, False, 0.02, "offset"),
    # large experts: 4096 tokens, 384 experts, hidden 7168, intermediate 2048, Zipf(1.2) popularity
    "large": MoEConfig("large", 4, 4096, 384, 8, 7168, 2048, False, 0.015, "zipf"),
}

QUANT_CONFIG = {"name": "quantize_8192x7168", "cid": 1, "M": 8192, "K": 7168}


def rng(*ids):
    return np.random.Generator(np.random.SFC64(np.random.SeedSequence([ROOT_SEED, *ids])))


def to_bf16_bits(a):
    """float array -> uint16 bf16 bit patterns (torch's round-to-nearest-even cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def custom_moe_config(name, T, E, k, H, I, bias=True, w_sigma=0.02, logits="normal", renormalize=True,
                      cid=100):
    return MoEConfig(name, cid, T, E, k, H, I, bias, w_sigma, logits, renormalize)


def moe_activations(cfg: MoEConfig):
    """x: bf16 bits [T, H] drawn N(0, 1); logits: float32 [T, E].

    normal: N(0, 1).  offset: N(0, 1) plus one N(0, 1.5) offset per expert (uneven expert loads).
    zipf: log p_{pi(e)} + Gumbel(0, 1) with p_r proportional to r**-1.2 over ranks r = 1..E and pi a
    seeded permutation, so the top-1 expert is Zipf(1.2)-distributed (Gumbel-max) and the top-k is a
    Zipf-weighted draw without replacement.
    """
    x = to_bf16_bits(rng(cfg.cid, _X).standard_normal((cfg.T, cfg.H), dtype=np.float32))
    g = rng(cfg.cid, _LOGITS)
    if cfg.logits == "zipf":
        ranks = np.arange(1, cfg.E + 1, dtype=np.float64)
        logp = -1.2 * np.log(ranks)
        perm = rng(cfg.cid, _OFFSETS).permutation(cfg.E)
        logits = logp[perm][None, :] + g.gumbel(size=(cfg.T, cfg.E))
    else:
        logits = g.standard_normal((cfg.T, cfg.E))
        if cfg.logits == "offset":
            logits = logits + rng(cfg.cid, _OFFSETS).normal(0.0, 1.5, size=cfg.E)[None, :]
    return x, np.ascontiguousarray(logits, dtype=np.float32)


def moe_master_expert(cfg: MoEConfig, e: int):
    """bf16 master weights of expert e: w13 [2I, H] (rows [w1; w3]) and w2 [H, I], N(0, w_sigma)."""
    w13 = rng(cfg.cid, _W13, e).standard_normal((2 * cfg.I, cfg.H), dtype=np.float32) * np.float32(cfg.w_sigma)
    w2 = rng(cfg.cid, _W2, e).standard_normal((cfg.H, cfg.I), dtype=np.float32) * np.float32(cfg.w_sigma)
    return to_bf16_bits(w13), to_bf16_bits(w2)


def moe_biases(cfg: MoEConfig):
    """bf16 biases b13 [E, 2I] and b2 [E, H] drawn N(0, 0.01), or (None, None)."""
    if not cfg.bias:
        return None, None
    b13 = rng(cfg.cid, _B13).normal(0.0, 0.01, size=(cfg.E, 2 * cfg.I))
    b2 = rng(cfg.cid, _B2).normal(0.0, 0.01, size=(cfg.E, cfg.H))
    return to_bf16_bits(b13), to_bf16_bits(b2)


def quant_matrix(M: int, K: int, cid: int = 1, zero_frac: float = 0.01, block: int = 32):
    """bf16 bits [M, K]: Student-t(3) values times a per-row 2**U(-8, 8) factor (U continuous), with
    round(zero_frac * blocks) of the `block`-element blocks set to zero, chosen without replacement."""
    g = rng(cid, _QMAT)
    v = g.standard_t(3, size=(M, K))
    v *= np.exp2(g.uniform(-8.0, 8.0, size=(M, 1)))
    nblk = M * (K // block)
    nz = int(round(zero_frac * nblk))
    if nz:
        zb = rng(cid, _ZERO).choice(nblk, size=nz, replace=False)
        v.reshape(nblk, block)[zb] = 0.0
    return to_bf16_bits(v)


def random_bits_matrix(M: int, K: int, seed: int):
    """Arbitrary finite bf16 patterns (every sign, exponent and mantissa), for edge-case tests."""
    g = rng(900, seed)
    b = g.integers(0, 1 << 16, size=(M, K), dtype=np.uint32).astype(np.uint16)
    expo = (b >> 7) & 0xFF
    b[expo == 0xFF] &= 0x807F  # map Inf/NaN exponents to zero/subnormal patterns
    return b
