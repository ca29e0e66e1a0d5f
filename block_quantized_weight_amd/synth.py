"""Seeded synthetic inputs for the block-scaled small-M GEMV.

This module only draws random numbers and packs them into the byte layouts the
library consumes. It holds none of the method's arithmetic (no decoding, no
dequantisation, no products), so both the GPU path and the CPU oracle can take
their inputs from here without sharing any computation.

Workloads (shapes and value distributions) follow the decode projections the
pages measure: the 8-bit Qwen3-8B-class qkv weight 4096x4096 ("MatMulNBits
8-bit: wide fp16 M=1 kernel", Results table), the FP8 5120x6144 projection
("Pin FP8 GEMV residency", H200 measurement table), the NVFP4 lm_head
N=248320, K=2048 ("Block-scaled MatMul decode GEMV", FP4 mma paragraph), the
4-bit lm_head K=4096, N=151936 ("Batched small-M GEMV for MatMulNBits", 4-bit
tables) and the small-N split-K corner M<=8, N<=1024 ("opt-in split-K GEMV for
small-N fp16 shapes", Description).

Draw order for every workload: one ``numpy.random.default_rng(seed)`` draws
A, then the weight codes, then the zero points, then the scales. A is drawn
at the workload's largest M so that rows are shared across an M sweep.
"""

from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Optional, Tuple

import numpy as np

FORMATS = ("u4", "u8", "fp8", "nvfp4")
ACT_DTYPES = ("f16", "bf16")

# E4M3 (OCP E4M3FN) byte codes 0x7F and 0xFF are NaN; every other code is finite.
FP8_FINITE_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
# Positive normal E4M3 codes from 2^-6 (0x08) up to 2^2 (0x48), inclusive.
NVFP4_SCALE_CODES = np.arange(0x08, 0x49, dtype=np.uint8)


@dataclasses.dataclass
class Problem:
    """One quantized weight plus the activations that multiply it.

    Byte layouts (all row-major, C order):
      u4    W [N, K/bs, bs/2] uint8, two codes per byte, low nibble = lower k
            scales [N, K/bs] fp16 bits (uint16)
            zp [N, ceil((K/bs)/2)] uint8, two 4-bit zero points per byte,
            low nibble = even block
      u8    W [N, K/bs, bs] uint8; scales [N, K/bs] fp16 bits; zp [N, K/bs] uint8
      fp8   W [N, K] uint8 E4M3 codes; scales [N, K/bs] float32; no zp
      nvfp4 W [N, K/2] uint8 packed E2M1, low nibble = lower k;
            scales [N, K/16] uint8 E4M3 codes; tensor_scale float32; no zp
    A is [M_max, K] activation bits (uint16) of dtype ``act`` (f16 or bf16); the
    optional bias is [N] bits of the same dtype, added to every row of Y.
    """

    name: str
    fmt: str
    act: str
    N: int
    K: int
    bs: int
    W: np.ndarray
    scales: np.ndarray
    zp: Optional[np.ndarray]
    tensor_scale: float
    A: np.ndarray
    ms: Tuple[int, ...] = (1,)
    seed: int = 0
    bias: Optional[np.ndarray] = None  # [N] activation bits (uint16), or None

    @property
    def m_max(self) -> int:
        return int(self.A.shape[0])

    def weight_bytes(self) -> int:
        """Codes + block scales + zero points (+4 B tensor scale for nvfp4)."""
        n = self.W.nbytes + self.scales.nbytes + (0 if self.zp is None else self.zp.nbytes)
        return n + (4 if self.fmt == "nvfp4" else 0)

    def code_bytes(self) -> int:
        return int(self.W.nbytes)

    def hashes(self) -> Dict[str, str]:
        out = {"A": sha256(self.A), "W": sha256(self.W), "scales": sha256(self.scales)}
        if self.zp is not None:
            out["zp"] = sha256(self.zp)
        return out


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


# --------------------------------------------------------------------------------------
# packing helpers (pure byte shuffling)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit values two per byte along the last axis, low nibble first."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[-1] % 2:
        pad = np.zeros(codes.shape[:-1] + (1,), dtype=np.uint8)
        codes = np.concatenate([codes, pad], axis=-1)
    lo = codes[..., 0::2]
    hi = codes[..., 1::2]
    return (lo & 0x0F) | ((hi & 0x0F) << 4)


def unpack_nibbles(packed: np.ndarray, count: int) -> np.ndarray:
    """Inverse of :func:`pack_nibbles` (keeps the first ``count`` values)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out[..., :count]


def round_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> IEEE binary16 (numpy's round-to-nearest-even), returned as bits."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bfloat16 with round-to-nearest-even, returned as bits."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def activation_bits(x: np.ndarray, act: str) -> np.ndarray:
    if act == "f16":
        return round_to_f16_bits(x)
    if act == "bf16":
        return round_to_bf16_bits(x)
    raise ValueError(f"unknown activation dtype {act!r}")


# --------------------------------------------------------------------------------------
# generic generator


def make_problem(
    fmt: str,
    act: str,
    N: int,
    K: int,
    bs: int,
    m_max: int,
    seed: int,
    *,
    name: str = "custom",
    ms: Tuple[int, ...] = (1,),
    zp_range: Tuple[int, int] = (0, 15),
    scale_sigma: float = 0.02,
    fp8_scale_exp: Tuple[float, float] = (-8.0, -4.0),
    tensor_scale: float = 0.01,
    with_zp: bool = True,
    with_bias: bool = False,
    bias_sigma: float = 0.5,
) -> Problem:
    """Draw one problem: A, then codes, then zero points, then scales, then (when
    asked) the bias, N(0, bias_sigma) rounded to the activation dtype. The bias is
    drawn last so the other arrays do not depend on whether it is drawn."""
    if fmt not in FORMATS:
        raise ValueError(f"unknown format {fmt!r}")
    if fmt == "nvfp4" and bs != 16:
        raise ValueError("nvfp4 uses one scale per 16 elements")
    if K % bs:
        raise ValueError("K must be a multiple of the block size")
    rng = np.random.default_rng(seed)
    A = activation_bits(rng.standard_normal((m_max, K)), act).reshape(m_max, K)
    nblk = K // bs
    zp = None
    ts = 1.0
    if fmt == "u4":
        codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
        W = pack_nibbles(codes).reshape(N, nblk, bs // 2)
        del codes
        if with_zp:
            z = rng.integers(zp_range[0], zp_range[1] + 1, size=(N, nblk), dtype=np.uint8)
            zp = pack_nibbles(z)
        scales = round_to_f16_bits(np.abs(rng.standard_normal((N, nblk))) * scale_sigma)
    elif fmt == "u8":
        W = rng.integers(0, 256, size=(N, nblk, bs), dtype=np.uint8)
        if with_zp:
            zp = rng.integers(zp_range[0], zp_range[1] + 1, size=(N, nblk), dtype=np.uint8)
        scales = round_to_f16_bits(np.abs(rng.standard_normal((N, nblk))) * scale_sigma)
    elif fmt == "fp8":
        idx = rng.integers(0, FP8_FINITE_CODES.size, size=(N, K))
        W = FP8_FINITE_CODES[idx]
        del idx
        e = rng.uniform(fp8_scale_exp[0], fp8_scale_exp[1], size=(N, nblk))
        scales = np.exp2(e).astype(np.float32)
    else:  # nvfp4
        codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
        W = pack_nibbles(codes)
        del codes
        idx = rng.integers(0, NVFP4_SCALE_CODES.size, size=(N, nblk))
        scales = NVFP4_SCALE_CODES[idx]
        ts = float(np.float32(tensor_scale))
    bias = activation_bits(rng.standard_normal(N) * bias_sigma, act).reshape(N) if with_bias else None
    return Problem(
        name=name, fmt=fmt, act=act, N=N, K=K, bs=bs, W=np.ascontiguousarray(W),
        scales=np.ascontiguousarray(scales), zp=None if zp is None else np.ascontiguousarray(zp),
        tensor_scale=ts, A=np.ascontiguousarray(A), ms=tuple(ms), seed=seed,
        bias=None if bias is None else np.ascontiguousarray(bias),
    )


def make_zero_point_problem(
    fmt: str,
    act: str,
    N: int,
    K: int,
    bs: int,
    seed: int,
    *,
    frac: float = 1.0,
    rows: Tuple[Tuple[float, float], ...] = ((16.0, 0.0), (64.0, 0.0), (1.0, 8192.0), (0.0, 8192.0)),
    scale_sigma: Optional[float] = None,
) -> Problem:
    """A 4- or 8-bit problem whose codes equal their block's zero point in a fraction
    ``frac`` of the (column, block) pairs (every pair for frac = 1): the weight those
    blocks dequantize to is zero, so the outputs are sums over the other blocks only
    (all zero for frac = 1), while the codes and zero points themselves span their
    whole range. Row i of A is N(0, rows[i][0]) plus, when rows[i][1] is nonzero, one
    entry of +-rows[i][1] at a random k (a single large activation). Drawn after
    make_problem's own draws with the same generator: the block choice, then per row
    the normal values, the spike position and its sign. Zero points are uniform over
    the full code range (0..15 or 0..255); scales are |N(0,1)| * scale_sigma (by default
    0.02 for 4-bit and 0.004 for 8-bit codes, as in the named workloads)."""
    if fmt not in ("u4", "u8"):
        raise ValueError("zero points exist for the 4- and 8-bit codes only")
    if scale_sigma is None:
        scale_sigma = 0.02 if fmt == "u4" else 0.004
    zr = (0, 15) if fmt == "u4" else (0, 255)
    base = make_problem(fmt, act, N, K, bs, 1, seed, name=f"zp_{fmt}_{act}", zp_range=zr,
                        scale_sigma=scale_sigma)
    rng = np.random.default_rng(seed + 7919)
    nblk = K // bs
    if fmt == "u4":
        z = unpack_nibbles(base.zp, nblk)  # [N, nblk]
        fill = (z | (z << 4)).astype(np.uint8)  # both nibbles of a byte hold z
    else:
        z = base.zp
        fill = z.astype(np.uint8)
    pick = rng.random((N, nblk)) < frac
    W = base.W.copy()
    W[pick] = fill[pick][:, None]
    A = np.zeros((len(rows), K), dtype=np.float64)
    for i, (sigma, spike) in enumerate(rows):
        A[i] = rng.standard_normal(K) * sigma
        if spike:
            k = int(rng.integers(0, K))
            A[i, k] = spike if rng.random() < 0.5 else -spike
    Abits = activation_bits(A, act).reshape(len(rows), K)
    return dataclasses.replace(base, W=np.ascontiguousarray(W), A=np.ascontiguousarray(Abits),
                               ms=(len(rows),))


# --------------------------------------------------------------------------------------
# the named workloads

WORKLOADS = {
    # tiny 4-bit case the oracle finishes instantly
    "u4_m1_k512_n256": dict(fmt="u4", act="f16", N=256, K=512, bs=32, ms=(1,), seed=0,
                            zp_range=(0, 15), scale_sigma=0.02),
    # 8-bit weight-only qkv-class projection at M=1
    "u8_m1_k4096_n4096": dict(fmt="u8", act="f16", N=4096, K=4096, bs=128, ms=(1,), seed=1,
                              zp_range=(96, 160), scale_sigma=0.004),
    # FP8 block-scaled projection, M in {1,4,8}
    "fp8_k6144_n5120": dict(fmt="fp8", act="f16", N=5120, K=6144, bs=128, ms=(1, 4, 8), seed=2),
    # NVFP4 multi-token verify, small shape
    "nvfp4_m4_k2048_n2048": dict(fmt="nvfp4", act="bf16", N=2048, K=2048, bs=16, ms=(4,), seed=3),
    # NVFP4 lm_head
    "nvfp4_m4_k2048_n248320": dict(fmt="nvfp4", act="bf16", N=248320, K=2048, bs=16, ms=(4,), seed=3),
    # 4-bit lm_head small-M sweep
    "u4_k4096_n151936": dict(fmt="u4", act="bf16", N=151936, K=4096, bs=32, ms=(1, 2, 4, 8, 16),
                             seed=4, zp_range=(0, 15), scale_sigma=0.02),
    # small-N split-K corner
    "u4_m8_k2048_n1024": dict(fmt="u4", act="f16", N=1024, K=2048, bs=32, ms=(8,), seed=40,
                              zp_range=(0, 15), scale_sigma=0.02),
    # a tall-K shape in the same corner (N <= 1024, large K), where the K range is also
    # split across workgroups (FP8 codes and scales drawn as for the FP8 projection)
    "fp8_m8_k16384_n1024": dict(fmt="fp8", act="f16", N=1024, K=16384, bs=128, ms=(8,), seed=41),
}


def workload(name: str, *, n_override: Optional[int] = None, with_bias: bool = False) -> Problem:
    """Generate a named workload. ``n_override`` keeps the seed and the draw order
    but changes N (used to make small slices with the same distributions);
    ``with_bias`` also draws a per-column bias, after everything else."""
    spec = dict(WORKLOADS[name])
    ms = spec.pop("ms")
    N = spec.pop("N") if n_override is None else (spec.pop("N"), n_override)[1]
    return make_problem(spec.pop("fmt"), spec.pop("act"), N, spec.pop("K"), spec.pop("bs"),
                        max(ms), spec.pop("seed"), name=name, ms=ms, with_bias=with_bias, **spec)
