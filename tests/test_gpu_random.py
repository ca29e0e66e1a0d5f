"""Seeded random parity: many shapes, row counts, entry points and forced plan choices
against the oracle.

Each case draws a format, activation dtype and block size, a ragged N, a K that is a
whole number of blocks, M from 1 to 40 (so 16-row chunks and row passes occur), and
either the automatic plan or a forced family, K split, part count, staging or ring
choice, through qgemv_run or qgemv_run_ws. K is drawn as a whole number of the units the
case's forced choice walks (four 16-byte chunks per column for the matrix family, one
chunk for the streaming family, one block otherwise), so every case runs. Every output
must lie within |y - y_ref| <= 1e-3 * sum|a*w| + 1e-3 of the oracle (plus a bf16
output's final rounding: strict=False), and a run with a workspace must leave it all
zero.
"""

import numpy as np
import pytest

import block_quantized_weight_amd as bqw
from block_quantized_weight_amd import synth

pytestmark = pytest.mark.gpu

from tests import gpu_util as gu

FORMATS = [("u4", 16), ("u4", 32), ("u4", 64), ("u4", 128), ("u8", 32), ("u8", 128), ("fp8", 32), ("fp8", 128),
           ("nvfp4", 16)]


KPC = {"u4": 32, "nvfp4": 32, "u8": 16, "fp8": 16}


def k_unit(fmt, bs, flags):
    """The K granularity the case's forced family needs: four chunks per column for the
    matrix family, a chunk for the streaming family, a block otherwise (NVFP4: two
    blocks, a byte of codes)."""
    fam = flags & 0xF
    unit = {2: 4 * KPC[fmt], 1: KPC[fmt]}.get(fam, 32 if fmt == "nvfp4" else bs)
    return int(np.lcm(unit, bs))


def draw_cases(n, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        fmt, bs = FORMATS[rng.integers(len(FORMATS))]
        act = "bf16" if rng.random() < 0.5 else "f16"
        N = int(rng.choice([1, 7, 16, 33, 100, 255, 640, 1000, 1500, 2047]))
        kraw = int(rng.integers(1, 8192 + 1))  # the K range, before rounding to the case's unit
        M = int(rng.choice([1, 2, 3, 4, 5, 8, 9, 12, 16, 17, 23, 33, 40]))
        kind = rng.integers(7)
        flags = 0
        if kind == 1:
            flags = int(rng.integers(1, 4))  # a forced family
        elif kind == 2:
            flags = 2 | (int(rng.choice([1, 2, 4, 8])) << 8)  # matrix family, forced K split
        elif kind == 3:
            flags = 2 | (int(rng.integers(1, 5)) << 4)  # matrix family, forced part count
        elif kind == 4:
            flags = 2 | int(rng.choice([bqw.FLAG_STAGE_A_ON, bqw.FLAG_STAGE_A_OFF]))
        elif kind == 5:
            flags = 2 | int(rng.choice([bqw.FLAG_RING_ON, bqw.FLAG_RING_OFF]))
        ws = bool(rng.random() < 0.5)
        unit = k_unit(fmt, bs, flags)
        K = max(unit, (kraw + unit - 1) // unit * unit)
        if N * K * M > 60_000_000:
            M = max(1, 60_000_000 // (N * K))
        cases.append((i, fmt, act, bs, N, K, M, flags, ws))
    return cases


@pytest.mark.parametrize("i,fmt,act,bs,N,K,M,flags,ws", draw_cases(200))
def test_random_case_against_the_oracle(i, fmt, act, bs, N, K, M, flags, ws):
    prob = synth.make_problem(fmt, act, N, K, bs, M, seed=1000 + i)
    plan = bqw.select(fmt, act, N, K, bs, min(M, 16), flags=flags, with_workspace=ws,
                      zero_points=0x2000 if prob.zp is not None else None)
    gu.say(f"[random {i}] {fmt}/{act} bs={bs} N={N} K={K} M={M} flags={flags:#x} ws={ws} plan={plan}")
    Y, got = gu.run_gpu(prob, M, flags=flags, ws=ws)
    if ws:
        assert got["ws_zero"], got
    ok, ratio, _, _ = gu.check_full(prob, M, Y, strict=False)
    assert ok, (i, ratio, got)


def draw_wide_cases(n, seed=2025):
    """Wide weights (N from 20000 to 70000, ragged), where the dispatcher's choices turn
    on how many tile groups fill the CUs: the DMA ring and its band, the K split, row
    passes, the streaming kernel at one or two rows. The automatic plan, K a whole number
    of four chunks (so the matrix family can take every case) up to 4096, M up to 16."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        fmt, bs = FORMATS[rng.integers(len(FORMATS))]
        act = "bf16" if rng.random() < 0.5 else "f16"
        N = int(rng.integers(20000, 70001))
        unit = int(np.lcm(4 * KPC[fmt], bs))
        K = unit * int(rng.integers(1, 4096 // unit + 1))
        M = int(rng.choice([1, 2, 3, 4, 5, 8, 9, 12, 16]))
        ws = bool(rng.random() < 0.5)
        cases.append((i, fmt, act, bs, N, K, M, ws))
    return cases


@pytest.mark.parametrize("i,fmt,act,bs,N,K,M,ws", draw_wide_cases(40))
def test_random_wide_case_against_the_oracle(i, fmt, act, bs, N, K, M, ws):
    """3000 sampled outputs and the first and last 40 columns of every row, against the
    oracle (plus a bf16 output's final rounding, as for the cases above)."""
    prob = synth.make_problem(fmt, act, N, K, bs, M, seed=5000 + i)
    gu.say(f"[random wide {i}] {fmt}/{act} bs={bs} N={N} K={K} M={M} ws={ws}")
    Y, got = gu.run_gpu(prob, M, ws=ws)
    if ws:
        assert got["ws_zero"], got
    ms, ns = gu.sample_points(M, N, 3000, i)
    yr, s = gu.oracle.gemv_points(prob, ms, ns, M=M)
    ok, ratio = gu.oracle.within_tolerance(Y[ms, ns], yr, s, out_dtype=prob.act)
    assert ok, (i, ratio, got)


def draw_long_cases(n, seed=2026):
    """Long rows (K from 8192 to 32768), where the activation rows outgrow the LDS: the
    streaming kernel's wide workgroups, the long-rows K parts, row passes. The automatic
    plan, N from 1000 to 40000 (at most 200 M weight elements), M up to 16."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        fmt, bs = FORMATS[rng.integers(len(FORMATS))]
        act = "bf16" if rng.random() < 0.5 else "f16"
        N = int(rng.integers(1000, 40001))
        unit = int(np.lcm(4 * KPC[fmt], bs))
        K = unit * int(rng.integers(8192 // unit, 32768 // unit + 1))
        N = min(N, 200_000_000 // K)  # at most 200 M weight elements to draw on the host
        M = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16]))
        ws = bool(rng.random() < 0.5)
        cases.append((i, fmt, act, bs, N, K, M, ws))
    return cases


@pytest.mark.parametrize("i,fmt,act,bs,N,K,M,ws", draw_long_cases(30))
def test_random_long_case_against_the_oracle(i, fmt, act, bs, N, K, M, ws):
    """3000 sampled outputs and the first and last 40 columns of every row, against the
    oracle (plus a bf16 output's final rounding)."""
    prob = synth.make_problem(fmt, act, N, K, bs, M, seed=7000 + i)
    gu.say(f"[random long {i}] {fmt}/{act} bs={bs} N={N} K={K} M={M} ws={ws}")
    Y, got = gu.run_gpu(prob, M, ws=ws)
    if ws:
        assert got["ws_zero"], got
    ms, ns = gu.sample_points(M, N, 3000, i)
    yr, s = gu.oracle.gemv_points(prob, ms, ns, M=M)
    ok, ratio = gu.oracle.within_tolerance(Y[ms, ns], yr, s, out_dtype=prob.act)
    assert ok, (i, ratio, got)


def draw_mid_cases(n, seed=2027):
    """Mid-size weights (N from 2048 to 20000, K from 1024 to 16384, at most 150 M weight
    elements), where the K split, its reduction area over the staged rows, K parts, row
    passes and the residency cut meet: the automatic plan or a forced K split, part
    count, DMA ring or unstaged rows, M up to 20."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        fmt, bs = FORMATS[rng.integers(len(FORMATS))]
        act = "bf16" if rng.random() < 0.5 else "f16"
        N = int(rng.integers(2048, 20001))
        kind = rng.integers(5)
        flags = 0
        if kind == 1:
            flags = 2 | (int(rng.choice([1, 2, 4, 8])) << 8)
        elif kind == 2:
            flags = 2 | (int(rng.integers(1, 5)) << 4)
        elif kind == 3:
            flags = 2 | int(rng.choice([bqw.FLAG_RING_ON | (1 << 8), bqw.FLAG_STAGE_A_OFF]))
        unit = int(np.lcm(4 * KPC[fmt], bs))
        K = unit * int(rng.integers(max(1, 1024 // unit), 16384 // unit + 1))
        N = min(N, 150_000_000 // K)
        M = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 9, 12, 16, 20]))
        ws = bool(rng.random() < 0.5)
        cases.append((i, fmt, act, bs, N, K, M, flags, ws))
    return cases


@pytest.mark.parametrize("i,fmt,act,bs,N,K,M,flags,ws", draw_mid_cases(40))
def test_random_mid_case_against_the_oracle(i, fmt, act, bs, N, K, M, flags, ws):
    """3000 sampled outputs and the first and last 40 columns of every row, against the
    oracle (plus a bf16 output's final rounding)."""
    prob = synth.make_problem(fmt, act, N, K, bs, M, seed=9000 + i)
    gu.say(f"[random mid {i}] {fmt}/{act} bs={bs} N={N} K={K} M={M} flags={flags:#x} ws={ws}")
    Y, got = gu.run_gpu(prob, M, flags=flags, ws=ws)
    if ws:
        assert got["ws_zero"], got
    ms, ns = gu.sample_points(M, N, 3000, i)
    yr, s = gu.oracle.gemv_points(prob, ms, ns, M=M)
    ok, ratio = gu.oracle.within_tolerance(Y[ms, ns], yr, s, out_dtype=prob.act)
    assert ok, (i, ratio, got)
