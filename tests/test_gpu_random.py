"""Seeded random parity: many shapes, row counts, entry points and forced plan choices
against the oracle.

Each case draws a format, activation dtype and block size, a ragged N, a K that is a
whole number of blocks, M from 1 to 40 (so 16-row chunks and row passes occur), and
either the automatic plan or a forced family, K split, part count, staging or ring
choice, through qgemv_run or qgemv_run_ws. A forced choice the shape cannot take is
rejected by the host before any launch (status 7) and the case is skipped. Every output
must lie within |y - y_ref| <= 1e-3 * sum|a*w| + 1e-3 of the oracle (plus the output
type's final rounding: strict=False), and a run with a workspace must leave it all zero.
"""

import numpy as np
import pytest

import block_quantized_weight_amd as bqw
from block_quantized_weight_amd import synth

pytestmark = pytest.mark.gpu

from tests import gpu_util as gu

FORMATS = [("u4", 16), ("u4", 32), ("u4", 64), ("u4", 128), ("u8", 32), ("u8", 128), ("fp8", 32), ("fp8", 128),
           ("nvfp4", 16)]


def draw_cases(n, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        fmt, bs = FORMATS[rng.integers(len(FORMATS))]
        act = "f16" if (fmt == "u8" and rng.random() < 0.5) else ("bf16" if rng.random() < 0.5 else "f16")
        N = int(rng.choice([1, 7, 16, 33, 100, 255, 640, 1000, 1500, 2047]))
        K = int(bs * rng.integers(1, max(2, 8192 // bs // 2) + 1))
        if fmt == "nvfp4" and K % 32:
            K += 16  # NVFP4 codes pack two per byte: K even per 32-k chunk
        M = int(rng.choice([1, 2, 3, 4, 5, 8, 9, 12, 16, 17, 23, 33, 40]))
        if N * K * M > 60_000_000:
            M = max(1, 60_000_000 // (N * K))
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
        cases.append((i, fmt, act, bs, N, K, M, flags, ws))
    return cases


@pytest.mark.parametrize("i,fmt,act,bs,N,K,M,flags,ws", draw_cases(200))
def test_random_case_against_the_oracle(i, fmt, act, bs, N, K, M, flags, ws):
    prob = synth.make_problem(fmt, act, N, K, bs, M, seed=1000 + i)
    try:
        plan = bqw.select(fmt, act, N, K, bs, min(M, 16), flags=flags, with_workspace=ws,
                          zero_points=0x2000 if prob.zp is not None else None)
    except bqw.QGemvError as e:
        assert e.status == 7, e
        pytest.skip(f"the forced choice does not fit this shape (status {e.status})")
    gu.say(f"[random {i}] {fmt}/{act} bs={bs} N={N} K={K} M={M} flags={flags:#x} ws={ws} plan={plan}")
    Y, got = gu.run_gpu(prob, M, flags=flags, ws=ws)
    if ws:
        assert got["ws_zero"], got
    ok, ratio, _, _ = gu.check_full(prob, M, Y, strict=False)
    assert ok, (i, ratio, got)
