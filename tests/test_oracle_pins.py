"""Pins for the CPU oracle: each check ties it to something other than itself.

- library decoders (numpy float16, torch bfloat16 / float8_e4m3fn) over every code;
- the values the pages print for the minifloat formats (tests/golden/minifloat_pins.txt);
- the exactness facts the pages state (lossless widening, exact scale folding,
  exact (q - zp)) checked exhaustively;
- exact rational brute force (fractions.Fraction) on tiny shapes of every format,
  computed from *unpacked* logical arrays, so packing and indexing are checked too;
- integer special cases that reduce to an exact numpy integer matmul;
- one-hot and K-ramp probes that catch swapped or permuted indices.
"""

import os
import zlib
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from block_quantized_weight_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pins():
    out = {}
    with open(os.path.join(GOLDEN, "minifloat_pins.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                out[k] = float(v)
    return out


# ----------------------------------------------------------------------------------
# decoders


def test_e4m3_table_matches_torch_float8_on_all_codes():
    _, e4 = oracle.tables()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(e4))
    assert np.array_equal(ref[~nan], e4[~nan])
    # signed zero is kept
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(e4[~nan]))


def test_e4m3_table_matches_page_values():
    pins = _pins()
    _, e4 = oracle.tables()
    fin = e4[~np.isnan(e4)]
    assert fin.size == 254
    assert sorted(np.nonzero(np.isnan(e4))[0].tolist()) == [0x7F, 0xFF]
    assert fin.max() == pins["e4m3_max"]
    assert fin[fin > 0].min() == pins["e4m3_min_positive"]
    # every finite value carries at most 4 significand bits
    nz = np.abs(fin[fin != 0])
    mant = nz / np.exp2(np.floor(np.log2(nz)))
    # normals: 1 + m/8; subnormals scaled the same way also land on multiples of 1/8
    assert np.all(np.abs(mant * 8 - np.round(mant * 8)) == 0)
    assert int(pins["e4m3_significand_bits"]) == 4


def test_e2m1_table_matches_page_values_and_float_structure():
    pins = _pins()
    e2, e4 = oracle.tables()
    assert e2[0] == 0.0
    mags = e2[:8]
    # sign bit is bit 3: codes c and c|8 are negatives of each other
    assert np.array_equal(e2[8:], -mags)
    assert np.signbit(e2[8])
    # magnitudes strictly increase with the code (ordering property of a float format)
    assert np.all(np.diff(mags) > 0)
    assert mags.max() == pins["e2m1_max"]
    assert mags[mags > 0].min() == pins["e2m1_min_nonzero"]
    # 2 significand bits: every nonzero magnitude is 1.0 or 1.5 times a power of two
    nz = mags[1:]
    frac = nz / np.exp2(np.floor(np.log2(nz)))
    assert set(frac.tolist()) <= {1.0, 1.5}
    assert int(pins["e2m1_significand_bits"]) == 2
    # IEEE-style binades: one exponent field value per pair of codes (1 mantissa bit),
    # so each binade above the subnormal one holds exactly two codes
    expo = np.floor(np.log2(mags[2:]))
    assert np.array_equal(expo, np.repeat(np.arange(0, 3), 2))
    # every E2M1 value is also an E4M3 value (the two formats nest)
    assert set(e2.tolist()) <= set(e4[~np.isnan(e4)].tolist())


def test_half_decoder_matches_numpy_on_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_activation_bits(bits, "f16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_bf16_decoder_matches_torch_on_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_activation_bits(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


# ----------------------------------------------------------------------------------
# exactness facts the GPU path relies on


def _exact_in_f16(x):
    x = np.asarray(x, dtype=np.float64)
    return np.array_equal(x.astype(np.float16).astype(np.float64), x)


def _exact_in_bf16(x):
    t = torch.from_numpy(np.asarray(x, dtype=np.float64))
    return torch.equal(t.to(torch.bfloat16).to(torch.float64), t)


def test_e4m3_widening_is_lossless():
    _, e4 = oracle.tables()
    fin = e4[~np.isnan(e4)]
    assert _exact_in_f16(fin) and _exact_in_bf16(fin)


def test_nvfp4_scale_fold_is_exact_and_in_range():
    pins = _pins()
    e2, e4 = oracle.tables()
    fin = e4[~np.isnan(e4)]
    prod = np.outer(e2, fin).ravel()
    assert _exact_in_f16(prod) and _exact_in_bf16(prod)
    assert np.abs(prod).max() == pins["fold_max"]
    assert np.abs(prod[prod != 0]).min() == pins["fold_min_nonzero"]


def test_q_minus_zp_is_exact_in_half_and_bf16():
    q = np.arange(256)
    d = (q[:, None] - q[None, :]).ravel().astype(np.float64)
    assert _exact_in_f16(d) and _exact_in_bf16(d)


def test_products_are_exact_in_fp32():
    rng = np.random.default_rng(7)
    a16 = rng.standard_normal(4096).astype(np.float16).astype(np.float64)
    abf = torch.from_numpy(rng.standard_normal(4096)).to(torch.bfloat16).to(torch.float64).numpy()
    d = np.arange(-255, 256, dtype=np.float64)
    _, e4 = oracle.tables()
    fin = e4[~np.isnan(e4)]
    for a in (a16, abf):
        for w in (d, fin):
            p = np.outer(a, w).ravel()
            assert np.array_equal(p.astype(np.float32).astype(np.float64), p)


# ----------------------------------------------------------------------------------
# packing convention


def test_nibble_packing_matches_golden_fixture():
    with open(os.path.join(GOLDEN, "nibble_order.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("->")
            codes = np.array([int(t, 16) for t in lhs.split()], dtype=np.uint8)
            want = np.array([int(t, 16) for t in rhs.split()], dtype=np.uint8)
            got = synth.pack_nibbles(codes)
            assert np.array_equal(got, want), line
            assert np.array_equal(synth.unpack_nibbles(got, codes.size), codes)


# ----------------------------------------------------------------------------------
# brute force with exact rationals on tiny shapes


def _seed(*key):
    """A seed that is the same in every process (Python's str hash is salted)."""
    return zlib.crc32(repr(key).encode())


def _f16_fraction(bits):
    return Fraction(float(np.uint16(bits).view(np.float16)))


def _bf16_fraction(bits):
    t = torch.tensor([int(np.int16(np.uint16(bits).view(np.int16)))], dtype=torch.int16)
    return Fraction(float(t.view(torch.bfloat16).to(torch.float64).item()))


def _e4m3_fraction(code):
    t = torch.tensor([int(code)], dtype=torch.uint8).view(torch.float8_e4m3fn)
    return Fraction(float(t.to(torch.float64).item()))


def _logical_problem(fmt, act, M, N, K, bs, rng, with_zp=True):
    """Random *unpacked* arrays plus the packed Problem built from them."""
    nblk = K // bs
    a_bits = synth.activation_bits(rng.standard_normal((M, K)), act)
    logical = {"a_bits": a_bits}
    zp_packed = None
    if fmt in ("u4", "u8"):
        hi = 16 if fmt == "u4" else 256
        q = rng.integers(0, hi, size=(N, K))
        z = rng.integers(0, hi, size=(N, nblk)) if with_zp else np.full((N, nblk), hi // 2)
        s_bits = synth.round_to_f16_bits(rng.uniform(0.01, 2.0, size=(N, nblk)))
        logical.update(q=q, z=z, s_bits=s_bits)
        if fmt == "u4":
            W = synth.pack_nibbles(q.astype(np.uint8)).reshape(N, nblk, bs // 2)
            zp_packed = synth.pack_nibbles(z.astype(np.uint8)) if with_zp else None
        else:
            W = q.astype(np.uint8).reshape(N, nblk, bs)
            zp_packed = z.astype(np.uint8) if with_zp else None
        scales = s_bits
        ts = 1.0
    elif fmt == "fp8":
        q = synth.FP8_FINITE_CODES[rng.integers(0, 254, size=(N, K))]
        s = np.exp2(rng.uniform(-8, 2, size=(N, nblk))).astype(np.float32)
        logical.update(q=q, s=s)
        W, scales, ts = q, s, 1.0
    else:
        q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
        sc = rng.integers(0, 0x7F, size=(N, K // 16)).astype(np.uint8)  # any finite positive code
        ts = float(np.float32(rng.uniform(0.001, 3.0)))
        logical.update(q=q, sc=sc, ts=ts)
        W, scales = synth.pack_nibbles(q), sc
    prob = synth.Problem(name="tiny", fmt=fmt, act=act, N=N, K=K, bs=bs, W=W, scales=scales,
                         zp=zp_packed, tensor_scale=ts, A=a_bits)
    return prob, logical


def _exact_result(fmt, act, M, N, K, bs, L):
    e2, _ = oracle.tables()  # E2M1 values are pinned separately (test above)
    act_frac = _f16_fraction if act == "f16" else _bf16_fraction
    a = [[act_frac(L["a_bits"][m, k]) for k in range(K)] for m in range(M)]
    Y = [[Fraction(0)] * N for _ in range(M)]
    S = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        for k in range(K):
            b = k // bs
            if fmt in ("u4", "u8"):
                w = _f16_fraction(L["s_bits"][n, b]) * (int(L["q"][n, k]) - int(L["z"][n, b]))
            elif fmt == "fp8":
                w = Fraction(float(L["s"][n, b])) * _e4m3_fraction(L["q"][n, k])
            else:
                w = Fraction(L["ts"]) * _e4m3_fraction(L["sc"][n, k // 16]) * Fraction(float(e2[L["q"][n, k]]))
            for m in range(M):
                t = a[m][k] * w
                Y[m][n] += t
                S[m][n] += abs(t)
    return Y, S


CASES = [
    ("u4", "f16", 32, True), ("u4", "bf16", 16, True), ("u4", "f16", 64, False),
    ("u8", "f16", 16, True), ("u8", "bf16", 32, True), ("u8", "f16", 16, False),
    ("fp8", "f16", 32, None), ("fp8", "bf16", 16, None),
    ("nvfp4", "bf16", 16, None), ("nvfp4", "f16", 16, None),
]


@pytest.mark.parametrize("fmt,act,bs,with_zp", CASES)
def test_brute_force_exact_rationals(fmt, act, bs, with_zp):
    rng = np.random.default_rng(_seed(fmt, act, bs, with_zp))
    for M, N, nblk in ((1, 1, 1), (2, 3, 3), (3, 5, 2)):
        K = nblk * bs
        prob, L = _logical_problem(fmt, act, M, N, K, bs, rng, with_zp=bool(with_zp))
        Y, S = oracle.gemv(prob)
        Ye, Se = _exact_result(fmt, act, M, N, K, bs, L)
        for m in range(M):
            for n in range(N):
                ye, se = float(Ye[m][n]), float(Se[m][n])
                assert abs(Y[m, n] - ye) <= 1e-12 * se + 1e-300, (m, n, Y[m, n], ye)
                assert abs(S[m, n] - se) <= 1e-12 * se + 1e-300


def _dequant_matrix(fmt, bs, L):
    """W as an fp64 [N, K] matrix from the unpacked arrays: library decoders for the
    scales and E4M3 codes (numpy float16, torch float8_e4m3fn), E2M1 from the pinned
    table, and no packed byte at all."""
    if fmt in ("u4", "u8"):
        s = L["s_bits"].astype(np.uint16).view(np.float16).astype(np.float64)
        return np.repeat(s, bs, axis=1) * (L["q"].astype(np.float64) - np.repeat(L["z"], bs, axis=1))
    e4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    if fmt == "fp8":
        return np.repeat(L["s"].astype(np.float64), bs, axis=1) * e4[L["q"]]
    e2, _ = oracle.tables()
    return L["ts"] * np.repeat(e4[L["sc"]], 16, axis=1) * np.asarray(e2)[L["q"]]


@pytest.mark.parametrize("fmt,act,bs,with_zp", CASES)
def test_numpy_dequant_matmul_agrees_on_larger_shapes(fmt, act, bs, with_zp):
    """A second implementation, numpy's: dequantize the unpacked arrays to fp64 and
    multiply with A @ W.T. On shapes past the brute force (odd block counts, so the
    4-bit zero-point rows end in half a byte; several rows; N not a multiple of
    anything) it checks the oracle's unpacking and indexing of the packed bytes."""
    rng = np.random.default_rng(_seed("numpy", fmt, act, bs, with_zp))
    for M, N, nblk in ((5, 37, 7), (1, 64, 33)):
        K = nblk * bs
        prob, L = _logical_problem(fmt, act, M, N, K, bs, rng, with_zp=bool(with_zp))
        Y, S = oracle.gemv(prob)
        a = L["a_bits"].astype(np.uint16)
        if act == "f16":
            A = a.view(np.float16).astype(np.float64)
        else:
            A = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
        W = _dequant_matrix(fmt, bs, L)
        Yn = A @ W.T
        Sn = np.abs(A) @ np.abs(W).T
        assert np.all(np.abs(Y - Yn) <= 1e-12 * Sn + 1e-300), (fmt, M, N, K)
        assert np.allclose(S, Sn, rtol=1e-12, atol=0.0)


def test_integer_special_case_is_exact():
    """scale 1, zero point 0 and small integer activations: Y = A_int @ Q^T exactly."""
    rng = np.random.default_rng(11)
    M, N, K, bs = 3, 7, 96, 32
    a_int = rng.integers(-8, 9, size=(M, K))
    q = rng.integers(0, 16, size=(N, K))
    nblk = K // bs
    prob = synth.Problem(
        name="int", fmt="u4", act="f16", N=N, K=K, bs=bs,
        W=synth.pack_nibbles(q.astype(np.uint8)).reshape(N, nblk, bs // 2),
        scales=np.full((N, nblk), 0x3C00, dtype=np.uint16),  # fp16 1.0
        zp=synth.pack_nibbles(np.zeros((N, nblk), dtype=np.uint8)), tensor_scale=1.0,
        A=synth.round_to_f16_bits(a_int.astype(np.float64)))
    Y, _ = oracle.gemv(prob)
    assert np.array_equal(Y, (a_int @ q.T).astype(np.float64))
    # same for 8-bit codes with zero point 0
    q8 = rng.integers(0, 256, size=(N, K))
    prob8 = synth.Problem(
        name="int8", fmt="u8", act="bf16", N=N, K=K, bs=bs, W=q8.astype(np.uint8).reshape(N, nblk, bs),
        scales=np.full((N, nblk), 0x3C00, dtype=np.uint16), zp=np.zeros((N, nblk), dtype=np.uint8),
        tensor_scale=1.0, A=synth.round_to_bf16_bits(a_int.astype(np.float64)))
    Y8, _ = oracle.gemv(prob8)
    assert np.array_equal(Y8, (a_int @ q8.T).astype(np.float64))


@pytest.mark.parametrize("fmt", ["u4", "u8", "fp8", "nvfp4"])
def test_one_hot_probes_pick_single_elements(fmt):
    """One-hot A selects one k; the result must equal that single dequantized weight
    computed from the logical (unpacked) arrays. Catches row/column/k swaps."""
    rng = np.random.default_rng(3)
    bs = 16 if fmt in ("nvfp4",) else 32
    M, N, K = 2, 6, 4 * bs
    prob, L = _logical_problem(fmt, "f16", M, N, K, bs, rng)
    e2, _ = oracle.tables()
    for k in (0, 1, bs - 1, bs, K - 2, K - 1):
        A = np.zeros((M, K), dtype=np.uint16)
        A[1, k] = 0x3C00  # 1.0 in row 1 only
        Y, _ = oracle.gemv(prob, A=A)
        assert np.all(Y[0] == 0.0)
        for n in range(N):
            b = k // bs
            if fmt in ("u4", "u8"):
                w = float(_f16_fraction(L["s_bits"][n, b])) * (int(L["q"][n, k]) - int(L["z"][n, b]))
            elif fmt == "fp8":
                w = float(L["s"][n, b]) * float(_e4m3_fraction(L["q"][n, k]))
            else:
                w = L["ts"] * float(_e4m3_fraction(L["sc"][n, k // 16])) * e2[L["q"][n, k]]
            assert Y[1, n] == w, (fmt, k, n)


def test_k_ramp_with_single_live_block_per_column():
    """Column n has nonzero codes only in block n; A varies along K. Any permutation
    of k inside or across blocks changes the result."""
    rng = np.random.default_rng(5)
    N, bs = 4, 32
    K = N * bs
    nblk = K // bs
    q = np.full((N, K), 8, dtype=np.uint8)
    for n in range(N):
        q[n, n * bs:(n + 1) * bs] = rng.integers(0, 16, size=bs)
    z = np.full((N, nblk), 8, dtype=np.uint8)
    a = (np.arange(K) % 97 + 1).astype(np.float64)  # exact in fp16
    prob = synth.Problem(name="ramp", fmt="u4", act="f16", N=N, K=K, bs=bs,
                         W=synth.pack_nibbles(q).reshape(N, nblk, bs // 2),
                         scales=np.full((N, nblk), 0x3C00, dtype=np.uint16), zp=synth.pack_nibbles(z),
                         tensor_scale=1.0, A=synth.round_to_f16_bits(a[None, :]))
    Y, _ = oracle.gemv(prob)
    want = np.array([np.dot(a[n * bs:(n + 1) * bs], q[n, n * bs:(n + 1) * bs].astype(np.float64) - 8)
                     for n in range(N)])
    assert np.array_equal(Y[0], want)


# ----------------------------------------------------------------------------------
# the oracle's own consistency and the bound it is used with


def test_points_match_full_product():
    p = synth.workload("u4_m8_k2048_n1024", n_override=64)
    Y, S = oracle.gemv(p)
    ms = np.repeat(np.arange(8), 5)
    ns = np.tile(np.array([0, 1, 17, 40, 63]), 8)
    y, s = oracle.gemv_points(p, ms, ns)
    assert np.array_equal(y, Y[ms, ns]) and np.array_equal(s, S[ms, ns])


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_data_is_not_vacuous(name):
    """|y_ref| is large against the bound, so an all-zero (or garbage) output fails."""
    p = synth.workload(name, n_override=32)
    Y, S = oracle.gemv(p)
    ok, ratio = oracle.within_tolerance(np.zeros_like(Y), Y, S)
    assert not ok and ratio > 5.0
    assert np.median(np.abs(Y) / oracle.tolerance(S)) > 1.0
    # a result off by a single dropped block also fails somewhere
    K, bs = p.K, p.bs
    p2 = synth.Problem(**{**p.__dict__})
    A2 = p.A.copy()
    A2[:, :bs] = 0
    Y2, _ = oracle.gemv(p2, A=A2)
    assert not oracle.within_tolerance(Y2, Y, S)[0]


@pytest.mark.parametrize("fmt,act,bs,with_zp", [("u4", "f16", 32, True), ("u8", "bf16", 16, True),
                                                ("fp8", "bf16", 16, None), ("nvfp4", "bf16", 16, None),
                                                ("nvfp4", "f16", 16, None)])
def test_brute_force_with_bias(fmt, act, bs, with_zp):
    """Optional bias: y[m, n] = sum_k a*w + bias[n] exactly (one value per output
    column, the same for every row, outside the NVFP4 tensor scale), S unchanged.
    Distinct rows and columns catch a bias indexed by the row, and NVFP4's tensor
    scale (not 1) catches a bias scaled with the product."""
    rng = np.random.default_rng(_seed("bias", fmt, act, bs))
    act_frac = _f16_fraction if act == "f16" else _bf16_fraction
    for M, N, nblk in ((2, 3, 2), (3, 5, 1)):
        K = nblk * bs
        prob, L = _logical_problem(fmt, act, M, N, K, bs, rng, with_zp=bool(with_zp))
        bias_bits = synth.activation_bits(rng.standard_normal(N) * 4.0, act).reshape(N)
        prob_b = synth.Problem(**{**prob.__dict__, "bias": bias_bits})
        Y, S = oracle.gemv(prob_b)
        Y0, S0 = oracle.gemv(prob)
        Ye, Se = _exact_result(fmt, act, M, N, K, bs, L)
        assert np.array_equal(S, S0)
        for m in range(M):
            for n in range(N):
                ye = float(Ye[m][n] + act_frac(bias_bits[n]))
                assert abs(Y[m, n] - ye) <= 1e-12 * (float(Se[m][n]) + abs(ye)) + 1e-300, (m, n, Y[m, n], ye)
        ys, ss = oracle.gemv_points(prob_b, [M - 1, 0], [N - 1, 0])
        assert np.array_equal(ys, [Y[M - 1, N - 1], Y[0, 0]]) and np.array_equal(ss, [S[M - 1, N - 1], S[0, 0]])


def test_integer_special_case_with_bias_is_exact():
    """Integer codes, scale 1, zero point 0, integer activations and an integer bias:
    Y = A_int @ Q^T + bias exactly."""
    rng = np.random.default_rng(12)
    M, N, K, bs = 3, 7, 64, 32
    a_int = rng.integers(-8, 9, size=(M, K))
    q = rng.integers(0, 16, size=(N, K))
    b_int = rng.integers(-256, 257, size=N)  # integers of magnitude <= 256 are exact in bf16
    nblk = K // bs
    prob = synth.Problem(
        name="int_bias", fmt="u4", act="bf16", N=N, K=K, bs=bs,
        W=synth.pack_nibbles(q.astype(np.uint8)).reshape(N, nblk, bs // 2),
        scales=np.full((N, nblk), 0x3C00, dtype=np.uint16),
        zp=synth.pack_nibbles(np.zeros((N, nblk), dtype=np.uint8)), tensor_scale=1.0,
        A=synth.round_to_bf16_bits(a_int.astype(np.float64)),
        bias=synth.round_to_bf16_bits(b_int.astype(np.float64)))
    Y, _ = oracle.gemv(prob)
    assert np.array_equal(Y, (a_int @ q.T + b_int[None, :]).astype(np.float64))


@pytest.mark.parametrize("fmt,act,bs", [("u4", "f16", 32), ("u4", "bf16", 16), ("u8", "f16", 128),
                                         ("u8", "bf16", 32)])
def test_codes_at_their_zero_points_give_exact_zeros(fmt, act, bs):
    """Blocks whose codes all equal their zero point dequantize to w = s * 0 = 0, so with
    every block so, Y and S are exactly zero whatever the activations (large normal
    values and single large spikes here); with 90% of the blocks so, Y equals the product
    over the other blocks alone, computed by numpy from the unpacked codes and zero points
    with those blocks removed (fp64, within 1e-12 of S)."""
    prob = synth.make_zero_point_problem(fmt, act, 40, 1024, bs, seed=3)
    Y, S = oracle.gemv(prob)
    assert np.all(Y == 0.0) and np.all(S == 0.0)
    prob = synth.make_zero_point_problem(fmt, act, 40, 1024, bs, seed=3, frac=0.9)
    Y, S = oracle.gemv(prob)
    nblk = 1024 // bs
    if fmt == "u4":
        q = synth.unpack_nibbles(prob.W.reshape(40, -1), 1024).astype(np.float64)
        z = synth.unpack_nibbles(prob.zp, nblk).astype(np.float64)
    else:
        q = prob.W.reshape(40, 1024).astype(np.float64)
        z = prob.zp.astype(np.float64)
    s = prob.scales.view(np.float16).astype(np.float64)
    live = ~np.all(q.reshape(40, nblk, bs) == z[:, :, None], axis=2)  # blocks not at their zero point
    assert 0.03 < live.mean() < 0.2
    W = (np.repeat(s * live, bs, axis=1)) * (q - np.repeat(z, bs, axis=1))
    a = prob.A
    A = (a.view(np.float16).astype(np.float64) if act == "f16"
         else torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy())
    Yn = A @ W.T
    Sn = np.abs(A) @ np.abs(W).T
    assert np.all(np.abs(Y - Yn) <= 1e-12 * Sn + 1e-300)
    assert np.abs(Yn).max() > 1.0
