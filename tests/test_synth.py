"""The seeded input generators: determinism, ranges and layouts (CPU only)."""

import numpy as np
import pytest

from block_quantized_weight_amd import synth


def test_generation_is_deterministic():
    a = synth.workload("u4_m1_k512_n256")
    b = synth.workload("u4_m1_k512_n256")
    assert a.hashes() == b.hashes()
    c = synth.workload("u4_m8_k2048_n1024")
    assert c.hashes() != a.hashes()


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_layouts_and_ranges(name):
    p = synth.workload(name, n_override=48)
    spec = synth.WORKLOADS[name]
    N, K, bs = 48, spec["K"], spec["bs"]
    nblk = K // bs
    assert p.A.shape == (max(spec["ms"]), K) and p.A.dtype == np.uint16
    if p.fmt == "u4":
        assert p.W.shape == (N, nblk, bs // 2)
        assert p.scales.shape == (N, nblk) and p.scales.dtype == np.uint16
        assert p.zp.shape == (N, (nblk + 1) // 2)
        z = synth.unpack_nibbles(p.zp, nblk)
        lo, hi = spec.get("zp_range", (0, 15))
        assert z.min() >= lo and z.max() <= hi
    elif p.fmt == "u8":
        assert p.W.shape == (N, nblk, bs)
        assert p.zp.shape == (N, nblk)
        assert p.zp.min() >= 96 and p.zp.max() <= 160
    elif p.fmt == "fp8":
        assert p.W.shape == (N, K)
        assert not np.isin(p.W, [0x7F, 0xFF]).any()
        assert p.scales.dtype == np.float32 and p.scales.shape == (N, nblk)
        assert p.scales.min() >= 2.0 ** -8 and p.scales.max() <= 2.0 ** -4
        assert p.zp is None
    else:
        assert p.W.shape == (N, K // 2)
        assert p.scales.shape == (N, K // 16) and p.scales.dtype == np.uint8
        assert p.scales.min() >= 0x08 and p.scales.max() <= 0x48
        assert p.tensor_scale == float(np.float32(0.01))
        assert p.zp is None


def test_full_size_byte_counts():
    # weight bytes = codes + block scales + zero points (+4 B tensor scale for nvfp4),
    # computed from the shapes without generating the data
    def wb(fmt, N, K, bs):
        nblk = K // bs
        if fmt == "u4":
            return N * K // 2 + N * nblk * 2 + N * ((nblk + 1) // 2)
        if fmt == "u8":
            return N * K + N * nblk * 2 + N * nblk
        if fmt == "fp8":
            return N * K + N * nblk * 4
        return N * K // 2 + N * (K // 16) + 4
    want = {
        "u4_m1_k512_n256": 75_776, "u8_m1_k4096_n4096": 17_170_432, "fp8_k6144_n5120": 32_440_320,
        "nvfp4_m4_k2048_n2048": 2_359_300, "nvfp4_m4_k2048_n248320": 286_064_644,
        "u4_k4096_n151936": 359_784_448, "u4_m8_k2048_n1024": 1_212_416,
        "fp8_m8_k16384_n1024": 17_301_504,
    }
    for name, spec in synth.WORKLOADS.items():
        assert wb(spec["fmt"], spec["N"], spec["K"], spec["bs"]) == want[name]
    small = synth.workload("u4_m1_k512_n256")
    assert small.weight_bytes() == want["u4_m1_k512_n256"]


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0])
    bits = synth.round_to_bf16_bits(x)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6... = 0x3F82)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0000]
