"""The dispatcher's launch sizes against the matrix-family kernels' own LDS layouts.

The register-ring kernel (k_mfma) lays out its LDS from its arguments:
a 64-byte zero block, the staged rows of the longest K part (row stride: that part's k
plus 8 elements, 2 bytes each, rounded up to 16 bytes), for 4-bit codes on bf16
activations one 16-byte activation-sum entry per chunk, row group and scale block (the
other formats with zero points form q - z in the decode), then the K-split
reduction area (8 waves x row groups x 4 x 64 fp32), which overlays the staged rows from
byte 0 when the workgroup holds a single tile group (always with K parts), and, with K
parts, a 4-byte completion flag after both. The DMA-ring kernel (k_mfma_dma) stages
all of K the same way and follows it with two (variant bit 2: three) slots per wave. The host must launch
with at least that much. This recomputes the kernels' layouts for every automatic
plan over a grid of shapes, every M, with and without a workspace and zero points,
and checks them against the plan, with the plan's other invariants.
"""

import pytest

import block_quantized_weight_amd as bqw

KPC = {"u4": 32, "nvfp4": 32, "u8": 16, "fp8": 16}
LDS = 160 * 1024

SHAPES = [  # fmt, act, N, K, bs
    ("u4", "bf16", 151936, 4096, 32), ("u4", "f16", 1024, 2048, 32), ("u4", "bf16", 4096, 4096, 32),
    ("u4", "bf16", 16384, 8192, 32), ("u4", "bf16", 2048, 16384, 32), ("u4", "f16", 512, 8192, 32),
    ("u4", "f16", 777, 896, 16), ("u4", "bf16", 3000, 4096, 128), ("u8", "f16", 4096, 4096, 128),
    ("u8", "f16", 4096, 8192, 128), ("u8", "f16", 2048, 8192, 128), ("u8", "f16", 1900, 8192, 64),
    ("u8", "bf16", 4096, 4096, 32), ("u8", "bf16", 151936, 2048, 128), ("u4", "f16", 151936, 4096, 32),
    ("fp8", "f16", 5120, 6144, 128), ("fp8", "f16", 8192, 4096, 128), ("fp8", "f16", 1024, 16384, 128),
    ("fp8", "bf16", 2048, 8192, 128), ("fp8", "f16", 100, 256, 128), ("nvfp4", "bf16", 248320, 2048, 16),
    ("nvfp4", "bf16", 2048, 4096, 16), ("nvfp4", "f16", 999, 3104, 16),
]


def kernel_lds(fmt, act, N, K, bs, rows, plan, zpp=False):
    """Bytes the matrix-family kernel addresses for a pass of `rows` rows."""
    ks, kp = plan["ksplit"], plan["kparts"]
    rg = (rows + 3) // 4
    h = 2 if fmt == "nvfp4" or (fmt == "u4" and bs == 16) else 1
    if plan["variant"] & 2:
        # DMA ring: all of K staged, then 8 waves x 2 slots of 4 K steps: 4 KiB of codes,
        # the scale windows (4 DMAs of 256 bytes for FP8 and 16-wide 4-bit blocks, else
        # 2) and the zero-point window when there are zero points
        nch = K // KPC[fmt]
        rows_b = (rows * (K + 8) * 2 + 15) // 16 * 16
        sums = nch * rg * h * 16 if (fmt, act) == ("u4", "bf16") else 0
        nsd = 4 if (fmt == "fp8" or (fmt == "u4" and h == 2)) else 2
        slot = 4096 + 256 * nsd + (256 if zpp else 0)
        return 64 + rows_b + sums + 8 * (3 if plan["variant"] & 4 else 2) * slot
    steps = K // (4 * KPC[fmt])
    smax = (steps + kp - 1) // kp
    staged = bool(plan["variant"] & 1)
    tiles = (N + 15) // 16
    ngroups = (tiles + 8 // ks - 1) // (8 // ks)
    red = 8 * rg * 4 * 64 * 4 if ks > 1 else 0
    abytes = 0
    if staged:
        astride = smax * 4 * KPC[fmt] + 8
        rows_b = (rows * astride * 2 + 15) // 16 * 16
        sums = 4 * smax * rg * h * 16 if (fmt, act) == ("u4", "bf16") else 0
        abytes = 64 + rows_b + sums
    overlay = staged and ks > 1 and (kp > 1 or plan["grid"] // kp >= ngroups)
    end = max(abytes, red) if overlay else abytes + red
    return end + (4 if kp > 1 else 0)


CASES = [(fmt, act, N, K, bs, zp) for (fmt, act, N, K, bs) in SHAPES for zp in (False, True)
         if not zp or fmt in ("u4", "u8")]  # zero points are for the integer codes


@pytest.mark.parametrize("cu", [80, 256, 304])
@pytest.mark.parametrize("fmt,act,N,K,bs,zp", CASES)
def test_every_matrix_plan_holds_the_kernels_lds_layout(fmt, act, N, K, bs, zp, cu):
    """At 80, 256 and 304 CUs (plans move with the CU count; the layouts must hold at
    each)."""
    for M in (1, 2, 3, 4, 5, 8, 9, 12, 13, 16, 20, 37):
        for ws in (False, True):
            p = bqw.select(fmt, act, N, K, bs, M, cu_count=cu, with_workspace=ws, zero_points=0x2000 if zp else None)
            assert 1 <= p["grid"] and 0 <= p["lds_bytes"] <= LDS, (M, ws, cu, p)
            rows = min(M, 16)
            # passes of rows_per_pass rows cover every row of each 16-row chunk
            chunks = (M + 15) // 16
            per_chunk = p["passes"] // chunks
            assert p["passes"] % chunks == 0 and p["rows_per_pass"] * per_chunk >= rows, (M, p)
            if p["kparts"] > 1:
                assert p["family"] == "mfma" and ws and p["grid"] % p["kparts"] == 0
                assert p["kparts"] * 16 * N < 1 << 31
                assert p["workspace_bytes"] >= p["kparts"] * min(M, 16) * N * 4
            if p["family"] != "mfma":
                continue  # the streaming kernels' staged rows are sized by the same formula
            need = kernel_lds(fmt, act, N, K, bs, min(p["rows_per_pass"], rows), p, zpp=zp)
            assert need <= p["lds_bytes"], (fmt, N, K, bs, M, ws, p, need)


DEPTH = 29  # QGEMV_FLAG_MFMA_DEPTH_SHIFT


@pytest.mark.parametrize("cu", [80, 256, 304])
def test_dma_ring_depth_rule(cu):
    """Three DMA-ring slots per wave for the 16-k-per-chunk formats (FP8, 8-bit codes)
    where the LDS holds them, two for 4-bit and NVFP4 codes; the depth flag forces two
    (1) or three (2, where they fit). The plan's LDS covers the slots it launches with."""
    def ring(fmt, act, N, K, bs, M, flags=0, zp=False):
        p = bqw.select(fmt, act, N, K, bs, M, cu_count=cu, flags=flags, zero_points=0x2000 if zp else None)
        assert p["family"] == "mfma" and p["variant"] & 2, p
        assert kernel_lds(fmt, act, N, K, bs, min(p["rows_per_pass"], M), p, zpp=zp) <= p["lds_bytes"] <= LDS
        return 3 if p["variant"] & 4 else 2

    assert ring("fp8", "f16", 65536, 4096, 128, 4) == 3
    assert ring("u8", "f16", 65536, 4096, 128, 4, zp=True) == 3
    assert ring("fp8", "f16", 65536, 4096, 128, 8) == 2  # eight staged rows leave no room for a third
    assert ring("u4", "bf16", 151936, 4096, 32, 4, zp=True) == 2
    assert ring("nvfp4", "bf16", 248320, 2048, 16, 4) == 2
    assert ring("fp8", "f16", 65536, 4096, 128, 4, flags=1 << DEPTH) == 2
    assert ring("u4", "bf16", 151936, 4096, 32, 4, flags=2 << DEPTH, zp=True) == 3
    assert ring("u4", "bf16", 151936, 4096, 32, 8, flags=2 << DEPTH, zp=True) == 2  # does not fit: two
