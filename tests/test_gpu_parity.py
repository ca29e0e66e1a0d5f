"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: |y - y_ref| <= 1e-3 * sum|a*w| + 1e-3 per output (fp32 accumulation), checked
element by element on every output of every named workload, the lm_head sizes included
(the oracle runs on all host cores; its rows do not depend on M, so one 16-row product
serves the whole M sweep).
Integer-valued and one-hot cases must match bit for bit; rows must come out
bit-identical whatever tile carries them; repeated runs must be bitwise equal.
"""

import numpy as np
import pytest

import block_quantized_weight_amd as bqw
import oracle
from block_quantized_weight_amd import synth

pytestmark = pytest.mark.gpu

from tests import gpu_util as gu

FAMILY_FLAG = {"auto": 0, "stream": 1, "mfma": 2, "generic": 3, "stream_classic": 1 | bqw.FLAG_STREAM_CLASSIC,
               "mfma_lds": 2 | bqw.FLAG_STAGE_A_ON | bqw.FLAG_RING_OFF,
               "mfma_nolds": 2 | bqw.FLAG_STAGE_A_OFF | bqw.FLAG_RING_OFF,
               "mfma_ring": 2 | bqw.FLAG_RING_ON | (1 << 8)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.require_gpu()


# ----------------------------------------------------------------------------------
# named workloads


SMALL = [("u4_m1_k512_n256", 1), ("u8_m1_k4096_n4096", 1), ("fp8_k6144_n5120", 1), ("fp8_k6144_n5120", 4),
         ("fp8_k6144_n5120", 8), ("nvfp4_m4_k2048_n2048", 4), ("u4_m8_k2048_n1024", 8)]


@pytest.mark.parametrize("name,M", SMALL)
def test_named_workload_full_parity(name, M):
    prob = synth.workload(name)
    gu.say(f"[parity] {name} M={M}")
    Y, plan = gu.run_gpu(prob, M)
    ok, ratio, Yr, S = gu.check_full(prob, M, Y)
    gu.say(f"   plan={plan} max err/tol={ratio:.3e}")
    assert ok, (name, M, ratio, plan)


@pytest.fixture(scope="module")
def lm_head_u4():
    prob = synth.workload("u4_k4096_n151936")
    gu.say("[oracle] u4 lm_head, 16 rows")
    Yr, S = oracle.gemv(prob, M=16)
    return prob, Yr, S


@pytest.fixture(scope="module")
def lm_head_nvfp4():
    prob = synth.workload("nvfp4_m4_k2048_n248320")
    gu.say("[oracle] nvfp4 lm_head, 4 rows")
    Yr, S = oracle.gemv(prob, M=4)
    return prob, Yr, S


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_u4_lm_head_full_parity(lm_head_u4, M):
    prob, Yr, S = lm_head_u4
    gu.say(f"[parity] u4 lm_head M={M}")
    Y, plan = gu.run_gpu(prob, M)
    ok, ratio = oracle.within_tolerance(Y, Yr[:M], S[:M])
    gu.say(f"   plan={plan} max err/tol={ratio:.3e}")
    assert ok, (M, ratio, plan)


@pytest.mark.parametrize("M", [1, 2, 4])
def test_nvfp4_lm_head_full_parity(lm_head_nvfp4, M):
    """Every output at M = 1, 2 and 4 (the DMA ring at each: NVFP4 takes it from one row
    where N is wide)."""
    prob, Yr, S = lm_head_nvfp4
    gu.say(f"[parity] nvfp4 lm_head M={M}")
    Y, plan = gu.run_gpu(prob, M)
    assert plan["family"] == "mfma" and plan["variant"] & 2, plan
    ok, ratio = oracle.within_tolerance(Y, Yr[:M], S[:M])
    gu.say(f"   plan={plan} max err/tol={ratio:.3e}")
    assert ok, (M, ratio, plan)


def test_nvfp4_one_row_rows_match_the_four_row_launch():
    """NVFP4 on a wide weight runs the matrix family from one row, so a row's bits do not
    depend on M (the family's row invariance): rows of M = 1 and 2 equal the same rows of
    a four-row launch, bit for bit (65536 x 2048, the DMA ring at every M)."""
    prob = synth.make_problem("nvfp4", "bf16", 65536, 2048, 16, 4, seed=52)
    Y4, p4 = gu.run_gpu(prob, 4)
    for M in (1, 2):
        Ym, pm = gu.run_gpu(prob, M)
        assert pm["family"] == "mfma" and pm["variant"] & 2 and p4["variant"] & 2, (pm, p4)
        assert np.array_equal(Ym.view(np.int64), Y4[:M].view(np.int64)), M


@pytest.mark.parametrize("act", ["bf16", "f16"])
@pytest.mark.parametrize("M", [4, 8])
def test_dma_ring_walks_several_rounds(act, M):
    """A 4-bit weight of 40000 columns: 2500 tiles on 256 eight-wave workgroups, so every
    wave of the DMA ring walks more than one tile; every output against the oracle."""
    prob = synth.make_problem("u4", act, 40000, 1024, 32, M, seed=77)
    gu.say(f"[parity] dma ring u4/{act} 40000x1024 M={M}")
    Y, plan = gu.run_gpu(prob, M)
    assert plan["family"] == "mfma" and plan["variant"] & 2, plan
    assert (40000 + 15) // 16 > plan["grid"] * plan["waves_per_wg"], plan
    ok, ratio, _, _ = gu.check_full(prob, M, Y)
    gu.say(f"   plan={plan} max err/tol={ratio:.3e}")
    assert ok, (ratio, plan)


@pytest.mark.parametrize("fmt,act", [("fp8", "f16"), ("u8", "f16"), ("u8", "bf16"), ("u4", "bf16")])
@pytest.mark.parametrize("M", [3, 4])
def test_three_slot_dma_ring(fmt, act, M):
    """The DMA ring with three slots per wave (the automatic depth for FP8 and 8-bit
    codes, forced for 4-bit ones) on a ragged N that walks several tiles per wave:
    every output against the oracle, and the same bits as the two-slot ring."""
    depth = 29  # QGEMV_FLAG_MFMA_DEPTH_SHIFT
    ring = 2 | bqw.FLAG_RING_ON | (1 << 8)  # the matrix family, no K split, the DMA ring
    prob = synth.make_problem(fmt, act, 20003, 2048, 32 if fmt == "u4" else 128, M, seed=91)
    gu.say(f"[parity] three-slot dma ring {fmt}/{act} 20003x2048 M={M}")
    Y3, p3 = gu.run_gpu(prob, M, flags=ring | (2 << depth))
    Y2, p2 = gu.run_gpu(prob, M, flags=ring | (1 << depth))
    assert p3["variant"] & 6 == 6 and p2["variant"] & 6 == 2, (p3, p2)
    ok, ratio, _, _ = gu.check_full(prob, M, Y3)
    gu.say(f"   plan={p3} max err/tol={ratio:.3e}")
    assert ok, (ratio, p3)
    assert np.array_equal(Y3.view(np.int64), Y2.view(np.int64))


@pytest.mark.parametrize("fmt,act,N,K,bs,variant", [
    ("u4", "f16", 28672, 5120, 32, 2),     # 8 rows take the DMA ring
    ("fp8", "f16", 24576, 4096, 128, 1),   # 8 rows stage in the register ring, K split 4
    ("u8", "bf16", 4096, 8192, 128, 1),    # K split 8, 256 tile groups
])
def test_row_passes_where_the_rows_do_not_stage(fmt, act, N, K, bs, variant):
    """More than 8 rows whose activations do not fit in LDS run as passes of 8 rows, one
    launch each (M = 16 here; M = 9 stages its rows in one launch on the first two):
    sampled outputs against the oracle at M = 9 and 16, and every row's bits equal to
    those of the 8-row launch (rows 0..7) and across M (row 8)."""
    prob = synth.make_problem(fmt, act, N, K, bs, 16, seed=93)
    gu.say(f"[parity] row passes {fmt}/{act} {N}x{K}")
    Y8, p8 = gu.run_gpu(prob, 8)
    assert p8["family"] == "mfma" and p8["variant"] & 3 == variant, p8
    Ys = {}
    for M in (9, 16):
        Ys[M], p = gu.run_gpu(prob, M)
        assert p["family"] == "mfma" and p["ksplit"] == p8["ksplit"], (M, p)
        if M == 16:
            assert p["passes"] == 2 and p["rows_per_pass"] == 8 and p["variant"] == p8["variant"], (M, p)
        ok, ratio = gu.check_points(prob, M, Ys[M], count=4000, seed=M)
        gu.say(f"   M={M} plan={p} max err/tol={ratio:.3e}")
        assert ok, (M, ratio)
        assert np.array_equal(Ys[M][:8].view(np.int64), Y8.view(np.int64)), M
    assert np.array_equal(Ys[16][8].view(np.int64), Ys[9][8].view(np.int64))


@pytest.mark.parametrize("fmt,act,N,K,bs,ring_max,frac", [("u4", "bf16", 24576, 4096, 32, 8, (3, 4)),
                                                           ("fp8", "f16", 28672, 4096, 128, 8, (7, 8)),
                                                           ("u4", "bf16", 28672, 8192, 32, 4, (7, 8))])
def test_dma_ring_band_takes_no_k_split_at_any_m(fmt, act, N, K, bs, ring_max, frac):
    """A weight whose ring tile groups fill 3/4 (4-bit) or 7/8 (FP8; 4-bit where only
    four rows fit next to the ring) of the CUs: the DMA ring from M = 2 or 3 up to 8 (or
    4), the unsplit register ring above, one summation order throughout. Sampled
    outputs against the oracle and a row's bits across M."""
    import torch

    cu = torch.cuda.get_device_properties(0).multi_processor_count
    if ((N + 15) // 16 + 7) // 8 * frac[1] < frac[0] * cu:
        pytest.skip(f"{N} columns are below the band on {cu} CUs")
    prob = synth.make_problem(fmt, act, N, K, bs, 16, seed=95)
    gu.say(f"[parity] ring band {fmt}/{act} {N}x{K}")
    rows = {}
    for M in (4, 8, 12, 16):
        Y, p = gu.run_gpu(prob, M)
        assert p["family"] == "mfma" and p["ksplit"] == 1 and bool(p["variant"] & 2) == (M <= ring_max), (M, p)
        ok, ratio = gu.check_points(prob, M, Y, count=3000, seed=M)
        gu.say(f"   M={M} plan={p} max err/tol={ratio:.3e}")
        assert ok, (M, ratio)
        rows[M] = Y[:4]
    for M in (8, 12, 16):
        assert np.array_equal(rows[M].view(np.int64), rows[4].view(np.int64)), M


@pytest.mark.parametrize("M", [2, 3, 4])
def test_overlaid_reduction_keeps_one_tile_group_per_workgroup(M):
    """4-bit 16446 x 9600 (block size 64): a K split of 4 over 514 tile groups. At two
    rows the staged rows leave room for the reduction area over them, which needs one
    tile group per workgroup; the kernel's registers leave fewer workgroups resident
    than that, and the create-time residency cut must keep the grid (a cut grid made
    the kernel lay the area past the launch's LDS: wrong outputs). At three and four
    rows the area follows the rows in a persistent grid. Sampled outputs against the
    oracle."""
    prob = synth.make_problem("u4", "f16", 16446, 9600, 64, M, seed=148)
    gu.say(f"[parity] overlaid reduction u4/f16 16446x9600 M={M}")
    for ws in (False, True):
        Y, plan = gu.run_gpu(prob, M, ws=ws)
        assert plan["family"] == "mfma" and plan["ksplit"] == 4 and plan["variant"] & 1, plan
        assert M > 2 or plan["grid"] >= (16446 + 15) // 16 // 2, plan
        ok, ratio = gu.check_points(prob, M, Y, count=4000, seed=M)
        gu.say(f"   ws={ws} plan={plan} max err/tol={ratio:.3e}")
        assert ok, (ws, ratio)


@pytest.mark.parametrize("fmt", ["fp8", "u4"])
@pytest.mark.parametrize("M,family", [(5, "mfma"), (6, "stream"), (16, "stream")])
def test_tall_narrow_shapes_without_workspace(fmt, M, family):
    """1024 x 16384 through qgemv_run: the activation rows do not fit in LDS, not even 8
    at a time, and the tile groups fill a quarter of the CUs, so from M = 6 the
    dispatcher takes the streaming family (M = 5 stays on the matrix cores, activations
    in the register ring). Every output against the oracle."""
    bs = 128 if fmt == "fp8" else 32
    prob = synth.make_problem(fmt, "f16", 1024, 16384, bs, M, seed=91)
    gu.say(f"[parity] tall {fmt} 1024x16384 M={M}")
    Y, plan = gu.run_gpu(prob, M)
    assert plan["family"] == family and plan["kparts"] == 1, plan
    ok, ratio, _, _ = gu.check_full(prob, M, Y)
    gu.say(f"   plan={plan} max err/tol={ratio:.3e}")
    assert ok, (ratio, plan)


# ----------------------------------------------------------------------------------
# every family, every format, ragged shapes


FMT_CASES = [("u4", "f16", 32), ("u4", "bf16", 32), ("u4", "f16", 16), ("u4", "bf16", 128),
             ("u8", "f16", 128), ("u8", "bf16", 32), ("u8", "f16", 16),
             ("fp8", "f16", 128), ("fp8", "bf16", 32), ("nvfp4", "bf16", 16), ("nvfp4", "f16", 16)]


def ring_eligible(prob, M):
    """The DMA ring copies each column's metadata window as whole dwords, so the
    dispatcher takes it only when every scale (and zero-point) row is a whole number
    of dwords, and only for one or two row groups (M <= 8)."""
    nblk = prob.K // prob.bs
    sb = {"u4": 2, "u8": 2, "fp8": 4, "nvfp4": 1}[prob.fmt]
    zrow = 0 if prob.zp is None else ((nblk + 1) // 2 if prob.fmt == "u4" else nblk)
    return M <= 8 and (nblk * sb) % 4 == 0 and zrow % 4 == 0


@pytest.mark.parametrize("family", ["auto", "stream", "mfma_nolds", "mfma_lds", "mfma_ring", "generic"])
@pytest.mark.parametrize("fmt,act,bs", FMT_CASES)
def test_families_ragged_shapes(family, fmt, act, bs):
    for N, K, M in [(1, 256, 1), (17, 512, 3), (36, 1024, 5), (1169, 768, 16), (300, 4096, 2)]:
        if K % bs:
            continue
        prob = synth.make_problem(fmt, act, N, K, bs, M, seed=N + K, zp_range=(0, 15) if fmt == "u4" else (96, 160),
                                  scale_sigma=0.02 if fmt == "u4" else 0.004)
        gu.say(f"[ragged] {family} {fmt}/{act} bs={bs} N={N} K={K} M={M}")
        Y, plan = gu.run_gpu(prob, M, flags=FAMILY_FLAG[family])
        if family != "auto":
            assert plan["family"] == family.split("_")[0]
        if family == "mfma_lds":
            assert plan["variant"] & 1
        if family == "mfma_ring" and ring_eligible(prob, M):
            assert plan["variant"] & 2, plan
        ok, ratio, _, _ = gu.check_full(prob, M, Y, strict=False)
        assert ok, (family, fmt, act, bs, N, K, M, ratio, plan)


@pytest.mark.parametrize("fmt,act", [("u4", "f16"), ("u8", "f16"), ("u4", "bf16"), ("u8", "bf16")])
def test_missing_zero_points_mean_midpoint(fmt, act):
    prob = synth.make_problem(fmt, act, 200, 512, 32, 4, seed=9, with_zp=False)
    assert prob.zp is None
    Y, _ = gu.run_gpu(prob, 4)
    ok, ratio, _, _ = gu.check_full(prob, 4, Y, strict=False)
    assert ok, ratio


# ----------------------------------------------------------------------------------
# bit-exact properties


@pytest.mark.parametrize("family", ["stream", "stream_classic", "mfma_nolds", "mfma_lds", "mfma_ring", "generic"])
@pytest.mark.parametrize("fmt,act,bs", [("u4", "bf16", 32), ("u4", "f16", 32), ("fp8", "f16", 128),
                                         ("nvfp4", "bf16", 16), ("u8", "f16", 128), ("u4", "f16", 16),
                                         ("u8", "bf16", 64)])
def test_row_results_do_not_depend_on_the_tile(family, fmt, act, bs):
    """Row i of an M-row call equals the same row run alone, and in any other M. The
    two activation paths of the matrix family must also agree bit for bit."""
    prob = synth.make_problem(fmt, act, 777, 2048, bs, 16, seed=21)
    flags = FAMILY_FLAG[family]
    gu.say(f"[rows] {family} {fmt}/{act}")
    Y16, plan16 = gu.run_gpu(prob, 16, flags=flags)
    for M in (1, 2, 3, 4, 5, 8, 13):
        A = np.ascontiguousarray(prob.A[16 - M:])  # rows land in different slots
        Ym, _ = gu.run_gpu(prob, M, flags=flags, A=A)
        assert np.array_equal(Ym.view(np.int64), Y16[16 - M:].view(np.int64)), (family, fmt, M)
    if family in ("mfma_lds", "mfma_ring"):
        # same K split (it orders the fp32 sums), other activation / weight paths
        ks = plan16["ksplit"]
        Yo, po = gu.run_gpu(prob, 16, flags=FAMILY_FLAG["mfma_nolds"] | (ks << 8))
        assert po["ksplit"] == ks and not (po["variant"] & 3)
        assert np.array_equal(Yo.view(np.int64), Y16.view(np.int64))


def _stream1_flags(cpw, unr, wpc):
    code = {1: 1, 2: 2, 4: 3}[cpw]
    return (1 | (code << bqw.FLAG_STREAM_CPW_SHIFT) | ((unr - 1) << bqw.FLAG_STREAM_UNR_SHIFT)
            | (wpc << bqw.FLAG_STREAM_WPC_SHIFT))


@pytest.mark.parametrize("fmt,act,bs,N,K", [("u4", "bf16", 32, 1001, 4000 // 32 * 32 + 32 * 3),
                                            ("u4", "f16", 16, 517, 64 * 32 * 3 + 32),
                                            ("u8", "f16", 128, 333, 128 * 37),
                                            ("u8", "bf16", 64, 700, 64 * 40),
                                            ("fp8", "f16", 128, 1234, 128 * 41),
                                            ("nvfp4", "bf16", 16, 999, 32 * 97),
                                            ("nvfp4", "f16", 16, 64, 32 * 128),
                                            ("u4", "bf16", 32, 20011, 1024),
                                            ("fp8", "bf16", 128, 9001, 2048)])
def test_one_row_persistent_kernel_matches_the_classic_kernel_bitwise(fmt, act, bs, N, K):
    """The persistent M = 1 streaming kernel keeps the streaming family's per-row
    arithmetic: every columns-per-wave / batch / grid choice (including grids small
    enough that each wave walks many column groups, and ragged chunk counts) must give
    the classic kernel's bits, and both must meet the oracle bound."""
    prob = synth.make_problem(fmt, act, N, K, bs, 1, seed=31)
    gu.say(f"[stream1] {fmt}/{act} bs{bs} N={N} K={K}")
    Yc, pc = gu.run_gpu(prob, 1, flags=FAMILY_FLAG["stream_classic"])
    assert not (pc["variant"] & 1)
    ok, ratio, _, _ = gu.check_full(prob, 1, Yc, strict=False)
    assert ok, ratio
    Ya, pa = gu.run_gpu(prob, 1, flags=FAMILY_FLAG["stream"])
    assert pa["variant"] & 1, pa
    assert np.array_equal(Ya.view(np.int64), Yc.view(np.int64))
    for cpw in (1, 2, 4):
        for unr in (2, 3, 4):
            for wpc in (0, 1):
                Yv, pv = gu.run_gpu(prob, 1, flags=_stream1_flags(cpw, unr, wpc))
                assert pv["variant"] & 1 and pv["cols_per_wave"] == cpw, pv
                assert np.array_equal(Yv.view(np.int64), Yc.view(np.int64)), (cpw, unr, wpc, pv)
    for unr in (2, 3, 4):  # 16-wave workgroups
        Yv, pv = gu.run_gpu(prob, 1, flags=_stream1_flags(1, unr, 0) | bqw.FLAG_STREAM_WIDE_WG)
        assert pv["waves_per_wg"] == 16, pv
        assert np.array_equal(Yv.view(np.int64), Yc.view(np.int64)), (unr, pv)


@pytest.mark.parametrize("fmt,act,bs,N,K", [("u4", "bf16", 32, 1001, 4064), ("u8", "f16", 64, 333, 64 * 37),
                                            ("fp8", "bf16", 128, 700, 128 * 41), ("nvfp4", "bf16", 16, 517, 32 * 97),
                                            ("u4", "f16", 16, 9001, 1024)])
@pytest.mark.parametrize("M", [2, 3, 4])
def test_multi_row_persistent_kernel_matches_the_classic_kernel_bitwise(fmt, act, bs, N, K, M):
    """Two or four rows per pass in the persistent streaming kernel: each row equals
    the classic streaming kernel's bits, and the oracle bound holds."""
    prob = synth.make_problem(fmt, act, N, K, bs, M, seed=32)
    gu.say(f"[stream-rows] {fmt}/{act} bs{bs} N={N} K={K} M={M}")
    Yc, pc = gu.run_gpu(prob, M, flags=FAMILY_FLAG["stream_classic"])
    ok, ratio, _, _ = gu.check_full(prob, M, Yc, strict=False)
    assert ok, ratio
    for cpw in (1, 2):
        for nwg in (0, 1, 2, 3, 4):  # automatic, then 4, 8, 12 and 16 waves per workgroup
            Ya, pa = gu.run_gpu(prob, M, flags=1 | ({1: 1, 2: 2}[cpw] << bqw.FLAG_STREAM_CPW_SHIFT)
                                | (nwg << bqw.FLAG_STREAM_NWG_SHIFT))
            assert pa["variant"] & 1 and pa["rows_per_pass"] >= M and pa["cols_per_wave"] == cpw, pa
            cap = 8 if cpw == 2 else (12 if (fmt == "u4" and bs == 16 and M > 2) else 16)
            assert nwg == 0 or pa["waves_per_wg"] == min(4 * nwg, cap), pa
            assert np.array_equal(Ya.view(np.int64), Yc.view(np.int64)), (cpw, nwg, pa)


@pytest.mark.parametrize("fmt,act,bs,N,K,M", [("u4", "bf16", 32, 4096, 14336, 3), ("fp8", "bf16", 128, 3001, 28672, 2),
                                              ("u8", "f16", 128, 2500, 16384, 4), ("u4", "bf16", 32, 1024, 16384, 4),
                                              ("u4", "bf16", 32, 8192, 28672, 1)])
def test_long_rows_in_the_persistent_streaming_kernel(fmt, act, bs, N, K, M):
    """Rows past 64 KB of LDS in the persistent streaming kernel (one round of
    workgroups of up to 16 waves holding them; one row up to 64 KB): the automatic
    plan, every row equal to the classic kernel's bits, sampled outputs against the
    oracle."""
    prob = synth.make_problem(fmt, act, N, K, bs, M, seed=34)
    gu.say(f"[stream-rows] long {fmt}/{act} N={N} K={K} M={M}")
    Ya, pa = gu.run_gpu(prob, M)
    gu.say(f"   plan={pa}")
    assert pa["family"] == "stream" and pa["variant"] & 1 and pa["lds_bytes"] > (48 if M == 1 else 64) * 1024, pa
    Yc, pc = gu.run_gpu(prob, M, flags=FAMILY_FLAG["stream_classic"])
    assert np.array_equal(Ya.view(np.int64), Yc.view(np.int64)), (pa, pc)
    ok, ratio = gu.check_points(prob, M, Ya, count=3000, seed=M)
    assert ok, ratio


@pytest.mark.parametrize("act,N,K", [("f16", 700, 128 * 41), ("bf16", 1234, 128 * 24), ("f16", 5120, 6144)])
@pytest.mark.parametrize("M", [5, 6, 8])
def test_eight_row_persistent_kernel_matches_the_classic_kernel_bitwise(act, N, K, M):
    """FP8 codes at M = 5..8 in one pass of eight rows (the persistent streaming kernel's
    largest row tile): each row equals the classic kernel's bits (two passes of four
    rows), at every workgroup size, and the oracle bound holds."""
    prob = synth.make_problem("fp8", act, N, K, 128, M, seed=33)
    gu.say(f"[stream-8rows] fp8/{act} N={N} K={K} M={M}")
    Yc, pc = gu.run_gpu(prob, M, flags=FAMILY_FLAG["stream_classic"])
    assert pc["rows_per_pass"] == 4 and pc["passes"] == 2, pc
    ok, ratio, _, _ = gu.check_full(prob, M, Yc, strict=False)
    assert ok, ratio
    for nwg in (0, 1, 2, 3, 4):
        Ya, pa = gu.run_gpu(prob, M, flags=1 | (nwg << bqw.FLAG_STREAM_NWG_SHIFT))
        assert pa["variant"] & 1 and pa["rows_per_pass"] == 8 and pa["passes"] == 1, pa
        assert nwg == 0 or pa["waves_per_wg"] == 4 * nwg, pa
        assert np.array_equal(Ya.view(np.int64), Yc.view(np.int64)), (nwg, pa)


@pytest.mark.parametrize("fmt,act,N,K,bs", [("u4", "f16", 1001, 2080, 32), ("u4", "f16", 777, 4096, 16),
                                             ("u8", "f16", 999, 2048, 128), ("u8", "bf16", 1234, 4096, 64),
                                             ("nvfp4", "bf16", 1111, 2048, 16), ("nvfp4", "f16", 999, 3104, 16)])
@pytest.mark.parametrize("M", [5, 8])
def test_eight_row_pass_of_other_formats_matches_the_classic_kernel_bitwise(fmt, act, N, K, bs, M):
    """4-bit (fp16), 8-bit and NVFP4 codes with K >= 2048 at M = 5..8 in one pass of eight
    rows: each row equals the classic kernel's bits (two passes of four rows) at every
    workgroup size the kernel takes, and the oracle bound holds."""
    prob = synth.make_problem(fmt, act, N, K, bs, M, seed=35)
    gu.say(f"[stream-8rows] {fmt}/{act} N={N} K={K} bs={bs} M={M}")
    Yc, pc = gu.run_gpu(prob, M, flags=FAMILY_FLAG["stream_classic"])
    assert pc["rows_per_pass"] == 4 and pc["passes"] == 2, pc
    ok, ratio, _, _ = gu.check_full(prob, M, Yc, strict=False)
    assert ok, ratio
    for nwg in ((0, 1, 2) if fmt in ("u4", "nvfp4") else (0, 1, 2, 3, 4)):
        Ya, pa = gu.run_gpu(prob, M, flags=1 | (nwg << bqw.FLAG_STREAM_NWG_SHIFT))
        assert pa["variant"] & 1 and pa["rows_per_pass"] == 8 and pa["passes"] == 1, pa
        assert nwg == 0 or pa["waves_per_wg"] == 4 * nwg, pa
        assert np.array_equal(Ya.view(np.int64), Yc.view(np.int64)), (nwg, pa)


@pytest.mark.parametrize("name,M", [("u4_m8_k2048_n1024", 8), ("fp8_k6144_n5120", 4), ("u8_m1_k4096_n4096", 1)])
def test_repeated_runs_are_bitwise_equal(name, M):
    prob = synth.workload(name)
    outs, plan = gu.run_gpu(prob, M, repeat=4)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0]), plan


@pytest.mark.parametrize("fmt,act,bs", [("fp8", "f16", 128), ("u8", "f16", 128), ("u4", "bf16", 32)])
def test_reduction_area_overlaid_on_the_staged_rows(fmt, act, bs):
    """M = 16, K = 4096: the staged rows and the K-split reduction area fit in LDS only
    overlaid (one tile group per workgroup). Within the bound against the oracle, and
    bit for bit equal to the unstaged run, at a ragged N."""
    M, N, K = 16, 1000, 4096
    prob = synth.make_problem(fmt, act, N, K, bs, M, seed=11)
    base = 2 | (4 << 8) | bqw.FLAG_RING_OFF
    gu.say(f"[overlay] {fmt}/{act} bs={bs} N={N} K={K} M={M}")
    Y, plan = gu.run_gpu(prob, M, flags=base | bqw.FLAG_STAGE_A_ON)
    assert plan["ksplit"] == 4 and plan["variant"] & 1, plan
    red = 8 * 4 * 4 * 64 * 4
    assert plan["lds_bytes"] + red > 160 * 1024 >= plan["lds_bytes"], plan
    Yu, pu = gu.run_gpu(prob, M, flags=base | bqw.FLAG_STAGE_A_OFF)
    assert not (pu["variant"] & 1)
    assert np.array_equal(Y.view(np.int64), Yu.view(np.int64))
    ok, ratio, _, _ = gu.check_full(prob, M, Y, strict=False)
    assert ok, ratio


def test_sixteen_rows_full_size_with_the_overlaid_reduction_area():
    """FP8 8192 x 4096 at M = 16 under the automatic plan (K split 4, staged rows with
    the reduction area overlaid), on sampled outputs against the oracle."""
    prob = synth.make_problem("fp8", "f16", 8192, 4096, 128, 16, seed=12)
    gu.say("[overlay] fp8 8192 x 4096 M=16 auto")
    Y, plan = gu.run_gpu(prob, 16)
    assert plan["family"] == "mfma" and plan["ksplit"] == 4 and plan["variant"] & 1, plan
    ok, ratio = gu.check_points(prob, 16, Y)
    assert ok, ratio


@pytest.mark.parametrize("fmt,act,N,K,bs,M,bias", [("fp8", "f16", 2000, 8192, 128, 13, False),
                                                   ("fp8", "f16", 2048, 8192, 128, 16, False),
                                                   ("u8", "f16", 1900, 8192, 128, 12, False),
                                                   ("fp8", "f16", 2000, 8192, 128, 16, True)])
def test_row_passes_match_one_unstaged_launch(fmt, act, N, K, bs, M, bias):
    """Where M > 8 rows do not fit in LDS and there are no K parts, the plan runs passes
    of 8 rows (the last one shorter), one launch each. Every row comes out bit for bit
    as in one launch with the activations in the register ring, and within the bound
    against the oracle."""
    prob = synth.make_problem(fmt, act, N, K, bs, M, seed=27, with_bias=bias)
    gu.say(f"[passes] {fmt}/{act} N={N} K={K} M={M} bias={bias}")
    Y, plan = gu.run_gpu(prob, M)
    assert plan["family"] == "mfma" and plan["passes"] == 2 and plan["rows_per_pass"] == 8, plan
    assert plan["variant"] & 1
    Yu, pu = gu.run_gpu(prob, M, flags=bqw.FLAG_STAGE_A_OFF)
    assert pu["passes"] == 1 and not (pu["variant"] & 1) and pu["ksplit"] == plan["ksplit"], pu
    assert np.array_equal(Y.view(np.int64), Yu.view(np.int64))
    ok, ratio, _, _ = gu.check_full(prob, M, Y, strict=False)
    assert ok, ratio


@pytest.mark.parametrize("fmt,act,N,K,bs,flags,family", [("u4", "f16", 1000, 2048, 32, 0, "stream"),
                                                         ("fp8", "f16", 777, 4096, 128, 2, "mfma"),
                                                         ("u4", "bf16", 3000, 4096, 32, 0, "mfma"),
                                                         ("nvfp4", "bf16", 640, 1024, 16, 1, "stream"),
                                                         ("u8", "f16", 500, 1024, 128, 3, "generic")])
def test_more_than_sixteen_rows_run_as_chunks(fmt, act, N, K, bs, flags, family):
    """M = 37 runs as chunks of 16, 16 and 5 rows with the 16-row plan: every output
    within the bound against the oracle, and the middle chunk bit for bit the 16-row
    call on those rows."""
    M = 37
    prob = synth.make_problem(fmt, act, N, K, bs, M, seed=28)
    gu.say(f"[chunks] {fmt}/{act} N={N} K={K} M={M} flags={flags:#x}")
    Y, plan = gu.run_gpu(prob, M, flags=flags)
    assert plan["family"] == family, plan
    ok, ratio, _, _ = gu.check_full(prob, M, Y, strict=False)
    assert ok, ratio
    Y16, p16 = gu.run_gpu(prob, 16, flags=flags, A=prob.A[16:32])
    assert plan["passes"] == 3 * p16["passes"], (plan, p16)
    assert np.array_equal(Y[16:32].view(np.int64), Y16.view(np.int64))


@pytest.mark.parametrize("stage", [False, True])
@pytest.mark.parametrize("ks", [1, 2, 4, 8])
def test_forced_k_split_is_correct(ks, stage):
    prob = synth.make_problem("u4", "bf16", 100, 4096, 32, 6, seed=4)
    flags = 2 | (ks << 8) | (bqw.FLAG_STAGE_A_ON if stage else bqw.FLAG_STAGE_A_OFF)
    Y, plan = gu.run_gpu(prob, 6, flags=flags)
    assert plan["ksplit"] == ks and bool(plan["variant"] & 1) == stage
    ok, ratio, _, _ = gu.check_full(prob, 6, Y, strict=False)
    assert ok, (ks, ratio)


@pytest.mark.parametrize("fmt,act", [("u4", "f16"), ("u4", "bf16"), ("u8", "f16"), ("u8", "bf16")])
def test_integer_special_case_is_exact(fmt, act):
    """Scale 1, zero point 0, small integer activations: fp32 holds the integer result
    exactly, so the output must be that integer rounded once to the output type."""
    rng = np.random.default_rng(1)
    M, N, K, bs = 5, 333, 512, 32
    nblk = K // bs
    a_int = rng.integers(-2, 3, size=(M, K))
    hi = 16 if fmt == "u4" else 4
    q = rng.integers(0, hi, size=(N, K)).astype(np.uint8)
    W = synth.pack_nibbles(q).reshape(N, nblk, bs // 2) if fmt == "u4" else q.reshape(N, nblk, bs)
    zp = synth.pack_nibbles(np.zeros((N, nblk), np.uint8)) if fmt == "u4" else np.zeros((N, nblk), np.uint8)
    prob = synth.Problem(name="int", fmt=fmt, act=act, N=N, K=K, bs=bs, W=W,
                         scales=np.full((N, nblk), 0x3C00, dtype=np.uint16), zp=zp, tensor_scale=1.0,
                         A=synth.activation_bits(a_int.astype(np.float64), act))
    exact = (a_int @ q.astype(np.int64).T).astype(np.float64)
    assert np.abs(exact).max() > 128  # large enough that bf16 must round some results
    want = oracle.decode_activation_bits(synth.activation_bits(exact, act), act)
    for fam in ("stream", "generic", "mfma_nolds", "mfma_lds", "mfma_ring"):
        Y, _ = gu.run_gpu(prob, M, flags=FAMILY_FLAG[fam])
        assert np.array_equal(Y, want), fam


@pytest.mark.parametrize("fmt,act,bs", [("u4", "bf16", 32), ("u8", "f16", 128), ("fp8", "f16", 128),
                                         ("nvfp4", "bf16", 16), ("u4", "f16", 16)])
def test_bias_epilogue_every_family(fmt, act, bs):
    """Optional bias (one value per column, added after every scale): every family and
    M meet the oracle bound on ragged N; row i of an M-row call equals the same row of
    the 16-row call bit for bit within a family; and the persistent streaming kernel
    keeps the classic kernel's bits with the bias too."""
    prob = synth.make_problem(fmt, act, 1169, 2048, bs, 16, seed=37, with_bias=True,
                              zp_range=(0, 15) if fmt == "u4" else (96, 160),
                              scale_sigma=0.02 if fmt == "u4" else 0.004)
    assert prob.bias is not None
    gu.say(f"[bias] {fmt}/{act} bs{bs}")
    fams = ["auto", "stream", "stream_classic", "generic", "mfma_nolds", "mfma_lds", "mfma_ring"]
    for fam in fams:
        Y16, p16 = gu.run_gpu(prob, 16, flags=FAMILY_FLAG[fam])
        ok, ratio, _, _ = gu.check_full(prob, 16, Y16, strict=False)
        assert ok, (fam, ratio, p16)
        for M in (1, 3, 5):
            A = np.ascontiguousarray(prob.A[16 - M:])
            Ym, pm = gu.run_gpu(prob, M, flags=FAMILY_FLAG[fam], A=A)
            ok, ratio, _, _ = gu.check_full(prob, M, Ym, A=A, strict=False)
            assert ok, (fam, M, ratio, pm)
            if fam not in ("auto", "stream") and pm["family"] == p16["family"] and pm["ksplit"] == p16["ksplit"]:
                assert np.array_equal(Ym.view(np.int64), Y16[16 - M:].view(np.int64)), (fam, M)
    Yc, _ = gu.run_gpu(prob, 1, flags=FAMILY_FLAG["stream_classic"])
    Ys, ps = gu.run_gpu(prob, 1, flags=FAMILY_FLAG["stream"])
    assert ps["variant"] & 1 and np.array_equal(Ys.view(np.int64), Yc.view(np.int64))


@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_integer_case_with_bias_is_exact(act):
    """Integer codes with scale 1 and zero point 0, small integer activations and an
    integer bias: every output is an integer the output type holds, so each family
    must return it exactly."""
    rng = np.random.default_rng(5)
    M, N, K, bs = 5, 300, 512, 32
    nblk = K // bs
    a_int = rng.integers(-2, 3, size=(M, K))
    q = rng.integers(0, 4, size=(N, K)).astype(np.uint8)
    b_int = rng.integers(-64, 65, size=N)
    prob = synth.Problem(name="int_bias", fmt="u4", act=act, N=N, K=K, bs=bs,
                         W=synth.pack_nibbles(q).reshape(N, nblk, bs // 2),
                         scales=np.full((N, nblk), 0x3C00, dtype=np.uint16),
                         zp=synth.pack_nibbles(np.zeros((N, nblk), np.uint8)), tensor_scale=1.0,
                         A=synth.activation_bits(a_int.astype(np.float64), act),
                         bias=synth.activation_bits(b_int.astype(np.float64), act))
    exact = (a_int @ q.astype(np.int64).T + b_int[None, :]).astype(np.float64)
    assert np.abs(exact).max() <= 256  # exact in bf16 as well
    for fam in ("stream", "stream_classic", "generic", "mfma_nolds", "mfma_lds", "mfma_ring"):
        Y, _ = gu.run_gpu(prob, M, flags=FAMILY_FLAG[fam])
        assert np.array_equal(Y, exact), fam


@pytest.mark.parametrize("fmt", ["fp8", "nvfp4", "u4", "u8"])
@pytest.mark.parametrize("act", ["f16", "bf16"])
def test_one_hot_probes_decode_every_code_exactly(fmt, act):
    """One-hot activations pick single weights; every code of the format appears, so
    each decoded value (times its scale) must come out exactly. Catches any lane,
    byte, nibble or k permutation and any decoder error."""
    rng = np.random.default_rng(2)
    N, K = 48, 512
    bs = 16 if fmt == "nvfp4" else 32
    nblk = K // bs
    if fmt == "fp8":
        codes = np.resize(synth.FP8_FINITE_CODES, (N, K)).astype(np.uint8)
        for n in range(N):
            codes[n] = np.roll(codes[n], 5 * n)
        W = codes
        scales = np.ones((N, nblk), np.float32)
        zp = None
    elif fmt == "nvfp4":
        codes = (np.arange(N * K).reshape(N, K) + np.arange(N)[:, None]) % 16
        W = synth.pack_nibbles(codes.astype(np.uint8))
        scales = np.full((N, K // 16), 0x38, np.uint8)  # E4M3 1.0
        zp = None
    elif fmt == "u4":
        codes = ((np.arange(K)[None, :] * 3 + np.arange(N)[:, None]) % 16).astype(np.uint8)
        W = synth.pack_nibbles(codes).reshape(N, nblk, bs // 2)
        zp = synth.pack_nibbles(rng.integers(0, 16, size=(N, nblk)).astype(np.uint8))
        scales = np.full((N, nblk), 0x3C00, np.uint16)
    else:
        codes = ((np.arange(K)[None, :] + 37 * np.arange(N)[:, None]) % 256).astype(np.uint8)
        W = codes.reshape(N, nblk, bs)
        zp = rng.integers(0, 256, size=(N, nblk)).astype(np.uint8)
        scales = np.full((N, nblk), 0x3C00, np.uint16)
    base = synth.Problem(name="onehot", fmt=fmt, act=act, N=N, K=K, bs=bs, W=W, scales=scales, zp=zp,
                         tensor_scale=1.0, A=np.zeros((16, K), np.uint16))
    one = 0x3C00 if act == "f16" else 0x3F80
    deq = oracle.dequant_columns(base)  # [N, K] exact values
    for fam in ("stream", "generic", "mfma_nolds", "mfma_lds", "mfma_ring"):
        for k0 in range(0, K, 16):
            A = np.zeros((16, K), np.uint16)
            A[np.arange(16), k0 + np.arange(16)] = one
            Y, _ = gu.run_gpu(base, 16, flags=FAMILY_FLAG[fam], A=A)
            want = deq[:, k0:k0 + 16].T  # exact in fp16 and bf16
            assert np.array_equal(Y, want), (fam, fmt, act, k0)


def test_misaligned_activations_fall_back_and_stay_correct():
    prob = synth.workload("u4_m8_k2048_n1024", n_override=256)
    Y, plan = gu.run_gpu(prob, 8, a_offset_elems=1)  # A 2 bytes off a 16-byte boundary
    ok, ratio, _, _ = gu.check_full(prob, 8, Y)
    assert ok, ratio


def test_run_rejects_bad_arguments():
    import torch
    prob = synth.workload("u4_m1_k512_n256")
    q, t = bqw.upload(prob)
    Y = torch.empty((16, prob.N), dtype=t["A"].dtype, device="cuda")
    # rejected before any launch (17 rows and more are valid: chunks of 16)
    for M in (0, bqw.MAX_ROWS + 1, -1):
        with pytest.raises(bqw.QGemvError) as e:
            q.run(t["A"], Y, M=M)
        assert e.value.status == 2
    with pytest.raises(bqw.QGemvError) as e:
        q.run(0, Y, M=1)
    assert e.value.status == 1
    q.close()


@pytest.mark.parametrize("act,bs,K", [("f16", 16, 16 * 120), ("bf16", 32, 2048), ("f16", 32, 32 * 100),
                                      ("f16", 128, 4096), ("bf16", 128, 128 * 44), ("f16", 256, 256 * 20)])
@pytest.mark.parametrize("M", [1, 3])
@pytest.mark.parametrize("zp", [True, False])
def test_metadata_windows_match_per_chunk_loads(act, bs, K, M, zp):
    """8-bit codes: the persistent streaming kernel's round metadata windows (one dword
    per lane per column, values handed out across lanes) give the same bits as the
    per-chunk loads, including partial last rounds, ragged N and missing zero points
    (the midpoint), and meet the oracle."""
    prob = synth.make_problem("u8", act, 333, K, bs, M, seed=K + bs, zp_range=(96, 160), scale_sigma=0.004,
                              with_zp=zp)
    gu.say(f"[meta window] u8/{act} bs={bs} K={K} M={M} zp={zp}")
    Yw, pw = gu.run_gpu(prob, M, flags=1)
    Yc, pc = gu.run_gpu(prob, M, flags=1 | bqw.FLAG_STREAM_META_CHUNK)
    assert pw["variant"] & 1 and pw["variant"] & 8, pw
    assert pc["variant"] & 1 and not pc["variant"] & 8, pc
    assert np.array_equal(Yw.view(np.int64), Yc.view(np.int64))
    ok, ratio, _, _ = gu.check_full(prob, M, Yw, strict=False)
    assert ok, ratio
