"""The C ABI on the host: the library loads, exports every declared entry point, and
its pure-host pieces (validation, status strings, dispatcher) behave. No GPU needed."""

import ctypes
import os
import re

import pytest

import block_quantized_weight_amd as bqw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"^\s*(?:int|void|const char \*)\s*\**\s*(qgemv_\w+)\s*\(", text, re.M))
    return names


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"qgemv_create", "qgemv_run", "qgemv_run_ws", "qgemv_run_noalloc", "qgemv_workspace_size", "qgemv_plan",
            "qgemv_select", "qgemv_destroy", "qgemv_status_str", "qgemv_abi_version", "qgemv_tune",
            "qgemv_tune_candidates"} <= names
    L = bqw.lib()
    for n in sorted(names):
        assert hasattr(L, n), n
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def test_abi_version_and_struct_layout():
    assert bqw.lib().qgemv_abi_version() == 6
    # the descriptor is 8-byte aligned with int64 N, K after four 32-bit fields; the
    # bias pointer (version 2) follows the flags
    assert ctypes.sizeof(bqw.Desc) == 72
    assert bqw.Desc.N.offset == 16 and bqw.Desc.W.offset == 32 and bqw.Desc.flags.offset == 60
    assert bqw.Desc.bias.offset == 64
    # the plan report gains the K parts and the workspace size (version 3)
    assert ctypes.sizeof(bqw.PlanInfo) == 56
    assert bqw.PlanInfo.grid.offset == 24 and bqw.PlanInfo.variant.offset == 36
    assert bqw.PlanInfo.kparts.offset == 40 and bqw.PlanInfo.workspace_bytes.offset == 48
    # the tuner's report (version 6)
    assert ctypes.sizeof(bqw.TuneInfo) == 32
    assert bqw.TuneInfo.chosen_flags.offset == 8 and bqw.TuneInfo.auto_us.offset == 16


def test_status_strings():
    for s in range(0, 11):
        assert bqw.status_str(s) and bqw.status_str(s) != bqw.status_str(99)
    assert "workspace" in bqw.status_str(9)
    assert "scratch" in bqw.status_str(10)
    assert bqw.status_str(0) == "ok"
    assert "unknown" in bqw.status_str(99)


def _sel(**kw):
    base = dict(fmt="u4", act="bf16", N=151936, K=4096, block_size=32, M=1, cu_count=256)
    base.update(kw)
    return bqw.select(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(M=0), 2), (dict(M=65537), 2), (dict(M=-1), 2), (dict(N=0), 2), (dict(K=0), 2), (dict(K=4010), 2),
    (dict(block_size=48), 3), (dict(block_size=8), 3), (dict(fmt="nvfp4", block_size=32), 3),
    (dict(fmt="bogus"), 4), (dict(act="fp32"), 4), (dict(fmt="fp8", zero_points=0x2000), 4),
    (dict(fmt="nvfp4", block_size=16, zero_points=0x2000), 4),
    (dict(W=None), 1), (dict(scales=None), 1), (dict(flags=0x4), 7), (dict(flags=9 << 8), 7), (dict(flags=3 << 8), 7), (dict(flags=5 << 12), 7), (dict(flags=3 << 29), 7), (dict(flags=(1 << 19) | (1 << 20)), 7), (dict(flags=(1 << 17) | (1 << 18)), 7),
    (dict(cu_count=0), 7), (dict(bias=0x2001), 7), (dict(flags=5 << 4), 7), (dict(flags=7 << 4), 7),
])
def test_select_rejects_invalid_arguments(kw, status):
    with pytest.raises(bqw.QGemvError) as e:
        _sel(**kw)
    assert e.value.status == status


def test_null_pointers_are_rejected_before_anything_else():
    L = bqw.lib()
    assert L.qgemv_select(None, 1, 256, 0, None) == 1
    out = bqw.PlanInfo()
    assert L.qgemv_select(None, 1, 256, 0, ctypes.byref(out)) == 1
    assert L.qgemv_select(None, 1, 256, 1, ctypes.byref(out)) == 1
    assert L.qgemv_create(None, None, 0) == 1
    h = ctypes.c_void_p()
    assert L.qgemv_create(ctypes.byref(h), None, 0) == 1
    assert L.qgemv_run(None, None, None, 1, None) == 1
    assert L.qgemv_run_ws(None, None, None, 1, None, 0, None) == 1
    size = ctypes.c_size_t()
    assert L.qgemv_workspace_size(None, 1, ctypes.byref(size)) == 1
    assert L.qgemv_plan(None, 1, 0, ctypes.byref(out)) == 1
    L.qgemv_destroy(None)  # ignored


def test_create_validates_before_touching_the_device():
    L = bqw.lib()
    d = bqw.make_desc("u4", "f16", 16, 100, 32, 0x1000, 0x1000)  # K not a multiple of bs
    h = ctypes.c_void_p()
    assert L.qgemv_create(ctypes.byref(h), ctypes.byref(d), 0) == 2
    d.struct_size = 8
    assert L.qgemv_create(ctypes.byref(h), ctypes.byref(d), 0) == 7


def test_select_families_and_fallback():
    assert _sel()["family"] in ("stream", "mfma")
    # misaligned weight pointer -> generic kernel, never an error
    assert _sel(W=0x1001)["family"] == "generic"
    # K not a multiple of a 16-byte chunk -> generic
    assert _sel(fmt="u4", K=16 * 3, block_size=16)["family"] == "generic"
    assert _sel(flags=3)["family"] == "generic"
    with pytest.raises(bqw.QGemvError):
        _sel(W=0x1001, flags=1)  # a forced fast family needs its preconditions


def test_select_parameters_that_shape_row_arithmetic_do_not_depend_on_m():
    """The K split orders each row's fp32 sums, so it may depend on the weight only; so
    do the K parts on these shapes while their activation rows fit in LDS (up to M = 12
    here). With a workspace, FP8 5120 x 6144 at M = 16 is long rows: no split inside a
    workgroup and 4 parts (the tests below). (The matrix family's variants, register
    ring, LDS-staged activations or LDS DMA ring, feed identical MFMA operands in the
    same order; the GPU tests check that they agree bit for bit.)"""
    for fmt, act, N, K, bs in [("u4", "bf16", 151936, 4096, 32), ("fp8", "f16", 5120, 6144, 128),
                               ("nvfp4", "bf16", 248320, 2048, 16), ("u8", "f16", 4096, 4096, 128),
                               ("u4", "f16", 1024, 2048, 32)]:
        for ws in (False, True):
            plans = [_sel(fmt=fmt, act=act, N=N, K=K, block_size=bs, M=m, with_workspace=ws) for m in range(1, 17)]
            for key, upto in (("ksplit", 12 if ws else 16), ("kparts", 12)):
                fams = {}
                for p in plans[:upto]:
                    fams.setdefault(p["family"], set()).add(p[key])
                assert all(len(v) == 1 for v in fams.values()), (fmt, ws, key, fams)


# Automatic plans that leave more than 10% of the CUs without a workgroup although the
# work could be spread further, each with what was measured against the alternatives
# (MI355X, cold weights, one session): the FP8 projection's 320 tiles make 160 8-wave
# workgroups at K split 4 from M = 5; a K split of 8 (320 workgroups, 2 rounds at this
# LDS) took 18.5-18.9 against 16.1-16.6 us at M = 8, K parts 17.5-64.9 us, unstaged
# activations 27.9, one pass of eight rows in the streaming kernel (256 workgroups)
# 20.5, 16-wave workgroups 16.8.
UNDERFILLED = {("fp8", 5120, 6144, M) for M in range(5, 17)}


@pytest.mark.parametrize("cu", [80, 256, 304])
def test_select_covers_the_machine(cu):
    """Every automatic plan for the named workloads (and M = 1, 2, 4, 8, 16, with and
    without a workspace) puts a workgroup on at least 90% of the CUs, or has run out of
    work to spread: every column has a wave of its own (streaming family), or, on 256 CUs,
    every 16-column tile (and K part) has its own workgroup (matrix family); the one
    exception is listed above with its measurements. On 80 and 304 CUs, where nothing
    was measured, the matrix family's K split follows its cost model (ties go to the
    smaller split), so there every tile group (and part) has its own workgroup."""
    shapes = [("u4", "bf16", 151936, 4096, 32), ("fp8", "f16", 5120, 6144, 128), ("nvfp4", "bf16", 248320, 2048, 16),
              ("u8", "f16", 4096, 4096, 128), ("nvfp4", "bf16", 2048, 2048, 16), ("u4", "f16", 1024, 2048, 32),
              ("u4", "f16", 256, 512, 32), ("fp8", "f16", 1024, 16384, 128)]
    for fmt, act, N, K, bs in shapes:
        for M in (1, 2, 4, 8, 16):
            for ws in (False, True):
                p = _sel(fmt=fmt, act=act, N=N, K=K, block_size=bs, M=M, with_workspace=ws, cu_count=cu)
                if p["grid"] >= 0.9 * cu:
                    continue
                if p["family"] == "stream":
                    spread = p["grid"] * p["waves_per_wg"] * p["cols_per_wave"] >= N and p["cols_per_wave"] == 1
                else:
                    tiles = (N + 15) // 16
                    groups = -(-tiles // (8 // p["ksplit"]))
                    if cu == 256:
                        spread = p["grid"] >= tiles * p["kparts"] or (fmt, N, K, M) in UNDERFILLED
                    else:
                        spread = p["grid"] >= groups * p["kparts"]
                assert spread, (cu, fmt, N, K, M, ws, p)


def test_k_parts_only_with_a_workspace_where_tile_groups_leave_cus_idle():
    """qgemv_run_ws splits K across workgroups only where the tile groups leave CUs
    idle, with the most parts that keep the grid within one workgroup per CU; qgemv_run
    never splits."""
    # FP8 1024 x 16384: 64 tiles, K split 8 -> 64 tile groups -> 4 parts (256 workgroups)
    for M in (5, 8, 16):
        kw = dict(fmt="fp8", act="f16", N=1024, K=16384, block_size=128, M=M)
        p0, p1 = _sel(**kw), _sel(**kw, with_workspace=True)
        assert p0["kparts"] == 1 and p0["workspace_bytes"] == 0
        # without a workspace, from M = 6 the rows (K = 16384) fit in LDS not even 8 at
        # a time: the streaming family; the matrix family keeps the same K split
        assert p0["family"] == ("mfma" if M == 5 else "stream"), p0
        assert p1["family"] == "mfma" and p1["ksplit"] == _sel(**kw, flags=2)["ksplit"] == 8
        assert p1["kparts"] == 4 and p1["grid"] == 64 * 4 and not (p1["variant"] & 2)
        # 64 counters (256 bytes), then the [4, M, N] fp32 partials
        assert p1["workspace_bytes"] == 256 + (4 * M * 1024 * 4 + 255) // 256 * 256
    # 128 tile groups (half the CUs): 2 parts only with 16 K steps or more per wave and
    # part. FP8 2048 x 16384 (256 steps, K split 8): 2 parts; 4-bit 2048 x 8192 (64
    # steps, K split 8): none
    p = _sel(fmt="fp8", act="f16", N=2048, K=16384, block_size=128, M=8, with_workspace=True)
    assert p["ksplit"] == 8 and p["kparts"] == 2 and p["grid"] == 256
    p = _sel(fmt="u4", act="bf16", N=2048, K=8192, block_size=32, M=8, with_workspace=True)
    assert p["ksplit"] == 8 and p["kparts"] == 1
    # 8-bit 4096 x 4096 (64 steps, K split 8): 256 tile groups fill the CUs: none
    p = _sel(fmt="u8", act="f16", N=4096, K=4096, block_size=128, M=8, with_workspace=True)
    assert p["family"] == "mfma" and p["ksplit"] == 8 and p["kparts"] == 1
    # 32 tile groups: 4-bit 512 x 8192 -> 4 parts (8 would leave one K step per wave)
    p = _sel(fmt="u4", act="bf16", N=512, K=8192, block_size=32, M=8, with_workspace=True)
    assert p["ksplit"] == 8 and p["kparts"] == 4
    # FP8 5120 x 6144: 160 tile groups; 2 parts would need a second round: none
    p = _sel(fmt="fp8", act="f16", N=5120, K=6144, block_size=128, M=8, with_workspace=True)
    assert p["kparts"] == 1 and p["workspace_bytes"] == 0
    # parts keep two K steps per wave: 4-bit 1024 x 2048 (16 steps, K split 8) in the
    # matrix family takes none
    p = _sel(fmt="u4", act="f16", N=1024, K=2048, block_size=32, M=8, flags=2, with_workspace=True)
    assert p["ksplit"] == 8 and p["kparts"] == 1
    # wide N fills the machine with tile groups: no parts, no workspace
    for M in (2, 8, 16):
        p = _sel(M=M, with_workspace=True)
        assert p["kparts"] == 1 and p["workspace_bytes"] == 0, p
    # the streaming family never splits
    p = _sel(fmt="fp8", act="f16", N=1024, K=16384, block_size=128, M=1, with_workspace=True)
    assert p["family"] == "stream" and p["kparts"] == 1


def test_k_split_takes_the_least_work_on_the_busiest_cu():
    """While the workgroups do not fill the CUs, the K split minimizes (workgroups per
    CU, rounded up) x (K steps per wave), ties to the smaller split; fewer than 8
    steps per wave only while the tiles are fewer than 4 per CU."""
    def ks(fmt, N, K, bs=128, act="f16"):
        return _sel(fmt=fmt, act=act, N=N, K=K, block_size=bs, M=8, flags=2)["ksplit"]
    # 1024 tiles, 64 steps: split 1 -> 128 workgroups x 64 steps; 2 -> 256 x 32; 4 ->
    # 512 (two per CU) x 16 = the same work as 2: the smaller split
    assert ks("u8", 16384, 4096) == 2
    # 512 tiles, 64 steps: 4 -> 256 x 16 beats 2 -> 128 x 32; 8 ties 4
    assert ks("fp8", 8192, 4096) == 4
    # 4-bit 8192 x 4096 (32 steps): 4 (8 steps per wave); 8 would leave 4 steps
    assert ks("u4", 8192, 4096, 32, "bf16") == 4
    # 4-bit 4096 x 4096: 4, not 8 (8 would leave 4 steps per wave, with 256 tiles)
    assert ks("u4", 4096, 4096, 32, "bf16") == 4
    assert ks("nvfp4", 4096, 4096, 16, "bf16") == 4
    # 320 tiles, 96 steps: 4 -> 160 x 24 ties 8 -> 320 (two rounds) x 12: 4
    assert ks("fp8", 5120, 6144) == 4
    # 768 tiles, 32 steps: 2 -> 192 x 16 ties 4 -> 384 x 8
    assert ks("u4", 12288, 4096, 32, "bf16") == 2
    # few tiles: the finest split that keeps two K steps per wave
    assert ks("u4", 1024, 2048, 32) == 8
    assert ks("fp8", 1024, 2048) == 8
    # wide N: no split (the lm_head's unsplit tile groups already fill the CUs)
    assert ks("u4", 151936, 4096, 32, "bf16") == 1
    assert ks("nvfp4", 248320, 2048, 16, "bf16") == 1


def test_three_and_four_rows_take_the_matrix_family_where_its_tile_groups_fill_the_cus():
    """M = 3..4: the matrix family where its tile groups fill the 256 CUs, for 1-byte
    codes only from 64 MB of codes; M = 2 stays with the streaming kernel below the
    4-bit 64 MB rule."""
    def fams(fmt, act, N, K, bs):
        return [_sel(fmt=fmt, act=act, N=N, K=K, block_size=bs, M=M)["family"] for M in (2, 3, 4)]
    assert fams("u4", "bf16", 8192, 4096, 32) == ["stream", "mfma", "mfma"]  # 256 tile groups (split 4)
    assert fams("nvfp4", "bf16", 8192, 4096, 16) == ["stream", "mfma", "mfma"]
    assert fams("u8", "f16", 16384, 4096, 128) == ["stream", "mfma", "mfma"]  # 64 MiB of codes
    assert fams("fp8", "f16", 16384, 4096, 128) == ["stream", "mfma", "mfma"]
    assert fams("u8", "f16", 8192, 4096, 128) == ["stream"] * 3  # 32 MiB
    assert fams("u4", "bf16", 4096, 4096, 32) == ["stream"] * 3  # 128 tile groups
    assert fams("fp8", "f16", 5120, 6144, 128) == ["stream"] * 3  # 160 tile groups


def test_small_weights_take_the_streaming_family_at_every_m():
    """Up to N x K = 4 Mi elements with K <= 4096, the streaming family serves every M,
    with or without a workspace: up to M = 8 one persistent pass of eight rows (FP8
    codes; 4-bit on fp16, 8-bit and NVFP4 codes with K >= 2048), else the multi-pass
    kernel; past either bound, M >= 5 takes the matrix family, except FP8 at M = 5..8
    where the tile groups fill at most half the CUs."""
    for fmt, act, N, K, bs in (("u4", "f16", 1024, 2048, 32), ("u4", "f16", 2048, 2048, 32),
                               ("fp8", "f16", 1024, 4096, 128), ("u8", "f16", 2048, 2048, 128),
                               ("nvfp4", "bf16", 2048, 2048, 16), ("u4", "bf16", 1024, 2048, 32),
                               ("u4", "f16", 4096, 1024, 32), ("u8", "bf16", 1024, 4096, 128)):
        one_pass = fmt == "fp8" or (K >= 2048 and (fmt, act) != ("u4", "bf16"))
        for M in (5, 8, 12, 16):
            for ws in (False, True):
                p = _sel(fmt=fmt, act=act, N=N, K=K, block_size=bs, M=M, with_workspace=ws)
                assert p["family"] == "stream" and p["kparts"] == 1, (fmt, N, K, M, ws, p)
                if one_pass and M <= 8:
                    assert p["rows_per_pass"] == 8 and p["passes"] == 1 and p["variant"] & 1, (fmt, M, p)
                    assert p["waves_per_wg"] <= (8 if fmt in ("u4", "nvfp4") else 16), p
                else:
                    assert p["rows_per_pass"] == 4 and p["passes"] == (M + 3) // 4, (fmt, K, M, p)
    for fmt, act, N, K, bs in (("u4", "f16", 1536, 4096, 32), ("fp8", "f16", 2048, 4096, 128),
                               ("u4", "f16", 512, 8192, 32), ("fp8", "f16", 512, 8192, 128)):
        for M in (5, 8, 16):
            p = _sel(fmt=fmt, act=act, N=N, K=K, block_size=bs, M=M)
            if fmt == "fp8" and M <= 8:
                # 128 and 32 tile groups on 256 CUs: eight rows in one streaming pass
                assert p["family"] == "stream" and p["rows_per_pass"] == 8, (N, K, M, p)
            else:
                assert p["family"] == "mfma", (fmt, N, K, M, p)
    # FP8 5120 x 6144 (160 tile groups) and 8192 x 4096 (256) keep the matrix family
    for N, K in ((5120, 6144), (8192, 4096)):
        for M in (5, 8):
            assert _sel(fmt="fp8", act="f16", N=N, K=K, block_size=128, M=M)["family"] == "mfma"


def test_reduction_area_overlays_the_staged_rows_when_one_round_fits():
    """With one tile group per workgroup the K-split reduction area overlays the staged
    activations (LDS = the larger of the two); a persistent grid that walks several
    tile groups keeps them side by side."""
    # FP8 8192 x 4096, M = 16: 256 tile groups (K split 4) on 256 CUs; staged rows
    # 64 + 16 x (4096 + 8) x 2 bytes, reduction 8 waves x 4 row groups x 4 x 64 x 4
    p = _sel(fmt="fp8", act="f16", N=8192, K=4096, block_size=128, M=16)
    rows, red = 64 + 16 * 4104 * 2, 8 * 4 * 4 * 64 * 4
    assert rows + red > 160 * 1024
    assert p["family"] == "mfma" and p["ksplit"] == 4 and p["variant"] & 1 and p["grid"] == 256
    assert p["lds_bytes"] == max(rows, red)
    # with K parts (forced 2, one workgroup per tile group and part): overlaid, plus
    # the 16-byte flag; the longest part's rows are staged
    p = _sel(fmt="fp8", act="f16", N=8192, K=4096, block_size=128, M=16, flags=2 | (2 << 4), with_workspace=True)
    assert p["kparts"] == 2 and p["variant"] & 1
    assert p["lds_bytes"] == max(64 + 16 * 2056 * 2, red) + 16
    # a forced split 2 on the 4-bit lm_head at M = 8: 2374 tile groups, more than fit
    # at once, so the grid persists and the layout stays side by side
    p = _sel(M=8, flags=2 | (2 << 8))
    rows = 64 + 8 * (4096 + 8) * 2 + 4 * 32 * 2 * 16  # rows and activation sums
    assert p["ksplit"] == 2 and p["variant"] & 1 and not (p["variant"] & 2)
    assert p["lds_bytes"] == rows + 8 * 2 * 4 * 64 * 4
    assert p["grid"] == 256 * (160 * 1024 // p["lds_bytes"])


def test_two_k_parts_where_the_unsplit_rows_do_not_fit_in_lds():
    """With a workspace, where the unsplit plan's activation rows do not fit in LDS at
    this M, 2 K parts (the one choice of the K parts that depends on M): where the tile
    groups fill at most half the CUs, or all of them with 24 K steps or more per
    unsplit wave; never without a workspace, never when the part count is forced, and
    not where the rows fit."""
    kw = dict(fmt="fp8", act="f16", N=2048, K=8192, block_size=128)
    # 128 tile groups; M = 8: 8 x (8192 + 8) x 2 bytes of rows fit (staged, 1 part);
    # M = 12 and 16 do not: 2 parts, each staging half the K range
    for M, kp in ((5, 1), (8, 1), (12, 2), (16, 2)):
        p = _sel(**kw, M=M, with_workspace=True)
        assert p["kparts"] == kp and p["variant"] & 1, (M, p)
        assert _sel(**kw, M=M)["kparts"] == 1
    p = _sel(**kw, M=16, with_workspace=True)
    assert p["grid"] == 256 and p["workspace_bytes"] == 512 + 2 * 16 * 2048 * 4
    # a forced part count is taken as given
    assert _sel(**kw, M=16, flags=2 | (1 << 4), with_workspace=True)["kparts"] == 1
    # 4-bit 2048 x 16384: the rows do not fit from M = 5 on; at M = 12 and 16 not even
    # half of them do, and the 2 parts run with the activations in the ring
    for M, staged in ((5, True), (8, True), (12, False), (16, False)):
        p = _sel(fmt="u4", act="bf16", N=2048, K=16384, block_size=32, M=M, with_workspace=True)
        assert p["kparts"] == 2 and bool(p["variant"] & 1) == staged, (M, p)
    # past half the CUs, only while each unsplit wave walks 24 K steps or more: FP8
    # 5120 x 6144 (160 tile groups, 96 steps, split 4: 24 per wave) at M = 16; not at
    # M = 12, where the rows fit
    # M = 12, where the rows fit; at M = 16 the long-rows rule takes it instead: no split
    # inside a workgroup, 4 parts (40 unsplit tile groups: one round of 160 workgroups)
    kw = dict(fmt="fp8", act="f16", N=5120, K=6144, block_size=128, with_workspace=True)
    p = _sel(**kw, M=16)
    assert p["ksplit"] == 1 and p["kparts"] == 4 and p["variant"] & 1, p
    assert _sel(**kw, M=12)["kparts"] == 1 and _sel(**kw, M=12)["ksplit"] == 4
    # 8-bit 4096 x 8192 (256 tile groups, 128 steps, split 8: 16 per wave): not the
    # 2-part rule; long rows at M = 16 (32 unsplit groups: 8 parts)
    p = _sel(fmt="u8", act="f16", N=4096, K=8192, block_size=128, M=16, with_workspace=True)
    assert p["ksplit"] == 1 and p["kparts"] == 8 and p["variant"] & 1, p


def test_row_passes_where_the_rows_do_not_fit_and_there_are_no_k_parts():
    """Without K parts, more than 8 rows whose activations do not stage run as passes
    of 8 (one launch each), each staging its rows or taking the DMA ring, whatever the
    tile groups; a forced staging choice keeps one launch."""
    kw = dict(fmt="fp8", act="f16", N=2048, K=8192, block_size=128)
    for M, passes in ((8, 1), (9, 1), (12, 2), (13, 2), (16, 2)):
        p = _sel(**kw, M=M)
        assert p["passes"] == passes and p["variant"] & 1, (M, p)
        if passes > 1:
            # the passes are the matrix family's 8-row plan (8 rows alone take one
            # streaming pass of eight rows on this shape: 128 tile groups)
            assert p["rows_per_pass"] == 8 and p["kparts"] == 1 and p == _sel(**kw, M=8, flags=2) | {"passes": passes}
    assert _sel(**kw, M=8)["family"] == "stream" and _sel(**kw, M=9)["family"] == "mfma"
    # with a workspace: 2 K parts in one launch instead
    p = _sel(**kw, M=16, with_workspace=True)
    assert p["passes"] == 1 and p["kparts"] == 2
    # a forced part count of 1 with a workspace: passes again
    assert _sel(**kw, M=16, flags=1 << 4, with_workspace=True)["passes"] == 2
    # forced staging off: one unstaged launch
    p = _sel(**kw, M=16, flags=bqw.FLAG_STAGE_A_OFF)
    assert p["passes"] == 1 and p["rows_per_pass"] == 16 and not (p["variant"] & 1)
    # FP8 5120 x 6144 at M = 16 (160 tile groups, 24 K steps per wave): passes
    p = _sel(fmt="fp8", act="f16", N=5120, K=6144, block_size=128, M=16)
    assert p["passes"] == 2 and p["grid"] == 160
    # 8-bit 4096 x 8192 (16 K steps per wave; 2 K parts at a split of 8 lose here):
    # passes without a workspace (with one, the long-rows parts above)
    p = _sel(fmt="u8", act="f16", N=4096, K=8192, block_size=128, M=16)
    assert p["passes"] == 2 and p["kparts"] == 1 and p["variant"] & 1, p
    # the same at any number of tile groups: FP8 65536 x 8192 (512 groups) from M = 10
    kw8 = dict(fmt="fp8", act="f16", N=65536, K=8192, block_size=128)
    assert [_sel(**kw8, M=M)["passes"] for M in (9, 10, 16)] == [1, 2, 2]
    # where the 8-row plan is the DMA ring, the passes are ring launches: 4-bit on f16
    # 28672 x 5120 (224 tile groups) at M = 16
    kwr = dict(fmt="u4", act="f16", N=28672, K=5120, block_size=32)
    p = _sel(**kwr, M=16)
    assert p["passes"] == 2 and p["variant"] & 2 and p == _sel(**kwr, M=8) | {"passes": 2}, p
    # 4-bit 2048 x 16384: 8 rows do not fit either: one unstaged matrix launch (128 tile
    # groups: the streaming fallback is for a quarter of the CUs or fewer)
    kw = dict(fmt="u4", act="bf16", N=2048, K=16384, block_size=32)
    for M in (6, 16):
        p = _sel(**kw, M=M)
        assert p["family"] == "mfma" and p["passes"] == 1 and not (p["variant"] & 1), p
    # 4-bit 1024 x 16384 (64 tile groups): the streaming family from M = 6
    kw = dict(fmt="u4", act="f16", N=1024, K=16384, block_size=32)
    assert [_sel(**kw, M=M)["family"] for M in (5, 6, 16)] == ["mfma", "stream", "stream"]


def test_a_workspace_sized_for_sixteen_rows_serves_every_m():
    """The K parts may depend on M (2 parts where the rows do not fit), yet the
    workspace a plan needs never exceeds the one at M = 16."""
    for fmt, act, N, K, bs in [("fp8", "f16", 2048, 8192, 128), ("u4", "bf16", 2048, 16384, 32),
                               ("fp8", "f16", 5120, 6144, 128), ("fp8", "f16", 1024, 16384, 128),
                               ("u4", "bf16", 512, 8192, 32), ("u4", "bf16", 16384, 8192, 32)]:
        full = _sel(fmt=fmt, act=act, N=N, K=K, block_size=bs, M=16, with_workspace=True)["workspace_bytes"]
        for M in range(1, 17):
            p = _sel(fmt=fmt, act=act, N=N, K=K, block_size=bs, M=M, with_workspace=True)
            assert p["workspace_bytes"] <= full, (fmt, N, K, M, p, full)


def test_more_than_sixteen_rows_take_the_sixteen_row_plan_in_chunks():
    """M > 16 (up to 65536) runs as chunks of 16 rows with the plan for 16 rows; the
    reported passes count every chunk's passes, and the workspace is that of 16 rows."""
    shapes = [dict(), dict(fmt="fp8", act="f16", N=5120, K=6144, block_size=128),
              dict(fmt="u4", act="f16", N=1024, K=2048, block_size=32),
              dict(fmt="fp8", act="f16", N=1024, K=16384, block_size=128)]
    for kw in shapes:
        for ws in (False, True):
            p16 = _sel(**kw, M=16, with_workspace=ws)
            for M, chunks in ((17, 2), (32, 2), (33, 3), (100, 7), (65536, 4096)):
                p = _sel(**kw, M=M, with_workspace=ws)
                assert p == p16 | {"passes": p16["passes"] * chunks}, (kw, M, ws, p, p16)
    assert bqw.MAX_ROWS == 65536


def test_forced_k_parts_and_k_split_are_clamped():
    # 4 K steps (fp8, K = 256): 8 forced parts become 4, one step each
    p = _sel(fmt="fp8", act="f16", N=100, K=256, block_size=128, M=8, flags=2 | (4 << 4), with_workspace=True)
    assert p["kparts"] == 4 and p["grid"] % 4 == 0
    # forced parts on a wide N: exactly one workgroup per tile group and part, no ring
    p = _sel(M=4, flags=2 | (2 << 4), with_workspace=True)
    groups = (151936 // 16 + (8 // p["ksplit"]) - 1) // (8 // p["ksplit"])
    assert p["kparts"] == 2 and p["grid"] == 2 * groups and not (p["variant"] & 2)
    # the partial tiles are indexed with 32-bit offsets: kparts * 16 * N < 2^31
    p = _sel(N=1 << 24, M=1, flags=2 | (4 << 4), with_workspace=True)
    assert p["kparts"] == 4
    # a forced K split beyond the K steps falls to a power of two (whole tiles per
    # 8-wave workgroup): 3 steps of 4-bit codes (K = 384), forced 8 -> 2
    p = _sel(N=100, K=384, M=8, flags=2 | (8 << 8))
    assert p["ksplit"] == 2


def test_streaming_metadata_windows_where_they_fit():
    """Variant bit 3 (one metadata window per round) is taken for 8-bit codes where a
    round's scale and zero-point windows are whole dwords within 64 of them and the rows
    are whole dwords; the other formats keep the per-chunk loads, as does an odd block
    count, and flag bit 7 forces them."""
    u8 = dict(fmt="u8", act="f16", N=4096, K=4096, block_size=128)
    p = _sel(**u8)
    assert p["family"] == "stream" and p["variant"] & 8
    assert _sel(**dict(u8, block_size=32))["variant"] & 8
    assert _sel(**dict(u8, M=3, N=900))["variant"] & 8                   # several rows per pass
    assert not _sel(**dict(u8, K=128 * 33))["variant"] & 8               # 33 blocks: odd rows
    assert not _sel(**dict(u8, flags=bqw.FLAG_STREAM_META_CHUNK))["variant"] & 8
    assert not _sel()["variant"] & 8                                      # 4-bit lm_head
    assert not _sel(fmt="fp8", act="f16", N=5120, K=6144, block_size=128)["variant"] & 8


@pytest.mark.parametrize("cu", [80, 256, 304])
def test_one_row_workgroups_where_columns_fill_8_to_16_waves_per_cu(cu):
    """One row, one column per wave, columns for 8..16 waves per CU: 16-wave workgroups
    (at most one per CU), except for 8-bit codes, which take four 4-wave workgroups per CU and two
    chunks per lane per batch; a forced 16-wave flag still gives 16 waves."""
    for fmt, act, bs in (("u8", "f16", 128), ("u8", "bf16", 128), ("u4", "f16", 32), ("fp8", "f16", 128),
                         ("nvfp4", "bf16", 16)):
        N = 12 * cu  # 12 columns per CU
        p = _sel(fmt=fmt, act=act, N=N, K=4096, block_size=bs, M=1, cu_count=cu)
        assert p["family"] == "stream" and p["cols_per_wave"] == 1, p
        if fmt == "u8":
            assert p["waves_per_wg"] == 4 and p["grid"] == min(4 * cu, (N + 3) // 4) and (p["variant"] >> 1) & 3 == 2, p
            f = _sel(fmt=fmt, act=act, N=N, K=4096, block_size=bs, M=1, cu_count=cu, flags=bqw.FLAG_STREAM_WIDE_WG)
            assert f["waves_per_wg"] == 16, f
        else:
            assert p["waves_per_wg"] == 16 and p["grid"] == (N + 15) // 16, p


@pytest.mark.parametrize("cu", [80, 256, 304])
def test_dma_ring_band(cu):
    """The DMA ring takes a weight at every M up to 8 once its tile groups (8 tiles of
    16 columns, no K split) reach 3/4 of the CUs for 4-bit and NVFP4 codes, 7/8 for FP8
    and 8-bit codes, where eight staged rows fit next to its slots; such a weight takes
    no K split at any M (the split never depends on M), and 1-byte codes keep the
    streaming kernel at M = 2. Below the band the K split and the other families stay."""
    def shape(fmt, groups, K):
        return dict(fmt=fmt, act="f16", N=groups * 128, K=K, block_size=32 if fmt in ("u4",) else
                    (16 if fmt == "nvfp4" else 128), cu_count=cu)

    for fmt, frac in (("u4", (3, 4)), ("nvfp4", (3, 4)), ("fp8", (7, 8)), ("u8", (7, 8))):
        g_in = (cu * frac[0] + frac[1] - 1) // frac[1]  # the fewest groups in the band
        kw = shape(fmt, g_in, 2048)
        for M in range(2, 9):
            p = _sel(**kw, M=M)
            if fmt in ("fp8", "u8") and M == 2:
                assert p["family"] == "stream", (fmt, cu, p)
            else:
                assert p["family"] == "mfma" and p["variant"] & 2 and p["ksplit"] == 1, (fmt, cu, M, p)
                assert p["grid"] == min(g_in, cu)
        for M in range(9, 17):
            p = _sel(**kw, M=M)
            assert p["family"] == "mfma" and p["ksplit"] == 1 and not p["variant"] & 2, (fmt, cu, M, p)
        # one group fewer: no ring at M = 4 (a K split where it pays, or the streaming kernel)
        p = _sel(**shape(fmt, g_in - 1, 2048), M=4)
        assert not (p["family"] == "mfma" and p["variant"] & 2), (fmt, cu, p)
    # a K range whose eight rows do not fit next to the ring: the weight keeps its K split
    # at 3/4 of the CUs; from 7/8 of them 4-bit codes take the ring up to four rows and
    # no K split at any M, 1-byte codes keep theirs
    kw = dict(fmt="u4", act="bf16", N=24576 * cu // 256, K=8192, block_size=32, cu_count=cu)
    assert all(_sel(**kw, M=M)["ksplit"] > 1 for M in (4, 8, 16))
    g78 = (7 * cu + 7) // 8
    kw = dict(fmt="u4", act="bf16", N=g78 * 128, K=8192, block_size=32, cu_count=cu)
    for M in (2, 3, 4, 5, 8, 16):
        p = _sel(**kw, M=M)
        assert p["family"] == "mfma" and p["ksplit"] == 1 and bool(p["variant"] & 2) == (M <= 4), (cu, M, p)
    kw = dict(fmt="fp8", act="f16", N=g78 * 128, K=8192, block_size=128, cu_count=cu)
    assert all(_sel(**kw, M=M)["ksplit"] > 1 for M in (4, 8, 16))
    # NVFP4 at one row: the ring only where its groups outnumber the CUs
    kw = dict(fmt="nvfp4", act="bf16", K=2048, block_size=16, cu_count=cu)
    assert _sel(**kw, N=cu * 128, M=1)["family"] == "stream"
    assert _sel(**kw, N=(cu + 1) * 128, M=1)["variant"] & 2


def test_automatic_workspaces_fit_the_noalloc_array():
    """On 256 CUs every automatic plan of up to 16 rows needs at most the no-allocation
    entry point's array (16 MiB): the largest are the long-rows K parts over nearly
    32768 columns."""
    worst = 0
    for fmt, act, bs in [("u4", "bf16", 32), ("fp8", "f16", 128), ("u8", "f16", 128), ("nvfp4", "bf16", 16)]:
        for K in (4096, 16384, 20480, 32768, 65536):
            for N in (1024, 4096, 8192, 20480, 30720, 32256, 32768, 151936):
                p = _sel(fmt=fmt, act=act, N=N, K=K, block_size=bs, M=16, with_workspace=True)
                worst = max(worst, p["workspace_bytes"])
    assert 8 << 20 < worst <= bqw.NOALLOC_SCRATCH_BYTES == 16 << 20, worst
