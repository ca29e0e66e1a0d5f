"""The tuner's candidate list on the host (no GPU): qgemv_tune_candidates.

The online per-shape choice that the pages' batched small-M review asks for ("[CUDA]
Batched small-M GEMV for MatMulNBits (4-bit/8-bit)", review: an online profiler in
place of thresholds tuned on one machine) may only pick launches that give the
automatic plan's bits. Those are the plans with the automatic plan's kernel family, K
split and K parts: those three fix the order of every fp32 sum, and the GPU tests show
each other choice (columns per wave, batch depth, workgroup size, grid, staging, ring)
bit-identical. Checked here as pure predicates at fixed compute-unit counts (80, 256
and 304), as the pages test their occupancy window ("[CUDA] Pin FP8 GEMV residency for
grids just past two blocks per SM", Tests).
"""

import ctypes

import pytest

import block_quantized_weight_amd as bqw

SHAPES = [  # fmt, act, N, K, bs
    ("u4", "bf16", 151936, 4096, 32), ("fp8", "f16", 5120, 6144, 128), ("u8", "f16", 4096, 4096, 128),
    ("nvfp4", "bf16", 248320, 2048, 16), ("nvfp4", "bf16", 2048, 2048, 16), ("u4", "bf16", 1024, 2048, 32),
    ("fp8", "f16", 1024, 16384, 128), ("u4", "f16", 777, 896, 16), ("u8", "bf16", 333, 128 * 37, 128),
    ("fp8", "f16", 100, 256, 128),
]

KEY = ("family", "rows_per_pass", "passes", "cols_per_wave", "ksplit", "waves_per_wg", "grid", "lds_bytes",
       "variant", "kparts", "workspace_bytes")


@pytest.mark.parametrize("cu", [80, 256, 304])
@pytest.mark.parametrize("fmt,act,N,K,bs", SHAPES)
def test_candidates_keep_the_automatic_sum_order(fmt, act, N, K, bs, cu):
    for M in (1, 2, 3, 4, 5, 8, 12, 16):
        for ws in (False, True):
            auto = bqw.select(fmt, act, N, K, bs, M, cu_count=cu, with_workspace=ws)
            cands = bqw.tune_candidates(fmt, act, N, K, bs, M, cu_count=cu, with_workspace=ws)
            assert cands[0] == 0 and 1 <= len(cands) <= bqw.TUNE_MAX_CANDIDATES, (M, ws, cands)
            seen = set()
            for f in cands:
                p = bqw.select(fmt, act, N, K, bs, M, cu_count=cu, flags=f, with_workspace=ws)
                assert (p["family"], p["ksplit"], p["kparts"]) == (auto["family"], auto["ksplit"], auto["kparts"]), \
                    (M, ws, hex(f), p, auto)
                key = tuple(p[k] for k in KEY) + (bool(f & bqw.FLAG_NO_RESIDENCY_FIT),)
                assert key not in seen, (M, ws, hex(f))  # one flag set per distinct launch
                seen.add(key)
                # the residency bit is listed only for persistent grids (it changes
                # nothing elsewhere)
                if f & bqw.FLAG_NO_RESIDENCY_FIT:
                    assert p["kparts"] == 1 and (p["family"] != "stream" or p["variant"] & 1), (hex(f), p)


def test_each_dimension_is_tried_where_it_can_matter():
    # the 4-bit lm_head at M = 1 (persistent streaming kernel): every batch depth,
    # columns per wave and the classic kernel are among the candidates
    c = bqw.tune_candidates("u4", "bf16", 151936, 4096, 32, 1)
    plans = [bqw.select("u4", "bf16", 151936, 4096, 32, 1, flags=f) for f in c]
    assert {p["cols_per_wave"] for p in plans} >= {1, 2, 4}
    assert {p["variant"] & 1 for p in plans} == {0, 1}
    assert {(p["variant"] >> 1) & 3 for p in plans if p["variant"] & 1} == {0, 2, 3}  # 4, 2 and 3 chunks
    # FP8 5120 x 6144 at M = 4: 4-, 8-, 12- and 16-wave workgroups
    c = bqw.tune_candidates("fp8", "f16", 5120, 6144, 128, 4)
    assert {bqw.select("fp8", "f16", 5120, 6144, 128, 4, flags=f)["waves_per_wg"] for f in c} >= {4, 8, 12, 16}
    # matrix family: the register ring at both depths and the LDS DMA ring
    c = bqw.tune_candidates("u4", "bf16", 151936, 4096, 32, 8)
    v = {bqw.select("u4", "bf16", 151936, 4096, 32, 8, flags=f)["variant"] & 0xA for f in c}
    assert v >= {0, 2, 8}, v
    # 8-bit codes: per-chunk metadata loads against the one-window form
    c = bqw.tune_candidates("u8", "f16", 4096, 4096, 128, 1)
    assert any(f & bqw.FLAG_STREAM_META_CHUNK for f in c) and any(not f & bqw.FLAG_STREAM_META_CHUNK for f in c)


def test_dimensions_fixed_by_the_descriptor_are_left_alone():
    fixed = (2 << bqw.FLAG_STREAM_CPW_SHIFT) | (3 << bqw.FLAG_STREAM_UNR_SHIFT)
    c = bqw.tune_candidates("u4", "bf16", 151936, 4096, 32, 1, flags=fixed)
    mask = (3 << bqw.FLAG_STREAM_CPW_SHIFT) | (3 << bqw.FLAG_STREAM_UNR_SHIFT)
    assert len(c) > 1 and all(f & mask == 0 for f in c)
    for f in c:
        p = bqw.select("u4", "bf16", 151936, 4096, 32, 1, flags=fixed | f)
        assert p["cols_per_wave"] == 2 and (p["variant"] >> 1) & 3 == 0, (hex(f), p)
    # a forced family and K split keep their values too
    c = bqw.tune_candidates("fp8", "f16", 5120, 6144, 128, 8, flags=2 | (8 << bqw.FLAG_KSPLIT_SHIFT))
    for f in c:
        p = bqw.select("fp8", "f16", 5120, 6144, 128, 8, flags=2 | (8 << bqw.FLAG_KSPLIT_SHIFT) | f)
        assert p["family"] == "mfma" and p["ksplit"] == 8


def test_invalid_requests():
    L = bqw.lib()
    d = bqw.make_desc("u4", "bf16", 1024, 2048, 32, 0x1000, 0x1000)
    buf = (ctypes.c_uint32 * 4)()
    n = ctypes.c_int()
    assert L.qgemv_tune_candidates(ctypes.byref(d), 0, 256, 0, buf, 4, ctypes.byref(n)) == 2
    assert L.qgemv_tune_candidates(ctypes.byref(d), 17, 256, 0, buf, 4, ctypes.byref(n)) == 2
    assert L.qgemv_tune_candidates(ctypes.byref(d), 1, 0, 0, buf, 4, ctypes.byref(n)) == 7
    assert L.qgemv_tune_candidates(ctypes.byref(d), 1, 256, 0, buf, 0, ctypes.byref(n)) == 7
    assert L.qgemv_tune_candidates(None, 1, 256, 0, buf, 4, ctypes.byref(n)) == 1
    assert L.qgemv_tune_candidates(ctypes.byref(d), 1, 256, 0, None, 4, ctypes.byref(n)) == 1
    # a short buffer takes the first entries
    assert L.qgemv_tune_candidates(ctypes.byref(d), 1, 256, 0, buf, 4, ctypes.byref(n)) == 0
    assert n.value == 4 and buf[0] == 0
    # the handle-side call validates before touching any device
    assert L.qgemv_tune(None, None, None, 1, 0, None, 0, 0, 0, None, None) == 1
