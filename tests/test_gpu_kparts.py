"""GPU parity of qgemv_run_ws: the K range of a tile group split across workgroups,
fp32 partial tiles in a caller-owned workspace, and the last workgroup to finish
adding them in part order ("[CUDA] MatMul: add an opt-in split-K GEMV", Cross-block
reduction).

Same bar as the other parity tests (|y - y_ref| <= 1e-3 * sum|a*w| + 1e-3 against the
oracle). In addition: rows are bit-identical whatever tile carries them (with the part
count forced, across M too), the staged and unstaged activation paths agree bit for bit,
repeated runs are bitwise equal, one workspace serves several handles in turn, and
every completed run leaves the whole workspace zero.
"""

import numpy as np
import pytest
import torch

import block_quantized_weight_amd as bqw
from block_quantized_weight_amd import synth

pytestmark = pytest.mark.gpu

from tests import gpu_util as gu

KPFLAG = {1: 1, 2: 2, 4: 3, 8: 4}  # parts -> value of flag bits 4..6


def kp_flags(kp):
    return KPFLAG[kp] << bqw.FLAG_KPARTS_SHIFT


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.require_gpu()


@pytest.mark.parametrize("M", [5, 8])
def test_tall_k_fp8_with_automatic_k_parts(M):
    """FP8 1024 x 16384 (64 tile groups for 256 CUs): the automatic plan takes four K
    parts."""
    prob = synth.make_problem("fp8", "f16", 1024, 16384, 128, 8, seed=25)
    gu.say(f"[kparts] fp8 1024x16384 M={M}")
    Y, plan = gu.run_gpu(prob, M, ws=True)
    gu.say(f"   plan={plan}")
    assert plan["family"] == "mfma" and plan["kparts"] == 4, plan
    assert plan["ws_zero"]
    ok, ratio, _, _ = gu.check_full(prob, M, Y)
    gu.say(f"   max err/tol={ratio:.3e}")
    assert ok, ratio


@pytest.mark.parametrize("fmt,act,N,K,bs,M,staged", [("fp8", "f16", 2048, 8192, 128, 16, True),
                                                      ("u4", "bf16", 2048, 16384, 32, 8, True),
                                                      ("u4", "bf16", 2048, 16384, 32, 12, False)])
def test_two_automatic_k_parts_where_the_unsplit_rows_do_not_fit(fmt, act, N, K, bs, M, staged):
    """Where the unsplit plan's activation rows do not fit in LDS at this M (128 tile
    groups, too few unsplit groups for the long-rows rule), the automatic plan takes 2 parts;
    sampled outputs against the oracle, and bit for bit the run with 2 parts forced."""
    prob = synth.make_problem(fmt, act, N, K, bs, M, seed=26)
    gu.say(f"[kparts] {fmt} {N}x{K} M={M} automatic 2 parts")
    Y, plan = gu.run_gpu(prob, M, ws=True)
    assert plan["family"] == "mfma" and plan["kparts"] == 2 and bool(plan["variant"] & 1) == staged, plan
    assert plan["ws_zero"]
    ok, ratio, _, _ = gu.check_full(prob, M, Y)
    assert ok, ratio
    Yf, pf = gu.run_gpu(prob, M, flags=2 | kp_flags(2), ws=True)
    assert pf["kparts"] == 2 and pf["ksplit"] == plan["ksplit"]
    assert np.array_equal(Y.view(np.int64), Yf.view(np.int64))


@pytest.mark.parametrize("fmt,act,N,K,bs,M,kp", [("u4", "bf16", 4096, 14336, 32, 8, 8),
                                                 ("u4", "bf16", 4096, 14336, 32, 16, 8),
                                                 ("fp8", "f16", 8192, 28672, 128, 4, 4),
                                                 ("nvfp4", "bf16", 8192, 28672, 16, 16, 8),
                                                 ("fp8", "f16", 5120, 6144, 128, 16, 4),
                                                 ("u8", "f16", 4096, 8192, 128, 16, 8),
                                                 ("u4", "bf16", 10240, 8192, 128, 12, 2)])
def test_long_rows_take_k_parts_without_an_in_workgroup_split(fmt, act, N, K, bs, M, kp):
    """Rows of the whole K that do not stage at this M, with 32 to 80 unsplit tile
    groups: no K split inside a workgroup, the most parts that keep one round of
    workgroups, more where the rows need them to stage. Sampled
    outputs against the oracle, the workspace left zero, and bit for bit the run with
    the same split and part count forced."""
    prob = synth.make_problem(fmt, act, N, K, bs, M, seed=27)
    gu.say(f"[kparts] long rows {fmt} {N}x{K} M={M}")
    Y, plan = gu.run_gpu(prob, M, ws=True)
    gu.say(f"   plan={plan}")
    assert plan["family"] == "mfma" and plan["ksplit"] == 1 and plan["kparts"] == kp and plan["variant"] & 1, plan
    assert plan["ws_zero"]
    ok, ratio = gu.check_points(prob, M, Y, count=4000, seed=M)
    gu.say(f"   max err/tol={ratio:.3e}")
    assert ok, ratio
    Yf, pf = gu.run_gpu(prob, M, flags=2 | (1 << 8) | kp_flags(kp), ws=True)
    assert pf["kparts"] == kp and pf["ksplit"] == 1
    assert np.array_equal(Y.view(np.int64), Yf.view(np.int64))


def test_more_than_sixteen_rows_share_the_workspace_chunk_by_chunk():
    """M = 20 with K parts (FP8 1024 x 16384, 4 parts): chunks of 16 and 4 rows run
    through the same workspace in turn, which ends all zero; outputs against the
    oracle, and rows 16..19 bit for bit a 4-row call held to the matrix family (on its
    own, 4 rows of 1-byte codes take the streaming family)."""
    prob = synth.make_problem("fp8", "f16", 1024, 16384, 128, 20, seed=29)
    gu.say("[kparts] fp8 1024x16384 M=20 in chunks")
    Y, plan = gu.run_gpu(prob, 20, ws=True)
    assert plan["kparts"] == 4 and plan["ws_zero"], plan
    ok, ratio, _, _ = gu.check_full(prob, 20, Y)
    assert ok, ratio
    Y4, p4 = gu.run_gpu(prob, 4, flags=2, ws=True, A=prob.A[16:20])
    assert p4["kparts"] == 4 and p4["ksplit"] == plan["ksplit"]
    assert np.array_equal(Y[16:20].view(np.int64), Y4.view(np.int64))


def test_fp8_projection_with_forced_k_parts():
    """The FP8 5120 x 6144 workload at M = 8 in two forced parts (the automatic plan
    keeps it whole)."""
    prob = synth.workload("fp8_k6144_n5120")
    Y, plan = gu.run_gpu(prob, 8, flags=2 | kp_flags(2), ws=True)
    assert plan["kparts"] == 2 and plan["ws_zero"], plan
    ok, ratio, _, _ = gu.check_full(prob, 8, Y)
    assert ok, ratio


def test_u8_projection_with_k_parts_and_bias():
    """The 8-bit 4096 x 4096 weight of the M = 1 workload at M = 8 in two forced K
    parts, with the fused bias added by the last workgroup."""
    prob = synth.make_problem("u8", "f16", 4096, 4096, 128, 8, seed=1, zp_range=(96, 160), scale_sigma=0.004,
                              with_bias=True)
    gu.say("[kparts] u8 4096x4096 M=8 bias")
    Y, plan = gu.run_gpu(prob, 8, flags=2 | kp_flags(2), ws=True)
    assert plan["kparts"] == 2 and plan["ws_zero"], plan
    ok, ratio, _, _ = gu.check_full(prob, 8, Y)
    assert ok, ratio


@pytest.mark.parametrize("fmt,act,bs", [("u4", "bf16", 32), ("u4", "f16", 16), ("u8", "f16", 128),
                                         ("fp8", "f16", 128), ("fp8", "bf16", 64), ("nvfp4", "bf16", 16)])
@pytest.mark.parametrize("kp", [2, 4, 8])
def test_forced_k_parts_every_format(fmt, act, bs, kp):
    """N = 777 (a ragged last tile) and K = 896: 7 K steps for 4-bit codes (parts of
    one or two steps, waves with no step of their own) and 14 for 8-bit ones. Checked
    against the oracle, across M (rows moved between tiles), and staged against
    unstaged activations."""
    K = 896
    steps = K // (4 * (32 if fmt in ("u4", "nvfp4") else 16))
    prob = synth.make_problem(fmt, act, 777, K, bs, 16, seed=23)
    gu.say(f"[kparts-forced] {fmt}/{act} bs{bs} kp={kp}")
    base = 2 | kp_flags(kp)
    Y16, p16 = gu.run_gpu(prob, 16, flags=base | bqw.FLAG_STAGE_A_ON, ws=True)
    want = kp
    while want > steps:
        want //= 2
    assert p16["kparts"] == want and (p16["variant"] & 1) and p16["ws_zero"], p16
    ok, ratio, _, _ = gu.check_full(prob, 16, Y16, strict=False)
    assert ok, ratio
    Yu, pu = gu.run_gpu(prob, 16, flags=base | bqw.FLAG_STAGE_A_OFF, ws=True)
    assert pu["kparts"] == want and not (pu["variant"] & 1) and pu["ksplit"] == p16["ksplit"], pu
    assert np.array_equal(Yu.view(np.int64), Y16.view(np.int64))
    for M in (1, 5, 13):
        A = np.ascontiguousarray(prob.A[16 - M:])
        Ym, pm = gu.run_gpu(prob, M, flags=base | bqw.FLAG_STAGE_A_ON, A=A, ws=True)
        assert pm["kparts"] == want and pm["ws_zero"], pm
        assert np.array_equal(Ym.view(np.int64), Y16[16 - M:].view(np.int64)), M


@pytest.mark.parametrize("ks", [1, 2, 8])
def test_forced_k_parts_with_every_k_split(ks):
    """K parts on top of each K split inside the workgroup (4-bit codes, K = 4096: 32
    steps, 4 parts of 8)."""
    prob = synth.make_problem("u4", "bf16", 300, 4096, 32, 6, seed=24)
    Y, plan = gu.run_gpu(prob, 6, flags=2 | kp_flags(4) | (ks << bqw.FLAG_KSPLIT_SHIFT), ws=True)
    assert plan["kparts"] == 4 and plan["ksplit"] == ks and plan["ws_zero"], plan
    ok, ratio, _, _ = gu.check_full(prob, 6, Y, strict=False)
    assert ok, (ks, ratio)


def test_repeated_runs_and_shared_workspace():
    """Three rounds of two handles, alternating on one workspace whose regions overlap
    (one plan's partials lie over the other's counters): each handle's output is
    bitwise the same every round, and the workspace ends all zero."""
    p1 = synth.workload("fp8_k6144_n5120")
    p2 = synth.make_problem("u4", "f16", 1000, 4096, 32, 8, seed=5)
    q1, t1 = bqw.upload(p1, flags=2 | kp_flags(2))
    q2, t2 = bqw.upload(p2, flags=2 | kp_flags(4))
    need = max(q1.workspace_size(8), q2.workspace_size(8))
    assert q1.plan(8, with_workspace=True)["kparts"] == 2 and q2.plan(8, with_workspace=True)["kparts"] == 4
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    A1, A2 = t1["A"][:8].contiguous(), t2["A"][:8].contiguous()
    outs1, outs2 = [], []
    for _ in range(3):
        Y1 = torch.full((8, p1.N), float("nan"), dtype=A1.dtype, device="cuda")
        Y2 = torch.full((8, p2.N), float("nan"), dtype=A2.dtype, device="cuda")
        q1.run(A1, Y1, M=8, workspace=ws)
        q2.run(A2, Y2, M=8, workspace=ws)
        torch.cuda.synchronize()
        outs1.append(Y1.cpu())
        outs2.append(Y2.cpu())
    for o in outs1[1:]:
        assert torch.equal(o.view(torch.int16), outs1[0].view(torch.int16))
    for o in outs2[1:]:
        assert torch.equal(o.view(torch.int16), outs2[0].view(torch.int16))
    # the u4 plan's partials lie over the fp8 plan's counters: both are zero at rest
    assert bool((ws == 0).all().item())
    ok, ratio, _, _ = gu.check_full(p1, 8, outs1[0].float().numpy().astype(np.float64))
    assert ok, ratio
    ok, ratio, _, _ = gu.check_full(p2, 8, outs2[0].float().numpy().astype(np.float64), strict=False)
    assert ok, ratio
    q1.close()
    q2.close()


def test_workspace_is_checked_before_launch():
    prob = synth.workload("fp8_k6144_n5120")
    q, t = bqw.upload(prob, flags=2 | kp_flags(2))
    A = t["A"][:8].contiguous()
    Y = torch.zeros((8, prob.N), dtype=A.dtype, device="cuda")
    need = q.workspace_size(8)
    assert 0 < need <= q.workspace_size(16)
    ws = torch.zeros(need + 512, dtype=torch.uint8, device="cuda")
    for kw in (dict(workspace_bytes=0), dict(workspace=ws, workspace_bytes=need - 4),
               dict(workspace=ws[1:], workspace_bytes=need)):
        with pytest.raises(bqw.QGemvError) as e:
            q.run(A, Y, M=8, **kw)
        assert e.value.status == bqw.QGEMV_E_WORKSPACE
    torch.cuda.synchronize()
    assert not Y.any().item()  # nothing was launched
    q.close()
    # a plan without K parts (the automatic plan of this shape) needs no workspace
    q, t = bqw.upload(prob)
    assert q.workspace_size(8) == 0
    Y = torch.zeros((8, prob.N), dtype=A.dtype, device="cuda")
    q.run(A, Y, M=8, workspace_bytes=0)
    torch.cuda.synchronize()
    ok, ratio, _, _ = gu.check_full(prob, 8, Y.float().cpu().numpy().astype(np.float64))
    assert ok, ratio
    q.close()


def test_k_parts_replay_in_a_captured_graph():
    """qgemv_run_ws needs no memset (every run leaves the workspace zero), so it can be
    captured in a graph. Four replays, with eager work on the stream between them, must
    each give the eager result bit for bit and leave the workspace zero."""
    prob = synth.workload("fp8_m8_k16384_n1024")
    q, t = bqw.upload(prob)
    assert q.plan(8, with_workspace=True)["kparts"] == 4
    A = t["A"][:8].contiguous()
    ws = torch.zeros(q.workspace_size(8), dtype=torch.uint8, device="cuda")
    Y = torch.zeros((8, prob.N), dtype=A.dtype, device="cuda")
    q.run(A, Y, M=8, workspace=ws)
    torch.cuda.synchronize()
    Y_eager = Y.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q.run(A, Y, M=8, workspace=ws)  # a run on the capture's side of the allocator first
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.run(A, Y, M=8, workspace=ws)
    x = torch.randn(256, 256, device="cuda")
    for _ in range(4):
        Y.fill_(float("nan"))
        x = (x @ x.T).tanh()  # eager work between the replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Y_eager.view(torch.int16))
        assert bool((ws == 0).all().item())
    ok, ratio, _, _ = gu.check_full(prob, 8, Y.float().cpu().numpy().astype(np.float64))
    assert ok, ratio
    del g
    q.close()


def test_one_handle_on_two_streams_with_their_own_workspaces():
    """The handle is immutable, so runs on two streams may overlap as long as each has
    its own workspace: both streams' outputs equal the serial result bit for bit, and
    both workspaces end zero."""
    prob = synth.workload("fp8_m8_k16384_n1024")
    q, t = bqw.upload(prob)
    A = t["A"][:8].contiguous()
    need = q.workspace_size(8)
    ref = torch.zeros((8, prob.N), dtype=A.dtype, device="cuda")
    q.run(A, ref, M=8, workspace=torch.zeros(need, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [torch.zeros(need, dtype=torch.uint8, device="cuda") for _ in streams]
    outs = [[torch.full((8, prob.N), float("nan"), dtype=A.dtype, device="cuda") for _ in range(10)] for _ in streams]
    torch.cuda.synchronize()
    for i in range(10):
        for s, ws, ys in zip(streams, wss, outs):
            with torch.cuda.stream(s):
                q.run(A, ys[i], M=8, workspace=ws)
    torch.cuda.synchronize()
    for ys in outs:
        for y in ys:
            assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
    for ws in wss:
        assert bool((ws == 0).all().item())
    q.close()
