"""qgemv_run_noalloc, the entry point that allocates nothing: the qgemv_run_ws plans and
kernels with the library's own device scratch array as the workspace.

Checked through the C ABI on the GPU: two calls in a row (the second with a smaller
input: fewer rows and a narrower weight) give the same bits as qgemv_run_ws with a
caller workspace, inside the oracle's bound; the shared array is reused between
handles; a plan whose workspace exceeds the array is rejected before any launch; and a
plan without K parts runs as qgemv_run does.
"""

import numpy as np
import pytest
import torch

import block_quantized_weight_amd as bqw
from block_quantized_weight_amd import synth

pytestmark = pytest.mark.gpu

from tests import gpu_util as gu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.require_gpu()


def _pair(prob, M, flags=0):
    """(qgemv_run_noalloc output, qgemv_run_ws output, plan) for the first M rows."""
    q, t = bqw.upload(prob, flags=flags)
    A = t["A"][:M].contiguous()
    Y1 = torch.full((M, prob.N), float("nan"), dtype=A.dtype, device="cuda")
    Y2 = torch.full((M, prob.N), float("nan"), dtype=A.dtype, device="cuda")
    q.run_noalloc(A, Y1, M=M)
    ws = gu.new_workspace(q, M)
    q.run(A, Y2, M=M, workspace=ws)
    torch.cuda.synchronize()
    plan = q.plan(M, with_workspace=True)
    q.close()
    return Y1.float().cpu().numpy().astype(np.float64), Y2.float().cpu().numpy().astype(np.float64), plan


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    big = synth.workload("fp8_m8_k16384_n1024")  # K parts across workgroups
    gu.say("[noalloc] fp8 1024x16384 M=8, then u4 512x8192 M=3")
    Y1, Y2, plan = _pair(big, 8)
    assert plan["kparts"] > 1 and 0 < plan["workspace_bytes"] <= bqw.NOALLOC_SCRATCH_BYTES, plan
    assert np.array_equal(Y1.view(np.int64), Y2.view(np.int64))
    ok, ratio, _, _ = gu.check_full(big, 8, Y1)
    assert ok, ratio
    small = synth.make_problem("u4", "bf16", 512, 8192, 32, 3, seed=5)
    Y1, Y2, plan = _pair(small, 3)
    assert plan["kparts"] > 1, plan
    assert np.array_equal(Y1.view(np.int64), Y2.view(np.int64))
    ok, ratio, _, _ = gu.check_full(small, 3, Y1, strict=False)
    assert ok, ratio


def test_noalloc_with_more_than_16_rows():
    prob = synth.make_problem("u8", "f16", 777, 2048, 64, 20, seed=6)
    Y1, Y2, plan = _pair(prob, 20)
    assert np.array_equal(Y1.view(np.int64), Y2.view(np.int64))
    ok, ratio, _, _ = gu.check_full(prob, 20, Y1)
    assert ok, ratio


def test_noalloc_rejects_a_plan_larger_than_its_array():
    # 8 forced K parts on 65536 columns: 8 x 16 x 65536 x 4 bytes of partials at M = 16,
    # 32 MiB, twice the array; the same handle at M = 1 needs 2 MiB and runs
    prob = synth.make_problem("fp8", "f16", 65536, 1024, 128, 16, seed=8)
    flags = 2 | (4 << 4)
    q, t = bqw.upload(prob, flags=flags)
    assert q.workspace_size(16) > bqw.NOALLOC_SCRATCH_BYTES >= q.workspace_size(1)
    Y = torch.zeros((16, prob.N), dtype=torch.float16, device="cuda")
    with pytest.raises(bqw.QGemvError) as e:
        q.run_noalloc(t["A"][:16].contiguous(), Y, M=16)
    assert e.value.status == bqw.QGEMV_E_SCRATCH
    torch.cuda.synchronize()
    assert bool((Y == 0).all().item())  # nothing was launched
    Y1 = torch.full((1, prob.N), float("nan"), dtype=torch.float16, device="cuda")
    q.run_noalloc(t["A"][:1].contiguous(), Y1, M=1)
    torch.cuda.synchronize()
    q.close()
    ok, ratio, _, _ = gu.check_full(prob, 1, Y1.float().cpu().numpy().astype(np.float64))
    assert ok, ratio
