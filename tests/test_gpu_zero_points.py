"""Zero points at full code range: blocks whose codes all equal their zero point.

A block whose codes all sit at its zero point dequantizes to zero (all-zero blocks of a
pruned or padded weight quantize that way). With every block so, every output is 0 and
the bound is the absolute 1e-3; with 90% of the blocks so, the outputs are sums over the
other 10%. The activations are large where this is hardest for a kernel that would add
an offset to the codes and take it back out of the block sum: N(0, 16), N(0, 64), and
single large values (+-8192) alone or on top of N(0, 1).

The pages form (q - zp) exactly before the multiply ("[CUDA] MatMulNBits 8-bit: wide fp16
M=1 kernel", Description). Every decode that does so here (4- and 8-bit codes on fp16,
8-bit codes on bf16) must give exactly 0 where every block is at its zero point, in
every kernel family. 4-bit codes on bf16 decode the bare codes and take -z * sum(a) in
fp32 (there is no packed bf16 subtract on gfx950); they must stay inside the bound.
Every output is compared with the oracle.
"""

import numpy as np
import pytest

import block_quantized_weight_amd as bqw
from block_quantized_weight_amd import synth

pytestmark = pytest.mark.gpu

from tests import gpu_util as gu

RING_OFF = bqw.FLAG_RING_OFF
CONFIGS = {
    # name: (flags, M, workspace)
    "auto_m4": (0, 4, False),
    "stream_m1": (1, 1, False),
    "stream_rows_m4": (1, 4, False),
    "stream_classic_m4": (1 | bqw.FLAG_STREAM_CLASSIC, 4, False),
    "mfma_staged_m4": (2 | bqw.FLAG_STAGE_A_ON | RING_OFF, 4, False),
    "mfma_unstaged_m4": (2 | bqw.FLAG_STAGE_A_OFF | RING_OFF, 4, False),
    "mfma_dma_ring_m4": (2 | bqw.FLAG_RING_ON | (1 << 8), 4, False),
    "mfma_kparts_m4": (2 | (2 << 4), 4, True),
    "generic_m4": (3, 4, False),
}
CASES = [("u4", "f16", 32), ("u4", "bf16", 32), ("u4", "f16", 16), ("u4", "bf16", 16), ("u8", "f16", 128),
         ("u8", "bf16", 128), ("u8", "bf16", 32)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.require_gpu()


def exact_decode(fmt, act):
    return not (fmt == "u4" and act == "bf16")


@pytest.mark.parametrize("frac", [1.0, 0.9])
@pytest.mark.parametrize("config", sorted(CONFIGS))
@pytest.mark.parametrize("fmt,act,bs", CASES)
def test_codes_at_their_zero_points(fmt, act, bs, config, frac):
    flags, M, ws = CONFIGS[config]
    prob = synth.make_zero_point_problem(fmt, act, 300, 4096, bs, seed=11 + bs, frac=frac)
    gu.say(f"[zero points] {fmt}/{act} bs={bs} {config} frac={frac}")
    outs = []
    if M == 1:
        # the one-row kernel, once per activation row
        for r in range(prob.A.shape[0]):
            Y, plan = gu.run_gpu(prob, 1, flags=flags, A=prob.A[r:r + 1], ws=ws)
            outs.append(Y[0])
        Y = np.stack(outs)
    else:
        Y, plan = gu.run_gpu(prob, M, flags=flags, ws=ws)
    if flags & 0xF:
        assert plan["family"] == {1: "stream", 2: "mfma", 3: "generic"}[flags & 0xF], plan
    if config == "mfma_dma_ring_m4":
        assert plan["variant"] & 2, plan
    if config == "mfma_kparts_m4":
        assert plan["kparts"] == 2 and plan["ws_zero"], plan
    Mr = prob.A.shape[0]
    ok, ratio, Yr, S = gu.check_full(prob, Mr, Y, strict=False)
    gu.say(f"   plan={plan} max err/tol={ratio:.3e}")
    assert ok, (fmt, act, bs, config, frac, ratio, plan)
    if frac == 1.0:
        assert np.all(Yr == 0.0) and np.all(S == 0.0)
        if exact_decode(fmt, act):
            # (q - z) formed exactly: nothing but exact zeros is summed
            assert np.all(Y == 0.0), (config, np.abs(Y).max())
