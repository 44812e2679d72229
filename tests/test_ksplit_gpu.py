"""GPU parity of the key-split prefill (256-wide 16-bit heads on grids too small
for 32-row tiles) against the CPU float64 oracle, every output element.

The kernel's workgroup holds 16 query rows of up to four heads and splits each
64-key step between two lanes of wavefronts, which merge at the end. The cases
cover one, two and four heads per workgroup (64, 32 and 16 rows of a head),
key counts on both sides of the 32-key lane and 64-key step edges, causal calls
whose early rows see no key, windows, boolean masks, sinks, and batches."""
import numpy as np
import pytest

from oracle import attention as orc
from scaled_dot_product_06_amd import inputs as gen
from tests.gpu_util import assert_parity, from_device, oracle_rows, run_gpu, say

pytestmark = pytest.mark.gpu

F16, BF16 = gen.F16, gen.BF16
DT = {"f16": F16, "bf16": BF16}


def _plan(p, window=0):
    import scaled_dot_product_06_amd as sd
    if window:
        return sd.sdpa_plan_windowed(*p.shape_args(), window, p.sinks is not None, p.dtype)
    return sd.sdpa_plan(*p.shape_args(), p.mask_kind, p.mask is not None, p.sinks is not None, p.dtype)


def _check(p, what):
    plan = _plan(p)
    assert (plan["rows_per_wave"], plan["splits"], plan["waves"]) == (16, 2, 8), plan
    say(f"{what}: {p!r}")
    got = from_device(run_gpu(p), p.dtype)
    want = oracle_rows(p)
    assert_parity(p, got, want, what)


# (B, Hq, Hkv, Lq): four heads per workgroup (group 8 and 4), two (group 2) and one (group 1)
HEAD_SHAPES = [(1, 16, 2, 70), (2, 8, 2, 33), (1, 4, 2, 100), (1, 2, 2, 77)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", HEAD_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_heads_per_workgroup_every_mask(shape, dtype):
    B, Hq, Hkv, Lq = shape
    for mask_kind in (0, 1, 2):
        for sinks in (False, True):
            p = gen.make_problem(8100 + Hq * 7 + Lq + mask_kind * 3 + sinks, B, Hq, Hkv, Lq, 157, 256, 256, DT[dtype],
                                 mask_kind, sinks=sinks)
            _check(p, f"ksplit heads mask={mask_kind} sinks={sinks}")


@pytest.mark.parametrize("Lk", [1, 2, 31, 32, 33, 63, 64, 65, 95, 96, 97, 128, 129, 1801])
def test_key_counts_across_lane_and_step_edges(Lk):
    for mask_kind in (0, 1, 2):
        p = gen.make_problem(8200 + Lk + mask_kind, 1, 8, 2, 45, Lk, 256, 256, BF16, mask_kind, sinks=True)
        _check(p, f"ksplit Lk={Lk} mask={mask_kind}")


@pytest.mark.parametrize("Lq,Lk", [(100, 40), (300, 64), (17, 1000), (1024, 1801)])
def test_causal_rows_that_see_few_or_no_keys(Lq, Lk):
    # Lq > Lk: the first Lq - Lk rows see no key (zeros, sink or not); the rest see a
    # few keys, all in the first step's first lane
    for sinks in (False, True):
        p = gen.make_problem(8300 + Lq + Lk + sinks, 1, 8, 2, Lq, Lk, 256, 256, F16, 1, sinks=sinks)
        _check(p, f"ksplit causal Lq={Lq} Lk={Lk} sinks={sinks}")


@pytest.mark.parametrize("window", [1, 20, 64, 100, 700])
def test_windows(window):
    import torch
    from scaled_dot_product_06_amd import attention
    from tests.gpu_util import device_inputs
    p = gen.make_problem(8400 + window, 1, 8, 2, 200, 900, 256, 256, BF16, 1, sinks=True)
    plan = _plan(p, window)
    assert (plan["rows_per_wave"], plan["splits"]) == (16, 2)
    q, k, v, _, s = device_inputs(p)
    got = from_device(attention(q, k, v, p.scale, 1, None, s, window=window), p.dtype)
    torch.cuda.synchronize()
    qw, kw, vw, _, sw = p.widened()
    want = orc.sdpa(qw, kw, vw, p.scale, 1, None, sw, window=window)
    assert_parity(p, got, want, f"ksplit window={window}")


def test_peaked_scores_across_both_lanes():
    # scale 1.0: each row follows its few top keys, which fall in either lane of any
    # step, so the merge's weights are of order one and a wrong merge shows
    p = gen.make_problem(8500, 1, 16, 2, 256, 1801, 256, 256, F16, 2, sinks=True, scale=1.0)
    _check(p, "ksplit peaked bool mask")
    p = gen.make_problem(8501, 1, 8, 2, 130, 700, 256, 256, BF16, 1, sinks=False, scale=1.0)
    _check(p, "ksplit peaked causal")


def test_batch_items_equal_each_item_alone():
    p = gen.make_problem(8600, 3, 16, 2, 90, 333, 256, 256, BF16, 2, sinks=True)
    plan = _plan(p)
    assert plan["splits"] == 2
    whole = from_device(run_gpu(p), BF16)
    for b in range(p.B):
        pb = gen.Problem(1, p.Hq, p.Hkv, p.Lq, p.Lk, p.D, p.Dv, BF16, p.mask_kind, p.scale, p.q[b:b + 1],
                         p.k[b:b + 1], p.v[b:b + 1], p.mask, p.sinks)
        alone = from_device(run_gpu(pb), BF16)
        assert np.array_equal(whole[b:b + 1], alone), f"batch item {b} differs"
