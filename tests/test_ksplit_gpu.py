"""GPU parity of the key-split prefill (every 16-bit call with heads of 192 or 256
columns, (192,192), (192,128) and (256,256); 128-wide calls with an additive mask;
calls with narrower heads, (64,64), (80,80), (96,96), (128,128) and (96,64), on small
grids) against the CPU float64 oracle, every output element.

The kernel's workgroup holds 16 query rows of up to four heads and splits each
64-key step between two lanes of wavefronts, which merge at the end. The cases
cover one, two and four heads per workgroup (64, 32 and 16 rows of a head),
key counts on both sides of the 32-key lane and 64-key step edges, causal calls
whose early rows see no key, windows, boolean and additive masks, sinks, and
batches."""
import numpy as np
import pytest

from oracle import attention as orc
from scaled_dot_product_06_amd import inputs as gen
from tests.gpu_util import assert_parity, from_device, oracle_rows, run_gpu, say

pytestmark = pytest.mark.gpu

F16, BF16 = gen.F16, gen.BF16
DT = {"f16": F16, "bf16": BF16}
# head pairs (D, Dv) the key-split kernel is built for
WIDTHS = [(64, 64), (80, 80), (96, 96), (128, 128), (96, 64), (192, 192), (192, 128), (256, 256)]
PAIR_IDS = ["x".join(map(str, w)) for w in WIDTHS]


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


@pytest.mark.parametrize("D,Dv", WIDTHS, ids=PAIR_IDS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("shape", HEAD_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_heads_per_workgroup_every_mask(shape, dtype, D, Dv):
    B, Hq, Hkv, Lq = shape
    for mask_kind in (0, 1, 2):
        for sinks in (False, True):
            p = gen.make_problem(8100 + Hq * 7 + Lq + mask_kind * 3 + sinks + D, B, Hq, Hkv, Lq, 157, D, Dv, DT[dtype],
                                 mask_kind, sinks=sinks)
            _check(p, f"ksplit heads mask={mask_kind} sinks={sinks}")


@pytest.mark.parametrize("D,Dv", WIDTHS, ids=PAIR_IDS)
@pytest.mark.parametrize("Lk", [1, 2, 31, 32, 33, 63, 64, 65, 95, 96, 97, 128, 129, 1801])
def test_key_counts_across_lane_and_step_edges(Lk, D, Dv):
    for mask_kind in (0, 1, 2):
        p = gen.make_problem(8200 + Lk + mask_kind + D, 1, 8, 2, 45, Lk, D, Dv, BF16, mask_kind, sinks=True)
        _check(p, f"ksplit Lk={Lk} mask={mask_kind}")


@pytest.mark.parametrize("D,Dv", WIDTHS, ids=PAIR_IDS)
@pytest.mark.parametrize("Lq,Lk", [(100, 40), (300, 64), (17, 1000), (1024, 1801)])
def test_causal_rows_that_see_few_or_no_keys(Lq, Lk, D, Dv):
    # Lq > Lk: the first Lq - Lk rows see no key (zeros, sink or not); the rest see a
    # few keys, all in the first step's first lane
    for sinks in (False, True):
        p = gen.make_problem(8300 + Lq + Lk + sinks + D, 1, 8, 2, Lq, Lk, D, Dv, F16, 1, sinks=sinks)
        _check(p, f"ksplit causal Lq={Lq} Lk={Lk} sinks={sinks}")


@pytest.mark.parametrize("D,Dv", WIDTHS, ids=PAIR_IDS)
@pytest.mark.parametrize("window", [1, 20, 64, 100, 700])
def test_windows(window, D, Dv):
    import torch
    from scaled_dot_product_06_amd import attention
    from tests.gpu_util import device_inputs
    p = gen.make_problem(8400 + window + D, 1, 8, 2, 200, 900, D, Dv, BF16, 1, sinks=True)
    plan = _plan(p, window)
    assert (plan["rows_per_wave"], plan["splits"]) == (16, 2)
    q, k, v, _, s = device_inputs(p)
    got = from_device(attention(q, k, v, p.scale, 1, None, s, window=window), p.dtype)
    torch.cuda.synchronize()
    qw, kw, vw, _, sw = p.widened()
    want = orc.sdpa(qw, kw, vw, p.scale, 1, None, sw, window=window)
    assert_parity(p, got, want, f"ksplit window={window}")


@pytest.mark.parametrize("D,Dv", WIDTHS, ids=PAIR_IDS)
def test_peaked_scores_across_both_lanes(D, Dv):
    # scale 1.0: each row follows its few top keys, which fall in either lane of any
    # step, so the merge's weights are of order one and a wrong merge shows
    p = gen.make_problem(8500 + D, 1, 16, 2, 256, 1801, D, Dv, F16, 2, sinks=True, scale=1.0)
    _check(p, "ksplit peaked bool mask")
    p = gen.make_problem(8501 + D, 1, 8, 2, 130, 700, D, Dv, BF16, 1, sinks=False, scale=1.0)
    _check(p, "ksplit peaked causal")


@pytest.mark.parametrize("D,Dv", WIDTHS, ids=PAIR_IDS)
def test_batch_items_equal_each_item_alone(D, Dv):
    p = gen.make_problem(8600 + D, 3, 16, 2, 90, 333, D, Dv, BF16, 2, sinks=True)
    plan = _plan(p)
    assert plan["splits"] == 2
    whole = from_device(run_gpu(p), BF16)
    for b in range(p.B):
        pb = gen.Problem(1, p.Hq, p.Hkv, p.Lq, p.Lk, p.D, p.Dv, BF16, p.mask_kind, p.scale, p.q[b:b + 1],
                         p.k[b:b + 1], p.v[b:b + 1], p.mask, p.sinks)
        alone = from_device(run_gpu(pb), BF16)
        assert np.array_equal(whole[b:b + 1], alone), f"batch item {b} differs"


@pytest.mark.parametrize("D,Dv", [(64, 64), (128, 128), (96, 64)], ids=["64x64", "128x128", "96x64"])
def test_a_full_batch_of_small_items_keeps_each_items_bits(D, Dv):
    # 8 items of 32 heads x 256 rows: each item's pipelined grid is 64 workgroups, the
    # whole batch's 512. The plan looks at one item, so the batch runs the key-split
    # kernel like each item alone, and every item's bits equal its bits alone.
    p = gen.make_problem(8650 + D + Dv, 8, 32, 8, 256, 256, D, Dv, BF16, 1, sinks=True)
    plan = _plan(p)
    assert (plan["rows_per_wave"], plan["splits"]) == (16, 2), plan
    whole = from_device(run_gpu(p), BF16)
    for b in (0, 3, 7):
        pb = gen.Problem(1, p.Hq, p.Hkv, p.Lq, p.Lk, p.D, p.Dv, BF16, p.mask_kind, p.scale, p.q[b:b + 1],
                         p.k[b:b + 1], p.v[b:b + 1], p.mask, p.sinks)
        assert _plan(pb)["splits"] == 2
        alone = from_device(run_gpu(pb), BF16)
        assert np.array_equal(whole[b:b + 1], alone), f"batch item {b} differs"
    from tests.gpu_util import sample_rows
    rows = sample_rows(p, 64, seed=5)
    assert_parity(p, np.stack([whole[b, h, i] for b, h, i in rows]), oracle_rows(p, rows), "full batch, sampled rows")


# --- additive masks (the key-split path: heads of 192 or more and 128-wide ones on every grid,
# narrower ones on small grids)

def _additive_call(p, add, sinks, offset=0):
    """Run with `add` (any broadcast shape) as an additive mask, `offset` elements into its buffer."""
    import torch
    from scaled_dot_product_06_amd import attention
    from tests.gpu_util import to_device
    flat = np.concatenate([np.zeros(offset, dtype=add.dtype), add.ravel()])
    dmask = to_device(flat, p.dtype)[offset:].view(add.shape)
    dq, dk, dv = (to_device(a, p.dtype) for a in (p.q, p.k, p.v))
    ds = None if sinks is None else to_device(sinks, p.dtype)
    got = attention(dq, dk, dv, p.scale, 3, dmask, ds)
    torch.cuda.synchronize()
    return from_device(got, p.dtype)


def _additive_plan(p):
    import scaled_dot_product_06_amd as sd
    plan = sd.sdpa_plan(*p.shape_args(), 3, True, True, p.dtype)
    assert (plan["rows_per_wave"], plan["splits"], plan["waves"]) == (16, 2, 8), plan


@pytest.mark.parametrize("D,Dv", WIDTHS, ids=PAIR_IDS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("Lq,Lk", [(9, 300), (45, 1), (45, 63), (70, 257), (100, 1801)])
def test_additive_mask_layouts(Lq, Lk, dtype, D, Dv):
    # full, per-head, per-batch and 2-D masks; a buffer starting one element in
    # (unaligned rows); -inf holes and one row hidden entirely (zeros, sinks or not)
    B, Hq, Hkv = 2, 8, 2
    dt = DT[dtype]
    seed = 8700 + Lq + Lk + D
    p = gen.make_problem(seed, B, Hq, Hkv, Lq, Lk, D, Dv, dt, 0, sinks=True)
    _additive_plan(p)
    q, k, v, _, s = p.widened()
    for shape in [(B, Hq, Lq, Lk), (1, Hq, Lq, Lk), (B, 1, Lq, Lk), (Lq, Lk)]:
        add = gen.additive_mask(seed + len(shape), shape, dt, holes=0.2)
        add[..., Lq // 2, :] = gen.NEG_INF_BITS[dt]
        for offset, sinks in ((0, p.sinks), (1, None)):
            got = _additive_call(p, add, sinks, offset)
            want = orc.sdpa(q, k, v, p.scale, 3, gen.widen(add, dt), None if sinks is None else s)
            assert not got[:, :, Lq // 2].any()
            assert_parity(p, got, want, f"additive {shape} offset {offset} sinks={sinks is not None}")


@pytest.mark.parametrize("D,Dv", WIDTHS, ids=PAIR_IDS)
@pytest.mark.parametrize("shape", HEAD_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_additive_mask_heads_per_workgroup(shape, D, Dv):
    B, Hq, Hkv, Lq = shape
    p = gen.make_problem(8800 + Hq + Lq + D, B, Hq, Hkv, Lq, 333, D, Dv, F16, 0, sinks=True, scale=1.0)
    _additive_plan(p)
    add = gen.additive_mask(8801 + D, (B, Hq, Lq, 333), F16, holes=0.1)
    got = _additive_call(p, add, p.sinks)
    q, k, v, _, s = p.widened()
    want = orc.sdpa(q, k, v, p.scale, 3, gen.widen(add, F16), s)
    assert_parity(p, got, want, "additive, peaked scores")


@pytest.mark.parametrize("D,Dv", WIDTHS, ids=PAIR_IDS)
def test_additive_mask_with_zero_scale(D, Dv):
    # scale 0: the scores are the mask values alone
    p = gen.make_problem(8900 + D, 1, 8, 2, 40, 200, D, Dv, BF16, 0, sinks=True, scale=0.0)
    add = gen.additive_mask(8901 + D, (1, 8, 40, 200), BF16, holes=0.3)
    got = _additive_call(p, add, p.sinks)
    q, k, v, _, s = p.widened()
    want = orc.sdpa(q, k, v, 0.0, 3, gen.widen(add, BF16), s)
    assert_parity(p, got, want, "additive, scale 0")


@pytest.mark.parametrize("D,Dv", [(256, 256), (192, 128)], ids=["256x256", "192x128"])
def test_additive_mask_on_a_full_grid_sampled_rows(D, Dv):
    # 32 heads x 1040 rows: 520 workgroups, two per compute unit and more
    from tests.gpu_util import sample_rows
    p = gen.make_problem(8950 + D + Dv, 1, 32, 4, 1040, 1297, D, Dv, BF16, 0, sinks=True)
    _additive_plan(p)
    add = gen.additive_mask(8951, (1, 32, 1040, 1297), BF16, holes=0.1)
    got = _additive_call(p, add, p.sinks)
    rows = sample_rows(p, 160, seed=3)
    q, k, v, _, s = p.widened()
    want = orc.sdpa(q, k, v, p.scale, 3, gen.widen(add, BF16), s, rows=rows)
    assert_parity(p, np.stack([got[b, h, i] for b, h, i in rows]), want, "additive, full grid, sampled rows")
