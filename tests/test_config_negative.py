"""Negative controls for the workload parity tests (CPU only).

Each workload test on the GPU compares the library's output with the oracle's
under the pages' predicate (nuvec-core "tests/fast.rs", ``assert_close`` with
``tolerance()``) and, for 16-bit types, the row-scaled check of
``tests/gpu_util.py``. A test that cannot fail proves nothing, so here the
same checks run on results that are known to be wrong, made from the oracle's
own output on the same inputs: all zeros, the keys of one decode split or one
prefill tile dropped, the sink ignored. Each test must reject every defect it
claims to catch (``tests/config_cases.py``, ``expected_catches``); between them
the tests of each workload catch every defect listed.
"""
import numpy as np
import pytest

from oracle import attention as orc
from tests import config_cases as cc
from tests.gpu_util import compare, parity_failures, row_scaled

# workload 3 is checked here on two whole (batch, head) slices, the first and the last
SLICES_3 = ((0, 0), (1, 31))


def _rows(p, number):
    if number != 3:
        return None
    return [(b, h, i) for b, h in SLICES_3 for i in range(p.Lq)]


def _visible(p):
    """The workload's own [Lq, Lk] visibility (causal, boolean or none)."""
    i = np.arange(p.Lq)[:, None]
    j = np.arange(p.Lk)[None, :]
    if p.mask_kind == orc.MASK_CAUSAL:
        return j <= i + p.Lk - p.Lq
    if p.mask_kind == orc.MASK_BOOL:
        return np.asarray(p.mask) != 0
    return np.ones((p.Lq, p.Lk), dtype=bool)


def _oracle(p, rows, drop=None, sinks=True):
    q, k, v, m, s = p.widened()
    if not sinks:
        s = None
    if drop is None:
        return orc.sdpa(q, k, v, p.scale, p.mask_kind, m, s, rows=rows)
    vis = _visible(p)
    vis[:, drop[0]:drop[1]] = False
    return orc.sdpa(q, k, v, p.scale, orc.MASK_BOOL, vis, s, rows=rows)


@pytest.mark.parametrize("number,kind", cc.all_cases(), ids=lambda x: str(x))
def test_each_workload_test_can_fail(number, kind):
    p = cc.case(number, kind)
    rows = _rows(p, number)
    want = _oracle(p, rows)
    assert parity_failures(want, want, p.dtype) == 0
    ranges = cc.dropped_ranges(number)
    caught = {}
    for name in cc.defects(number, kind):
        if name == "zeros":
            bad = np.zeros_like(want)
        elif name == "sink ignored":
            bad = _oracle(p, rows, sinks=False)
        else:
            bad = _oracle(p, rows, drop=ranges[name])
        pages = compare(bad, want, p.dtype)[0]
        rbad, ratio = row_scaled(bad, want, p.dtype)
        caught[name] = parity_failures(bad, want, p.dtype) > 0
        print(f"workload {number} {kind}: {name}: pages' predicate fails {pages} elements, "
              f"row-scaled fails {rbad} (worst ratio {ratio:.3g})")
    missed = sorted(n for n in cc.expected_catches(number, kind) if not caught[n])
    assert not missed, f"workload {number} {kind}: the test would pass {missed}"


@pytest.mark.parametrize("number", sorted(cc.VARIANTS))
def test_every_defect_is_caught_by_some_test_of_the_workload(number):
    claimed = set()
    listed = set()
    for kind in cc.VARIANTS[number]:
        claimed |= cc.expected_catches(number, kind)
        listed |= set(cc.defects(number, kind))
    assert listed <= claimed, f"workload {number}: no test catches {sorted(listed - claimed)}"


def test_planted_keys_sit_where_claimed():
    # the planted positions cover the first key, both sides of a split edge, a middle
    # split, and the final one-key split of both decode workloads
    for number in cc.DECODE:
        p = cc.case(number, "planted")
        kps = cc.KEYS_PER_SPLIT[number]
        assert (p.Lk - 1) % kps == 0, "the final split holds exactly one key"
        pos = [j for pair in range(p.B * p.Hkv) for f, s in cc.planted_positions(number, pair)
               for j in (f, s) if j is not None]
        assert {0, kps - 1, kps, p.Lk - 1} <= set(pos)
        group = p.Hq // p.Hkv
        for b in range(p.B):
            for hkv in range(p.Hkv):
                for i, (f, s) in enumerate(cc.planted_positions(number, b * p.Hkv + hkv)):
                    for j in (f, s):
                        if j is not None:
                            assert np.array_equal(p.k[b, hkv, j], p.q[b, hkv * group + i, 0])


@pytest.mark.parametrize("number,kind", [(2, "planted"), (5, "planted"), (3, "peaked"), (4, "peaked")])
def test_variant_outputs_are_of_order_one(number, kind):
    # what makes these tests able to fail: outputs near 1 in size, where the pages'
    # floor of 1 no longer hides an error
    p = cc.case(number, kind)
    rows = _rows(p, number)
    want = _oracle(p, rows)
    big = np.max(np.abs(want), axis=-1)
    share = float(np.mean(big > 0.5))
    print(f"workload {number} {kind}: rows with max |r| above the mark: {share:.3f}, max |r| {want.max():.3f}")
    if kind == "planted":
        # every head owns a planted key: every row is order one
        assert share == 1.0
    else:
        assert share > 0.9
