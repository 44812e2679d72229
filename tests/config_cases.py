"""The five workloads and the variants of them that the parity tests run, with
the defects each test must be able to see.

With N(0,1) inputs averaged over thousands of keys, the decode outputs and the
late prefill rows are a few hundredths. That is under the absolute floor of
the pages' predicate, |g - r| <= tol * max(|r|, 1) (nuvec-core "tests/fast.rs",
``assert_close`` with ``tolerance()``), so on the plain workloads that
predicate alone cannot see a lost key split. The variants keep each
workload's exact shape, dtype, mask and route, and make outputs of order one:

* ``peaked``: scale 1.0, so scores spread by about sqrt(D) and each row's
  output is close to the value rows of its few top-scoring keys, wherever
  they fall;
* ``planted`` (decode workloads): the key at a chosen position is a copy of one
  query head's row, which gives that head a score well above the rest; the
  head's output is then mostly that key's value row. The positions cover the
  first key, both sides of a split edge, a middle split, the split before the
  last, and the final split, which holds one key. Odd heads of a group get a
  second copy in another split: two equal weights, so the output is close to
  the mean of two value rows from two different splits;
* ``heavy_sinks`` (workload 4): each sink logit is moved up by the log of the
  row's mass of key weights, so the sink takes between about a tenth and nine
  tenths of the denominator, and an ignored or misread sink is visible.

``defects`` lists, per test, results that a correct test must reject: all
zeros, the keys of one split (decode) or one 32-key tile (prefill) dropped,
and the sink ignored. ``expected_catches`` says which of them each test is
claimed to reject; the CPU negative controls check the claim on the oracle's
own output.
"""
from __future__ import annotations

import functools
import math

import numpy as np

from scaled_dot_product_06_amd import inputs as gen

# keys per decode split that the router gives the two decode workloads
KEYS_PER_SPLIT = {2: 128, 5: 1024}
DECODE = (2, 5)
PREFILL = (1, 3, 4)


@functools.lru_cache(maxsize=None)
def _base(number: int) -> gen.Problem:
    return gen.workload(number)


def _copy(p: gen.Problem, **kw) -> gen.Problem:
    f = dict(B=p.B, Hq=p.Hq, Hkv=p.Hkv, Lq=p.Lq, Lk=p.Lk, D=p.D, Dv=p.Dv, dtype=p.dtype, mask_kind=p.mask_kind,
             scale=p.scale, q=p.q, k=p.k, v=p.v, mask=p.mask, sinks=p.sinks, name=p.name)
    f.update(kw)
    return gen.Problem(**f)


def planted_positions(number: int, pair: int):
    """[(first, second or None)] per head of one (batch, kv head) pair's group."""
    p = _base(number)
    kps = KEYS_PER_SPLIT[number]
    Lk = p.Lk
    nsplit = -(-Lk // kps)
    first = [Lk - 1, 0, kps - 1, kps, (nsplit // 2) * kps + 17 + pair, Lk - 2, 2 * kps + 5 + pair,
             (nsplit - 2) * kps + 33 + pair]
    group = p.Hq // p.Hkv
    assert group <= len(first)
    out = []
    for i in range(group):
        second = (nsplit // 3 + i) * kps + 7 + pair if i % 2 else None
        out.append((first[i], second))
    return out


def _planted(number: int) -> gen.Problem:
    p = _base(number)
    assert p.Lq == 1
    k = np.array(p.k)
    group = p.Hq // p.Hkv
    for b in range(p.B):
        for hkv in range(p.Hkv):
            pair = b * p.Hkv + hkv
            taken = set()
            for i, (j1, j2) in enumerate(planted_positions(number, pair)):
                h = hkv * group + i
                for j in (j1, j2):
                    if j is None:
                        continue
                    assert 0 <= j < p.Lk and j not in taken
                    taken.add(j)
                    k[b, hkv, j] = p.q[b, h, 0]
    return _copy(p, k=k, name=p.name + " planted")


def _heavy_sinks(number: int) -> gen.Problem:
    p = _base(number)
    assert p.sinks is not None and p.dtype != gen.F32
    # log of a row's key-weight mass under uniform[-1,1) inputs: about 0.9 * Lk
    # visible keys, each weighing about exp(var(score) / 2) with
    # var(score) = scale^2 * D / 9
    var = p.scale ** 2 * p.D / 9.0
    shift = math.log(0.9 * p.Lk) + var / 2.0
    s = gen.widen(p.sinks, p.dtype) + shift
    return _copy(p, sinks=gen.to_storage(s, p.dtype), name=p.name + " heavy sinks")


VARIANTS = {
    1: ("plain",),
    2: ("plain", "peaked", "planted"),
    3: ("plain", "peaked"),
    4: ("plain", "peaked", "heavy_sinks"),
    5: ("plain", "peaked", "planted"),
}


@functools.lru_cache(maxsize=None)
def case(number: int, kind: str) -> gen.Problem:
    """Workload `number` as the parity tests run it."""
    if kind not in VARIANTS[number]:
        raise ValueError(f"workload {number} has no variant {kind!r}")
    if kind == "plain":
        return _base(number)
    if kind == "peaked":
        p = _base(number)
        return _copy(p, scale=1.0, name=p.name + " peaked")
    if kind == "planted":
        return _planted(number)
    return _heavy_sinks(number)


def all_cases():
    return [(n, kind) for n in sorted(VARIANTS) for kind in VARIANTS[n]]


def dropped_ranges(number: int):
    """Key ranges whose loss a test may be asked to see: decode splits (the first,
    a middle one and the final one) or one 32-key prefill tile."""
    p = _base(number)
    if number in DECODE:
        kps = KEYS_PER_SPLIT[number]
        nsplit = -(-p.Lk // kps)
        return {"first split": (0, kps), "middle split": ((nsplit // 2) * kps, (nsplit // 2 + 1) * kps),
                "final split": ((nsplit - 1) * kps, p.Lk)}
    t = p.Lk // 64   # a tile in the middle of the keys
    return {"one tile": (32 * t, 32 * t + 32)}


def defects(number: int, kind: str):
    """Names of the defects checked for one test."""
    names = ["zeros"] + list(dropped_ranges(number))
    if case(number, kind).sinks is not None:
        names.append("sink ignored")
    return names


# Which defects each test is claimed to reject (the CPU negative controls assert it).
# The plain decode workloads cannot see the loss of their one-key final split, and
# the plain workload 4 is not claimed to see its sinks (one logit among about 1,600
# similar ones); the planted and heavy-sink variants are.
def expected_catches(number: int, kind: str):
    names = set(defects(number, kind))
    if kind == "plain" and number in DECODE:
        names.discard("final split")
    if kind == "peaked" and number in DECODE:
        # a dropped split shows only if it holds some row's top keys, which depends
        # on where they fall; the planted variant places them
        names -= set(dropped_ranges(number))
    if kind in ("plain", "peaked") and number == 4:
        names.discard("sink ignored")
    return names
