"""The router's rules, restated: for random valid shapes, sdpa_plan must give the
plan these rules give (route, kernel geometry, grid, scratch). Host only, no GPU.

The rules are the ones include/sdpa.h documents for sdpa_plan_t, written out
again here independently of the C planner:

  * nothing to do (B, Hq or Lq zero) -> "empty"; no keys -> "zero_fill";
  * 16-bit inputs with Lq <= 8 and (Hq/Hkv)*Lq <= 32 -> "decode": splits of a
    power-of-two number of keys, about a 64th of the keys the rows read,
    clamped to [64, 1024]; a (splits, Hkv, B) grid; a 16-byte {max, sum} slot
    and Dv floats per (batch, kv head, split, packed row) of scratch;
  * otherwise "prefill" on one of four kernels: the key-split kernel for
    16-bit (192,192), (192,128) and (256,256) heads, for 16-bit 128-wide heads
    with an additive mask, and for 16-bit (64,64), (80,80), (96,96), (128,128)
    and (96,64) heads whose pipelined grid for one batch item is under 256
    workgroups; the pipelined kernel for
    other 16-bit calls at (64,64), (80,80), (96,96), (128,128) or (96,64)
    without an additive mask; the f32 key-split kernel for f32 calls whose
    32-row grid for one batch item is under 256 workgroups (no additive
    mask); else the generic kernel. 16-bit boolean masks outside the
    key-split kernel are packed into Lq x ceil(Lk/32) words first.
"""
import math

import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import scaled_dot_product_06_amd as sd  # noqa: E402

F32, F16, BF16 = 0, 1, 2
PAIRS = [(64, 64), (80, 80), (96, 96), (128, 128), (192, 192), (256, 256), (512, 512), (96, 64), (192, 128)]
WAVES = 4   # wavefronts of a prefill workgroup (the key-split kernel doubles them)


def pow2_floor(x):
    return 1 << (x.bit_length() - 1)


def first_window_key(Lq, Lk, window):
    return max(0, Lk - Lq - window + 1) if window > 0 else 0


def expected_plan(B, Hq, Hkv, Lq, Lk, D, Dv, mask_kind, dtype, window=0):
    base = dict(kernels=0, rows_per_wave=0, waves=0, block_n=0, heads_per_group=0, keys_per_split=0, splits=0,
                grid=(0, 0, 0), scratch_bytes=0)
    if B == 0 or Hq == 0 or Lq == 0:
        return dict(base, route="empty")
    if Lk == 0:
        return dict(base, route="zero_fill", kernels=1)   # grid: a fill kernel's, not checked here
    g = Hq // Hkv
    if dtype != F32 and Lq <= 8 and g * Lq <= 32:
        rows = g * Lq
        nkeys = Lk - first_window_key(Lq, Lk, window)
        kps = min(max(pow2_floor(max(nkeys // 64, 1)), 64), 1024)
        splits = -(-nkeys // kps)
        return dict(base, route="decode", kernels=2, rows_per_wave=16 if rows <= 16 and D % 32 == 0 else 32,
                    waves=4, block_n=32, heads_per_group=g, keys_per_split=kps, splits=splits,
                    grid=(splits, Hkv, B), scratch_bytes=B * Hkv * splits * rows * (Dv + 4) * 4)
    heads = math.gcd(g, WAVES)
    hmax = max(D, Dv)
    pipelined_grid = (Hq // heads) * -(-Lq // ((WAVES // heads) * 32))   # per batch item
    if dtype != F32 and ((D, Dv) in ((192, 192), (192, 128), (256, 256))
                         or ((D, Dv) == (128, 128) and mask_kind == 3)
                         or ((D, Dv) in ((64, 64), (80, 80), (96, 96), (128, 128), (96, 64))
                             and pipelined_grid < 256)):
        bm = (WAVES // heads) * 16
        return dict(base, route="prefill", kernels=1, rows_per_wave=16, waves=2 * WAVES, block_n=32,
                    heads_per_group=heads, splits=2, grid=(B * Hq // heads * -(-Lq // bm), 1, 1))
    pipelined = dtype != F32 and (D, Dv) in ((64, 64), (80, 80), (96, 96), (128, 128), (96, 64)) and mask_kind != 3
    rows = 32 if pipelined or hmax <= 128 else 16
    if dtype == F32 and rows == 32 and (Hq // heads) * -(-Lq // ((WAVES // heads) * 32)) < 256:
        rows = 16
        if mask_kind != 3:
            return dict(base, route="prefill", kernels=1, rows_per_wave=16, waves=WAVES,
                        block_n=32 if hmax <= 64 else 16, heads_per_group=1, splits=WAVES,
                        grid=(B * Hq * -(-Lq // 16), 1, 1))
    if pipelined:
        block_n = 32
    elif dtype == F32:
        block_n = 32 if hmax <= 128 else 16
    else:
        block_n = 32 if hmax > 256 else 64
    bm = (WAVES // heads) * rows
    plan = dict(base, route="prefill", kernels=1, rows_per_wave=rows, waves=WAVES, block_n=block_n,
                heads_per_group=heads, grid=(B * Hq // heads * -(-Lq // bm), 1, 1))
    if dtype != F32 and mask_kind == 2:
        plan.update(kernels=2, scratch_bytes=Lq * -(-Lk // 32) * 4)
    return plan


def _compare(got, want):
    if want["route"] == "zero_fill":
        got = dict(got, grid=(0, 0, 0))
    assert got == want


shapes = st.tuples(
    st.integers(0, 3),                                   # B
    st.integers(1, 8),                                   # Hkv
    st.sampled_from([1, 2, 3, 4, 5, 8, 16, 32]),         # group
    st.one_of(st.integers(0, 40), st.integers(41, 5000)),   # Lq
    st.one_of(st.integers(0, 300), st.integers(301, 70000)),  # Lk
    st.sampled_from(PAIRS),
    st.integers(0, 3),                                   # mask kind
    st.sampled_from([F32, F16, BF16]),
    st.booleans(),                                       # sinks
)


@settings(max_examples=400, deadline=None)
@given(shapes)
def test_plans_follow_the_documented_rules(shape):
    B, Hkv, g, Lq, Lk, (D, Dv), mask_kind, dtype, sinks = shape
    Hq = Hkv * g
    got = sd.sdpa_plan(B, Hq, Hkv, Lq, Lk, D, Dv, mask_kind, mask_kind >= 2, sinks, dtype)
    _compare(got, expected_plan(B, Hq, Hkv, Lq, Lk, D, Dv, mask_kind, dtype))


@settings(max_examples=300, deadline=None)
@given(shapes, st.integers(1, 20000))
def test_windowed_plans_follow_the_documented_rules(shape, window):
    # a window needs the causal mask; a window of at least Lk keys plans as causal attention
    B, Hkv, g, Lq, Lk, (D, Dv), _, dtype, sinks = shape
    Hq = Hkv * g
    got = sd.sdpa_plan_windowed(B, Hq, Hkv, Lq, Lk, D, Dv, window, sinks, dtype)
    _compare(got, expected_plan(B, Hq, Hkv, Lq, Lk, D, Dv, 1, dtype, window if window < Lk else 0))


def test_the_restatement_matches_the_workload_plans():
    # the five workloads, fixed: the restatement itself reproduces known plans
    assert expected_plan(2, 32, 8, 4096, 4096, 128, 128, 1, BF16)["grid"] == (2048, 1, 1)
    dec = expected_plan(4, 16, 2, 1, 65537, 256, 256, 0, BF16)
    # 4 x 2 (batch, kv head) x 65 splits x 8 packed rows x (16 B + 256 floats)
    assert (dec["keys_per_split"], dec["splits"], dec["scratch_bytes"]) == (1024, 65, 4326400)
    short = expected_plan(1, 32, 4, 1, 8193, 128, 128, 0, BF16)
    assert (short["keys_per_split"], short["splits"], short["scratch_bytes"]) == (128, 65, 1098240)
    ks = expected_plan(1, 16, 2, 1024, 1801, 256, 256, 2, F16)
    assert (ks["rows_per_wave"], ks["splits"], ks["grid"], ks["kernels"]) == (16, 2, (256, 1, 1), 1)
    f32 = expected_plan(1, 8, 8, 128, 128, 64, 64, 1, F32)
    assert (f32["rows_per_wave"], f32["splits"], f32["grid"]) == (16, 4, (64, 1, 1))
