"""GPU parity: the HIP library (through its C ABI) against the CPU float64
oracle, element by element, on seeded inputs. Tolerance per element:
|g - r| <= tol * max(|r|, 1), tol = 2e-5 (f32), 4e-3 (f16), 5e-2 (bf16)."""
import json
import os
import zlib

import numpy as np
import pytest

from oracle import attention as orc
from scaled_dot_product_06_amd import inputs as gen
from tests import config_cases as cc
from tests.gpu_util import (TOL, assert_parity, compare, device_inputs, from_device, oracle_rows, run_gpu,
                            sample_rows, say, to_device)

pytestmark = pytest.mark.gpu

F32, F16, BF16 = gen.F32, gen.F16, gen.BF16
DT = {"f32": F32, "f16": F16, "bf16": BF16}
HEAD_PAIRS = [(64, 64), (80, 80), (96, 96), (128, 128), (192, 192), (256, 256), (512, 512), (96, 64), (192, 128)]


def _full_check(p, what=""):
    got = from_device(run_gpu(p), p.dtype)
    want = oracle_rows(p)
    assert got.shape == want.shape
    assert_parity(p, got, want, what)
    return got


# --- the five workloads ---------------------------------------------------------------------
# Each workload at its exact shape, plus the variants of tests/config_cases.py whose outputs
# are of order one (peaked scores, planted keys in chosen decode splits, heavy sinks), so a
# lost split, tile or sink fails the check (the CPU negative controls show that it would).
# Every output element is compared with the oracle, one (batch, head) slice at a time.

@pytest.mark.parametrize("number,kind", cc.all_cases(), ids=lambda x: str(x))
def test_workload(number, kind):
    import scaled_dot_product_06_amd as sd
    p = cc.case(number, kind)
    say(f"workload {number} {kind}: {p!r}")
    plan = sd.sdpa_plan(*p.shape_args(), p.mask_kind, p.mask is not None, p.sinks is not None, p.dtype)
    if number in cc.DECODE:
        assert plan["route"] == "decode" and plan["keys_per_split"] == cc.KEYS_PER_SPLIT[number]
    else:
        assert plan["route"] == "prefill"
    _full_check(p, f"workload {number} {kind}")


# --- coverage grids -------------------------------------------------------------------------

# (B, Hq, Hkv, Lq, Lk, D, Dv): the shapes of nuvec-core's kernel-vs-fallback test
PAGE_SHAPES = [
    (2, 4, 4, 1, 37, 64, 64), (1, 8, 2, 4, 50, 128, 128), (1, 4, 4, 2, 33, 96, 64), (1, 2, 1, 1, 20, 192, 128),
    (1, 8, 1, 1, 1100, 128, 128), (1, 16, 2, 1, 9000, 128, 128), (2, 4, 2, 33, 45, 64, 64),
    (1, 2, 2, 100, 100, 80, 80), (1, 4, 4, 64, 96, 128, 128), (1, 2, 2, 40, 40, 96, 64),
]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", PAGE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_page_shapes(shape, dtype):
    B, Hq, Hkv, Lq, Lk, D, Dv = shape
    for mask_kind in (0, 1, 2):
        for sinks in (False, True):
            seed = 1000 + zlib.crc32(repr((shape, dtype, mask_kind, sinks)).encode()) % 100000
            p = gen.make_problem(seed, B, Hq, Hkv, Lq, Lk, D, Dv, DT[dtype], mask_kind, dist="uniform",
                                 sinks=sinks, scale=0.3)
            _full_check(p, f"mask={mask_kind} sinks={sinks}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D,Dv", HEAD_PAIRS)
def test_prefill_head_grid(D, Dv, dtype):
    for mask_kind in (0, 1, 2):
        for sinks in (False, True):
            p = gen.make_problem(7 + D + Dv + mask_kind, 2, 4, 2, 77, 150, D, Dv, DT[dtype], mask_kind,
                                 sinks=sinks)
            _full_check(p, f"prefill mask={mask_kind} sinks={sinks}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D,Dv", HEAD_PAIRS)
def test_decode_head_grid(D, Dv, dtype):
    # (Hq, Hkv, Lq): 8 rows, 12 rows with causal cuts, 32 rows (32-row tiles)
    for Hq, Hkv, Lq in ((8, 1, 1), (8, 2, 3), (16, 2, 4)):
        for mask_kind in (0, 1, 2):
            p = gen.make_problem(11 + D + Lq + mask_kind, 2, Hq, Hkv, Lq, 1000, D, Dv, DT[dtype], mask_kind,
                                 sinks=(mask_kind == 2))
            _full_check(p, f"decode Hq={Hq} Hkv={Hkv} Lq={Lq} mask={mask_kind}")


@pytest.mark.parametrize("Lk", [1, 2, 31, 32, 33, 63, 64, 65, 1023, 1024, 1025, 8193])
def test_decode_key_lengths(Lk):
    p = gen.make_problem(500 + Lk, 1, 32, 4, 1, Lk, 128, 128, BF16, 1)
    _full_check(p, f"decode Lk={Lk}")


@pytest.mark.parametrize("Lq,Lk", [(9, 9), (33, 33), (64, 64), (65, 700), (128, 128), (129, 64), (200, 1),
                                   (342, 1119)])
def test_prefill_lengths(Lq, Lk):
    for dtype in (BF16, F16):
        p = gen.make_problem(900 + Lq, 1, 8, 2, Lq, Lk, 128, 128, dtype, 1, sinks=True)
        _full_check(p, f"prefill Lq={Lq} Lk={Lk}")


def _mask_patterns(Lq, Lk):
    """Boolean masks that probe the 16-bit prefill's packed 32-key mask words: keys on
    word edges only (bits 0 and 31, and the ragged last key), a diagonal stripe that
    shifts by row, and rows hidden entirely (whose output is zero, sinks or not)."""
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    return {
        "word_edges": (j % 32 == 0) | (j % 32 == 31) | (j == Lk - 1),
        "stripes": (i + j) % 3 == 0,
        "rows_off": (i % 5 != 2) & (j % 7 != 3),
    }


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("Lk", [1, 31, 32, 33, 63, 64, 65, 100, 1025])
def test_prefill_bool_mask_word_edges(D, Lk):
    for dtype in (BF16, F16):
        p = gen.make_problem(1300 + Lk + D, 1, 4, 2, 70, Lk, D, D, dtype, 2, sinks=True)
        for name, pattern in _mask_patterns(p.Lq, Lk).items():
            p.mask = np.ascontiguousarray(np.broadcast_to(pattern, (p.Lq, Lk)).astype(np.uint8))
            _full_check(p, f"bool mask {name} D={D} Lk={Lk}")


# --- full grids at 64- to 256-wide heads -------------------------------------------------------
# Two batch items of 32 heads, ragged on both axes: 1040 query rows over 1297 keys. At
# heads of 192 and 256 columns the key-split kernel (520 workgroups of 16-row blocks per
# batch item); at 64-, 96- and 128-wide heads the pipelined kernel, whose grid here (264
# workgroups of 32-row blocks per batch item) is large enough that the plan keeps it (the
# small-grid tests of the 64- and 128-wide heads run the key-split kernel).

WIDE = dict(B=2, Hq=32, Hkv=4, Lq=1040, Lk=1297)
WIDE_PAIRS = [(64, 64), (96, 96), (128, 128), (192, 192), (192, 128), (256, 256)]
WIDE_IDS = ["x".join(map(str, w)) for w in WIDE_PAIRS]


def _wide_plan_check(p):
    import scaled_dot_product_06_amd as sd
    plan = sd.sdpa_plan(*p.shape_args(), p.mask_kind, p.mask is not None, p.sinks is not None, p.dtype)
    # the plan's key lanes: 0 = pipelined kernel, 2 = key-split
    assert plan["splits"] == (2 if p.D >= 192 else 0), plan


@pytest.mark.parametrize("D,Dv", WIDE_PAIRS, ids=WIDE_IDS)
@pytest.mark.parametrize("mask_kind,sinks", [(0, False), (1, False), (1, True), (2, True)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_wide_heads_full_grid_sampled_rows(mask_kind, sinks, dtype, D, Dv):
    w = WIDE
    p = gen.make_problem(1700 + 10 * mask_kind + sinks + D, w["B"], w["Hq"], w["Hkv"], w["Lq"], w["Lk"], D, Dv,
                         DT[dtype], mask_kind, sinks=sinks)
    _wide_plan_check(p)
    say(f"full grid: {p!r}")
    got = from_device(run_gpu(p), p.dtype)
    assert np.all(np.isfinite(got))
    rows = sample_rows(p, 120, seed=17 + mask_kind)
    want = oracle_rows(p, rows)
    assert_parity(p, np.stack([got[b, h, i] for b, h, i in rows]), want,
                  f"({D},{Dv}) full grid mask {mask_kind} sinks {sinks}, sampled rows")


@pytest.mark.parametrize("D,Dv", WIDE_PAIRS, ids=WIDE_IDS)
def test_wide_heads_full_grid_batch_items_equal_each_item_alone(D, Dv):
    w = WIDE
    p = gen.make_problem(1795 + D, w["B"], w["Hq"], w["Hkv"], w["Lq"], w["Lk"], D, Dv, BF16, 1, sinks=True)
    _wide_plan_check(p)
    whole = from_device(run_gpu(p), BF16)
    for b in range(w["B"]):
        pb = gen.Problem(1, w["Hq"], w["Hkv"], w["Lq"], w["Lk"], D, Dv, BF16, 1, p.scale, p.q[b:b + 1],
                         p.k[b:b + 1], p.v[b:b + 1], None, p.sinks)
        alone = from_device(run_gpu(pb), BF16)
        assert np.array_equal(whole[b:b + 1], alone), f"batch item {b} differs"


@pytest.mark.parametrize("D,Dv", WIDE_PAIRS, ids=WIDE_IDS)
def test_wide_heads_full_grid_window_sampled_rows(D, Dv):
    from scaled_dot_product_06_amd import attention
    import torch
    w = WIDE
    p = gen.make_problem(1790 + D, w["B"], w["Hq"], w["Hkv"], w["Lq"], w["Lk"], D, Dv, BF16, 1, sinks=True)
    _wide_plan_check(p)
    q, k, v, _, sinks = device_inputs(p)
    got = from_device(attention(q, k, v, p.scale, 1, None, sinks, window=300), p.dtype)
    torch.cuda.synchronize()
    rows = sample_rows(p, 96, seed=23)
    qq, kk, vv, _, ss = p.widened()
    want = orc.sdpa(qq, kk, vv, p.scale, 1, None, ss, window=300, rows=rows)
    assert_parity(p, np.stack([got[b, h, i] for b, h, i in rows]), want, f"({D},{Dv}) full grid window 300")


# --- sliding windows (nuvec-core tests/fast.rs, windowed-kernel tests) -------------------------

# (Lq, Lk, D, Hq, Hkv, window): one-query decode over windows below the keys (short and long
# caches), few-query decode, prefill chunks with windows of 1 to above the keys
WINDOW_CASES = [(1, 300, 64, 8, 1, 128), (1, 4096, 64, 8, 8, 128), (1, 9000, 128, 8, 1, 3),
                (1, 2000, 256, 4, 1, 1024), (4, 600, 128, 4, 2, 7), (8, 1500, 64, 4, 4, 128),
                (40, 300, 64, 4, 2, 7), (97, 400, 128, 2, 1, 33), (64, 640, 64, 2, 2, 1),
                (300, 700, 256, 2, 1, 128), (33, 45, 64, 4, 2, 100), (2, 5000, 256, 4, 2, 1024),
                (130, 130, 128, 4, 4, 64), (200, 900, 96, 4, 2, 50)]


def _window_check(p, w, what):
    from scaled_dot_product_06_amd import attention
    import torch
    q, k, v, _, sinks = device_inputs(p)
    got = from_device(attention(q, k, v, p.scale, 1, None, sinks, window=w), p.dtype)
    torch.cuda.synchronize()
    qq, kk, vv, _, ss = p.widened()
    want = orc.sdpa(qq, kk, vv, p.scale, 1, None, ss, window=w)
    assert_parity(p, got, want, what)
    assert np.isfinite(got).all()


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_windows(case, dtype):
    Lq, Lk, D, Hq, Hkv, w = case
    dt = {"f32": F32, "f16": F16, "bf16": BF16}[dtype]
    for sinks in (False, True):
        p = gen.make_problem(2000 + Lq + Lk + w, 1, Hq, Hkv, Lq, Lk, D, D, dt, 1, sinks=sinks)
        _window_check(p, w, f"window {w} sinks={sinks}")


def test_full_window_is_causal_bit_for_bit():
    import torch
    from scaled_dot_product_06_amd import attention
    for (Lq, Lk, dt) in [(1, 3000, BF16), (70, 70, F16), (5, 9, F32), (130, 400, BF16)]:
        p = gen.make_problem(3100 + Lq, 1, 4, 2, Lq, Lk, 128, 128, dt, 1, sinks=True)
        q, k, v, _, s = device_inputs(p)
        causal = attention(q, k, v, p.scale, 1, None, s)
        for w in (Lk, Lk + 5):
            win = attention(q, k, v, p.scale, 1, None, s, window=w)
            torch.cuda.synchronize()
            assert torch.equal(win.view(torch.int16) if dt != F32 else win,
                               causal.view(torch.int16) if dt != F32 else causal), (Lq, Lk, w)


@pytest.mark.parametrize("Lk,w", [(300, 128), (4096, 128), (9000, 300), (2000, 1024)])
def test_one_query_window_equals_its_keys_alone(Lk, w):
    # a decode row over a window gives the same bits as an unmasked call over exactly its keys
    import torch
    from scaled_dot_product_06_amd import attention
    p = gen.make_problem(3200 + Lk, 1, 8, 2, 1, Lk, 128, 128, BF16, 1, sinks=True)
    q, k, v, _, s = device_inputs(p)
    win = attention(q, k, v, p.scale, 1, None, s, window=w)
    alone = attention(q, k[:, :, Lk - w:].contiguous(), v[:, :, Lk - w:].contiguous(), p.scale, 0, None, s)
    torch.cuda.synchronize()
    assert torch.equal(win.view(torch.int16), alone.view(torch.int16))


# --- edge cases -------------------------------------------------------------------------------

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("name", ["masked_key_sentinel.json", "all_masked_single_tile.json",
                                  "all_masked_multi_tile.json"])
@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_printed_examples_on_gpu(name, dtype):
    """The lattice-inference worked examples, zero-padded to a 64-wide head."""
    g = json.load(open(os.path.join(GOLDEN, name)))
    Lq, Lk, D, Dv = g["Lq"], g["Lk"], g["D"], g["Dv"]
    q = np.zeros((1, 1, Lq, 64))
    k = np.zeros((1, 1, Lk, 64))
    v = np.zeros((1, 1, Lk, 64))
    q[0, 0, :, :D] = np.array(g["q"]).reshape(Lq, D)
    k[0, 0, :, :D] = np.array(g["k"]).reshape(Lk, D)
    v[0, 0, :, :Dv] = np.array(g["v"]).reshape(Lk, Dv)
    dt = DT[dtype]
    p = gen.Problem(1, 1, 1, Lq, Lk, 64, 64, dt, 2, g["scale"], gen.to_storage(q, dt), gen.to_storage(k, dt),
                    gen.to_storage(v, dt), np.array(g["mask"], np.uint8), None, name)
    got = from_device(run_gpu(p), dt)[0, 0, :, :Dv].reshape(-1)
    want = np.array(g["expected"])
    assert np.all(np.isfinite(got))
    if g["tolerance"] == 0:
        assert np.array_equal(got, want), (got, want)
    else:
        # the printed bound, widened to the element type's own tolerance
        tol = max(g["tolerance"], TOL[dt])
        assert np.all(np.abs(got - want) <= tol * np.maximum(np.abs(want), 1.0)), (got, want)


def test_empty_and_keyless_calls():
    import torch
    from scaled_dot_product_06_amd import SDPA_MASK_CAUSAL, attention
    q = torch.randn(1, 2, 3, 64, device="cuda").to(torch.bfloat16)
    kv = torch.zeros(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    sinks = torch.randn(2, device="cuda").to(torch.bfloat16)
    for kind, s in ((0, None), (1, None), (1, sinks)):
        out = torch.full((1, 2, 3, 64), 7.0, device="cuda", dtype=torch.bfloat16)
        attention(q, kv, kv, 0.125, kind, None, s, out=out)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out).item() == 0
    # no queries: nothing is written, the call succeeds
    qe = torch.zeros(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(1, 2, 5, 64, device="cuda").to(torch.bfloat16)
    out = attention(qe, k, k, 0.125, SDPA_MASK_CAUSAL)
    assert tuple(out.shape) == (1, 2, 0, 64)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_rows_without_visible_keys_are_zero(dtype):
    dt = DT[dtype]
    # causal with more queries than keys: the first Lq - Lk rows see nothing (prefill and decode routes)
    for (Hq, Hkv, Lq, Lk) in ((4, 2, 100, 40), (2, 2, 5, 3)):
        for sinks in (False, True):
            p = gen.make_problem(40 + Lq, 1, Hq, Hkv, Lq, Lk, 64, 64, dt, 1, sinks=sinks)
            got = _full_check(p, f"causal Lq={Lq} > Lk={Lk} sinks={sinks}")
            assert np.all(got[:, :, : Lq - Lk] == 0)
    # boolean rows with no true entry
    p = gen.make_problem(77, 1, 4, 1, 70, 90, 128, 128, dt, 2, sinks=True)
    p.mask = np.array(p.mask)
    p.mask[[0, 5, 69]] = 0
    got = _full_check(p, "bool mask with empty rows")
    assert np.all(got[:, :, [0, 5, 69]] == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("scale", [-0.7, 0.0, 1.0])
def test_scale_values(dtype, scale):
    for Lq in (1, 50):
        p = gen.make_problem(60 + Lq, 1, 4, 2, Lq, 300, 64, 64, DT[dtype], 0, scale=scale)
        _full_check(p, f"scale={scale} Lq={Lq}")


@pytest.mark.parametrize("scale", [-0.7, 0.0])
@pytest.mark.parametrize("route", ["fast-f16", "fast-bf16", "generic-256", "decode-f16", "window", "additive",
                                   "paged", "paged-f32"])
def test_negative_and_zero_scale_on_every_path(route, scale):
    # q's sign is flipped in the kernels (scores use |scale|); zero scale gives the mean
    # of the visible rows
    import torch
    from scaled_dot_product_06_amd import attention, paged_attention
    dt = {"fast-f16": F16, "decode-f16": F16, "paged-f32": F32}.get(route, BF16)
    D = 256 if route == "generic-256" else 128
    Lq = 1 if route.startswith(("decode", "paged")) else 70
    p = gen.make_problem(4000 + len(route) + int(10 * scale), 2, 8, 2, Lq, 333, D, D, dt, 1, sinks=True,
                         scale=scale)
    qq, kk, vv, _, ss = p.widened()
    q, k, v, _, sk = device_inputs(p)
    if route == "window":
        got = attention(q, k, v, scale, 1, None, sk, window=50)
        want = orc.sdpa(qq, kk, vv, scale, 1, None, ss, window=50)
    elif route == "additive":
        add = gen.additive_mask(5, (1, 8, Lq, 333), dt, 0.1)
        got = attention(q, k, v, scale, 3, to_device(add, dt), sk)
        want = orc.sdpa(qq, kk, vv, scale, 3, gen.widen(add, dt), ss)
    elif route.startswith("paged"):
        from oracle import paged as pgd
        bs, blocks = 16, 2 * 21 + 3
        kc, table = gen.paged_cache(p.k, bs, gen.block_order(4, blocks), blocks)
        vc, _ = gen.paged_cache(p.v, bs, gen.block_order(4, blocks), blocks)
        lengths = np.array([333, 200], dtype=np.int32)
        got = paged_attention(q, to_device(kc, dt), to_device(vc, dt), torch.from_numpy(table).cuda(),
                              torch.from_numpy(lengths).cuda(), scale, 1, 0, sk)
        want = pgd.paged_sdpa(qq, gen.widen(kc, dt), gen.widen(vc, dt), table, lengths, scale, 1, ss)
    else:
        got = attention(q, k, v, scale, 1, None, sk)
        want = orc.sdpa(qq, kk, vv, scale, 1, None, ss)
    torch.cuda.synchronize()
    assert_parity(p, from_device(got, dt), want, f"{route} scale={scale}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_wide_score_range(dtype):
    """Scores spread over tens of units: the running maximum moves many times.

    f32 runs at half the score spread (std 8 instead of 16): at std 16 the f32
    rounding of the scores alone (about 2^-24 * |s| * scale, then exponentiated)
    reaches the 2e-5 bound, which the float32 tolerance of the pages was set
    for scores near zero."""
    scale = 1.0 if dtype == "f32" else 2.0
    for Lq in (1, 96):
        p = gen.make_problem(80 + Lq, 1, 4, 1, Lq, 2000, 64, 64, DT[dtype], 1, scale=scale, sinks=True)
        _full_check(p, f"scale {scale} Lq={Lq}")


def test_largest_heads_long_keys():
    for Lq, Lk in ((1, 5000), (130, 700)):
        p = gen.make_problem(90 + Lq, 1, 8, 2, Lq, Lk, 512, 512, BF16, 1, sinks=True)
        _full_check(p, f"D=512 Lq={Lq} Lk={Lk}")


@pytest.mark.parametrize("scale", [None, 1.0], ids=["rsqrtD", "peaked"])
@pytest.mark.parametrize("Lk,D,mask_kind", [(262145, 128, 0), (300001, 64, 1), (1 << 20, 64, 0)])
def test_decode_more_splits_than_one_reduce_chunk(Lk, D, mask_kind, scale):
    # 1024-key splits: 257, 293 and 1024 of them, so the reduce walks its splits in
    # several chunks of 256 (and the last split holds one key in the first case). At
    # scale 1/sqrt(D) the outputs are a few thousandths; at scale 1.0 each row's output
    # is close to its top keys' value rows (order one), wherever they fall
    p = gen.make_problem(600 + Lk % 97, 1, 8, 1, 1, Lk, D, D, BF16, mask_kind, sinks=True, scale=scale)
    plan = __import__("scaled_dot_product_06_amd").sdpa_plan(*p.shape_args(), mask_kind, False, True, BF16)
    assert plan["route"] == "decode" and plan["splits"] > 256
    _full_check(p, f"decode Lk={Lk} splits={plan['splits']} scale={p.scale}")


@pytest.mark.parametrize("B,Hq,Hkv,Lk", [(1000, 4, 2, 70), (65535, 2, 1, 5)])
def test_decode_large_batch(B, Hq, Hkv, Lk):
    # the decode grid's z dimension is the batch; 65,535 is its limit
    p = gen.make_problem(700 + B % 13, B, Hq, Hkv, 1, Lk, 64, 64, F16, 1, dist="uniform")
    got = from_device(run_gpu(p), p.dtype)
    rows = sample_rows(p, 300, seed=B)
    want = oracle_rows(p, rows)
    assert_parity(p, np.stack([got[b, h, i] for b, h, i in rows]), want, f"decode B={B}, sampled rows")


def test_long_prefill_sampled_rows():
    # 16,384 x 16,384 causal, one head pair: positions well past 2^13 in every index
    p = gen.make_problem(801, 1, 2, 1, 16384, 16384, 64, 64, BF16, 1)
    got = from_device(run_gpu(p), p.dtype)
    rows = sample_rows(p, 200, seed=801)
    want = oracle_rows(p, rows)
    assert_parity(p, np.stack([got[b, h, i] for b, h, i in rows]), want, "prefill 16k x 16k, sampled rows")


# --- properties -------------------------------------------------------------------------------

@pytest.mark.parametrize("Lq,Lk,dtype", [(1, 3000, BF16), (4, 777, F16), (150, 300, BF16), (60, 60, F32)])
def test_batch_items_equal_each_item_alone(Lq, Lk, dtype):
    p = gen.make_problem(123, 3, 8, 2, Lq, Lk, 128, 128, dtype, 1, sinks=True)
    whole = from_device(run_gpu(p), dtype)
    for b in range(3):
        pb = gen.Problem(1, 8, 2, Lq, Lk, 128, 128, dtype, 1, p.scale, p.q[b:b + 1], p.k[b:b + 1],
                         p.v[b:b + 1], None, p.sinks)
        alone = from_device(run_gpu(pb), dtype)
        assert np.array_equal(whole[b:b + 1], alone), f"batch item {b} differs"


@pytest.mark.parametrize("Lq,Lk", [(1, 9000), (300, 500)])
def test_run_to_run_determinism(Lq, Lk):
    p = gen.make_problem(321, 2, 16, 2, Lq, Lk, 128, 128, BF16, 2 if Lq > 1 else 1)
    dev = device_inputs(p)
    a = from_device(run_gpu(p, dev), BF16)
    b = from_device(run_gpu(p, dev), BF16)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("Lq", [1, 70])
def test_gqa_equals_repeated_heads(Lq):
    p = gen.make_problem(55, 1, 8, 2, Lq, 400, 128, 128, F16, 1, sinks=True)
    rep = gen.Problem(1, 8, 8, Lq, 400, 128, 128, F16, 1, p.scale, p.q, np.repeat(p.k, 4, axis=1),
                      np.repeat(p.v, 4, axis=1), None, p.sinks)
    a = from_device(run_gpu(p), F16)
    b = from_device(run_gpu(rep), F16)
    bad, _, _ = compare(a, b, F16)
    assert bad == 0
