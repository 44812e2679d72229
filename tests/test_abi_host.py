"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/sdpa.h declares, and sdpa_plan validates and routes as
documented (errors are return codes with a message naming the argument)."""
import ctypes
import os
import re
import subprocess
import sys
import threading

import pytest

import scaled_dot_product_06_amd as sd
from scaled_dot_product_06_amd import inputs as gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdpa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char\*)\s+(sdpa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_expected_entry_points():
    assert _declared_functions() == sorted(sd.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(sd.library_path())
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert sd.sdpa_abi_version() == 5
    out = subprocess.run(["nm", "-D", "--defined-only", sd.library_path()], capture_output=True, text=True).stdout
    for name in _declared_functions():
        assert re.search(rf"\bT {name}$", out, flags=re.M), f"{name} not exported with C linkage"


def _plan(B=1, Hq=8, Hkv=2, Lq=128, Lk=128, D=128, Dv=128, mask=0, has_mask=None, sinks=0, dtype=2):
    if has_mask is None:
        has_mask = mask == 2
    return sd.sdpa_plan(B, Hq, Hkv, Lq, Lk, D, Dv, mask, has_mask, sinks, dtype, check=False)


@pytest.mark.parametrize("number,route", [(1, "prefill"), (2, "decode"), (3, "prefill"), (4, "prefill"),
                                          (5, "decode")])
def test_workload_routes(number, route):
    w = gen.WORKLOADS[number]
    p = sd.sdpa_plan(w["B"], w["Hq"], w["Hkv"], w["Lq"], w["Lk"], w["D"], w["Dv"], w["mask_kind"],
                     w["mask_kind"] == 2, w["sinks"], w["dtype"])
    assert p["route"] == route
    if route == "decode":
        assert p["kernels"] == 2
        rows = w["Hq"] // w["Hkv"] * w["Lq"]
        assert p["splits"] * p["keys_per_split"] >= w["Lk"] > (p["splits"] - 1) * p["keys_per_split"]
        assert p["scratch_bytes"] == w["B"] * w["Hkv"] * p["splits"] * rows * (w["Dv"] + 4) * 4
        assert p["grid"] == (p["splits"], w["Hkv"], w["B"])
    elif w["mask_kind"] == 2 and w["dtype"] != 0 and p["splits"] != 2:
        # 16-bit prefill with a boolean mask: the mask is first packed into bits
        assert p["kernels"] == 2 and p["scratch_bytes"] == w["Lq"] * -(-w["Lk"] // 32) * 4
    else:
        assert p["kernels"] == 1 and p["scratch_bytes"] == 0
    if route == "prefill":
        if p["splits"] and w["dtype"] == 0:
            # the waves of a workgroup split the keys of one query block
            assert p["splits"] == p["waves"] and p["heads_per_group"] == 1
            rows_per_block = p["rows_per_wave"]
        elif p["splits"]:
            # 256-wide 16-bit heads: two key lanes of wavefronts
            assert (w["D"], p["splits"], p["rows_per_wave"], p["block_n"]) == (256, 2, 16, 32)
            rows_per_block = p["waves"] // p["splits"] // p["heads_per_group"] * p["rows_per_wave"]
        else:
            rows_per_block = p["waves"] // p["heads_per_group"] * p["rows_per_wave"]
        head_blocks = w["B"] * w["Hq"] // p["heads_per_group"]
        assert p["grid"] == (head_blocks * -(-w["Lq"] // rows_per_block), 1, 1)


def test_small_f32_calls_split_keys_within_a_workgroup():
    # workload 1: 8 heads x 128 rows; a 32-row grid would have 8 workgroups
    p = _plan(B=1, Hq=8, Hkv=8, Lq=128, Lk=128, D=64, Dv=64, mask=1, dtype=0)
    assert (p["rows_per_wave"], p["splits"], p["heads_per_group"], p["grid"]) == (16, 4, 1, (64, 1, 1))
    # the rule looks at one batch item, so the batch keeps the tiles
    q = _plan(B=5, Hq=8, Hkv=8, Lq=128, Lk=128, D=64, Dv=64, mask=1, dtype=0)
    assert (q["rows_per_wave"], q["splits"], q["grid"]) == (16, 4, (320, 1, 1))
    # large f32 calls keep the 32-row walk; 16-bit calls never take this split (small
    # 16-bit grids of heads up to 128 wide take the key-split kernel's two key lanes of eight waves
    # instead, large ones the pipelined kernel)
    big = _plan(B=1, Hq=32, Hkv=8, Lq=4096, Lk=4096, D=128, Dv=128, mask=1, dtype=0)
    assert (big["rows_per_wave"], big["splits"]) == (32, 0)
    assert (_plan(dtype=2)["splits"], _plan(dtype=2)["waves"]) == (2, 8)
    assert _plan(D=64, Dv=64, dtype=2)["splits"] == 2
    assert _plan(B=1, Hq=64, Hkv=8, Lq=1024, Lk=1024, D=64, Dv=64, dtype=2)["splits"] == 0
    # additive masks keep the generic walk at 16 rows
    add = _plan(B=1, Hq=8, Hkv=8, Lq=128, Lk=128, D=64, Dv=64, mask=3, has_mask=True, dtype=0)
    assert (add["rows_per_wave"], add["splits"]) == (16, 0)


def test_decode_split_size_depends_on_keys_not_batch():
    a = _plan(B=1, Hq=32, Hkv=4, Lq=1, Lk=20000)
    b = _plan(B=7, Hq=32, Hkv=4, Lq=1, Lk=20000)
    assert a["keys_per_split"] == b["keys_per_split"] and a["splits"] == b["splits"]


def test_routing_thresholds():
    assert _plan(Lq=8, Hq=4, Hkv=1)["route"] == "decode"        # 32 rows
    assert _plan(Lq=9, Hq=4, Hkv=1)["route"] == "prefill"       # more than 8 queries
    assert _plan(Lq=5, Hq=8, Hkv=1)["route"] == "prefill"       # 40 rows do not fit a tile
    assert _plan(Lq=1, dtype=0)["route"] == "prefill"           # f32 always tiles


def test_empty_and_keyless_routes():
    assert _plan(Lq=0)["route"] == "empty"
    assert _plan(B=0)["route"] == "empty"
    assert _plan(Hq=0, Hkv=0)["route"] == "empty"
    p = _plan(Lk=0, mask=1, sinks=1)
    assert p["route"] == "zero_fill" and p["kernels"] == 1


@pytest.mark.parametrize("kwargs,code,needle", [
    (dict(Hq=3, Hkv=2), -1, "multiple of Hkv"),
    (dict(Hq=4, Hkv=0), -1, "Hkv"),
    (dict(B=-1), -1, "B must be"),
    (dict(Lk=-5), -1, "Lk must be"),
    (dict(dtype=3), -1, "dtype"),
    (dict(mask=3), -1, "mask_kind"),
    (dict(mask=2, has_mask=False), -1, "mask is NULL"),
    (dict(D=100, Dv=100), -2, "head sizes"),
    (dict(D=128, Dv=64), -2, "head sizes"),
    (dict(B=1 << 40, Hq=1 << 20, Hkv=1 << 20, Lq=1 << 20), -1, "overflow"),
])
def test_invalid_arguments_are_rejected(kwargs, code, needle):
    rc = _plan(**kwargs)
    assert rc == code
    assert needle in sd.sdpa_last_error()


def test_forward_validates_before_touching_memory():
    # No GPU needed: every one of these fails validation before any HIP call.
    f = sd.sdpa_forward
    assert f(None, None, None, None, 1, 3, 2, 4, 4, 64, 64, 0.1, 0, None, None, 2, None, check=False) == -1
    assert "multiple" in sd.sdpa_last_error()
    assert f(None, None, None, None, 1, 2, 2, 4, 4, 64, 64, float("nan"), 0, None, None, 2, None,
             check=False) == -1
    assert "scale" in sd.sdpa_last_error()
    assert f(None, None, None, None, 1, 2, 2, 4, 4, 64, 64, 0.1, 2, None, None, 2, None, check=False) == -1
    assert "mask" in sd.sdpa_last_error()
    assert f(None, None, None, None, 1, 2, 2, 4, 4, 64, 64, 0.1, 0, None, None, 2, None, check=False) == -1
    assert "NULL" in sd.sdpa_last_error()
    assert f(16, 16, 16, 8, 1, 2, 2, 4, 4, 64, 64, 0.1, 0, None, None, 2, None, check=False) == -1
    assert "aligned" in sd.sdpa_last_error()
    # an empty call is a successful no-op, even with null pointers
    assert f(None, None, None, None, 1, 2, 2, 0, 4, 64, 64, 0.1, 0, None, None, 2, None, check=False) == 0


def test_plans_are_pure_across_repeats_and_threads():
    cases = [dict(Lq=1, Lk=65537, Hq=16, Hkv=2, D=256, Dv=256), dict(Lq=4096, Lk=4096, Hq=32, Hkv=8),
             dict(Lq=1024, Lk=1801, Hq=16, Hkv=2, D=256, Dv=256, mask=2, sinks=1, dtype=1)]
    first = [_plan(**c) for c in cases]
    for _ in range(100):
        assert [_plan(**c) for c in cases] == first
    got = []
    t = threading.Thread(target=lambda: got.extend(_plan(**c) for c in cases))
    t.start()
    t.join()
    assert got == first
    code = ("import scaled_dot_product_06_amd as sd, json; "
            f"print(json.dumps([sd.sdpa_plan(*a) for a in {[(1, c.get('Hq', 8), c.get('Hkv', 2), c.get('Lq', 128), c.get('Lk', 128), c.get('D', 128), c.get('Dv', 128), c.get('mask', 0), c.get('mask', 0) == 2, c.get('sinks', 0), c.get('dtype', 2)) for c in cases]}]))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert out.returncode == 0, out.stderr
    import json
    other = json.loads(out.stdout)
    for a, b in zip(other, first):
        b = dict(b)
        b["grid"] = list(b["grid"])
        assert a == b


def test_errors_are_per_thread():
    assert _plan(Hq=3, Hkv=2) == -1
    msgs = []
    t = threading.Thread(target=lambda: msgs.append(sd.sdpa_last_error()))
    t.start()
    t.join()
    assert msgs == [""]
    assert "multiple" in sd.sdpa_last_error()


# --- windowed calls ---------------------------------------------------------------------------

def test_full_window_plans_as_causal():
    for lq, lk in [(1, 4096), (5, 300), (300, 700)]:
        causal = sd.sdpa_plan(1, 8, 2, lq, lk, 128, 128, 1, False, True, 2)
        for w in (lk, lk + 1, 1 << 30):
            assert sd.sdpa_plan_windowed(1, 8, 2, lq, lk, 128, 128, w, True, 2) == causal


def test_windowed_decode_splits_follow_the_window():
    # attention_plan.rs, windowed_decode_plans_from_the_window_keys: the partitions follow
    # the keys the rows read, not the cache length
    causal = sd.sdpa_plan(1, 64, 8, 1, 4096, 64, 64, 1, False, False, 1)
    win = sd.sdpa_plan_windowed(1, 64, 8, 1, 4096, 64, 64, 128, False, 1)
    alone = sd.sdpa_plan(1, 64, 8, 1, 128, 64, 64, 0, False, False, 1)
    assert win["route"] == causal["route"] == "decode"
    assert win["splits"] * win["keys_per_split"] >= 128 > (win["splits"] - 1) * win["keys_per_split"]
    assert win["splits"] < causal["splits"]
    assert (win["keys_per_split"], win["splits"]) == (alone["keys_per_split"], alone["splits"])
    # several query rows read the union of their windows
    w4 = sd.sdpa_plan_windowed(1, 8, 2, 4, 9000, 128, 128, 300, False, 2)
    assert w4["splits"] * w4["keys_per_split"] >= 303


@pytest.mark.parametrize("window", [0, -1, -(1 << 40)])
def test_invalid_windows_are_rejected(window):
    assert sd.sdpa_plan_windowed(1, 4, 2, 5, 9, 64, 64, window, False, 2, check=False) == -1
    assert "window" in sd.sdpa_last_error()
    f = sd.sdpa_forward_windowed
    assert f(None, None, None, None, 1, 4, 2, 5, 9, 64, 64, 0.1, window, None, 2, None, check=False) == -1
    assert "window" in sd.sdpa_last_error()


# --- paged calls ------------------------------------------------------------------------------

def _plan_paged(B=2, Hq=8, Hkv=2, Lq=1, D=128, Dv=128, blocks=40, bs=16, max_blocks=20, mask=1, window=0,
                sinks=0, dtype=2):
    return sd.sdpa_plan_paged(B, Hq, Hkv, Lq, D, Dv, blocks, bs, max_blocks, mask, window, sinks, dtype,
                              check=False)


def test_paged_plans_are_decode_plans_over_the_capacity():
    # fast.rs, paged_attention_equals_contiguous_attention: with two passes the key
    # partitions follow the table's capacity (max_blocks * bs), not the lengths
    for (B, Hq, Hkv, Lq, D, bs, mb) in [(2, 8, 2, 1, 128, 32, 94), (1, 8, 2, 4, 128, 64, 33),
                                        (3, 8, 2, 1, 128, 32, 10), (2, 4, 1, 4, 64, 16, 5)]:
        p = _plan_paged(B=B, Hq=Hq, Hkv=Hkv, Lq=Lq, D=D, Dv=D, bs=bs, max_blocks=mb)
        c = sd.sdpa_plan(B, Hq, Hkv, Lq, mb * bs, D, D, 1, False, False, 2)
        assert p == c, (p, c)


def test_paged_window_plans_follow_the_window():
    full = _plan_paged(Lq=1, bs=32, max_blocks=128)
    win = _plan_paged(Lq=1, bs=32, max_blocks=128, window=128)
    assert win["splits"] * win["keys_per_split"] >= 128 and win["splits"] < full["splits"]
    four = _plan_paged(Lq=4, bs=32, max_blocks=128, window=300)
    assert four["splits"] * four["keys_per_split"] >= 303
    assert _plan_paged(window=1 << 30) == _plan_paged()


@pytest.mark.parametrize("kwargs,code,needle", [
    (dict(mask=2), -1, "mask_kind"),
    (dict(mask=0, window=5), -1, "window"),
    (dict(window=-1), -1, "window"),
    (dict(blocks=0), -1, "blocks"),
    (dict(bs=0), -1, "bs"),
    (dict(max_blocks=0), -1, "max_blocks"),
    (dict(Hq=4, Hkv=3), -1, "multiple"),
    (dict(dtype=7), -1, "dtype"),
    (dict(Lq=9), -2, "decode"),
    (dict(Hq=66, Hkv=2, Lq=1), -2, "decode"),
    (dict(D=72, Dv=72), -2, "head sizes"),
    (dict(bs=1 << 20, max_blocks=1 << 20), -2, "capacity"),
])
def test_invalid_paged_arguments_are_rejected(kwargs, code, needle):
    assert _plan_paged(**kwargs) == code
    assert needle in sd.sdpa_last_error()


def test_paged_forward_validates_before_touching_memory():
    f = sd.sdpa_paged_forward
    args = dict(B=1, Hq=4, Hkv=2, Lq=1, D=64, Dv=64, blocks=4, bs=8, max_blocks=2, scale=0.1, mask_kind=1,
                window=0, sinks=None, dtype=2, stream=None)

    def call(ptrs, **over):
        a = dict(args, **over)
        return f(*ptrs, a["B"], a["Hq"], a["Hkv"], a["Lq"], a["D"], a["Dv"], a["blocks"], a["bs"],
                 a["max_blocks"], a["scale"], a["mask_kind"], a["window"], a["sinks"], a["dtype"], a["stream"],
                 check=False)

    none = (None,) * 6
    assert call(none) == -1 and "NULL" in sd.sdpa_last_error()
    assert call((16, 16, 16, 16, None, 16)) == -1 and "table" in sd.sdpa_last_error()
    assert call((16, 16, 16, 8, 16, 16)) == -1 and "aligned" in sd.sdpa_last_error()
    assert call((16, 16, 16, 16, 16, 18)) == -1 and "aligned" in sd.sdpa_last_error()
    assert call(none, scale=float("inf")) == -1 and "scale" in sd.sdpa_last_error()
    assert call(none, Hkv=3) == -1 and "multiple" in sd.sdpa_last_error()
    # empty calls are successful no-ops, even with null pointers
    assert call(none, Lq=0) == 0
    assert call(none, B=0) == 0


def test_paged_write_validates_before_touching_memory():
    w = sd.sdpa_paged_write
    assert w(None, None, None, 3, 6, 2, 4, 64, 2, None, check=False) == -1
    assert "NULL" in sd.sdpa_last_error()
    assert w(None, None, None, -1, 6, 2, 4, 64, 2, None, check=False) == -1
    assert w(None, None, None, 3, 6, 2, 0, 64, 2, None, check=False) == -1
    assert "bs" in sd.sdpa_last_error()
    assert w(None, None, None, 3, 6, 2, 4, 63, 2, None, check=False) == -2
    assert "16 bytes" in sd.sdpa_last_error()
    assert w(None, None, None, 3, 6, 2, 4, 64, 9, None, check=False) == -1
    assert w(16, 16, 18, 3, 6, 2, 4, 64, 2, None, check=False) == -1
    assert "aligned" in sd.sdpa_last_error()
    assert w(None, None, None, 0, 6, 2, 4, 64, 2, None, check=False) == 0
    # f32 rows of 4 elements are 16 bytes
    assert w(None, None, None, 0, 6, 2, 4, 4, 0, None, check=False) == 0


# --- strided views and additive masks ----------------------------------------------------------

def _strided(q=(16, 4 * 5 * 64, 5 * 64, 64), k=(16, 2 * 9 * 64, 9 * 64, 64), v=(16, 2 * 9 * 64, 9 * 64, 64),
             mask_kind=0, mask=None, window=0, B=1, Hq=4, Hkv=2, Lq=5, Lk=9, D=64, Dv=64, dtype=2, out=16,
             scale=0.1):
    return sd.sdpa_forward_strided(q, k, v, out, B, Hq, Hkv, Lq, Lk, D, Dv, scale, mask_kind, mask, None, window,
                                   dtype, None, check=False)


def test_additive_masks_plan_off_the_pipelined_kernel():
    # the pipelined kernel reads no additive mask: on a grid it fills (32 heads x 4096
    # rows), 128-wide heads with an additive mask take the key-split kernel and
    # 64- and 96-wide ones the generic kernel
    fast = sd.sdpa_plan(1, 32, 8, 4096, 4096, 128, 128, 0, False, False, 2)
    add = sd.sdpa_plan(1, 32, 8, 4096, 4096, 128, 128, 3, True, False, 2)
    assert fast["route"] == add["route"] == "prefill"
    assert (fast["block_n"], fast["splits"], add["block_n"], add["splits"]) == (32, 0, 32, 2)
    for d in (64, 96):
        gen_add = sd.sdpa_plan(1, 32, 8, 4096, 4096, d, d, 3, True, False, 2)
        assert (gen_add["rows_per_wave"], gen_add["block_n"], gen_add["splits"]) == (32, 64, 0)
    # on a small grid heads up to 128 wide take the key-split kernel
    small = sd.sdpa_plan(1, 8, 2, 300, 300, 128, 128, 3, True, False, 2)
    assert (small["splits"], small["rows_per_wave"]) == (2, 16)
    for d, dv in ((64, 64), (80, 80), (96, 96), (96, 64)):
        small = sd.sdpa_plan(1, 8, 2, 300, 300, d, dv, 3, True, False, 2)
        assert (small["splits"], small["rows_per_wave"], small["block_n"]) == (2, 16, 32)
    dec = sd.sdpa_plan(1, 8, 2, 1, 3000, 128, 128, 3, True, False, 2)
    assert dec["route"] == "decode"
    assert sd.sdpa_plan(1, 8, 2, 1, 3000, 128, 128, 3, False, False, 2, check=False) == -1
    assert "ADDITIVE" in sd.sdpa_last_error()


def test_strided_call_validates_before_touching_memory():
    assert _strided(q=None) == -1 and "views" in sd.sdpa_last_error()
    assert _strided(k=(16, -64, 64, 64)) == -1 and ">= 0" in sd.sdpa_last_error()
    assert _strided(v=(16, 0, 0, 36)) == -1 and "16-byte" in sd.sdpa_last_error()   # 72-byte rows
    assert _strided(q=(8, 0, 0, 64)) == -1 and "aligned" in sd.sdpa_last_error()
    assert _strided(k=(16, 0, 0, 1 << 25)) == -2 and "2^26" in sd.sdpa_last_error()
    assert _strided(q=(16, 1 << 62, 0, 64), B=3) == -1 and "overflow" in sd.sdpa_last_error()
    assert _strided(mask_kind=2) == -1 and "mask view" in sd.sdpa_last_error()
    assert _strided(mask_kind=2, mask=(16, 0, 0, 10)) == -2 and "boolean" in sd.sdpa_last_error()
    assert _strided(mask_kind=3) == -1 and "mask view" in sd.sdpa_last_error()
    assert _strided(mask_kind=3, mask=(17, 0, 0, 9)) == -1 and "element size" in sd.sdpa_last_error()
    assert _strided(mask_kind=3, mask=(16, 0, 0, 9), window=4) == -1 and "window" in sd.sdpa_last_error()
    assert _strided(mask_kind=1, window=-2) == -1 and "window" in sd.sdpa_last_error()
    assert _strided(scale=float("nan")) == -1 and "scale" in sd.sdpa_last_error()
    # empty calls are successful no-ops
    assert _strided(Lq=0) == 0 and _strided(B=0) == 0


def test_contiguous_call_refuses_an_additive_mask():
    f = sd.sdpa_forward
    assert f(16, 16, 16, 16, 1, 2, 2, 4, 4, 64, 64, 0.1, 3, 16, None, 2, None, check=False) == -1
    assert "sdpa_forward_strided" in sd.sdpa_last_error()


def test_f32_paged_plans_are_prefill_plans():
    # f32 paged calls run the f32 tiled kernel over the capacity's keys, for any Lq
    for Lq in (1, 4, 9, 300):
        p = _plan_paged(Lq=Lq, dtype=0)
        assert p["route"] == "prefill" and p["scratch_bytes"] == 0
        assert p == sd.sdpa_plan(2, 8, 2, Lq, 20 * 16, 128, 128, 1, False, False, 0)


def test_key_split_plans_for_wide_heads_and_small_64_and_128_wide_grids():
    # 256-wide 16-bit heads take the key-split 16-row kernel whatever the grid (it
    # measured faster than 32-row tiles, one wavefront per SIMD, on full grids too);
    # the batch size never changes the geometry
    def shape(p):
        return p["rows_per_wave"], p["block_n"], p["splits"], p["waves"]
    big = sd.sdpa_plan(1, 32, 4, 1040, 1297, 256, 256, 1, False, False, 2)   # 8 x 65 workgroups
    assert shape(big) + (big["grid"][0],) == (16, 32, 2, 8, 8 * 65)
    assert shape(sd.sdpa_plan(3, 32, 4, 1040, 1297, 256, 256, 1, False, False, 2)) == (16, 32, 2, 8)
    under = sd.sdpa_plan(1, 32, 4, 992, 1297, 256, 256, 1, False, False, 2)  # 8 x 62
    assert shape(under) + (under["grid"][0],) == (16, 32, 2, 8, 8 * 62)
    small = sd.sdpa_plan(1, 16, 2, 1024, 1801, 256, 256, 2, True, True, 1)  # workload 4: 4 x 64
    # the key-split kernel reads the boolean mask's bytes: one kernel, no scratch
    assert shape(small) + (small["grid"][0], small["kernels"], small["scratch_bytes"]) == (16, 32, 2, 8, 4 * 64, 1, 0)
    # the pipelined kernel (128-wide heads on a grid it fills) packs it first
    packed = sd.sdpa_plan(1, 64, 8, 1024, 1801, 128, 128, 2, True, True, 1)   # 16 x 32 workgroups
    assert (packed["kernels"], packed["scratch_bytes"]) == (2, 1024 * 57 * 4)
    # 128-wide heads on a small grid: the key-split kernel, which reads the bytes itself
    small128 = sd.sdpa_plan(1, 16, 2, 1024, 1801, 128, 128, 2, True, True, 1)  # 4 x 32 for the pipelined kernel
    assert shape(small128) + (small128["kernels"], small128["scratch_bytes"]) == (16, 32, 2, 8, 1, 0)
    # the threshold: 256 pipelined workgroups per batch item keep the pipelined kernel,
    # at every head pair up to 128 wide; the batch size never changes the kernel
    for d, dv in ((64, 64), (80, 80), (96, 96), (128, 128), (96, 64)):
        assert shape(sd.sdpa_plan(1, 32, 4, 1024, 1024, d, dv, 1, False, False, 2)) == (32, 32, 0, 4)   # 8 x 32
        assert shape(sd.sdpa_plan(1, 32, 4, 992, 1024, d, dv, 1, False, False, 2)) == (16, 32, 2, 8)    # 8 x 31
        assert shape(sd.sdpa_plan(4, 32, 4, 992, 1024, d, dv, 1, False, False, 2)) == (16, 32, 2, 8)    # per item
        assert shape(sd.sdpa_plan(9, 32, 4, 1024, 1024, d, dv, 1, False, False, 2)) == (32, 32, 0, 4)   # per item
    batched = sd.sdpa_plan(8, 16, 2, 1024, 1801, 256, 256, 2, True, True, 1)  # the same per batch item
    assert shape(batched) + (batched["grid"][0],) == (16, 32, 2, 8, 8 * 4 * 64)
    # one or two heads per workgroup: 64 or 32 rows of a head per key lane
    assert sd.sdpa_plan(1, 4, 4, 100, 300, 256, 256, 0, False, False, 2)["grid"][0] == 4 * 2
    assert sd.sdpa_plan(1, 4, 2, 100, 300, 256, 256, 0, False, False, 2)["grid"][0] == 2 * 4
    # additive masks take the key-split kernel at 192- and 256-wide heads too, at
    # 128-wide heads on every grid and at 64-, 80- and 96-wide heads on small grids; other calls
    # keep the generic kernel (the pipelined kernel reads no additive mask)
    add = sd.sdpa_plan(1, 64, 8, 1024, 1801, 256, 256, 3, True, True, 1)
    assert shape(add) + (add["kernels"], add["scratch_bytes"]) == (16, 32, 2, 8, 1, 0)
    big_add = sd.sdpa_plan(1, 32, 4, 1040, 1297, 256, 256, 3, True, False, 2)
    assert shape(big_add) == (16, 32, 2, 8)
    assert shape(sd.sdpa_plan(1, 64, 8, 1024, 1801, 128, 128, 3, True, True, 1)) == (16, 32, 2, 8)
    assert shape(sd.sdpa_plan(1, 64, 8, 1024, 1801, 64, 64, 3, True, True, 1)) == (32, 64, 0, 4)
    assert shape(sd.sdpa_plan(1, 16, 2, 1024, 1801, 128, 128, 3, True, True, 1)) == (16, 32, 2, 8)
    # heads of 192 columns take the key-split kernel on every grid, with every mask kind
    for dv in (192, 128):
        for mk in (0, 1, 2, 3):
            big192 = sd.sdpa_plan(1, 64, 8, 1024, 1801, 192, dv, mk, mk >= 2, True, 1)
            assert shape(big192) + (big192["kernels"], big192["scratch_bytes"]) == (16, 32, 2, 8, 1, 0)
