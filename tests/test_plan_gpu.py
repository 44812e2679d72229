"""Plans against what runs, on the GPU (nuvec-core "tests/attention_plan.rs":
plans_name_the_kernels_that_run, scratch_is_within_the_plan, plans_are_pure).

Kernels: one call is captured into a HIP graph (never launched) and its kernel
nodes are counted and their launch shapes read back; the count must be the
plan's `kernels`, and the attention kernel's grid and block the plan's `grid`
and `waves` x 64. Scratch: the library takes its scratch from the device's
default stream-ordered memory pool, which nothing else in the process uses, so
the pool's used bytes after a call (from a released workspace) are the
scratch the call holds: at least the plan's `scratch_bytes`, and no more than
that rounded up to the library's 1 MiB granule."""
import ctypes

import numpy as np
import pytest

import scaled_dot_product_06_amd as sd
from scaled_dot_product_06_amd import inputs as gen
from tests.gpu_util import say, to_device

pytestmark = pytest.mark.gpu

F32, F16, BF16 = gen.F32, gen.F16, gen.BF16
MIB = 1 << 20


class Dim3(ctypes.Structure):
    _fields_ = [("x", ctypes.c_uint32), ("y", ctypes.c_uint32), ("z", ctypes.c_uint32)]


class KernelNodeParams(ctypes.Structure):
    # hipKernelNodeParams (hip_runtime_api.h)
    _fields_ = [("blockDim", Dim3), ("extra", ctypes.c_void_p), ("func", ctypes.c_void_p), ("gridDim", Dim3),
                ("kernelParams", ctypes.c_void_p), ("sharedMemBytes", ctypes.c_uint32)]


_HIP = None


def hip():
    """The HIP runtime torch has loaded (same soname as the library's)."""
    global _HIP
    if _HIP is None:
        import torch
        torch.cuda.init()
        h = ctypes.CDLL("libamdhip64.so.7")
        vp, P = ctypes.c_void_p, ctypes.POINTER
        h.hipStreamBeginCapture.argtypes = [vp, ctypes.c_int]
        h.hipStreamEndCapture.argtypes = [vp, P(vp)]
        h.hipGraphGetNodes.argtypes = [vp, vp, P(ctypes.c_size_t)]
        h.hipGraphNodeGetType.argtypes = [vp, P(ctypes.c_int)]
        h.hipGraphKernelNodeGetParams.argtypes = [vp, P(KernelNodeParams)]
        h.hipGraphDestroy.argtypes = [vp]
        h.hipDeviceGetDefaultMemPool.argtypes = [P(vp), ctypes.c_int]
        h.hipMemPoolGetAttribute.argtypes = [vp, ctypes.c_int, vp]
        _HIP = h
    return _HIP


def captured_kernels(call, stream):
    """[(grid, block)] of the kernel nodes one call records on `stream`, plus the
    types of any other nodes. The graph is destroyed, never launched."""
    h = hip()
    assert h.hipStreamBeginCapture(stream, 2) == 0          # relaxed capture mode
    graph = ctypes.c_void_p()
    try:
        call()
    finally:
        rc = h.hipStreamEndCapture(stream, ctypes.byref(graph))
    assert rc == 0
    n = ctypes.c_size_t(0)
    assert h.hipGraphGetNodes(graph, None, ctypes.byref(n)) == 0
    nodes = (ctypes.c_void_p * max(n.value, 1))()
    assert h.hipGraphGetNodes(graph, nodes, ctypes.byref(n)) == 0
    kernels, others = [], []
    for i in range(n.value):
        t = ctypes.c_int(-1)
        assert h.hipGraphNodeGetType(nodes[i], ctypes.byref(t)) == 0
        if t.value == 0:
            prm = KernelNodeParams()
            assert h.hipGraphKernelNodeGetParams(nodes[i], ctypes.byref(prm)) == 0
            kernels.append(((prm.gridDim.x, prm.gridDim.y, prm.gridDim.z),
                            (prm.blockDim.x, prm.blockDim.y, prm.blockDim.z)))
        else:
            others.append(t.value)
    assert h.hipGraphDestroy(graph) == 0
    return kernels, others


def pool_used_bytes():
    h = hip()
    pool = ctypes.c_void_p()
    assert h.hipDeviceGetDefaultMemPool(ctypes.byref(pool), 0) == 0
    used = ctypes.c_uint64(0)
    assert h.hipMemPoolGetAttribute(pool, 7, ctypes.byref(used)) == 0   # hipMemPoolAttrUsedMemCurrent
    return used.value


def _case(kind, B, Hq, Hkv, Lq, Lk, D, Dv, dtype, window=0, bs=16):
    """(plan, call(stream)) of one case: kind 0/1/2 the plain mask kinds, 3 additive,
    'win' a window, 'paged' a paged cache of blocks of bs positions."""
    import torch
    mask_kind = {"win": 1, "paged": 1}.get(kind, kind)
    p = gen.make_problem(8000 + Lq + Lk + D, B, Hq, Hkv, Lq, Lk, D, Dv, dtype, mask_kind if mask_kind != 3 else 0,
                         sinks=True)
    q, k, v = (to_device(a, dtype) for a in (p.q, p.k, p.v))
    s = to_device(p.sinks, dtype)
    out = torch.empty((B, Hq, Lq, Dv), dtype=q.dtype, device="cuda")
    if kind == "paged":
        n = max(Lk, 1)
        per = -(-n // bs)
        blocks = B * per + 3
        order = gen.block_order(1, blocks)
        kc, table = gen.paged_cache(p.k, bs, order, blocks)
        vc, _ = gen.paged_cache(p.v, bs, order, blocks)
        dk, dv = to_device(kc, dtype), to_device(vc, dtype)
        dt = torch.from_numpy(table).cuda()
        dl = torch.full((B,), Lk, dtype=torch.int32, device="cuda")
        plan = sd.sdpa_plan_paged(B, Hq, Hkv, Lq, D, Dv, blocks, bs, per, 1, window, True, dtype)
        return plan, lambda st: sd.paged_attention(q, dk, dv, dt, dl, p.scale, 1, window, s, out=out, stream=st)
    if kind == "win":
        plan = sd.sdpa_plan_windowed(B, Hq, Hkv, Lq, Lk, D, Dv, window, True, dtype)
        return plan, lambda st: sd.attention(q, k, v, p.scale, 1, None, s, out=out, stream=st, window=window)
    mask = None
    if kind == 2:
        mask = torch.from_numpy(p.mask).cuda()
    elif kind == 3:
        mask = to_device(gen.additive_mask(1, (1, Hq, Lq, Lk), dtype, 0.1), dtype)
    plan = sd.sdpa_plan(B, Hq, Hkv, Lq, Lk, D, Dv, kind, mask is not None, True, dtype)
    return plan, lambda st: sd.attention(q, k, v, p.scale, kind, mask, s, out=out, stream=st)


# (kind, B, Hq, Hkv, Lq, Lk, D, Dv, dtype[, window]): every route and launch count
CASES = [
    (1, 1, 64, 8, 512, 300, 128, 128, BF16),       # pipelined prefill (a grid it fills)
    (2, 1, 64, 8, 512, 300, 128, 128, F16),        # mask packing + pipelined prefill
    (1, 2, 8, 2, 300, 300, 128, 128, BF16),        # key-split prefill (128-wide heads, small grid)
    (0, 1, 8, 2, 77, 150, 256, 256, F16),          # key-split prefill (256-wide heads)
    (2, 1, 16, 2, 100, 300, 256, 256, BF16),       # key-split prefill reading the mask bytes: one kernel
    (0, 1, 8, 2, 77, 150, 192, 128, F16),          # key-split prefill (192-wide K, 128-wide V)
    (0, 1, 8, 2, 77, 150, 512, 512, F16),          # generic prefill (512-wide heads)
    (1, 1, 64, 8, 512, 300, 96, 96, BF16),         # pipelined prefill (96-wide heads in the 128-wide layout)
    (2, 1, 8, 2, 200, 333, 64, 64, F16),           # key-split prefill (64-wide heads, small grid), byte mask
    (2, 1, 64, 8, 512, 333, 64, 64, F16),          # mask packing + pipelined prefill (64-wide heads)
    (2, 1, 4, 2, 70, 90, 128, 128, F32),           # f32 prefill, byte mask
    (3, 1, 64, 8, 512, 257, 128, 128, BF16),       # additive mask: key-split prefill (128-wide heads, a large grid)
    (3, 1, 64, 8, 512, 257, 64, 64, BF16),         # additive mask: generic prefill (64-wide heads, a large grid)
    (3, 1, 8, 2, 100, 257, 128, 128, BF16),        # additive mask: key-split prefill (small grid)
    (1, 2, 16, 2, 1, 65537, 256, 256, BF16),       # long decode: split + reduce
    (2, 1, 32, 4, 1, 8193, 128, 128, BF16),        # decode with a byte mask
    (3, 1, 8, 2, 3, 999, 96, 64, F16),             # decode with an additive mask
    (0, 1, 8, 2, 5, 0, 128, 128, BF16),            # no keys: zero fill
    (0, 1, 8, 2, 0, 100, 128, 128, BF16),          # no queries: nothing
    ("win", 4, 16, 2, 1, 65537, 256, 256, BF16, 4096),
    ("win", 2, 32, 8, 700, 700, 128, 128, BF16, 128),
    ("paged", 2, 8, 2, 1, 3000, 128, 128, BF16, 0),
    ("paged", 2, 8, 2, 4, 2100, 64, 64, F16, 300),
]


def _ids(c):
    return "-".join(str(x) for x in c)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_plans_name_the_kernels_that_run(case):
    import torch
    kind, B, Hq, Hkv, Lq, Lk, D, Dv, dtype = case[:9]
    window = case[9] if len(case) > 9 else 0
    plan, call = _case(kind, B, Hq, Hkv, Lq, Lk, D, Dv, dtype, window)
    say(f"{_ids(case)}: {plan}")
    stream = torch.cuda.Stream()
    call(stream.cuda_stream)              # the first call may grow the scratch (not captured)
    torch.cuda.synchronize()
    kernels, others = captured_kernels(lambda: call(stream.cuda_stream), stream.cuda_stream)
    say(f"  captured kernels {kernels}, other nodes {others}")
    assert others == []
    assert len(kernels) == plan["kernels"]
    if plan["route"] in ("prefill", "decode"):
        want = (tuple(int(g) for g in plan["grid"]), (plan["waves"] * 64, 1, 1))
        assert want in kernels, (want, kernels)
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", [c for c in CASES if c[0] != "paged"], ids=_ids)
def test_scratch_is_within_the_plan(case):
    import torch
    kind, B, Hq, Hkv, Lq, Lk, D, Dv, dtype = case[:9]
    window = case[9] if len(case) > 9 else 0
    plan, call = _case(kind, B, Hq, Hkv, Lq, Lk, D, Dv, dtype, window)
    torch.cuda.synchronize()
    sd.sdpa_release_workspace()
    base = pool_used_bytes()
    stream = torch.cuda.Stream()
    call(stream.cuda_stream)
    torch.cuda.synchronize()
    used = pool_used_bytes() - base
    want = plan["scratch_bytes"]
    say(f"{_ids(case)}: plan scratch {want} B, pool holds {used} B")
    assert want <= used <= -(-want // MIB) * MIB
    sd.sdpa_release_workspace()
    assert pool_used_bytes() == base


def test_paged_scratch_is_within_the_plan():
    import torch
    plan, call = _case("paged", 2, 8, 2, 1, 3000, 128, 128, BF16, 0)
    torch.cuda.synchronize()
    sd.sdpa_release_workspace()
    base = pool_used_bytes()
    call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    used = pool_used_bytes() - base
    assert plan["scratch_bytes"] <= used <= -(-plan["scratch_bytes"] // MIB) * MIB
    sd.sdpa_release_workspace()


def test_plans_are_pure_under_memory_pressure():
    import torch
    args = [(1, 16, 2, 1, 65537, 256, 256, 0, False, False, BF16), (2, 32, 8, 4096, 4096, 128, 128, 1, False, False, BF16),
            (1, 16, 2, 1024, 1801, 256, 256, 2, True, True, F16), (1, 8, 8, 128, 128, 64, 64, 1, False, False, F32)]
    before = [sd.sdpa_plan(*a) for a in args]
    big = torch.empty(256 << 20, dtype=torch.float32, device="cuda")   # 1 GiB held
    big.fill_(1.0)
    torch.cuda.synchronize()
    assert [sd.sdpa_plan(*a) for a in args] == before
    del big
    torch.cuda.empty_cache()
