"""Calls in captured graphs and on concurrent streams.

The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph): each
route is captured once, after an eager call on the capture stream has sized the
stream's scratch (so the capture allocates nothing), then replayed several
times with eager work on the output in between; every replay must give the
eager call's bits. The library enqueues no memset nodes (zeros come from a
fill kernel), so replays after the first see the same work. And calls issued
from several host threads, each on its own stream, at once."""
import numpy as np
import pytest

import scaled_dot_product_06_amd as sd
from scaled_dot_product_06_amd import inputs as gen
from tests.gpu_util import to_device

pytestmark = pytest.mark.gpu

F32, F16, BF16 = gen.F32, gen.F16, gen.BF16


def _call(kind, B, Hq, Hkv, Lq, Lk, D, dtype):
    """(name, call(out, stream), out shape): one call of each route."""
    import torch
    mask_kind = {"window": 1, "paged": 1, "views": 1, "additive": 0}.get(kind, kind)
    p = gen.make_problem(9000 + Lq + Lk, B, Hq, Hkv, Lq, Lk, D, D, dtype, mask_kind, sinks=True)
    q, k, v = (to_device(a, dtype) for a in (p.q, p.k, p.v))
    s = to_device(p.sinks, dtype)
    mask = None if p.mask is None else torch.from_numpy(p.mask).cuda()
    if kind == "window":
        return lambda out, st: sd.attention(q, k, v, p.scale, 1, None, s, out=out, stream=st, window=33)
    if kind == "additive":
        add = to_device(gen.additive_mask(9, (1, Hq, Lq, Lk), dtype, 0.1), dtype)
        return lambda out, st: sd.attention(q, k, v, p.scale, 3, add, s, out=out, stream=st)
    if kind == "views":
        kt = to_device(np.ascontiguousarray(p.k.transpose(0, 2, 1, 3)), dtype).transpose(1, 2)
        return lambda out, st: sd.attention(q, kt, v, p.scale, 1, None, s, out=out, stream=st)
    if kind == "paged":
        bs = 16
        per = -(-Lk // bs)
        blocks = B * per + 3
        order = gen.block_order(3, blocks)
        kc, table = gen.paged_cache(p.k, bs, order, blocks)
        vc, _ = gen.paged_cache(p.v, bs, order, blocks)
        dk, dv = to_device(kc, dtype), to_device(vc, dtype)
        dt = torch.from_numpy(table).cuda()
        dl = torch.full((B,), Lk, dtype=torch.int32, device="cuda")
        return lambda out, st: sd.paged_attention(q, dk, dv, dt, dl, p.scale, 1, 0, s, out=out, stream=st)
    return lambda out, st: sd.attention(q, k, v, p.scale, mask_kind, mask, s, out=out, stream=st)


CASES = [
    (1, 1, 64, 8, 512, 300, 128, BF16),     # pipelined prefill (a grid it fills: 256 workgroups)
    (2, 1, 64, 8, 512, 257, 128, F16),      # mask packing + pipelined prefill (two kernels, scratch)
    (1, 2, 8, 2, 300, 300, 128, BF16),      # key-split prefill (128-wide heads, small grid)
    (2, 1, 8, 2, 300, 300, 64, F16),        # key-split prefill (64-wide heads, small grid), mask bytes
    (2, 1, 16, 2, 100, 300, 256, F16),      # key-split prefill reading the mask bytes
    (0, 1, 8, 2, 77, 150, 512, BF16),       # generic prefill (512-wide heads)
    (1, 1, 4, 2, 40, 70, 64, F32),          # f32 prefill
    (0, 2, 16, 2, 1, 9000, 256, BF16),      # decode split + reduce (scratch)
    (1, 1, 32, 4, 1, 8193, 128, BF16),      # the 8193-key decode: split + reduce
    (1, 1, 8, 2, 5, 0, 128, BF16),          # no keys: the fill kernel
    ("window", 1, 8, 2, 3, 2000, 128, BF16),
    ("additive", 1, 8, 2, 70, 257, 128, BF16),
    ("views", 1, 8, 2, 64, 200, 128, F16),
    ("paged", 2, 8, 2, 1, 3000, 128, BF16),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_graph_replays_equal_the_eager_call(case):
    import torch
    kind, B, Hq, Hkv, Lq, Lk, D, dtype = case
    call = _call(kind, B, Hq, Hkv, Lq, Lk, D, dtype)
    tdt = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}[dtype]
    stream = torch.cuda.Stream()
    want = torch.empty((B, Hq, Lq, D), dtype=tdt, device="cuda")
    with torch.cuda.stream(stream):
        call(want, stream.cuda_stream)          # sizes this stream's scratch
    torch.cuda.synchronize()
    out = torch.full_like(want, float("nan"))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        call(out, stream.cuda_stream)
    torch.cuda.synchronize()
    bits = torch.int32 if dtype == F32 else torch.int16
    for replay in range(4):
        out.fill_(float("nan"))                 # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(bits), want.view(bits)), f"replay {replay}"
    del graph
    torch.cuda.synchronize()


def test_concurrent_streams_and_threads():
    """Decode and masked-prefill calls (both use scratch) issued from four host threads,
    each on its own stream, with no synchronisation between them: the library keeps
    one scratch buffer per (device, stream), so every result is the single-stream one."""
    import threading

    import torch
    cases = [_call(0, 2, 16, 2, 1, 9000, 256, BF16), _call(2, 1, 8, 2, 100, 257, 128, F16),
             _call("window", 1, 8, 2, 3, 2000, 128, BF16), _call("paged", 2, 8, 2, 1, 3000, 128, BF16)]
    shapes = [(2, 16, 1, 256, torch.bfloat16), (1, 8, 100, 128, torch.float16), (1, 8, 3, 128, torch.bfloat16),
              (2, 8, 1, 128, torch.bfloat16)]
    wants = []
    for call, (B, H, L, D, dt) in zip(cases, shapes):
        w = torch.empty((B, H, L, D), dtype=dt, device="cuda")
        call(w, torch.cuda.current_stream().cuda_stream)
        wants.append(w)
    torch.cuda.synchronize()
    outs = [[torch.empty_like(w) for _ in range(8)] for w in wants]
    errors = []

    def worker(i):
        try:
            torch.cuda.set_device(0)
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for o in outs[i]:
                    cases[i](o, st.cuda_stream)
            st.synchronize()
        except Exception as e:          # reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for w, os_ in zip(wants, outs):
        bits = torch.int16
        for o in os_:
            assert torch.equal(o.view(bits), w.view(bits))


def test_graph_replays_after_a_larger_eager_call_on_its_stream():
    """A graph keeps the scratch it was captured with: a later eager call on the same
    stream that needs more scratch gets a new, larger buffer, and the captured graph's
    buffer stays allocated (retired, not freed), so replays still give the eager bits."""
    import torch
    small = _call(0, 2, 16, 2, 1, 9000, 256, BF16)
    large = _call(0, 2, 16, 2, 1, 262145, 256, BF16)
    plans = [sd.sdpa_plan(2, 16, 2, 1, L, 256, 256, 0, False, True, BF16) for L in (9000, 262145)]
    assert plans[1]["scratch_bytes"] > 2 * plans[0]["scratch_bytes"]
    stream = torch.cuda.Stream()
    want = torch.empty((2, 16, 1, 256), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(stream):
        small(want, stream.cuda_stream)         # sizes this stream's scratch for the small call
    torch.cuda.synchronize()
    out = torch.full_like(want, float("nan"))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        small(out, stream.cuda_stream)
    torch.cuda.synchronize()
    big_out = torch.empty((2, 16, 1, 256), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(stream):
        large(big_out, stream.cuda_stream)      # grows the stream's scratch
    torch.cuda.synchronize()
    for replay in range(3):
        out.fill_(float("nan"))
        with torch.cuda.stream(stream):
            large(big_out, stream.cuda_stream)  # eager work on the new buffer between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {replay}"
    del graph
    torch.cuda.synchronize()


def test_first_call_needing_scratch_inside_a_capture_is_refused():
    """A capture cannot allocate the stream's scratch: the call returns
    SDPA_ERR_UNSUPPORTED, names the plan's scratch_bytes, and enqueues nothing. A call
    that needs no scratch (an unmasked prefill) is captured as the stream's first call."""
    import torch
    decode = _call(0, 2, 16, 2, 1, 9000, 256, BF16)
    prefill = _call(1, 2, 8, 2, 300, 300, 128, BF16)
    stream = torch.cuda.Stream()
    out = torch.full((2, 16, 1, 256), 3.0, dtype=torch.bfloat16, device="cuda")
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(sd.SdpaError) as err:
        with torch.cuda.graph(graph, stream=stream):
            decode(out, stream.cuda_stream)
    assert err.value.code == sd.SDPA_ERR_UNSUPPORTED
    assert "scratch_bytes" in err.value.message
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
    del graph
    want = torch.empty((2, 8, 300, 128), dtype=torch.bfloat16, device="cuda")
    prefill(want, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    fresh = torch.cuda.Stream()
    got = torch.full_like(want, float("nan"))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=fresh):
        prefill(got, fresh.cuda_stream)
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    del graph
    torch.cuda.synchronize()
