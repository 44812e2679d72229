#!/usr/bin/env python3
"""Benchmark of the fused attention forward hot path on one MI355X.

One step = one pass over the whole path on one batch of synthetic input:
  * prefill: bf16 GQA causal prefill, B=2, Hq=32, Hkv=8, Lq=Lk=4096, D=Dv=128
    (one sdpa_forward call, routed to the tiled MFMA kernel);
  * decode:  bf16 GQA decode, B=4, Hq=16, Hkv=2, Lq=1, Lk=65537, D=Dv=256
    (one sdpa_forward call, routed to the split-key kernel and its reduce).
Inputs are resident in HBM before timing starts. The decode K/V alternates
between two copies (1.07 GB together, over four times the 256 MB MALL) so that
every decode step streams its K/V from HBM; prefill runs warm.

`value` is prefill TFLOP/s (causal pairs only, 2 FLOP per multiply-add over
QK^T and PV); the decode K/V GB/s sits in `decode`. Per-call kernel time is
taken with HIP events on the stream the library launches on. The printed JSON
line also carries the roofline fraction of the dominant kernel and the CPU
float64 oracle timed on a bounded sample of the same prefill workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PREFILL_WORKLOAD, DECODE_WORKLOAD = 3, 5


def causal_pairs(Lq: int, Lk: int, window: int = 0) -> int:
    """Visible (query, key) pairs of a bottom-right aligned causal mask, and of
    its sliding-window band (row at position pos reads pos - window < j <= pos)."""
    total = 0
    for i in range(Lq):
        pos = i + Lk - Lq
        hi = min(Lk, pos + 1)
        lo = max(0, pos - window + 1) if window else 0
        total += max(0, hi - lo)
    return total


def prefill_flop(p, window: int = 0) -> int:
    pairs = causal_pairs(p.Lq, p.Lk, window) if p.mask_kind == 1 else p.Lq * p.Lk
    return p.B * p.Hq * pairs * 2 * (p.D + p.Dv)


def decode_bytes(p, window: int = 0) -> int:
    """K/V bytes a decode call reads: every key, or the rows' windows."""
    esize = 4 if p.dtype == 0 else 2
    keys = min(p.Lk, window + p.Lq - 1) if window else p.Lk
    return p.B * p.Hkv * keys * (p.D + p.Dv) * esize


# The sources that define each profiled kernel (its code, its argument block and
# the device helpers it uses); a change to any of them voids its stored traffic.
KERNEL_SOURCES = {
    "prefill": ("attn_device.h", "kernels.h", "prefill_fast.h", "prefill_f16bf16.hip"),
    "decode": ("attn_device.h", "kernels.h", "decode_impl.h", "decode.hip"),
}


def _traffic_for(kernel_tag: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the kernel's current sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel_tag)
    except Exception:
        return None
    if not rec or rec.get("source_sha256") != kernel_source_hash(kernel_tag):
        return None
    return rec.get("bytes_per_launch")


def kernel_source_hash(kernel_tag: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "scaled_dot_product_06_amd", "csrc")
    for name in KERNEL_SOURCES[kernel_tag]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return 1


def _time_oracle(p, rows=None):
    """Seconds for one oracle evaluation of problem p (all rows, or the given ones)."""
    from oracle import attention as orc
    q, k, v, m, s = p.widened()
    t0 = time.perf_counter()
    orc.sdpa(q, k, v, p.scale, p.mask_kind, m, s, rows=rows)
    return time.perf_counter() - t0


def cpu_baseline(p, seconds: float, gen, dec=None):
    """Time the float64 oracle on the host cores: whole (batch, head) slices of
    the prefill workload `p` for about `seconds` (the reported value, in
    TFLOP/s), then each of the five workloads once, in its own unit, with all
    BLAS threads and, for the three small ones, on one thread. Input
    generation is outside the timed regions."""
    from oracle import attention as orc
    threads = _blas_threads()
    q, k, v, m, s = p.widened()
    group = p.Hq // p.Hkv
    per_head = causal_pairs(p.Lq, p.Lk) * 2 * (p.D + p.Dv)
    done = 0
    t0 = time.perf_counter()
    for b in range(p.B):
        for h in range(p.Hq):
            hk = h // group
            orc.sdpa(q[b:b + 1, h:h + 1], k[b:b + 1, hk:hk + 1], v[b:b + 1, hk:hk + 1],
                     p.scale, p.mask_kind, m, None if s is None else s[h:h + 1])
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    per = {}
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        threadpool_limits = None
    for num in (1, 2, 4, 5, 3):
        w = p if num == PREFILL_WORKLOAD else (dec if num == DECODE_WORKLOAD and dec is not None else gen.workload(num))
        if w.Lq == 1:
            unit, work = "GB/s", decode_bytes(w) / 1e9
        else:
            unit, work = "TFLOP/s", prefill_flop(w) / 1e12
        entry = {"workload": gen.WORKLOADS[num]["name"], "unit": unit}
        if num == PREFILL_WORKLOAD:
            # the slices timed above stand for the whole call
            entry.update({"threads": threads, "seconds": round(dt * p.B * p.Hq / done, 2),
                          "value": round(done * per_head / dt / 1e12, 5), "sample": f"{done} of {p.B * p.Hq} slices"})
        else:
            sec = _time_oracle(w)
            entry.update({"threads": threads, "seconds": round(sec, 3), "value": round(work / sec, 5)})
            if num in (1, 2, 5) and threadpool_limits is not None:
                with threadpool_limits(limits=1):
                    sec1 = _time_oracle(w)
                entry["one_thread"] = {"seconds": round(sec1, 3), "value": round(work / sec1, 5)}
        per[str(num)] = entry
    try:
        affinity = len(os.sched_getaffinity(0))
    except Exception:
        affinity = None
    return {"value": done * per_head / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {p.B * p.Hq} (batch, head) slices of the prefill workload, all {p.Lq} rows "
                      f"each; numpy float64 on {threads} BLAS threads, {dt:.1f} s",
            "cpu_model": _cpu_model(), "os_cpu_count": os.cpu_count(), "cpus_allowed": affinity,
            "blas_threads": threads, "per_workload": per}


PEAK_FP32_MFMA_TFLOPS = 157.3
OTHER_WORKLOADS = (1, 2, 4)   # timed and reported; not the headline metric
# sliding-window calls on the headline shapes (reported): (workload, window)
WINDOWED_WORKLOADS = ((5, 4096), (3, 1024))


# caps on the reported-only workloads' timing batches (--other-calls, --other-rounds):
# profiling runs shorten them; "settle" is the untimed load (seconds) before each
# workload's batches (at most --settle)
OTHER_CAPS = {"calls": 1 << 30, "rounds": 1 << 30, "settle": 0.25}


def measure_other_workloads(torch, sd, gen, dev, to_dev, stream, log, calls=50, rounds=5):
    """Per-call kernel time (HIP events on the library's stream, median of
    `rounds` batches of `calls`) of the f32 causal prefill, the 8193-key bf16
    decode, the f16 prefill with a boolean mask and sinks, and sliding-window
    calls on the headline shapes, each against its own roofline (windowed work
    counts only the keys in the band). Decode K/V rotates over copies whose
    windows together span > 2x the 256 MB MALL, so every call streams from HBM."""
    import numpy as np
    res = {}
    for num, window in [(n, 0) for n in OTHER_WORKLOADS] + list(WINDOWED_WORKLOADS):
        p = gen.workload(num)
        if window:
            p.name += f" window {window}"
            p.mask_kind = 1   # windows are causal (the same as no mask for a single query)
        q = to_dev(p.q, p.dtype)
        mask = None if p.mask is None else torch.from_numpy(np.ascontiguousarray(p.mask)).to(dev)
        sinks = None if p.sinks is None else to_dev(p.sinks, p.dtype)
        decode = p.Lq == 1
        copies = 1
        if decode:
            copies = max(1, -(-2 * 256 * 2 ** 20 // decode_bytes(p, window)))
        ks = [to_dev(p.k, p.dtype)]
        vs = [to_dev(p.v, p.dtype)]
        for _ in range(copies - 1):
            ks.append(ks[0].clone())
            vs.append(vs[0].clone())
        out = torch.empty((p.B, p.Hq, p.Lq, p.Dv), dtype=q.dtype, device=dev)

        def call(i):
            sd.attention(q, ks[i % copies], vs[i % copies], p.scale, p.mask_kind, mask, sinks, out=out,
                         stream=stream.cuda_stream, window=window or None)

        us = _time_calls(torch, stream, call, calls, rounds)
        rec = {"workload": p.name, "us_per_call": round(us, 2)}
        if window:
            rec["window"] = window
        if decode:
            gbps = decode_bytes(p, window) / us / 1e3
            rec.update({"kv_bytes_per_call": decode_bytes(p, window), "GB/s": round(gbps, 1),
                        "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4), "kv_copies": copies})
        else:
            flop = prefill_flop(p, window)
            tf = flop / us / 1e6
            peak = PEAK_FP32_MFMA_TFLOPS if p.dtype == gen.F32 else PEAK_BF16_TFLOPS
            rec.update({"flop_per_call": flop, "TFLOP/s": round(tf, 2), "peak_TFLOP/s": peak,
                        "frac_mfma_peak": round(tf / peak, 4)})
        res[f"{num}w{window}" if window else str(num)] = rec
        log(f"{p.name}: {us:.1f} us/call " + (f"{rec['GB/s']} GB/s" if decode else f"{rec['TFLOP/s']} TFLOP/s"))
        del ks, vs, q, out
        torch.cuda.empty_cache()
    return res


def measure_wide_workloads(torch, sd, gen, dev, to_dev, stream, log):
    """The headline prefill shape at 256-wide heads (bf16, causal; seed 31), which
    runs the key-split kernel: per-call kernel time against the bf16 MFMA peak
    (reported)."""
    p = gen.make_problem(31, 2, 32, 8, 4096, 4096, 256, 256, gen.BF16, 1,
                         name="bf16 GQA causal prefill B2 H32/8 L4096x4096 D256")
    q, k, v = (to_dev(a, p.dtype) for a in (p.q, p.k, p.v))
    out = torch.empty((p.B, p.Hq, p.Lq, p.Dv), dtype=q.dtype, device=dev)
    plan = sd.sdpa_plan(p.B, p.Hq, p.Hkv, p.Lq, p.Lk, p.D, p.Dv, 1, False, False, p.dtype)

    def call(i):
        sd.attention(q, k, v, p.scale, 1, out=out, stream=stream.cuda_stream)

    us = _time_calls(torch, stream, call, calls=10, rounds=5)
    flop = prefill_flop(p)
    tf = flop / us / 1e6
    log(f"{p.name}: {us:.1f} us/call {tf:.1f} TFLOP/s")
    del q, k, v, out
    torch.cuda.empty_cache()
    return {"3d256": {"workload": p.name, "us_per_call": round(us, 2), "flop_per_call": flop,
                      "TFLOP/s": round(tf, 2), "peak_TFLOP/s": PEAK_BF16_TFLOPS,
                      "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4), "rows_per_wave": plan["rows_per_wave"],
                      "block_n": plan["block_n"], "key_lanes": plan["splits"]}}


# paged-cache decode on the long-context decode shape (reported): (workload, block size, window)
PAGED_WORKLOADS = ((5, 16, 0), (5, 16, 4096))


def measure_paged_workloads(torch, sd, gen, dev, to_dev, stream, log, calls=50, rounds=5):
    """Per-call kernel time of decode over a paged cache: the long-context decode
    workload's K/V copied into blocks of 16 positions at shuffled places (three
    spare blocks), every sequence at its full length, with and without a sliding
    window. Counted bytes are the K/V rows the call reads (block ids excluded)."""
    import numpy as np
    res = {}
    for num, bs, window in PAGED_WORKLOADS:
        p = gen.workload(num)
        per = -(-p.Lk // bs)
        blocks = p.B * per + 3
        order = gen.block_order(num, blocks)
        kc, table = gen.paged_cache(p.k, bs, order, blocks)
        vc, _ = gen.paged_cache(p.v, bs, order, blocks)
        q = to_dev(p.q, p.dtype)
        kd, vd = to_dev(kc, p.dtype), to_dev(vc, p.dtype)
        del kc, vc
        td = torch.from_numpy(table).to(dev)
        ld = torch.full((p.B,), p.Lk, dtype=torch.int32, device=dev)
        out = torch.empty((p.B, p.Hq, p.Lq, p.Dv), dtype=q.dtype, device=dev)
        nbytes = decode_bytes(p, window)
        mask_kind = 1 if window else p.mask_kind

        def call(i):
            sd.paged_attention(q, kd, vd, td, ld, p.scale, mask_kind, window, out=out, stream=stream.cuda_stream)

        us = _time_calls(torch, stream, call, calls, rounds)
        gbps = nbytes / us / 1e3
        name = f"{p.name} paged bs={bs}" + (f" window {window}" if window else "")
        res[f"{num}p{bs}" + (f"w{window}" if window else "")] = {
            "workload": name, "us_per_call": round(us, 2), "block_size": bs, "blocks": blocks,
            "window": window or None, "kv_bytes_per_call": nbytes, "GB/s": round(gbps, 1),
            "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4)}
        log(f"{name}: {us:.1f} us/call {gbps:.0f} GB/s")
        del q, kd, vd, td, ld, out
        torch.cuda.empty_cache()
    return res


def _time_calls(torch, stream, call, calls=50, rounds=5):
    """Median per-call time (us) over `rounds` batches of `calls`, HIP events on
    `stream`. `call(i)` makes the i-th call. Untimed calls for OTHER_CAPS["settle"]
    seconds (at least 20) come first: the clocks fall while the host builds a
    workload's inputs, and a few ms of calls after such a pause run up to 15 %
    slow."""
    calls = max(1, min(calls, OTHER_CAPS["calls"]))
    rounds = max(1, min(rounds, OTHER_CAPS["rounds"]))
    n = 0
    t_end = time.perf_counter() + OTHER_CAPS["settle"]
    while True:
        for _ in range(20):
            call(n)
            n += 1
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            break
    times = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(calls):
            call(n)
            n += 1
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / calls * 1e3)
    return sorted(times)[len(times) // 2]


def measure_strided_workloads(torch, sd, gen, dev, to_dev, stream, log):
    """Calls through sdpa_forward_strided: the causal prefill with q, K and V as
    transposed views of [B, L, H, D] arrays (the layout a model's projections
    produce), and the f16 masked-prefill shape with an additive [1, Hq, Lq, Lk]
    mask (N(0,1) values, 10 % -inf) and sinks. Prefill FLOP as for the
    contiguous calls (the additive mask counts every pair); the additive line
    also reports the mask bytes it reads."""
    import numpy as np
    res = {}
    p = gen.workload(3)
    tv = lambda a: to_dev(np.ascontiguousarray(a.transpose(0, 2, 1, 3)), p.dtype).transpose(1, 2)
    q, k, v = tv(p.q), tv(p.k), tv(p.v)
    out = torch.empty((p.B, p.Hq, p.Lq, p.Dv), dtype=q.dtype, device=dev)
    us = _time_calls(torch, stream, lambda i: sd.attention(q, k, v, p.scale, p.mask_kind, out=out,
                                                           stream=stream.cuda_stream))
    flop = prefill_flop(p)
    tf = flop / us / 1e6
    res["3v"] = {"workload": p.name + ", q/k/v as transposed [B,L,H,D] views", "us_per_call": round(us, 2),
                 "flop_per_call": flop, "TFLOP/s": round(tf, 2), "peak_TFLOP/s": PEAK_BF16_TFLOPS,
                 "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    log(f"{res['3v']['workload']}: {us:.1f} us/call {tf:.1f} TFLOP/s")
    del q, k, v, out
    p = gen.workload(4)
    add = gen.additive_mask(4, (1, p.Hq, p.Lq, p.Lk), p.dtype, holes=0.1)
    q, k, v = (to_dev(a, p.dtype) for a in (p.q, p.k, p.v))
    m, s = to_dev(add, p.dtype), to_dev(p.sinks, p.dtype)
    out = torch.empty((p.B, p.Hq, p.Lq, p.Dv), dtype=q.dtype, device=dev)
    us = _time_calls(torch, stream, lambda i: sd.attention(q, k, v, p.scale, 3, m, s, out=out,
                                                           stream=stream.cuda_stream))
    flop = p.B * p.Hq * p.Lq * p.Lk * 2 * (p.D + p.Dv)
    tf = flop / us / 1e6
    mbytes = add.size * add.itemsize
    res["4a"] = {"workload": "f16 GQA prefill additive-mask+sinks B1 H16/2 L1024x1801 D256",
                 "us_per_call": round(us, 2), "flop_per_call": flop, "TFLOP/s": round(tf, 2),
                 "peak_TFLOP/s": PEAK_BF16_TFLOPS, "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                 "mask_bytes_per_call": mbytes, "mask_GB/s": round(mbytes / us / 1e3, 1)}
    log(f"{res['4a']['workload']}: {us:.1f} us/call {tf:.1f} TFLOP/s, mask {mbytes / us / 1e3:.0f} GB/s")
    del q, k, v, m, s, out
    torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle", type=float, default=2.0,
                    help="extra untimed stepping (seconds) after the warmup steps, so GPU clocks settle")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time budget for cpu_baseline's "
                    "prefill sample (the other workloads add about 10 s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true", help="skip the reported-only workloads (f32 prefill, "
                    "8193-key decode, f16 masked prefill with sinks, sliding windows, paged decode, "
                    "strided views, additive mask, 256-wide prefill)")
    ap.add_argument("--other-calls", type=int, default=None,
                    help="at most this many calls per timed batch of a reported-only workload (profiling runs)")
    ap.add_argument("--other-rounds", type=int, default=None,
                    help="at most this many timed batches per reported-only workload (profiling runs)")
    args = ap.parse_args()
    if args.other_calls:
        OTHER_CAPS["calls"] = args.other_calls
    if args.other_rounds:
        OTHER_CAPS["rounds"] = args.other_rounds
    OTHER_CAPS["settle"] = max(0.0, min(OTHER_CAPS["settle"], args.settle))
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library has no "
              f"multi-GPU path)", file=sys.stderr)
        return 2

    import torch

    import scaled_dot_product_06_amd as sd
    from scaled_dot_product_06_amd import inputs as gen

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)

    def to_dev(a, dtype):
        import numpy as np
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if dtype == gen.BF16 else torch.from_numpy(a)
        return t.to(dev)

    t0 = time.perf_counter()
    pre = gen.workload(PREFILL_WORKLOAD)
    dec = gen.workload(DECODE_WORKLOAD)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
    pq, pk, pv = (to_dev(a, pre.dtype) for a in (pre.q, pre.k, pre.v))
    pout = torch.empty((pre.B, pre.Hq, pre.Lq, pre.Dv), dtype=pq.dtype, device=dev)
    dq = to_dev(dec.q, dec.dtype)
    dk = [to_dev(dec.k, dec.dtype)]
    dv = [to_dev(dec.v, dec.dtype)]
    dk.append(dk[0].clone())
    dv.append(dv[0].clone())
    dout = torch.empty((dec.B, dec.Hq, dec.Lq, dec.Dv), dtype=dq.dtype, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def step(i):
        sd.attention(pq, pk, pv, pre.scale, pre.mask_kind, out=pout, stream=stream.cuda_stream)
        sd.attention(dq, dk[i % 2], dv[i % 2], dec.scale, dec.mask_kind, out=dout, stream=stream.cuda_stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # let the clocks settle: keep stepping (untimed) for at least --settle seconds
    t_settle = time.perf_counter() + args.settle
    i = args.warmup
    while time.perf_counter() < t_settle:
        step(i)
        i += 1
        if i % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(K):
            ev[i][0].record(stream)
            sd.attention(pq, pk, pv, pre.scale, pre.mask_kind, out=pout, stream=stream.cuda_stream)
            ev[i][1].record(stream)
            sd.attention(dq, dk[i % 2], dv[i % 2], dec.scale, dec.mask_kind, out=dout,
                         stream=stream.cuda_stream)
            ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    pre_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    dec_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    step_ms = ev[0][0].elapsed_time(ev[-1][2]) / K

    flop = prefill_flop(pre)
    nbytes = decode_bytes(dec)
    tflops = flop / (pre_ms * 1e-3) / 1e12
    gbps = nbytes / (dec_ms * 1e-3) / 1e9
    log(f"prefill {pre_ms * 1e3:.1f} us/call = {tflops:.1f} TFLOP/s ({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of "
        f"bf16 MFMA peak); decode {dec_ms * 1e3:.1f} us/call = {gbps:.0f} GB/s "
        f"({100 * gbps / PEAK_HBM_GBPS:.1f}% of HBM peak); step {step_ms:.3f} ms; wall {wall:.2f} s")

    others = None
    if not args.no_others:
        others = measure_other_workloads(torch, sd, gen, dev, to_dev, stream, log)
        others.update(measure_paged_workloads(torch, sd, gen, dev, to_dev, stream, log))
        others.update(measure_strided_workloads(torch, sd, gen, dev, to_dev, stream, log))
        others.update(measure_wide_workloads(torch, sd, gen, dev, to_dev, stream, log))

    pre_plan = sd.sdpa_plan(pre.B, pre.Hq, pre.Hkv, pre.Lq, pre.Lk, pre.D, pre.Dv, pre.mask_kind, False, False,
                            pre.dtype)
    dec_plan = sd.sdpa_plan(dec.B, dec.Hq, dec.Hkv, dec.Lq, dec.Lk, dec.D, dec.Dv, dec.mask_kind, False, False,
                            dec.dtype)
    traffic_pre = _traffic_for("prefill")
    traffic_dec = _traffic_for("decode")

    result = {
        "metric": "prefill TFLOP/s (% MFMA peak) + decode K/V GB/s (% HBM peak), 1 GPU",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based N(0,1) inputs, no dataset)",
        "config": {
            "workload": "bf16 GQA causal prefill B=2 Hq=32 Hkv=8 Lq=Lk=4096 D=Dv=128 + "
                        "bf16 GQA decode B=4 Hq=16 Hkv=2 Lq=1 Lk=65537 D=Dv=256",
            "prefill_flop_per_call": flop,
            "decode_kv_bytes_per_call": nbytes,
            "prefill_plan": pre_plan,
            "decode_plan": dec_plan,
        },
        "decode": {
            "value": round(gbps, 1), "unit": "GB/s", "us_per_call": round(dec_ms * 1e3, 2),
            "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
        },
        "roofline": {
            "kernel": "prefill_fast_kernel (bf16, 32x32x16 MFMA, D=Dv=128)",
            "bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_pre,
        },
        "roofline_decode": {
            "kernel": "decode_split_kernel + decode_reduce_kernel (bf16, D=256)",
            "bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBPS, 4),
            "traffic": traffic_dec,
        },
        "cpu_baseline": None,
        "other_workloads": others,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of the prefill workload ...")
        result["cpu_baseline"] = cpu_baseline(pre, args.cpu_seconds, gen, dec)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
