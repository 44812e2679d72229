"""Seeded, counter-based synthetic inputs for attention workloads.

This module draws random numbers and rounds them to storage types. It holds
none of the attention arithmetic: the GPU path, the tests and the CPU oracle
all receive the tensors it returns.

Element ``n`` of tensor ``t`` under seed ``s`` is driven by the 64-bit word
``x(n) = mix64(mix64(s) ^ (t << 56) ^ n)``, where ``mix64`` is the splitmix64
finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014). From that word:

* uniform on [-1, 1): ``(x >> 40) * 2**-23 - 1`` (24 random bits, exact in f32);
* standard normal: Box-Muller in float64 on the 53-bit uniforms of words
  ``n`` and ``n + 2**55``, ``sqrt(-2 ln u1) * cos(2 pi u2)``;
* Bernoulli(0.9): ``(x >> 40) < 15099494`` (probability 0.89999998).

Values are rounded to nearest-even into the storage type; normals are rounded
to float32 first and then to float16/bfloat16. Storage arrays are numpy
``float32`` / ``float16`` and, for bfloat16, ``uint16`` holding the bit
pattern. Tensor ids: q=1, k=2, v=3, mask=4, sinks=5, block order=6, additive
mask values=7, additive mask -inf positions=8.

Paged caches (``block_order``, ``paged_cache``) only move these arrays into
blocks at shuffled places; the block order is a Fisher-Yates shuffle whose
step i swaps with index ``x(i) mod (i + 1)`` of stream 6.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}
DTYPE_BY_NAME = {"f32": F32, "f16": F16, "bf16": BF16}
STORAGE = {F32: np.float32, F16: np.float16, BF16: np.uint16}

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_MASK, TENSOR_SINKS, TENSOR_PAGES = 1, 2, 3, 4, 5, 6
TENSOR_ADD, TENSOR_ADD_HOLES = 7, 8

_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def _mix64(z: np.ndarray) -> np.ndarray:
    z = z.copy()
    z ^= z >> np.uint64(30)
    z *= _M1
    z ^= z >> np.uint64(27)
    z *= _M2
    z ^= z >> np.uint64(31)
    return z


def _stream_key(seed: int, tensor: int) -> np.uint64:
    s = _mix64(np.array([seed & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64))[0]
    return np.uint64(int(s) ^ ((tensor & 0xFF) << 56))


def words(seed: int, tensor: int, start: int, count: int) -> np.ndarray:
    """The 64-bit words x(start) .. x(start+count-1) of one tensor stream."""
    key = _stream_key(seed, tensor)
    n = np.arange(start, start + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(n ^ key)


def _chunked(count: int, dtype, fill) -> np.ndarray:
    """Fill out[s:s+c] = fill(s, c) over fixed chunks, on a few threads (numpy
    releases the GIL); the values do not depend on the thread count."""
    out = np.empty(count, dtype=dtype)
    starts = list(range(0, count, _CHUNK))

    def work(s):
        c = min(_CHUNK, count - s)
        out[s:s + c] = fill(s, c)

    workers = min(16, os.cpu_count() or 1, max(1, len(starts)))
    if workers <= 1:
        for s in starts:
            work(s)
    else:
        with _cf.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(work, starts))
    return out


def uniform_pm1(seed: int, tensor: int, count: int) -> np.ndarray:
    """float32 draws on [-1, 1), exact."""
    def fill(s, c):
        u = (words(seed, tensor, s, c) >> np.uint64(40)).astype(np.float64)
        return (u * 2.0 ** -23 - 1.0).astype(np.float32)
    return _chunked(count, np.float32, fill)


def normal(seed: int, tensor: int, count: int) -> np.ndarray:
    """float64 standard-normal draws (Box-Muller)."""
    def fill(s, c):
        a = words(seed, tensor, s, c) >> np.uint64(11)
        b = words(seed, tensor, s + (1 << 55), c) >> np.uint64(11)
        u1 = (a.astype(np.float64) + 1.0) * 2.0 ** -53  # (0, 1]
        u2 = b.astype(np.float64) * 2.0 ** -53          # [0, 1)
        return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    return _chunked(count, np.float64, fill)


def bernoulli(seed: int, tensor: int, count: int, threshold: int = 15099494) -> np.ndarray:
    """uint8 draws, 1 with probability threshold / 2**24."""
    def fill(s, c):
        return (words(seed, tensor, s, c) >> np.uint64(40)) < np.uint64(threshold)
    return _chunked(count, np.uint8, fill)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float values into the storage array of ``dtype`` (nearest-even)."""
    x32 = np.asarray(x).astype(np.float32)
    if dtype == F32:
        return x32
    if dtype == F16:
        return x32.astype(np.float16)
    if dtype == BF16:
        return f32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype}")


def widen(a: np.ndarray, dtype: int) -> np.ndarray:
    """Exact float64 values of a storage array."""
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a).astype(np.float64)


def tensor(seed: int, tensor_id: int, shape, dtype: int, dist: str) -> np.ndarray:
    """A storage array of ``shape`` with i.i.d. draws of ``dist`` ('uniform' or 'normal')."""
    count = int(np.prod(shape, dtype=np.int64)) if len(shape) else 1
    if dist == "uniform":
        x = uniform_pm1(seed, tensor_id, count)
    elif dist == "normal":
        x = normal(seed, tensor_id, count)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return to_storage(x, dtype).reshape(shape)


def diagonal_bool_mask(seed: int, lq: int, lk: int) -> np.ndarray:
    """[lq, lk] uint8 mask: Bernoulli(0.9) entries, with column lk-lq+i forced on in row i
    (when that column exists)."""
    m = bernoulli(seed, TENSOR_MASK, lq * lk).reshape(lq, lk)
    rows = np.arange(lq)
    cols = rows + (lk - lq)
    ok = (cols >= 0) & (cols < lk)
    m[rows[ok], cols[ok]] = 1
    return m


class Problem:
    """One attention call's inputs, in storage arrays, plus their shape parameters."""

    def __init__(self, B, Hq, Hkv, Lq, Lk, D, Dv, dtype, mask_kind, scale,
                 q, k, v, mask=None, sinks=None, name=""):
        self.B, self.Hq, self.Hkv, self.Lq, self.Lk, self.D, self.Dv = B, Hq, Hkv, Lq, Lk, D, Dv
        self.dtype, self.mask_kind, self.scale = dtype, mask_kind, float(scale)
        self.q, self.k, self.v, self.mask, self.sinks = q, k, v, mask, sinks
        self.name = name

    def shape_args(self):
        return (self.B, self.Hq, self.Hkv, self.Lq, self.Lk, self.D, self.Dv)

    def widened(self):
        """(q, k, v, mask, sinks) as exact float64 arrays (mask as bool)."""
        f = lambda a: None if a is None else widen(a, self.dtype)
        m = None if self.mask is None else (np.asarray(self.mask) != 0)
        return f(self.q), f(self.k), f(self.v), m, f(self.sinks)

    def __repr__(self):
        return (f"Problem({self.name} B={self.B} Hq={self.Hq} Hkv={self.Hkv} Lq={self.Lq} "
                f"Lk={self.Lk} D={self.D} Dv={self.Dv} {DTYPE_NAMES[self.dtype]} "
                f"mask={self.mask_kind} sinks={self.sinks is not None})")


def make_problem(seed, B, Hq, Hkv, Lq, Lk, D, Dv, dtype, mask_kind, dist="normal",
                 sinks=False, scale=None, name=""):
    """Inputs for one call. mask_kind: 0 none, 1 causal, 2 boolean ([Lq, Lk],
    Bernoulli(0.9) with the bottom-right diagonal forced on). Sinks are N(0,1)."""
    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    q = tensor(seed, TENSOR_Q, (B, Hq, Lq, D), dtype, dist)
    k = tensor(seed, TENSOR_K, (B, Hkv, Lk, D), dtype, dist)
    v = tensor(seed, TENSOR_V, (B, Hkv, Lk, Dv), dtype, dist)
    mask = diagonal_bool_mask(seed, Lq, Lk) if mask_kind == 2 else None
    s = tensor(seed, TENSOR_SINKS, (Hq,), dtype, "normal") if sinks else None
    return Problem(B, Hq, Hkv, Lq, Lk, D, Dv, dtype, mask_kind, scale, q, k, v, mask, s, name)


# The five workloads, seeded by their number. Scale is 1/sqrt(D) throughout.
WORKLOADS = {
    1: dict(name="f32 causal prefill B1 H8/8 L128x128 D64",
            B=1, Hq=8, Hkv=8, Lq=128, Lk=128, D=64, Dv=64, dtype=F32, mask_kind=1,
            dist="uniform", sinks=False),
    2: dict(name="bf16 GQA decode B1 H32/4 Lk8193 D128",
            B=1, Hq=32, Hkv=4, Lq=1, Lk=8193, D=128, Dv=128, dtype=BF16, mask_kind=1,
            dist="normal", sinks=False),
    3: dict(name="bf16 GQA causal prefill B2 H32/8 L4096x4096 D128",
            B=2, Hq=32, Hkv=8, Lq=4096, Lk=4096, D=128, Dv=128, dtype=BF16, mask_kind=1,
            dist="normal", sinks=False),
    4: dict(name="f16 GQA prefill bool-mask+sinks B1 H16/2 L1024x1801 D256",
            B=1, Hq=16, Hkv=2, Lq=1024, Lk=1801, D=256, Dv=256, dtype=F16, mask_kind=2,
            dist="uniform", sinks=True),
    5: dict(name="bf16 GQA decode B4 H16/2 Lk65537 D256",
            B=4, Hq=16, Hkv=2, Lq=1, Lk=65537, D=256, Dv=256, dtype=BF16, mask_kind=0,
            dist="normal", sinks=False),
}


def workload(number: int) -> Problem:
    w = dict(WORKLOADS[number])
    name = w.pop("name")
    return make_problem(number, name=name, **w)


# ---- paged caches -------------------------------------------------------------------------

NAN_BITS = {F32: np.float32(np.nan), F16: np.float16(np.nan), BF16: np.uint16(0x7FC0)}


def block_order(seed: int, blocks: int) -> np.ndarray:
    """A seeded permutation of range(blocks) (Fisher-Yates on stream 6)."""
    w = words(seed, TENSOR_PAGES, 0, max(blocks, 1))
    order = np.arange(blocks, dtype=np.int64)
    for i in range(blocks - 1, 0, -1):
        j = int(w[i] % np.uint64(i + 1))
        order[i], order[j] = order[j], order[i]
    return order


def paged_cache(x: np.ndarray, bs: int, order: np.ndarray, blocks: int, fill=0):
    """Copies a storage array x [B, Hkv, N, E] into a cache [blocks, Hkv, bs, E]:
    positions j*bs .. j*bs+bs-1 of sequence s go to block order[s * per + j],
    per = ceil(N / bs). Rows no sequence owns hold `fill` (a value, or "nan").
    Returns (cache, table [B, per] int32)."""
    B, hkv, n, e = x.shape
    per = -(-n // bs)
    assert blocks >= B * per and len(order) >= B * per
    cache = np.empty((blocks, hkv, bs, e), dtype=x.dtype)
    cache[...] = NAN_BITS[_storage_code(x.dtype)] if isinstance(fill, str) else fill
    for s in range(B):
        for j in range(per):
            m = min(bs, n - j * bs)
            cache[order[s * per + j], :, :m] = x[s, :, j * bs:j * bs + m]
    table = np.asarray(order[:B * per], dtype=np.int32).reshape(B, per)
    return cache, table


def _storage_code(dt) -> int:
    for code, st in STORAGE.items():
        if np.dtype(st) == np.dtype(dt):
            return code
    raise ValueError(f"not a storage dtype: {dt}")


# ---- additive masks -------------------------------------------------------------------------

NEG_INF_BITS = {F32: np.float32(-np.inf), F16: np.float16(-np.inf), BF16: np.uint16(0xFF80)}


def additive_mask(seed: int, shape, dtype: int, holes: float = 0.0) -> np.ndarray:
    """An additive mask in storage type: N(0,1) values (stream 7), with entries set to
    -inf where the uniform draw of stream 8 falls below 2*holes - 1 (probability
    `holes`)."""
    m = tensor(seed, TENSOR_ADD, shape, dtype, "normal")
    if holes > 0:
        count = m.size
        u = uniform_pm1(seed, TENSOR_ADD_HOLES, count).reshape(m.shape)
        m[u < 2.0 * holes - 1.0] = NEG_INF_BITS[dtype]
    return m
