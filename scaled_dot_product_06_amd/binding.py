"""ctypes binding of libsdpa.so (include/sdpa.h): the same entry points under
the same names, plus `attention`, which only marshals torch tensors into an
sdpa_forward call. Every step of the computation runs in the library's HIP
kernels; there is no Python or CPU fallback."""
from __future__ import annotations

import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdpa.so")

SDPA_F32, SDPA_F16, SDPA_BF16 = 0, 1, 2
SDPA_MASK_NONE, SDPA_MASK_CAUSAL, SDPA_MASK_BOOL, SDPA_MASK_ADDITIVE = 0, 1, 2, 3
SDPA_OK, SDPA_ERR_INVALID, SDPA_ERR_UNSUPPORTED, SDPA_ERR_HIP = 0, -1, -2, -3
SDPA_ROUTE_EMPTY, SDPA_ROUTE_ZERO_FILL, SDPA_ROUTE_PREFILL, SDPA_ROUTE_DECODE = 0, 1, 2, 3
ROUTE_NAMES = {0: "empty", 1: "zero_fill", 2: "prefill", 3: "decode"}

EXPORTED = ("sdpa_forward", "sdpa_plan", "sdpa_forward_windowed", "sdpa_plan_windowed", "sdpa_paged_forward",
            "sdpa_plan_paged", "sdpa_paged_write", "sdpa_forward_strided", "sdpa_last_error", "sdpa_release_workspace",
            "sdpa_abi_version", "sdpa_forward_noalloc", "sdpa_noalloc_scratch_bytes")


class SdpaPlan(ctypes.Structure):
    _fields_ = [
        ("route", ctypes.c_int32),
        ("kernels", ctypes.c_int32),
        ("rows_per_wave", ctypes.c_int32),
        ("waves", ctypes.c_int32),
        ("block_n", ctypes.c_int32),
        ("heads_per_group", ctypes.c_int32),
        ("keys_per_split", ctypes.c_int64),
        ("splits", ctypes.c_int64),
        ("grid", ctypes.c_int64 * 3),
        ("scratch_bytes", ctypes.c_int64),
    ]

    def as_dict(self):
        return {
            "route": ROUTE_NAMES.get(self.route, self.route),
            "kernels": self.kernels,
            "rows_per_wave": self.rows_per_wave,
            "waves": self.waves,
            "block_n": self.block_n,
            "heads_per_group": self.heads_per_group,
            "keys_per_split": self.keys_per_split,
            "splits": self.splits,
            "grid": tuple(self.grid),
            "scratch_bytes": self.scratch_bytes,
        }


class SdpaView(ctypes.Structure):
    """sdpa_view_t: a data pointer and element strides (batch, head, row)."""
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("stride_l", ctypes.c_int64)]


class SdpaError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"sdpa error {code}: {message}")
        self.code = code
        self.message = message


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libsdpa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m scaled_dot_product_06_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, c_int, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.sdpa_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, ctypes.c_float,
                                 c_int, vp, vp, c_int, vp]
    lib.sdpa_forward.restype = c_int
    lib.sdpa_forward_noalloc.argtypes = list(lib.sdpa_forward.argtypes)
    lib.sdpa_forward_noalloc.restype = c_int
    lib.sdpa_noalloc_scratch_bytes.argtypes = []
    lib.sdpa_noalloc_scratch_bytes.restype = i64
    lib.sdpa_plan.argtypes = [i64, i64, i64, i64, i64, i64, i64, c_int, c_int, c_int, c_int,
                              ctypes.POINTER(SdpaPlan)]
    lib.sdpa_plan.restype = c_int
    lib.sdpa_forward_windowed.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, ctypes.c_float,
                                          i64, vp, c_int, vp]
    lib.sdpa_forward_windowed.restype = c_int
    lib.sdpa_plan_windowed.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, c_int, c_int,
                                       ctypes.POINTER(SdpaPlan)]
    lib.sdpa_plan_windowed.restype = c_int
    lib.sdpa_paged_forward.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, i64,
                                       ctypes.c_float, c_int, i64, vp, c_int, vp]
    lib.sdpa_paged_forward.restype = c_int
    lib.sdpa_plan_paged.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, i64, c_int, i64, c_int, c_int,
                                    ctypes.POINTER(SdpaPlan)]
    lib.sdpa_plan_paged.restype = c_int
    lib.sdpa_paged_write.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, c_int, vp]
    lib.sdpa_paged_write.restype = c_int
    pv = ctypes.POINTER(SdpaView)
    lib.sdpa_forward_strided.argtypes = [pv, pv, pv, vp, i64, i64, i64, i64, i64, i64, i64, ctypes.c_float, c_int,
                                         pv, vp, i64, c_int, vp]
    lib.sdpa_forward_strided.restype = c_int
    lib.sdpa_last_error.argtypes = []
    lib.sdpa_last_error.restype = ctypes.c_char_p
    lib.sdpa_release_workspace.argtypes = []
    lib.sdpa_release_workspace.restype = c_int
    lib.sdpa_abi_version.argtypes = []
    lib.sdpa_abi_version.restype = c_int
    _lib = lib
    return lib


def sdpa_last_error() -> str:
    return load().sdpa_last_error().decode()


def _check(rc: int) -> int:
    if rc != SDPA_OK:
        raise SdpaError(rc, sdpa_last_error())
    return rc


def sdpa_forward(q, k, v, out, B, Hq, Hkv, Lq, Lk, D, Dv, scale, mask_kind, mask, sinks, dtype, stream,
                 check: bool = True) -> int:
    """Raw call: pointers are integers (device addresses) or None."""
    rc = load().sdpa_forward(q, k, v, out, B, Hq, Hkv, Lq, Lk, D, Dv, ctypes.c_float(scale), mask_kind,
                             mask, sinks, dtype, stream)
    return _check(rc) if check else rc


def sdpa_forward_noalloc(q, k, v, out, B, Hq, Hkv, Lq, Lk, D, Dv, scale, mask_kind, mask, sinks, dtype, stream,
                         check: bool = True) -> int:
    """Raw allocation-free call (the library's fixed per-device scratch): as sdpa_forward."""
    rc = load().sdpa_forward_noalloc(q, k, v, out, B, Hq, Hkv, Lq, Lk, D, Dv, ctypes.c_float(scale), mask_kind,
                                     mask, sinks, dtype, stream)
    return _check(rc) if check else rc


def sdpa_noalloc_scratch_bytes() -> int:
    return load().sdpa_noalloc_scratch_bytes()


def sdpa_plan(B, Hq, Hkv, Lq, Lk, D, Dv, mask_kind, has_mask, has_sinks, dtype, check: bool = True):
    """Returns the plan as a dict (or the return code when check=False and it fails)."""
    p = SdpaPlan()
    rc = load().sdpa_plan(B, Hq, Hkv, Lq, Lk, D, Dv, mask_kind, int(bool(has_mask)), int(bool(has_sinks)),
                          dtype, ctypes.byref(p))
    if rc != SDPA_OK:
        if check:
            _check(rc)
        return rc
    return p.as_dict()


def sdpa_forward_windowed(q, k, v, out, B, Hq, Hkv, Lq, Lk, D, Dv, scale, window, sinks, dtype, stream,
                          check: bool = True) -> int:
    """Raw windowed call (causal attention over a sliding window of keys)."""
    rc = load().sdpa_forward_windowed(q, k, v, out, B, Hq, Hkv, Lq, Lk, D, Dv, ctypes.c_float(scale), window,
                                      sinks, dtype, stream)
    return _check(rc) if check else rc


def sdpa_plan_windowed(B, Hq, Hkv, Lq, Lk, D, Dv, window, has_sinks, dtype, check: bool = True):
    """The windowed call's plan as a dict (or the return code when check=False and it fails)."""
    p = SdpaPlan()
    rc = load().sdpa_plan_windowed(B, Hq, Hkv, Lq, Lk, D, Dv, window, int(bool(has_sinks)), dtype,
                                   ctypes.byref(p))
    if rc != SDPA_OK:
        if check:
            _check(rc)
        return rc
    return p.as_dict()


def sdpa_paged_forward(q, kcache, vcache, out, table, lengths, B, Hq, Hkv, Lq, D, Dv, blocks, bs, max_blocks,
                       scale, mask_kind, window, sinks, dtype, stream, check: bool = True) -> int:
    """Raw paged call (attention over a paged key/value cache)."""
    rc = load().sdpa_paged_forward(q, kcache, vcache, out, table, lengths, B, Hq, Hkv, Lq, D, Dv, blocks, bs,
                                   max_blocks, ctypes.c_float(scale), mask_kind, window, sinks, dtype, stream)
    return _check(rc) if check else rc


def sdpa_plan_paged(B, Hq, Hkv, Lq, D, Dv, blocks, bs, max_blocks, mask_kind, window, has_sinks, dtype,
                    check: bool = True):
    """The paged call's plan as a dict (or the return code when check=False and it fails)."""
    p = SdpaPlan()
    rc = load().sdpa_plan_paged(B, Hq, Hkv, Lq, D, Dv, blocks, bs, max_blocks, mask_kind, window,
                                int(bool(has_sinks)), dtype, ctypes.byref(p))
    if rc != SDPA_OK:
        if check:
            _check(rc)
        return rc
    return p.as_dict()


def sdpa_paged_write(cache, rows, slots, n, blocks, Hkv, bs, E, dtype, stream, check: bool = True) -> int:
    """Raw paged cache write (rows into slots, in place)."""
    rc = load().sdpa_paged_write(cache, rows, slots, n, blocks, Hkv, bs, E, dtype, stream)
    return _check(rc) if check else rc


def sdpa_forward_strided(q, k, v, out, B, Hq, Hkv, Lq, Lk, D, Dv, scale, mask_kind, mask, sinks, window, dtype,
                         stream, check: bool = True) -> int:
    """Raw strided call: q, k, v (and mask, or None) are (data, stride_b, stride_h, stride_l) tuples
    or SdpaView objects (None for a NULL view)."""
    def view(x):
        if x is None:
            return None
        return ctypes.byref(x if isinstance(x, SdpaView) else SdpaView(*x))
    rc = load().sdpa_forward_strided(view(q), view(k), view(v), out, B, Hq, Hkv, Lq, Lk, D, Dv,
                                     ctypes.c_float(scale), mask_kind, view(mask), sinks, window, dtype, stream)
    return _check(rc) if check else rc


def sdpa_release_workspace() -> int:
    return _check(load().sdpa_release_workspace())


def sdpa_abi_version() -> int:
    return load().sdpa_abi_version()


# ---- torch marshalling -------------------------------------------------------------------

def _dtype_code(t):
    import torch
    codes = {torch.float32: SDPA_F32, torch.float16: SDPA_F16, torch.bfloat16: SDPA_BF16}
    if t.dtype not in codes:
        raise SdpaError(SDPA_ERR_INVALID, f"unsupported tensor dtype {t.dtype}")
    return codes[t.dtype]


def _view(name, t, shape):
    """(data, stride_b, stride_h, stride_l) of a 4-D GPU tensor whose last axis is contiguous."""
    if not t.is_cuda:
        raise SdpaError(SDPA_ERR_INVALID, f"{name} must be a GPU tensor")
    if tuple(t.shape) != tuple(shape):
        raise SdpaError(SDPA_ERR_INVALID, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise SdpaError(SDPA_ERR_INVALID, f"{name} must be contiguous along its last axis")
    return (t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _out_tensor(out, q, shape):
    """`out` as given (checked: a contiguous GPU tensor of q's dtype and device and the
    output shape, which the kernels overwrite whole) or a new one."""
    import torch
    if out is None:
        return torch.empty(shape, dtype=q.dtype, device=q.device)
    if not out.is_cuda or out.device != q.device:
        raise SdpaError(SDPA_ERR_INVALID, f"out must be a GPU tensor on {q.device}")
    if out.dtype != q.dtype:
        raise SdpaError(SDPA_ERR_INVALID, f"out has dtype {out.dtype}, q has {q.dtype}")
    if tuple(out.shape) != tuple(shape):
        raise SdpaError(SDPA_ERR_INVALID, f"out has shape {tuple(out.shape)}, expected {tuple(shape)}")
    if not out.is_contiguous():
        raise SdpaError(SDPA_ERR_INVALID, "out must be contiguous")
    return out


def _sinks_ptr(sinks, q, Hq):
    """Device address of the [Hq] sinks, or None. The tensor must be contiguous: a
    contiguous copy made here could be freed before the asynchronous kernels read it."""
    if sinks is None:
        return None
    if tuple(sinks.shape) != (Hq,) or sinks.dtype != q.dtype or not sinks.is_cuda or sinks.device != q.device:
        raise SdpaError(SDPA_ERR_INVALID, f"sinks must be a GPU tensor of shape ({Hq},) and dtype {q.dtype} on "
                        f"{q.device}")
    if not sinks.is_contiguous():
        raise SdpaError(SDPA_ERR_INVALID, "sinks must be contiguous")
    return sinks.data_ptr()


def attention(q, k, v, scale: float, mask_kind: int = SDPA_MASK_NONE, mask=None, sinks=None, out=None,
              stream=None, window=None):
    """softmax(scale * q k^T + mask) v on the GPU.

    q [B,Hq,Lq,D], k [B,Hkv,Lk,D], v [B,Hkv,Lk,Dv] GPU tensors of one dtype;
    contiguous ones go through sdpa_forward (sdpa_forward_windowed with a
    `window`, causal only), views whose last axis is contiguous (a transposed
    [B,L,H,D] array, a slice of a longer cache) through sdpa_forward_strided.
    mask: a contiguous uint8/bool [Lq,Lk] tensor (mask_kind 2), or an
    additive mask of q's dtype broadcastable to [B,Hq,Lq,Lk] (mask_kind 3,
    any strides with a contiguous last axis). sinks: [Hq] of q's dtype.
    Returns out [B,Hq,Lq,Dv] (contiguous).
    """
    import torch
    B, Hq, Lq, D = q.shape
    _, Hkv, Lk, _ = k.shape
    Dv = v.shape[3]
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise SdpaError(SDPA_ERR_INVALID, f"{name} must be a GPU tensor")
        if t.dtype != q.dtype:
            raise SdpaError(SDPA_ERR_INVALID, f"{name} has dtype {t.dtype}, q has {q.dtype}")
        if t.device != q.device:
            raise SdpaError(SDPA_ERR_INVALID, f"{name} is on {t.device}, q on {q.device}")
    if tuple(k.shape) != (B, Hkv, Lk, D) or tuple(v.shape[:3]) != (B, Hkv, Lk):
        raise SdpaError(SDPA_ERR_INVALID, f"k {tuple(k.shape)} / v {tuple(v.shape)} do not match q {tuple(q.shape)}")
    mptr = None
    mview = None
    if mask_kind == SDPA_MASK_BOOL:
        if mask is None or tuple(mask.shape) != (Lq, Lk) or not mask.is_contiguous() or not mask.is_cuda \
                or mask.device != q.device:
            raise SdpaError(SDPA_ERR_INVALID, f"mask must be a contiguous GPU tensor of shape ({Lq}, {Lk})")
        if mask.dtype == torch.bool:
            mask = mask.view(torch.uint8)
        if mask.dtype != torch.uint8:
            raise SdpaError(SDPA_ERR_INVALID, "mask must be uint8 or bool")
        mptr = mask.data_ptr()
        mview = (mptr, 0, 0, Lk)
    elif mask_kind == SDPA_MASK_ADDITIVE:
        if mask is None or mask.dtype != q.dtype or not mask.is_cuda or mask.device != q.device or mask.dim() < 2 \
                or mask.dim() > 4:
            raise SdpaError(SDPA_ERR_INVALID, f"an additive mask must be a 2-4 dimensional GPU tensor of {q.dtype}")
        m4 = mask.reshape((1,) * (4 - mask.dim()) + tuple(mask.shape)) if mask.dim() < 4 else mask
        try:
            m4 = m4.expand(B, Hq, Lq, Lk)
        except RuntimeError:
            raise SdpaError(SDPA_ERR_INVALID, f"additive mask {tuple(mask.shape)} does not broadcast to "
                            f"({B}, {Hq}, {Lq}, {Lk})")
        mview = _view("mask", m4, (B, Hq, Lq, Lk))
    sptr = _sinks_ptr(sinks, q, Hq)
    out = _out_tensor(out, q, (B, Hq, Lq, Dv))
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if window is not None and mask_kind != SDPA_MASK_CAUSAL:
        raise SdpaError(SDPA_ERR_INVALID, "a window needs the causal mask (mask_kind 1)")
    contiguous = q.is_contiguous() and k.is_contiguous() and v.is_contiguous()
    if not contiguous or mask_kind == SDPA_MASK_ADDITIVE:
        sdpa_forward_strided(_view("q", q, (B, Hq, Lq, D)), _view("k", k, (B, Hkv, Lk, D)),
                             _view("v", v, (B, Hkv, Lk, Dv)), out.data_ptr(), B, Hq, Hkv, Lq, Lk, D, Dv,
                             float(scale), mask_kind, mview, sptr, int(window or 0), _dtype_code(q), stream)
        return out
    if window is not None:
        sdpa_forward_windowed(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, Lq, Lk, D,
                              Dv, float(scale), int(window), sptr, _dtype_code(q), stream)
        return out
    sdpa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, Hq, Hkv, Lq, Lk, D, Dv,
                 float(scale), mask_kind, mptr, sptr, _dtype_code(q), stream)
    return out


def _gpu_tensor(name, t, dtype=None, device=None):
    if not t.is_cuda or not t.is_contiguous():
        raise SdpaError(SDPA_ERR_INVALID, f"{name} must be a contiguous GPU tensor")
    if device is not None and t.device != device:
        raise SdpaError(SDPA_ERR_INVALID, f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise SdpaError(SDPA_ERR_INVALID, f"{name} has dtype {t.dtype}, expected {dtype}")


def paged_attention(q, kcache, vcache, table, lengths, scale: float, mask_kind: int = SDPA_MASK_CAUSAL,
                    window: int = 0, sinks=None, out=None, stream=None):
    """Attention over a paged cache through sdpa_paged_forward.

    q [B,Hq,Lq,D]; kcache [blocks,Hkv,bs,D], vcache [blocks,Hkv,bs,Dv] of q's
    dtype; table [B,max_blocks] and lengths [B] int32; all contiguous GPU
    tensors. window 0 = none. Returns out [B,Hq,Lq,Dv].
    """
    import torch
    B, Hq, Lq, D = q.shape
    blocks, Hkv, bs, _ = kcache.shape
    Dv = vcache.shape[3]
    for name, t in (("q", q), ("kcache", kcache), ("vcache", vcache)):
        _gpu_tensor(name, t, q.dtype, q.device)
    for name, t in (("table", table), ("lengths", lengths)):
        _gpu_tensor(name, t, torch.int32, q.device)
    if tuple(kcache.shape) != (blocks, Hkv, bs, D) or tuple(vcache.shape[:3]) != (blocks, Hkv, bs):
        raise SdpaError(SDPA_ERR_INVALID, f"kcache {tuple(kcache.shape)} / vcache {tuple(vcache.shape)} do not "
                        f"match q {tuple(q.shape)}")
    if table.dim() != 2 or table.shape[0] != B or tuple(lengths.shape) != (B,):
        raise SdpaError(SDPA_ERR_INVALID, f"table must be [{B}, max_blocks] and lengths [{B}]")
    sptr = _sinks_ptr(sinks, q, Hq)
    out = _out_tensor(out, q, (B, Hq, Lq, Dv))
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    sdpa_paged_forward(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), out.data_ptr(), table.data_ptr(),
                       lengths.data_ptr(), B, Hq, Hkv, Lq, D, Dv, blocks, bs, table.shape[1], float(scale),
                       mask_kind, int(window), sptr, _dtype_code(q), stream)
    return out


def paged_write(cache, rows, slots, stream=None):
    """Writes rows [n,Hkv,E] into cache [blocks,Hkv,bs,E] at slots [n] (int32), in
    place, through sdpa_paged_write; slots outside the cache are skipped.
    Returns cache."""
    import torch
    blocks, Hkv, bs, E = cache.shape
    n = rows.shape[0]
    _gpu_tensor("cache", cache)
    _gpu_tensor("rows", rows, cache.dtype)
    _gpu_tensor("slots", slots, torch.int32)
    if tuple(rows.shape) != (n, Hkv, E) or tuple(slots.shape) != (n,):
        raise SdpaError(SDPA_ERR_INVALID, f"rows {tuple(rows.shape)} / slots {tuple(slots.shape)} do not match "
                        f"cache {tuple(cache.shape)}")
    if stream is None:
        stream = torch.cuda.current_stream(cache.device).cuda_stream
    sdpa_paged_write(cache.data_ptr(), rows.data_ptr(), slots.data_ptr(), n, blocks, Hkv, bs, E,
                     _dtype_code(cache), stream)
    return cache
