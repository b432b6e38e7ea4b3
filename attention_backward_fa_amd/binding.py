"""ctypes binding of ``libfa_bwd.so`` (C ABI in ``include/fa_bwd.h``).

Argument marshalling only: the functions keep the C names, check that torch
tensors match the shapes, dtypes, device and contiguity the C ABI assumes
(the C side sees bare pointers and cannot), pass their device pointers and
the current HIP stream, and turn status codes into exceptions
(invalid argument -> ValueError, unsupported -> NotImplementedError,
out of memory / HIP error -> RuntimeError). All compute runs in the library.
There is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa_bwd.so")

FA_BWD_OK = 0
FA_BWD_ERR_INVALID_ARGUMENT = 1
FA_BWD_ERR_UNSUPPORTED = 2
FA_BWD_ERR_OUT_OF_MEMORY = 3
FA_BWD_ERR_HIP = 4
FA_BWD_ERR_SCRATCH_LIMIT = 5
FA_BWD_NOALLOC_MAX_ROWS = 1 << 22

FA_BWD_ALGO_DEFAULT = 0
FA_BWD_ALGO_SINGLE_PASS = 1
FA_BWD_ALGO_RECOMPUTE_DQ = 2
FA_BWD_ALGO_SPLIT_REDUCE = 3
FA_BWD_ALGO_RECOMPUTE_DQ_8W = 4
FA_BWD_ALGO_RECOMPUTE_DQ_4W = 5
FA_BWD_ALGO_RECOMPUTE_DQ_64K = 6
FA_BWD_ALGO_STORED_DS = 7

FA_BWD_MASK_NONE = 0
FA_BWD_MASK_PADDING = 1
FA_BWD_MASK_CAUSAL = 2
FA_BWD_MASK_PADDING_CAUSAL = 3

# every symbol include/fa_bwd.h declares
EXPORTED = ("fa_bwd_create", "fa_bwd_run", "fa_bwd_run_lse", "fa_bwd_run_noalloc", "fa_fwd_run", "fa_bwd_plan",
            "fa_bwd_destroy", "fa_bwd_status_string", "fa_bwd_get_desc", "fa_bwd_dkdv_layout", "fa_bwd_dq_form",
            "fa_bwd_profile_enable", "fa_bwd_profile_collect")


class FaBwdDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_kv", ctypes.c_int32),
                ("total_q", ctypes.c_int64), ("total_kv", ctypes.c_int64), ("algorithm", ctypes.c_int32),
                ("num_heads_kv", ctypes.c_int32), ("window", ctypes.c_int32), ("head_dim_v", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Open the library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m attention_backward_fa_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    lib.fa_bwd_create.argtypes = [ctypes.POINTER(FaBwdDesc), ctypes.POINTER(vp)]
    lib.fa_bwd_create.restype = i32
    lib.fa_bwd_run.argtypes = [vp] * 10 + [f32, i32] + [vp] * 4
    lib.fa_bwd_run.restype = i32
    lib.fa_bwd_run_lse.argtypes = [vp] * 9 + [f32, i32] + [vp] * 4
    lib.fa_bwd_run_lse.restype = i32
    lib.fa_bwd_run_noalloc.argtypes = [ctypes.POINTER(FaBwdDesc)] + [vp] * 9 + [f32, i32] + [vp] * 4
    lib.fa_bwd_run_noalloc.restype = i32
    lib.fa_fwd_run.argtypes = [vp] * 6 + [f32, i32] + [vp] * 4
    lib.fa_fwd_run.restype = i32
    lib.fa_bwd_plan.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32), i32]
    lib.fa_bwd_plan.restype = i32
    lib.fa_bwd_destroy.argtypes = [vp]
    lib.fa_bwd_destroy.restype = i32
    lib.fa_bwd_status_string.argtypes = [i32]
    lib.fa_bwd_status_string.restype = ctypes.c_char_p
    lib.fa_bwd_get_desc.argtypes = [vp]
    lib.fa_bwd_get_desc.restype = ctypes.POINTER(FaBwdDesc)
    lib.fa_bwd_dkdv_layout.argtypes = [vp, i32]
    lib.fa_bwd_dkdv_layout.restype = i32
    lib.fa_bwd_dq_form.argtypes = [vp, i32]
    lib.fa_bwd_dq_form.restype = i32
    lib.fa_bwd_profile_enable.argtypes = [vp, i32]
    lib.fa_bwd_profile_enable.restype = i32
    lib.fa_bwd_profile_collect.argtypes = [vp, ctypes.POINTER(f32), i32, ctypes.POINTER(i32)]
    lib.fa_bwd_profile_collect.restype = i32
    _lib = lib
    return lib


def fa_bwd_status_string(status: int) -> str:
    return load_library().fa_bwd_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status == FA_BWD_OK:
        return
    msg = f"{what}: {fa_bwd_status_string(status)} (status {status})"
    if status in (FA_BWD_ERR_INVALID_ARGUMENT, FA_BWD_ERR_SCRATCH_LIMIT):
        raise ValueError(msg)
    if status == FA_BWD_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise RuntimeError(msg)


def fa_bwd_create(batch: int, num_heads: int, head_dim: int, max_seqlen_q: int, max_seqlen_kv: int,
                  total_q: int, total_kv: int, algorithm: int = FA_BWD_ALGO_DEFAULT,
                  num_heads_kv: int = 0, window: int = 0, head_dim_v: int = 0) -> ctypes.c_void_p:
    """Create a handle (and its device workspace on the current device); num_heads_kv 0 = num_heads;
    window 0 = none, w > 0 = each query i sees keys (i - w, i]; head_dim_v (V, O, dO, dV) 0 = head_dim."""
    desc = FaBwdDesc(batch, num_heads, head_dim, max_seqlen_q, max_seqlen_kv, total_q, total_kv, algorithm,
                     num_heads_kv, window, head_dim_v)
    handle = ctypes.c_void_p()
    _check(load_library().fa_bwd_create(ctypes.byref(desc), ctypes.byref(handle)), "fa_bwd_create")
    return handle


def fa_bwd_get_desc(handle) -> FaBwdDesc:
    ptr = load_library().fa_bwd_get_desc(handle)
    if not ptr:
        raise ValueError("fa_bwd_get_desc: null handle")
    return ptr.contents


def fa_bwd_dkdv_layout(handle, mask: int) -> int:
    """The algorithm code of the dK/dV layout runs under `mask` take on this handle (-1: invalid)."""
    return int(load_library().fa_bwd_dkdv_layout(handle, int(mask)))


def fa_bwd_dq_form(handle, mask: int) -> int:
    """The algorithm code of the way runs under `mask` form dQ on this handle (stored dS or recompute;
    -1: invalid)."""
    return int(load_library().fa_bwd_dq_form(handle, int(mask)))


def fa_bwd_destroy(handle) -> None:
    _check(load_library().fa_bwd_destroy(handle), "fa_bwd_destroy")


def fa_bwd_plan(handle, cu_seqlens_q, cu_seqlens_kv, mask: int) -> None:
    """Longest-first schedule from host sequence offsets (any int sequence, numpy array or CPU tensor of
    batch + 1 entries); later runs with this mask launch one workgroup per non-empty tile. Both None
    drops the plan."""
    if cu_seqlens_q is None and cu_seqlens_kv is None:
        _check(load_library().fa_bwd_plan(handle, None, None, int(mask)), "fa_bwd_plan")
        return
    d = fa_bwd_get_desc(handle)
    arrays = []
    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_kv", cu_seqlens_kv)):
        if cu is None:
            raise ValueError(f"{name}: both offset arrays or neither")
        if hasattr(cu, "device") and getattr(cu.device, "type", "cpu") != "cpu":
            raise ValueError(f"{name}: expected host values, got device {cu.device}")
        vals = [int(x) for x in (cu.tolist() if hasattr(cu, "tolist") else cu)]
        if len(vals) != d.batch + 1:
            raise ValueError(f"{name}: expected {d.batch + 1} entries, got {len(vals)}")
        arrays.append((ctypes.c_int32 * len(vals))(*vals))
    _check(load_library().fa_bwd_plan(handle, arrays[0], arrays[1], int(mask)), "fa_bwd_plan")


def _expect(t, name, shape, dtype, device):
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def fa_bwd_run(handle, q, k, v, o, dout, m, l, cu_seqlens_q, cu_seqlens_kv, scale: float, mask: int,
               dq, dk, dv, stream=None) -> None:
    """Enqueue the backward on ``stream`` (default: torch's current stream of q's device).

    Tensors: q, dq bf16 [total_q, H, d]; o, dout bf16 [total_q, H, d_v]; k, dk bf16 [total_kv, H_kv, d];
    v, dv bf16 [total_kv, H_kv, d_v]; m, l fp32 [total_q, H]; cu_seqlens_* int32 [batch + 1]; all on one GPU
    (d = head_dim, d_v = head_dim_v of the handle).
    """
    import torch
    d = fa_bwd_get_desc(handle)
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"q: expected a GPU tensor, got device {dev}")
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    qs, os_ = (d.total_q, d.num_heads, d.head_dim), (d.total_q, d.num_heads, d.head_dim_v)
    ks, vs = (d.total_kv, d.num_heads_kv, d.head_dim), (d.total_kv, d.num_heads_kv, d.head_dim_v)
    ptrs = [
        _expect(q, "q", qs, bf, dev), _expect(k, "k", ks, bf, dev), _expect(v, "v", vs, bf, dev),
        _expect(o, "o", os_, bf, dev), _expect(dout, "dout", os_, bf, dev),
        _expect(m, "m", qs[:2], f32, dev), _expect(l, "l", qs[:2], f32, dev),
        _expect(cu_seqlens_q, "cu_seqlens_q", (d.batch + 1,), i32, dev),
        _expect(cu_seqlens_kv, "cu_seqlens_kv", (d.batch + 1,), i32, dev),
    ]
    outs = [_expect(dq, "dq", qs, bf, dev), _expect(dk, "dk", ks, bf, dev), _expect(dv, "dv", vs, bf, dev)]
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    st = load_library().fa_bwd_run(handle, *ptrs, ctypes.c_float(scale), int(mask), *outs, ctypes.c_void_p(stream))
    _check(st, "fa_bwd_run")


def fa_bwd_run_noalloc(desc: FaBwdDesc, q, k, v, o, dout, m, l, cu_seqlens_q, cu_seqlens_kv, scale: float,
                       mask: int, dq, dk, dv, stream=None) -> None:
    """The allocation-free backward: no handle, the library's fixed scratch array (at most
    FA_BWD_NOALLOC_MAX_ROWS = total_q * num_heads); tensors as for ``fa_bwd_run`` with the sizes of
    ``desc`` (num_heads_kv, head_dim_v of 0 meaning num_heads, head_dim)."""
    import torch
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"q: expected a GPU tensor, got device {dev}")
    hk = desc.num_heads_kv or desc.num_heads
    dvd = desc.head_dim_v or desc.head_dim
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    qs, os_ = (desc.total_q, desc.num_heads, desc.head_dim), (desc.total_q, desc.num_heads, dvd)
    ks, vs = (desc.total_kv, hk, desc.head_dim), (desc.total_kv, hk, dvd)
    ptrs = [
        _expect(q, "q", qs, bf, dev), _expect(k, "k", ks, bf, dev), _expect(v, "v", vs, bf, dev),
        _expect(o, "o", os_, bf, dev), _expect(dout, "dout", os_, bf, dev),
        _expect(m, "m", qs[:2], f32, dev), _expect(l, "l", qs[:2], f32, dev),
        _expect(cu_seqlens_q, "cu_seqlens_q", (desc.batch + 1,), i32, dev),
        _expect(cu_seqlens_kv, "cu_seqlens_kv", (desc.batch + 1,), i32, dev),
    ]
    outs = [_expect(dq, "dq", qs, bf, dev), _expect(dk, "dk", ks, bf, dev), _expect(dv, "dv", vs, bf, dev)]
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    st = load_library().fa_bwd_run_noalloc(ctypes.byref(desc), *ptrs, ctypes.c_float(scale), int(mask), *outs,
                                           ctypes.c_void_p(stream))
    _check(st, "fa_bwd_run_noalloc")


def fa_bwd_run_lse(handle, q, k, v, o, dout, lse, cu_seqlens_q, cu_seqlens_kv, scale: float, mask: int,
                   dq, dk, dv, stream=None) -> None:
    """The backward with one log-sum-exp per row (lse = m + ln l, fp32 [total_q, H]) instead of (m, l)."""
    import torch
    d = fa_bwd_get_desc(handle)
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"q: expected a GPU tensor, got device {dev}")
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    qs, os_ = (d.total_q, d.num_heads, d.head_dim), (d.total_q, d.num_heads, d.head_dim_v)
    ks, vs = (d.total_kv, d.num_heads_kv, d.head_dim), (d.total_kv, d.num_heads_kv, d.head_dim_v)
    ptrs = [
        _expect(q, "q", qs, bf, dev), _expect(k, "k", ks, bf, dev), _expect(v, "v", vs, bf, dev),
        _expect(o, "o", os_, bf, dev), _expect(dout, "dout", os_, bf, dev), _expect(lse, "lse", qs[:2], f32, dev),
        _expect(cu_seqlens_q, "cu_seqlens_q", (d.batch + 1,), i32, dev),
        _expect(cu_seqlens_kv, "cu_seqlens_kv", (d.batch + 1,), i32, dev),
    ]
    outs = [_expect(dq, "dq", qs, bf, dev), _expect(dk, "dk", ks, bf, dev), _expect(dv, "dv", vs, bf, dev)]
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    st = load_library().fa_bwd_run_lse(handle, *ptrs, ctypes.c_float(scale), int(mask), *outs,
                                       ctypes.c_void_p(stream))
    _check(st, "fa_bwd_run_lse")


def fa_fwd_run(handle, q, k, v, cu_seqlens_q, cu_seqlens_kv, scale: float, mask: int, o, m, l,
               stream=None) -> None:
    """Enqueue the forward (O, m, l for the backward) on ``stream`` (default: torch's current stream).

    Tensors: q bf16 [total_q, H, d]; o bf16 [total_q, H, d_v] (written); k bf16 [total_kv, H_kv, d];
    v bf16 [total_kv, H_kv, d_v]; m, l fp32 [total_q, H] (written); cu_seqlens_* int32 [batch + 1]; all on
    one GPU.
    """
    import torch
    d = fa_bwd_get_desc(handle)
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"q: expected a GPU tensor, got device {dev}")
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    qs, os_ = (d.total_q, d.num_heads, d.head_dim), (d.total_q, d.num_heads, d.head_dim_v)
    ks, vs = (d.total_kv, d.num_heads_kv, d.head_dim), (d.total_kv, d.num_heads_kv, d.head_dim_v)
    ptrs = [
        _expect(q, "q", qs, bf, dev), _expect(k, "k", ks, bf, dev), _expect(v, "v", vs, bf, dev),
        _expect(cu_seqlens_q, "cu_seqlens_q", (d.batch + 1,), i32, dev),
        _expect(cu_seqlens_kv, "cu_seqlens_kv", (d.batch + 1,), i32, dev),
    ]
    outs = [_expect(o, "o", os_, bf, dev), _expect(m, "m", qs[:2], f32, dev), _expect(l, "l", qs[:2], f32, dev)]
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    st = load_library().fa_fwd_run(handle, *ptrs, ctypes.c_float(scale), int(mask), *outs, ctypes.c_void_p(stream))
    _check(st, "fa_fwd_run")


def fa_bwd_profile_enable(handle, enable: bool) -> None:
    _check(load_library().fa_bwd_profile_enable(handle, 1 if enable else 0), "fa_bwd_profile_enable")


def fa_bwd_profile_collect(handle, max_runs: int = 4096):
    """Per-run kernel times [(first_ms, second_ms, third_ms), ...] of the runs recorded since the last call:
    backward (row statistics, dK/dV or single-pass main kernel, dQ kernel or dQ cast); forward (fill,
    forward kernel, 0)."""
    buf = (ctypes.c_float * (3 * max_runs))()
    n = ctypes.c_int32()
    _check(load_library().fa_bwd_profile_collect(handle, buf, max_runs, ctypes.byref(n)), "fa_bwd_profile_collect")
    return [tuple(buf[3 * r:3 * r + 3]) for r in range(n.value)]


class FaBwd:
    """Owns one handle; ``run`` allocates nothing when the outputs are passed in."""

    def __init__(self, batch, num_heads, head_dim, max_seqlen_q, max_seqlen_kv, total_q, total_kv,
                 algorithm=FA_BWD_ALGO_DEFAULT, num_heads_kv=0, window=0, head_dim_v=0):
        self.handle = fa_bwd_create(batch, num_heads, head_dim, max_seqlen_q, max_seqlen_kv, total_q, total_kv,
                                    algorithm, num_heads_kv, window, head_dim_v)

    def run(self, q, k, v, o, dout, m, l, cu_seqlens_q, cu_seqlens_kv, scale, mask, dq=None, dk=None, dv=None,
            stream=None):
        import torch
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        fa_bwd_run(self.handle, q, k, v, o, dout, m, l, cu_seqlens_q, cu_seqlens_kv, scale, mask, dq, dk, dv, stream)
        return dq, dk, dv

    def run_lse(self, q, k, v, o, dout, lse, cu_seqlens_q, cu_seqlens_kv, scale, mask, dq=None, dk=None, dv=None,
                stream=None):
        import torch
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        fa_bwd_run_lse(self.handle, q, k, v, o, dout, lse, cu_seqlens_q, cu_seqlens_kv, scale, mask, dq, dk, dv,
                       stream)
        return dq, dk, dv

    def forward(self, q, k, v, cu_seqlens_q, cu_seqlens_kv, scale, mask, o=None, m=None, l=None, stream=None):
        import torch
        o = torch.empty(q.shape[:2] + v.shape[2:], dtype=q.dtype, device=q.device) if o is None else o
        m = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device) if m is None else m
        l = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device) if l is None else l
        fa_fwd_run(self.handle, q, k, v, cu_seqlens_q, cu_seqlens_kv, scale, mask, o, m, l, stream)
        return o, m, l

    def dkdv_layout(self, mask):
        return fa_bwd_dkdv_layout(self.handle, mask)

    def dq_form(self, mask):
        return fa_bwd_dq_form(self.handle, mask)

    def plan(self, cu_seqlens_q, cu_seqlens_kv, mask):
        fa_bwd_plan(self.handle, cu_seqlens_q, cu_seqlens_kv, mask)

    def close(self):
        if self.handle is not None and self.handle.value:
            fa_bwd_destroy(self.handle)
        self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def attention_backward(q, k, v, o, dout, m, l, cu_seqlens_q, cu_seqlens_kv, scale: float, mask: int,
                       max_seqlen_q: int, max_seqlen_kv: int, algorithm: int = FA_BWD_ALGO_DEFAULT,
                       window: int = 0):
    """One-shot call: create a handle, run on the current stream, destroy (which waits)."""
    with FaBwd(cu_seqlens_q.numel() - 1, q.shape[1], q.shape[2], max_seqlen_q, max_seqlen_kv,
               q.shape[0], k.shape[0], algorithm, k.shape[1], window, v.shape[2]) as op:
        return op.run(q, k, v, o, dout, m, l, cu_seqlens_q, cu_seqlens_kv, scale, mask)


def attention_forward(q, k, v, cu_seqlens_q, cu_seqlens_kv, scale: float, mask: int, max_seqlen_q: int,
                      max_seqlen_kv: int, window: int = 0):
    """One-shot forward: returns O (bf16), m, l (fp32) on q's device."""
    with FaBwd(cu_seqlens_q.numel() - 1, q.shape[1], q.shape[2], max_seqlen_q, max_seqlen_kv,
               q.shape[0], k.shape[0], num_heads_kv=k.shape[1], window=window, head_dim_v=v.shape[2]) as op:
        return op.forward(q, k, v, cu_seqlens_q, cu_seqlens_kv, scale, mask)
