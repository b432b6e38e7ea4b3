"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function ``include/fa_bwd.h`` declares, and rejects bad arguments before
any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

from attention_backward_fa_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_bwd.h")


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(fa_(?:bwd|fwd)_\w+)\s*\(", text, flags=re.M)))


def test_header_declarations_match_binding():
    assert declared_functions() == sorted(B.EXPORTED)


def test_header_enum_values_match_binding():
    """Every FA_BWD_* enumerator of the header has the same value in the binding (mask codes,
    algorithm codes, status codes)."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    values = {name: int(v) for name, v in re.findall(r"\b(FA_BWD_[A-Z0-9_]+)\s*=\s*(-?\d+)", text)}
    assert {"FA_BWD_ALGO_RECOMPUTE_DQ_8W", "FA_BWD_ALGO_RECOMPUTE_DQ_4W", "FA_BWD_MASK_CAUSAL", "FA_BWD_OK"} <= set(values)
    for name, v in values.items():
        assert getattr(B, name) == v, name


def test_library_exports_every_declared_symbol():
    lib = B.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\S+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_status_strings():
    assert B.fa_bwd_status_string(0) == "ok"
    assert B.fa_bwd_status_string(1) == "invalid argument"
    assert B.fa_bwd_status_string(2) == "unsupported configuration"
    assert B.fa_bwd_status_string(3) == "out of device memory"
    assert B.fa_bwd_status_string(4) == "HIP runtime error"
    assert B.fa_bwd_status_string(99) == "unknown status"


def _create(**kw):
    d = dict(batch=1, num_heads=1, head_dim=128, max_seqlen_q=128, max_seqlen_kv=128, total_q=128, total_kv=128,
             algorithm=0)
    d.update(kw)
    lib = B.load_library()
    h = ctypes.c_void_p(0x1234)
    st = lib.fa_bwd_create(ctypes.byref(B.FaBwdDesc(**d)), ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), B.FA_BWD_ERR_INVALID_ARGUMENT),
    (dict(num_heads=0), B.FA_BWD_ERR_INVALID_ARGUMENT),
    (dict(max_seqlen_q=0), B.FA_BWD_ERR_INVALID_ARGUMENT),
    (dict(max_seqlen_kv=-5), B.FA_BWD_ERR_INVALID_ARGUMENT),
    (dict(total_q=0), B.FA_BWD_ERR_INVALID_ARGUMENT),
    (dict(total_kv=-1), B.FA_BWD_ERR_INVALID_ARGUMENT),
    (dict(head_dim=0), B.FA_BWD_ERR_UNSUPPORTED),
    (dict(head_dim=4), B.FA_BWD_ERR_UNSUPPORTED),       # head dims: multiples of 8 in [8, 256]
    (dict(head_dim=100), B.FA_BWD_ERR_UNSUPPORTED),
    (dict(head_dim=264), B.FA_BWD_ERR_UNSUPPORTED),
    (dict(head_dim_v=12), B.FA_BWD_ERR_UNSUPPORTED),
    (dict(head_dim_v=-8), B.FA_BWD_ERR_UNSUPPORTED),
    (dict(head_dim=96, algorithm=1), B.FA_BWD_ERR_UNSUPPORTED),                 # single pass: 64 or 128,
    (dict(head_dim=256, algorithm=1), B.FA_BWD_ERR_UNSUPPORTED),                # equal head dims
    (dict(head_dim=128, head_dim_v=64, algorithm=1), B.FA_BWD_ERR_UNSUPPORTED),
    (dict(num_heads=1 << 14, head_dim=256), B.FA_BWD_ERR_INVALID_ARGUMENT),     # 128 rows >= 2^30 bytes
    (dict(head_dim=96, algorithm=3), B.FA_BWD_ERR_UNSUPPORTED),                 # split-reduce: the same
    (dict(head_dim=64, head_dim_v=128, algorithm=3), B.FA_BWD_ERR_UNSUPPORTED),
    (dict(num_heads=4, num_heads_kv=1, algorithm=3), B.FA_BWD_ERR_UNSUPPORTED),
    (dict(window=32, algorithm=3), B.FA_BWD_ERR_UNSUPPORTED),
    (dict(algorithm=8), B.FA_BWD_ERR_INVALID_ARGUMENT),
    (dict(algorithm=6, head_dim=64), B.FA_BWD_ERR_UNSUPPORTED),                 # 64-key layout: d = 128
    (dict(algorithm=6, head_dim_v=64), B.FA_BWD_ERR_UNSUPPORTED),
    (dict(algorithm=7, head_dim=64), B.FA_BWD_ERR_UNSUPPORTED),                 # stored dS: the same
    (dict(algorithm=7, head_dim=128, head_dim_v=64, window=16), B.FA_BWD_ERR_UNSUPPORTED),
    (dict(algorithm=7, head_dim=96), B.FA_BWD_ERR_UNSUPPORTED),                 # or one above 128, no window
    (dict(algorithm=7, head_dim=256, window=16), B.FA_BWD_ERR_UNSUPPORTED),
    (dict(algorithm=7, head_dim=64, head_dim_v=192, window=1), B.FA_BWD_ERR_UNSUPPORTED),
    # stored dS: a dS workspace past 2^47 bytes (here 2^24 x 2^21 blocks of 16 KiB per head)
    (dict(algorithm=7, max_seqlen_q=1 << 29, max_seqlen_kv=1 << 29, total_q=1 << 29, total_kv=1 << 29),
     B.FA_BWD_ERR_UNSUPPORTED),
    (dict(algorithm=-1), B.FA_BWD_ERR_INVALID_ARGUMENT),
    (dict(total_q=1 << 40, num_heads=8), B.FA_BWD_ERR_INVALID_ARGUMENT),          # index range
    (dict(max_seqlen_kv=1 << 30, num_heads=1 << 10, batch=1 << 10), B.FA_BWD_ERR_INVALID_ARGUMENT),  # grid size
    (dict(batch=1 << 19, num_heads=1 << 10, max_seqlen_q=1, max_seqlen_kv=1, total_q=1 << 19, total_kv=1 << 19,
          algorithm=3), B.FA_BWD_ERR_INVALID_ARGUMENT),                            # 8 split workgroups each
    (dict(num_heads=6, num_heads_kv=4), B.FA_BWD_ERR_INVALID_ARGUMENT),   # K/V heads must divide query heads
    (dict(num_heads=4, num_heads_kv=-2), B.FA_BWD_ERR_INVALID_ARGUMENT),
    (dict(num_heads=4, num_heads_kv=8), B.FA_BWD_ERR_INVALID_ARGUMENT),
    (dict(num_heads=4, num_heads_kv=2, algorithm=1), B.FA_BWD_ERR_UNSUPPORTED),  # grouped heads: recompute form
    (dict(window=-1), B.FA_BWD_ERR_INVALID_ARGUMENT),
    (dict(max_seqlen_q=(1 << 30) + 1, total_q=1 << 31), B.FA_BWD_ERR_INVALID_ARGUMENT),   # positions < 2^30
    (dict(max_seqlen_kv=(1 << 30) + 1, total_kv=1 << 31), B.FA_BWD_ERR_INVALID_ARGUMENT),
    (dict(window=64, algorithm=1), B.FA_BWD_ERR_UNSUPPORTED),                    # window: recompute form
])
def test_create_rejects_bad_descriptors_before_any_hip_call(kw, status):
    st, h = _create(**kw)
    assert st == status
    assert h.value is None   # *out is cleared on failure


def test_create_null_arguments():
    lib = B.load_library()
    h = ctypes.c_void_p()
    assert lib.fa_bwd_create(None, ctypes.byref(h)) == B.FA_BWD_ERR_INVALID_ARGUMENT
    assert lib.fa_bwd_create(ctypes.byref(B.FaBwdDesc(1, 1, 128, 1, 1, 1, 1, 0)), None) == B.FA_BWD_ERR_INVALID_ARGUMENT


def test_run_and_profile_reject_null_handle():
    lib = B.load_library()
    p = ctypes.c_void_p(256)
    assert lib.fa_bwd_run(None, *([p] * 9), ctypes.c_float(0.1), 0, p, p, p, None) == B.FA_BWD_ERR_INVALID_ARGUMENT
    assert lib.fa_bwd_run_lse(None, *([p] * 8), ctypes.c_float(0.1), 0, p, p, p, None) == B.FA_BWD_ERR_INVALID_ARGUMENT
    assert lib.fa_fwd_run(None, *([p] * 5), ctypes.c_float(0.1), 0, p, p, p, None) == B.FA_BWD_ERR_INVALID_ARGUMENT
    cu = (ctypes.c_int32 * 2)(0, 1)
    assert lib.fa_bwd_plan(None, cu, cu, 0) == B.FA_BWD_ERR_INVALID_ARGUMENT
    n = ctypes.c_int32()
    assert lib.fa_bwd_profile_collect(None, None, 0, ctypes.byref(n)) == B.FA_BWD_ERR_INVALID_ARGUMENT
    assert lib.fa_bwd_profile_enable(None, 1) == B.FA_BWD_ERR_INVALID_ARGUMENT
    assert not lib.fa_bwd_get_desc(None)
    assert lib.fa_bwd_dkdv_layout(None, 0) == -1
    assert lib.fa_bwd_dq_form(None, 0) == -1


def _noalloc(desc, ptr=256, l=True):
    p = ctypes.c_void_p(ptr)
    lp = p if l else None
    return B.load_library().fa_bwd_run_noalloc(ctypes.byref(desc) if desc is not None else None, p, p, p, p, p, p,
                                                lp, p, p, ctypes.c_float(0.1), 0, p, p, p, None)


@pytest.mark.parametrize("kw,status", [
    # total_q * num_heads above the fixed scratch (2^22 rows): rejected before any HIP call
    (dict(total_q=(1 << 22) + 1, max_seqlen_q=(1 << 22) + 1), B.FA_BWD_ERR_SCRATCH_LIMIT),
    (dict(num_heads=64, total_q=(1 << 16) + 1), B.FA_BWD_ERR_SCRATCH_LIMIT),
    (dict(algorithm=1), B.FA_BWD_ERR_UNSUPPORTED),       # single-pass and split-reduce need a dQ workspace
    (dict(algorithm=3), B.FA_BWD_ERR_UNSUPPORTED),
    (dict(algorithm=7), B.FA_BWD_ERR_UNSUPPORTED),       # the stored-dS form needs a dS workspace
    (dict(batch=0), B.FA_BWD_ERR_INVALID_ARGUMENT),      # the descriptor checks of fa_bwd_create
    (dict(head_dim=100), B.FA_BWD_ERR_UNSUPPORTED),
])
def test_noalloc_rejects_before_any_hip_call(kw, status):
    d = dict(batch=1, num_heads=1, head_dim=128, max_seqlen_q=128, max_seqlen_kv=128, total_q=128, total_kv=128,
             algorithm=0)
    d.update(kw)
    assert _noalloc(B.FaBwdDesc(**d)) == status


def test_noalloc_rejects_null_and_misaligned_pointers():
    desc = B.FaBwdDesc(1, 1, 128, 128, 128, 128, 128, 0)
    assert _noalloc(None) == B.FA_BWD_ERR_INVALID_ARGUMENT
    assert _noalloc(desc, l=False) == B.FA_BWD_ERR_INVALID_ARGUMENT
    assert _noalloc(desc, ptr=258) == B.FA_BWD_ERR_INVALID_ARGUMENT
    assert B.fa_bwd_status_string(B.FA_BWD_ERR_SCRATCH_LIMIT).startswith("problem exceeds")
    assert B.FA_BWD_NOALLOC_MAX_ROWS == 1 << 22


def test_destroy_null_is_ok():
    assert B.load_library().fa_bwd_destroy(None) == B.FA_BWD_OK


def test_binding_maps_status_to_exceptions():
    with pytest.raises(ValueError):
        B.fa_bwd_create(0, 1, 128, 1, 1, 1, 1)
    with pytest.raises(NotImplementedError):
        B.fa_bwd_create(1, 1, 84, 1, 1, 1, 1)


def test_missing_library_fails_loudly(tmp_path):
    saved = B._lib
    try:
        B._lib = None
        with pytest.raises(RuntimeError, match="missing"):
            B.load_library(str(tmp_path / "nope.so"))
    finally:
        B._lib = saved
