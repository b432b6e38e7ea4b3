"""The allocation-free entry point (fa_bwd_run_noalloc) against fa_bwd_run.

Two calls in a row through the C ABI, the second on a smaller problem (fewer
rows x heads, another head dim, a padded mask), so that it runs on the fixed
scratch array the first call left filled. Each call's dQ, dK, dV must equal
bitwise those of a handle of the recompute form created from the same sizes
(the same kernels and layout rule; the default's stored-dS form needs a dS
workspace, so the allocation-free default is the recompute form), lie within
the per-tensor tolerance of the fp64 oracle, and the output buffers (filled
with NaN beforehand) must be fully written.
"""
import numpy as np
import pytest
import torch

from attention_backward_fa_amd import binding as B
from attention_backward_fa_amd import inputs as I
from tests import parity as P

pytestmark = pytest.mark.gpu

CASES = [
    I.custom_case("noalloc_large", 4, 128, I.MASK_CAUSAL, 251, [1500, 700, 333]),
    I.custom_case("noalloc_small", 2, 64, I.MASK_PADDING_CAUSAL, 252, [200, 97], padded_len=256),
]


def _desc(inp, algorithm):
    tq, heads, d = inp["q"].shape
    return B.FaBwdDesc(inp["batch"], heads, d, inp["max_seqlen_q"], inp["max_seqlen_kv"], tq, inp["k"].shape[0],
                       algorithm, inp["k"].shape[1], inp["window"], inp["v"].shape[2])


def test_noalloc_equals_fa_bwd_run_on_two_calls_the_second_smaller():
    dev = torch.device("cuda:0")
    for case in CASES:
        print(f"[noalloc] {case.name}: H={case.heads} d={case.head_dim} mask={case.mask}", flush=True)
        inp = I.make(case)
        o, m, l = P.oracle_stats(inp)
        ref = P.oracle_backward(inp, o, m, l)
        t = {k: inp[k].to(dev) for k in ("q", "k", "v", "do", "cu_q", "cu_kv")}
        od, md, ld = o.to(dev), m.to(dev), l.to(dev)
        desc = _desc(inp, B.FA_BWD_ALGO_DEFAULT)
        with B.FaBwd(inp["batch"], case.heads, case.head_dim, inp["max_seqlen_q"], inp["max_seqlen_kv"],
                     inp["q"].shape[0], inp["k"].shape[0], B.FA_BWD_ALGO_RECOMPUTE_DQ) as op:
            want = op.run(t["q"], t["k"], t["v"], od, t["do"], md, ld, t["cu_q"], t["cu_kv"], inp["scale"],
                          inp["mask"])
        got = tuple(torch.full_like(x, float("nan")) for x in want)
        B.fa_bwd_run_noalloc(desc, t["q"], t["k"], t["v"], od, t["do"], md, ld, t["cu_q"], t["cu_kv"], inp["scale"],
                             inp["mask"], *got)
        torch.cuda.synchronize()
        for name, g, w in zip(("dq", "dk", "dv"), got, want):
            assert bool(torch.isfinite(g).all()), f"{name}: not every output element was written"
            assert torch.equal(g, w), f"{name}: differs from fa_bwd_run"
        res = P.check_full(inp, tuple(x.float().cpu() for x in got), ref)
        print(f"[noalloc] {case.name}: " + " ".join(f"{k}: rel_l2={v[0]:.2e}" for k, v in res.items()), flush=True)


def test_noalloc_rejects_a_problem_beyond_the_scratch():
    """total_q * num_heads above the fixed array: a clear error, nothing enqueued."""
    dev = torch.device("cuda:0")
    rows = B.FA_BWD_NOALLOC_MAX_ROWS // 8 + 1
    desc = B.FaBwdDesc(1, 8, 64, rows, rows, rows, rows, B.FA_BWD_ALGO_DEFAULT, 0, 0, 0)
    x = torch.zeros((rows, 8, 64), dtype=torch.bfloat16, device=dev)
    st = torch.zeros((rows, 8), dtype=torch.float32, device=dev)
    cu = torch.tensor([0, rows], dtype=torch.int32, device=dev)
    with pytest.raises(ValueError, match="fixed scratch"):
        B.fa_bwd_run_noalloc(desc, x, x, x, x, x, st, st, cu, cu, 0.125, 0, x, x, x)
    assert np.isfinite(float(x.float().sum()))
