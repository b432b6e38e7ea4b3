"""GPU parity of the forward that produces the backward's inputs (``fa_fwd_run``) against the fp64
oracle forward, on the small cases of the backward parity tests; and the chained GPU forward +
GPU backward against the oracle's exact forward + backward.

Tolerance: O per tensor as for the gradients (rel-L2 <= 1e-2, max-abs <= 3e-2 * max|ref|); the
statistics come from fp32 arithmetic on the same bf16 inputs, so m and the log-sum-exp m + ln(l) must
agree to 1e-3 absolute (the scaled logits are O(10)); rows outside every sequence must hold exactly
O = 0, m = 0, l = 1.
"""
import numpy as np
import pytest
import torch

import oracle
from attention_backward_fa_amd import binding as B
from attention_backward_fa_amd import inputs as I
from tests import parity as P
from tests.test_gpu_parity import CASES, GQA_CASES, WINDOW_CASES

pytestmark = pytest.mark.gpu

STAT_TOL = 1e-3


def gpu_forward(inp):
    dev = torch.device("cuda")
    t = {k: inp[k].to(dev) for k in ("q", "k", "v", "cu_q", "cu_kv")}
    o, m, l = B.attention_forward(t["q"], t["k"], t["v"], t["cu_q"], t["cu_kv"], inp["scale"], inp["mask"],
                                  inp["max_seqlen_q"], inp["max_seqlen_kv"], inp["window"])
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), m.cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64)


def check_forward(inp, gpu, ref, rows=None):
    o, m, l = gpu
    ro, rm, rl = ref
    P.assert_close("o", o, ro)
    assert np.all(np.isfinite(m)) and np.all(l > 0)
    dm = float(np.max(np.abs(m - rm))) if m.size else 0.0
    dlse = float(np.max(np.abs((m + np.log(l)) - (rm + np.log(rl))))) if m.size else 0.0
    assert dm <= STAT_TOL and dlse <= STAT_TOL, f"m err {dm:.2e}, lse err {dlse:.2e} (tol {STAT_TOL})"
    return dm, dlse


@pytest.mark.parametrize("case", CASES + GQA_CASES + WINDOW_CASES, ids=[c.name for c in CASES + GQA_CASES + WINDOW_CASES])
def test_forward_parity(case):
    inp = I.make(case)
    print(f"[forward] {case.name}: T_q={inp['q'].shape[0]} H={case.heads} d={case.head_dim} mask={case.mask}",
          flush=True)
    o, m, l = gpu_forward(inp)
    ro, rm, rl = oracle.forward(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_kv"], inp["scale"], inp["mask"],
                                inp["max_seqlen_q"], inp["max_seqlen_kv"], inp["window"])
    valid = oracle.valid_rows(inp["cu_q"], inp["mask"], inp["max_seqlen_q"], inp["q"].shape[0])
    assert np.all(o[~valid] == 0) and np.all(m[~valid] == 0) and np.all(l[~valid] == 1)
    dm, dlse = check_forward(inp, (o[valid], m[valid], l[valid]), (ro[valid], rm[valid], rl[valid]))
    print(f"[forward] {case.name}: m err {dm:.2e} lse err {dlse:.2e}", flush=True)


CHAIN = [c for c in CASES + GQA_CASES + WINDOW_CASES
         if c.name in ("sk16_t01", "ragged_causal_d128", "ragged_causal_d64", "kv_longer_causal", "empty_sequence",
                       "padded_causal_d128", "gqa_causal_d128", "gqa_padded_causal_d128", "window_causal_d128",
                       "window_gqa_causal_d128")]


@pytest.mark.parametrize("case", CHAIN, ids=[c.name for c in CHAIN])
def test_forward_then_backward(case):
    """GPU forward feeds the GPU backward; compared with the oracle's exact fp64 forward + backward."""
    inp = I.make(case)
    dev = torch.device("cuda")
    t = {k: inp[k].to(dev) for k in ("q", "k", "v", "do", "cu_q", "cu_kv")}
    with B.FaBwd(inp["batch"], case.heads, case.head_dim, inp["max_seqlen_q"], inp["max_seqlen_kv"],
                 inp["q"].shape[0], inp["k"].shape[0], num_heads_kv=inp["k"].shape[1], window=inp["window"]) as op:
        o, m, l = op.forward(t["q"], t["k"], t["v"], t["cu_q"], t["cu_kv"], inp["scale"], inp["mask"])
        dq, dk, dv = op.run(t["q"], t["k"], t["v"], o, t["do"], m, l, t["cu_q"], t["cu_kv"], inp["scale"],
                            inp["mask"])
        torch.cuda.synchronize()
    ro, rm, rl = oracle.forward(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_kv"], inp["scale"], inp["mask"],
                                inp["max_seqlen_q"], inp["max_seqlen_kv"], inp["window"])
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], ro, inp["do"], rm, rl, inp["cu_q"], inp["cu_kv"],
                          inp["scale"], inp["mask"], inp["max_seqlen_q"], inp["max_seqlen_kv"], inp["window"])
    res = P.check_full(inp, (dq.float().cpu(), dk.float().cpu(), dv.float().cpu()), ref)
    print(f"[chain] {case.name}: " + " ".join(f"{k}: rel_l2={v[0]:.2e}" for k, v in res.items()), flush=True)


LSE_CASES = [c for c in CASES if c.name in ("tiny", "ragged_causal_d128", "padded_causal_d64", "empty_sequence")]


@pytest.mark.parametrize("case", LSE_CASES, ids=[c.name for c in LSE_CASES])
def test_backward_from_lse(case):
    """fa_bwd_run_lse with lse = m + ln(l) against the oracle backward from the same statistic."""
    inp = I.make(case)
    o, m, l = P.oracle_stats(inp)
    lse = (m.double() + torch.log(l.double())).float()
    dev = torch.device("cuda")
    t = {k: inp[k].to(dev) for k in ("q", "k", "v", "do", "cu_q", "cu_kv")}
    with B.FaBwd(inp["batch"], case.heads, case.head_dim, inp["max_seqlen_q"], inp["max_seqlen_kv"],
                 inp["q"].shape[0], inp["k"].shape[0]) as op:
        dq, dk, dv = op.run_lse(t["q"], t["k"], t["v"], o.to(dev), t["do"], lse.to(dev), t["cu_q"], t["cu_kv"],
                                inp["scale"], inp["mask"])
        torch.cuda.synchronize()
    ref = oracle.backward_from_lse(inp["q"], inp["k"], inp["v"], o, inp["do"], lse, inp["cu_q"], inp["cu_kv"],
                                   inp["scale"], inp["mask"], inp["max_seqlen_q"], inp["max_seqlen_kv"])
    res = P.check_full(inp, (dq.float().cpu(), dk.float().cpu(), dv.float().cpu()), ref)
    print(f"[lse] {case.name}: " + " ".join(f"{k}: rel_l2={v[0]:.2e}" for k, v in res.items()), flush=True)
