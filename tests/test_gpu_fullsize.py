"""GPU parity at the full sizes of the benchmark workloads, over whole gradient tensors.

For each workload the seeded inputs are drawn once; the fp64 oracle's forward
(over query row blocks) gives O (bf16), m, l (fp32), and its backward gives
the reference dQ, dK, dV. Every algorithm then runs once on those inputs in
the launch configuration bench.py times (one handle, inputs resident on the
GPU, one ``fa_bwd_run`` on the current stream), and every valid row of every
output tensor is compared with the reference: relative L2 error <= 1e-2 and
max |gpu - ref| <= 3e-2 * max |ref| per tensor; rows outside every sequence
must be exactly zero. The forward is compared the same way on O, with bounds
on m and on the log-sum-exp m + ln l.

The oracle runs on a thread pool of the host's CPUs (at most 16); the longest
workload (two sequences in 32768-row slots, 16 heads) takes on the order of a
minute or two there. Setting FA_ORACLE_CACHE to a directory keeps the oracle's
results on disk between runs.
"""
import time

import numpy as np
import pytest
import torch

import oracle
from attention_backward_fa_amd import binding as B
from attention_backward_fa_amd import inputs
from tests import parity as P

pytestmark = pytest.mark.gpu

FULL = ["dense", "varlen", "causal", "longpad"]
ALGOS = {"default": B.FA_BWD_ALGO_DEFAULT, "eightwave": B.FA_BWD_ALGO_RECOMPUTE_DQ_8W,
         "fourwave": B.FA_BWD_ALGO_RECOMPUTE_DQ_4W, "keys64": B.FA_BWD_ALGO_RECOMPUTE_DQ_64K,
         "singlepass": B.FA_BWD_ALGO_SINGLE_PASS, "splitreduce": B.FA_BWD_ALGO_SPLIT_REDUCE,
         "storedds": B.FA_BWD_ALGO_STORED_DS}
# the variant workloads (grouped K/V heads, a window, other head dims) in the default form, and the
# window one also in the 64-key and stored-dS forms
VARIANTS = ["causal_gqa", "causal_window", "causal_d256", "causal_mla"]
# (workload, algorithm): every algorithm of a workload runs while its reference is held, then the
# forward of that workload where it is checked
CASES = ([(n, a) for n in FULL for a in list(ALGOS) + (["forward"] if n in ("causal", "longpad") else [])]
         + [(n, a) for n in VARIANTS for a in ["default"] + (["keys64", "storedds"] if n == "causal_window" else [])])

_held = {}


def _log(name):
    return lambda msg: print(f"[fullsize] {name}: {msg}", flush=True)


def _workload(name):
    """Inputs, the oracle's statistics and reference gradients, and device copies of one workload
    (one workload held at a time)."""
    if name not in _held:
        _held.clear()
        torch.cuda.empty_cache()
        inp = inputs.make(name)
        t0 = time.perf_counter()
        (o, m, l), ref = P.reference(inp, log=_log(name))
        _log(name)(f"reference ready in {time.perf_counter() - t0:.1f} s")
        dev = {k: inp[k].to("cuda:0") for k in ("q", "k", "v", "do", "cu_q", "cu_kv")}
        dev.update(o=o.to("cuda:0"), m=m.to("cuda:0"), l=l.to("cuda:0"))
        _held[name] = (inp, (o, m, l), ref, dev)
    return _held[name]


def _handle(inp, algo):
    tq, heads, d = inp["q"].shape
    return B.FaBwd(inp["batch"], heads, d, inp["max_seqlen_q"], inp["max_seqlen_kv"], tq, inp["k"].shape[0], algo,
                   num_heads_kv=inp["k"].shape[1], window=inp["window"], head_dim_v=inp["v"].shape[2])


@pytest.mark.parametrize("name,algo", CASES)
def test_fullsize_whole_tensors(name, algo):
    print(f"[fullsize] {name} ({algo})", flush=True)
    inp, (o, m, l), ref, dev = _workload(name)
    tq, heads, d = inp["q"].shape
    print(f"[fullsize] {name} ({algo}): T_q={tq} T_kv={inp['k'].shape[0]} H={heads} H_kv={inp['k'].shape[1]} "
          f"d={d} d_v={inp['v'].shape[2]} mask={inp['mask']} window={inp['window']}", flush=True)
    if algo == "forward":
        return _check_forward(name, inp, (o, m, l), dev)
    with _handle(inp, ALGOS[algo]) as op:
        dq, dk, dv = op.run(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["m"], dev["l"], dev["cu_q"],
                            dev["cu_kv"], inp["scale"], inp["mask"])
        torch.cuda.synchronize()
    gpu = tuple(x.float().cpu() for x in (dq, dk, dv))
    res = P.check_full(inp, gpu, ref)
    print(f"[fullsize] {name} ({algo}): " + " ".join(f"{k}: rel_l2={v[0]:.2e} max={v[1]:.2e}" for k, v in res.items()),
          flush=True)


def _check_forward(name, inp, stats, dev):
    """The forward at full size, in the configuration bench.py --path forward times, against the oracle
    forward over whole tensors."""
    o_ref, m_ref, l_ref = stats
    tq, heads, d = inp["q"].shape
    with B.FaBwd(inp["batch"], heads, d, inp["max_seqlen_q"], inp["max_seqlen_kv"], tq, inp["k"].shape[0]) as op:
        o, m, l = op.forward(dev["q"], dev["k"], dev["v"], dev["cu_q"], dev["cu_kv"], inp["scale"], inp["mask"])
        torch.cuda.synchronize()
    vq = oracle.valid_rows(inp["cu_q"], inp["mask"], inp["max_seqlen_q"], tq)
    o, m, l = o.float().cpu().numpy(), m.cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64)
    assert np.all(o[~vq] == 0) and np.all(m[~vq] == 0) and np.all(l[~vq] == 1)
    # the reference O is the oracle's fp64 O rounded to bf16 (the backward's input): the difference holds
    # both sides' final rounding, each at most half a bf16 unit, far inside the tolerance
    rel, mx = P.assert_close("o", o[vq], o_ref.float().numpy()[vq].astype(np.float64))
    dm = float(np.max(np.abs(m[vq] - m_ref.numpy()[vq])))
    dlse = float(np.max(np.abs(m[vq] + np.log(l[vq]) - m_ref.numpy()[vq] - np.log(l_ref.numpy()[vq]))))
    assert dm <= 1e-3 and dlse <= 1e-3, f"m err {dm:.2e}, lse err {dlse:.2e}"
    print(f"[fullsize] {name} (forward): o rel_l2={rel:.2e} max={mx:.2e} m err {dm:.2e} lse err {dlse:.2e}",
          flush=True)
