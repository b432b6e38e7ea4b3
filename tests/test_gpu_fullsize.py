"""GPU parity at the full sizes of the benchmark workloads, in the launch
configuration bench.py times: one handle per workload, inputs resident on the
GPU, O, m, l from the plain fp32 torch forward (bench.make_workload), one
``fa_bwd_run`` on the current stream.

The fp64 oracle computes sampled outputs one by one (``oracle.backward_rows``):
rows of dQ and rows of dK/dV of a few (sequence, head) pairs, at tile edges
(0, 31/32, 63/64, 127/128), the middle, the last rows and random rows. The
sampled rows of each tensor are compared as one set against the per-tensor
tolerance of the small-size tests. Every output is also checked for what holds
at any size: all values finite, rows outside every sequence exactly zero.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
from attention_backward_fa_amd import binding as B
from tests import parity as P

pytestmark = pytest.mark.gpu

FULL = ["dense", "varlen", "causal", "longpad"]
ALGOS = {"default": B.FA_BWD_ALGO_DEFAULT, "eightwave": B.FA_BWD_ALGO_RECOMPUTE_DQ_8W,
         "fourwave": B.FA_BWD_ALGO_RECOMPUTE_DQ_4W, "singlepass": B.FA_BWD_ALGO_SINGLE_PASS,
         "splitreduce": B.FA_BWD_ALGO_SPLIT_REDUCE}
# the workloads with grouped K/V heads, a window or other head dims run the recompute form only
VARIANTS = ["causal_gqa", "causal_window", "causal_d256", "causal_mla"]
BACKWARD = [(n, a) for n in FULL for a in ALGOS] + [(n, "default") for n in VARIANTS]

_cache = {}


def _workload(name):
    """Inputs and the torch-forward statistics of one workload (built once per module)."""
    if name not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        inp, dev = bench.make_workload(name, torch.device("cuda:0"))
        host = {k: dev[k].float().cpu() for k in ("o", "m", "l")}
        _cache[name] = (inp, dev, host)
    return _cache[name]


def _rows(length, rng, n_random=5):
    picks = {0, 1, 31, 32, 63, 64, 127, 128, length // 2, length - 2, length - 1}
    picks |= set(rng.integers(0, length, n_random).tolist())
    return sorted(r for r in picks if 0 <= r < length)


def _pairs(inp, rng):
    """(sequence, head) pairs to sample: first and last head of the longest
    sequence, a random head of the shortest non-empty one and of a random one."""
    lens = np.asarray(inp["seqlens_q"])
    heads = inp["q"].shape[1]
    nonempty = np.flatnonzero(lens > 0)
    longest = int(nonempty[np.argmax(lens[nonempty])])
    shortest = int(nonempty[np.argmin(lens[nonempty])])
    pairs = {(longest, 0), (longest, heads - 1), (shortest, int(rng.integers(heads))),
             (int(rng.choice(nonempty)), int(rng.integers(heads)))}
    return sorted(pairs)


@pytest.mark.parametrize("name,algo", BACKWARD)
def test_fullsize_sampled(name, algo):
    inp, dev, host = _workload(name)
    tq, heads, d = inp["q"].shape
    tk = inp["k"].shape[0]
    print(f"[fullsize] {name} ({algo}): T_q={tq} T_kv={tk} H={heads} H_kv={inp['k'].shape[1]} d={d} "
          f"d_v={inp['v'].shape[2]} mask={inp['mask']} window={inp['window']}", flush=True)
    with B.FaBwd(inp["batch"], heads, d, inp["max_seqlen_q"], inp["max_seqlen_kv"], tq, tk, ALGOS[algo],
                 num_heads_kv=inp["k"].shape[1], window=inp["window"], head_dim_v=inp["v"].shape[2]) as op:
        dq, dk, dv = op.run(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["m"], dev["l"], dev["cu_q"],
                            dev["cu_kv"], inp["scale"], inp["mask"])
        torch.cuda.synchronize()
    for nm, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), f"{nm}: non-finite values"
    vq = torch.from_numpy(oracle.valid_rows(inp["cu_q"], inp["mask"], inp["max_seqlen_q"], tq)).to(dq.device)
    vk = torch.from_numpy(oracle.valid_rows(inp["cu_kv"], inp["mask"], inp["max_seqlen_kv"], tk)).to(dk.device)
    assert int((dq[~vq] != 0).sum()) == 0, "dq: rows outside every sequence are not zero"
    assert int((dk[~vk] != 0).sum()) == 0 and int((dv[~vk] != 0).sum()) == 0, \
        "dk/dv: rows outside every sequence are not zero"

    rng = np.random.default_rng(1000 + inp["seed"])
    segq = oracle.segments(inp["cu_q"], inp["mask"], inp["max_seqlen_q"])
    segk = oracle.segments(inp["cu_kv"], inp["mask"], inp["max_seqlen_kv"])
    got = {"dq": [], "dk": [], "dv": []}
    ref = {"dq": [], "dk": [], "dv": []}
    for b, h in _pairs(inp, rng):
        (qs, lq), (ks, lk) = segq[b], segk[b]
        qr, kr = _rows(lq, rng), _rows(lk, rng)
        rq, rk, rv = oracle.backward_rows(inp["q"], inp["k"], inp["v"], host["o"], inp["do"], host["m"], host["l"],
                                          inp["cu_q"], inp["cu_kv"], inp["scale"], inp["mask"], b, h, qr, kr,
                                          inp["max_seqlen_q"], inp["max_seqlen_kv"], inp["window"])
        hk = h // (heads // inp["k"].shape[1])  # the K/V head whose dK/dV rows these are
        got["dq"].append(dq[[qs + r for r in qr], h].float().cpu().numpy())
        got["dk"].append(dk[[ks + r for r in kr], hk].float().cpu().numpy())
        got["dv"].append(dv[[ks + r for r in kr], hk].float().cpu().numpy())
        ref["dq"].append(rq)
        ref["dk"].append(rk)
        ref["dv"].append(rv)
    res = {nm: P.assert_close(nm, np.concatenate(got[nm]), np.concatenate(ref[nm])) for nm in got}
    print(f"[fullsize] {name} ({algo}): " + " ".join(f"{k}: rel_l2={v[0]:.2e} max={v[1]:.2e}"
                                                     for k, v in res.items()), flush=True)


@pytest.mark.parametrize("name", ["causal", "longpad"])
def test_fullsize_forward_sampled(name):
    """The forward at full size, in the configuration bench.py --path forward times."""
    from attention_backward_fa_amd import inputs
    inp = inputs.make(name)
    tq, heads, d = inp["q"].shape
    dev = torch.device("cuda:0")
    t = {k: inp[k].to(dev) for k in ("q", "k", "v", "cu_q", "cu_kv")}
    print(f"[fullsize-forward] {name}: T_q={tq} H={heads} d={d} mask={inp['mask']}", flush=True)
    with B.FaBwd(inp["batch"], heads, d, inp["max_seqlen_q"], inp["max_seqlen_kv"], tq, inp["k"].shape[0]) as op:
        o, m, l = op.forward(t["q"], t["k"], t["v"], t["cu_q"], t["cu_kv"], inp["scale"], inp["mask"])
        torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(m).all()) and bool((l > 0).all())
    vq = torch.from_numpy(oracle.valid_rows(inp["cu_q"], inp["mask"], inp["max_seqlen_q"], tq)).to(dev)
    assert int((o[~vq] != 0).sum()) == 0 and bool((m[~vq] == 0).all()) and bool((l[~vq] == 1).all())
    rng = np.random.default_rng(2000 + inp["seed"])
    segq = oracle.segments(inp["cu_q"], inp["mask"], inp["max_seqlen_q"])
    got_o, ref_o, dm, dlse = [], [], 0.0, 0.0
    for b, h in _pairs(inp, rng):
        qs, lq = segq[b]
        rows = _rows(lq, rng)
        ro, rm, rl = oracle.forward_rows(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_kv"], inp["scale"],
                                         inp["mask"], b, h, rows, inp["max_seqlen_q"], inp["max_seqlen_kv"])
        idx = [qs + r for r in rows]
        got_o.append(o[idx, h].float().cpu().numpy())
        ref_o.append(ro)
        gm = m[idx, h].cpu().numpy().astype(np.float64)
        gl = l[idx, h].cpu().numpy().astype(np.float64)
        dm = max(dm, float(np.max(np.abs(gm - rm))))
        dlse = max(dlse, float(np.max(np.abs(gm + np.log(gl) - rm - np.log(rl)))))
    rel, mx = P.assert_close("o", np.concatenate(got_o), np.concatenate(ref_o))
    assert dm <= 1e-3 and dlse <= 1e-3, f"m err {dm:.2e}, lse err {dlse:.2e}"
    print(f"[fullsize-forward] {name}: o rel_l2={rel:.2e} max={mx:.2e} m err {dm:.2e} lse err {dlse:.2e}", flush=True)
