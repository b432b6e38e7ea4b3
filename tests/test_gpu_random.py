"""Seeded random configurations of everything the recompute backward and the forward accept at once:
head dims (multiples of 8 up to 256, the value head dim equal or not), grouped K/V heads, every
mask, windows, packed and padded layouts, empty and one-token sequences, Lq != Lk. Each drawn
configuration is compared with the fp64 oracle on every valid row (backward and forward), and run
again from a host schedule (fa_bwd_plan), which must give bitwise the same gradients. The draws
are fixed by the seed below, so a failure names a reproducible case.
"""
import numpy as np
import pytest
import torch

import oracle
from attention_backward_fa_amd import binding as B
from attention_backward_fa_amd import inputs as I
from tests import parity as P
from tests.test_gpu_forward import check_forward, gpu_forward

pytestmark = pytest.mark.gpu

SEED = 20261202
DIMS = [8, 16, 32, 40, 64, 72, 96, 120, 128, 136, 160, 184, 192, 216, 256]


def _draw(n: int):
    rng = np.random.default_rng(SEED)
    cases = []
    for i in range(n):
        d = int(rng.choice(DIMS))
        dv = d if rng.random() < 0.6 else int(rng.choice(DIMS))
        hk = int(rng.integers(1, 4))
        heads = hk * int(rng.choice([1, 2, 4]))
        mask = int(rng.integers(0, 4))
        batch = int(rng.integers(1, 4))
        lq = [int(x) for x in rng.integers(0, 260, batch)]
        if max(lq) == 0:
            lq[0] = 1 + int(rng.integers(0, 200))
        if rng.random() < 0.3:
            lq[int(rng.integers(0, batch))] = 1
        lk = lq if rng.random() < 0.5 else [int(x) for x in rng.integers(1, 260, batch)]
        window = int(rng.integers(1, 160)) if rng.random() < 0.3 else 0
        padded_len = max(max(lq), max(lk)) + int(rng.integers(0, 40)) if I.is_padded_mask(mask) else 0
        cases.append(I.custom_case(f"rand{i:02d}_d{d}_dv{dv}_h{heads}_hk{hk}_m{mask}_w{window}", heads, d, mask,
                                   SEED + i, lq, lk, padded_len=padded_len, heads_kv=hk, window=window,
                                   head_dim_v=dv))
    return cases


CASES = _draw(40)


@pytest.mark.parametrize("case", CASES, ids=[c.name for c in CASES])
def test_random_configuration(case):
    inp = I.make(case)
    print(f"[random] {case.name}: lq {inp['seqlens_q']} lk {inp['seqlens_kv']} padded {case.padded_len}", flush=True)
    o, m, l = P.oracle_stats(inp)
    ref = P.oracle_backward(inp, o, m, l)
    # the two dK/dV layouts in turn (heads above 128 have one layout)
    algo = (B.FA_BWD_ALGO_RECOMPUTE_DQ_8W, B.FA_BWD_ALGO_RECOMPUTE_DQ_4W)[CASES.index(case) % 2]
    gpu = P.run_gpu(inp, o, m, l, algorithm=algo)
    res = P.check_full(inp, gpu, ref)
    # the same run from a host schedule: bitwise the same
    dev = torch.device("cuda")
    t = {k: inp[k].to(dev) for k in ("q", "k", "v", "do", "cu_q", "cu_kv")}
    with B.FaBwd(inp["batch"], case.heads, case.head_dim, inp["max_seqlen_q"], inp["max_seqlen_kv"],
                 inp["q"].shape[0], inp["k"].shape[0], algo, num_heads_kv=inp["k"].shape[1], window=inp["window"],
                 head_dim_v=inp["v"].shape[2]) as op:
        op.plan(inp["cu_q"], inp["cu_kv"], inp["mask"])
        planned = op.run(t["q"], t["k"], t["v"], o.to(dev), t["do"], m.to(dev), l.to(dev), t["cu_q"], t["cu_kv"],
                         inp["scale"], inp["mask"])
        torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv"), gpu, planned):
        assert torch.equal(x, y.float().cpu()), f"{name}: planned run differs from the dense grid"
    # the forward
    fo, fm, fl = gpu_forward(inp)
    ro, rm, rl = oracle.forward(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_kv"], inp["scale"], inp["mask"],
                                inp["max_seqlen_q"], inp["max_seqlen_kv"], inp["window"])
    valid = oracle.valid_rows(inp["cu_q"], inp["mask"], inp["max_seqlen_q"], inp["q"].shape[0])
    assert np.all(fo[~valid] == 0) and np.all(fm[~valid] == 0) and np.all(fl[~valid] == 1)
    check_forward(inp, (fo[valid], fm[valid], fl[valid]), (ro[valid], rm[valid], rl[valid]))
    print(f"[random] {case.name}: " + " ".join(f"{k}: rel_l2={v[0]:.2e}" for k, v in res.items()), flush=True)


# the stored-dS form (and the 64-key layout it runs on at head dims of 128) over a draw of its own: head
# dims of 128, with windows, and above 128 (the wide-head kernels' dS pieces, no window), grouped heads,
# every mask, packed and padded layouts, Lq != Lk; against the oracle, and planned runs bitwise equal
DS_SEED = 20261203
DS_DIMS = [128, 128, 128, 136, 160, 184, 192, 216, 256]


def _draw_ds(n: int):
    rng = np.random.default_rng(DS_SEED)
    cases = []
    for i in range(n):
        d = int(rng.choice(DS_DIMS))
        dv = 128 if d == 128 else (d if rng.random() < 0.5 else int(rng.choice([64, 96, 128, 176, 256])))
        hk = int(rng.integers(1, 4))
        heads = hk * int(rng.choice([1, 2, 4]))
        mask = int(rng.integers(0, 4))
        batch = int(rng.integers(1, 4))
        lq = [int(x) for x in rng.integers(0, 700, batch)]
        if max(lq) == 0:
            lq[0] = 1 + int(rng.integers(0, 500))
        lk = lq if rng.random() < 0.5 else [int(x) for x in rng.integers(1, 700, batch)]
        window = int(rng.integers(1, 400)) if d == 128 and rng.random() < 0.4 else 0
        padded_len = max(max(lq), max(lk)) + int(rng.integers(0, 40)) if I.is_padded_mask(mask) else 0
        cases.append(I.custom_case(f"rds{i:02d}_d{d}_dv{dv}_h{heads}_hk{hk}_m{mask}_w{window}", heads, d, mask,
                                   DS_SEED + i, lq, lk, padded_len=padded_len, heads_kv=hk, window=window,
                                   head_dim_v=dv))
    return cases


DS_CASES = _draw_ds(16)


@pytest.mark.parametrize("case", DS_CASES, ids=[c.name for c in DS_CASES])
def test_random_stored_ds(case):
    inp = I.make(case)
    print(f"[random-ds] {case.name}: lq {inp['seqlens_q']} lk {inp['seqlens_kv']} padded {case.padded_len}",
          flush=True)
    o, m, l = P.oracle_stats(inp)
    ref = P.oracle_backward(inp, o, m, l)
    algos = [B.FA_BWD_ALGO_STORED_DS] + ([B.FA_BWD_ALGO_RECOMPUTE_DQ_64K] if case.head_dim == 128 else [])
    dev = torch.device("cuda")
    t = {k: inp[k].to(dev) for k in ("q", "k", "v", "do", "cu_q", "cu_kv")}
    for algo in algos:
        gpu = P.run_gpu(inp, o, m, l, algorithm=algo)
        res = P.check_full(inp, gpu, ref)
        with B.FaBwd(inp["batch"], case.heads, case.head_dim, inp["max_seqlen_q"], inp["max_seqlen_kv"],
                     inp["q"].shape[0], inp["k"].shape[0], algo, num_heads_kv=inp["k"].shape[1],
                     window=inp["window"], head_dim_v=inp["v"].shape[2]) as op:
            op.plan(inp["cu_q"], inp["cu_kv"], inp["mask"])
            planned = op.run(t["q"], t["k"], t["v"], o.to(dev), t["do"], m.to(dev), l.to(dev), t["cu_q"],
                             t["cu_kv"], inp["scale"], inp["mask"])
            torch.cuda.synchronize()
        for name, x, y in zip(("dq", "dk", "dv"), gpu, planned):
            assert torch.equal(x, y.float().cpu()), f"{name}: planned run differs from the dense grid ({algo})"
        print(f"[random-ds] {case.name} algorithm {algo}: " +
              " ".join(f"{k}: rel_l2={v[0]:.2e}" for k, v in res.items()), flush=True)
