"""GPU tests of the host-side schedule (``fa_bwd_plan``): with a plan the recompute kernels and the
forward launch one workgroup per non-empty (tile, head, sequence), longest first, instead of the
dense grid. Each workgroup computes what it computes in the dense grid, so planned and dense runs
must agree bitwise; one planned case is also compared with the oracle. Host-side rejections of bad
offsets keep the previous plan."""
import pytest
import torch

from attention_backward_fa_amd import binding as B
from attention_backward_fa_amd import inputs as I
from tests import parity as P

pytestmark = pytest.mark.gpu

NONE, PAD, CAUSAL, PADC = I.MASK_NONE, I.MASK_PADDING, I.MASK_CAUSAL, I.MASK_PADDING_CAUSAL

CASES = [
    I.custom_case("plan_varlen_none", 4, 128, NONE, 401, [700, 65, 1, 300, 0, 129]),
    I.custom_case("plan_varlen_causal", 4, 128, CAUSAL, 402, [513, 64, 200, 1000]),
    I.custom_case("plan_kv_longer_causal", 2, 64, CAUSAL, 403, [100, 250], [380, 64]),
    I.custom_case("plan_padded_causal", 2, 128, PADC, 404, [300, 131], padded_len=320),
    I.custom_case("plan_gqa_window", 4, 128, CAUSAL, 405, [600, 90], heads_kv=2, window=100),
    I.custom_case("plan_wide_mla", 2, 192, CAUSAL, 406, [333, 70], head_dim_v=128),
    # d = 256: the stored-dS pass runs eight-wave workgroups on the dense grid, four-wave ones planned
    I.custom_case("plan_wide_d256", 2, 256, CAUSAL, 408, [300, 77, 260]),
    # 96 heads x 4 sequences of up to 1024 tokens, no mask: the dQ kernel's dense grid runs head-major
    # per XCD (384 (sequence, head) pairs divide over 8 XCDs; the largest workgroup, 16 key steps, is
    # under a quarter of the work per slot on 256 CUs)
    I.custom_case("plan_head_major_none", 96, 128, NONE, 407, [1024, 1000, 777, 1024]),
]


def _tensors(inp, dev):
    return {k: inp[k].to(dev) for k in ("q", "k", "v", "do", "cu_q", "cu_kv")}


def _op(inp, case, algorithm=B.FA_BWD_ALGO_DEFAULT):
    return B.FaBwd(inp["batch"], case.heads, case.head_dim, inp["max_seqlen_q"], inp["max_seqlen_kv"],
                   inp["q"].shape[0], inp["k"].shape[0], algorithm, num_heads_kv=inp["k"].shape[1],
                   window=inp["window"], head_dim_v=inp["v"].shape[2])


def _run(op, inp, t, o, m, l):
    dq, dk, dv = op.run(t["q"], t["k"], t["v"], o, t["do"], m, l, t["cu_q"], t["cu_kv"], inp["scale"], inp["mask"])
    fo, fm, fl = op.forward(t["q"], t["k"], t["v"], t["cu_q"], t["cu_kv"], inp["scale"], inp["mask"])
    torch.cuda.synchronize()
    return [x.clone() for x in (dq, dk, dv, fo, fm, fl)]


@pytest.mark.parametrize("algo", [B.FA_BWD_ALGO_DEFAULT, B.FA_BWD_ALGO_RECOMPUTE_DQ_4W, B.FA_BWD_ALGO_RECOMPUTE_DQ_64K,
                                  B.FA_BWD_ALGO_STORED_DS], ids=["default", "4w", "64k", "storedds"])
@pytest.mark.parametrize("case", CASES, ids=[c.name for c in CASES])
def test_planned_equals_dense_bitwise(case, algo):
    d128 = case.head_dim == 128 and case.head_dim_v in (0, 128)
    wide = max(case.head_dim, case.head_dim_v or case.head_dim) > 128 and case.window == 0
    if algo == B.FA_BWD_ALGO_RECOMPUTE_DQ_64K and not d128:
        pytest.skip("the 64-key layout needs head dims of 128")
    if algo == B.FA_BWD_ALGO_STORED_DS and not (d128 or wide):
        pytest.skip("the stored-dS form needs head dims of 128, or one above 128 and no window")
    inp = I.make(case)
    print(f"[plan] {case.name}: lengths {inp['seqlens_q']} mask {case.mask} algorithm {algo}", flush=True)
    dev = torch.device("cuda")
    t = _tensors(inp, dev)
    o, m, l = (x.to(dev) for x in P.oracle_stats(inp))
    with _op(inp, case, algo) as op:
        dense = _run(op, inp, t, o, m, l)
        op.plan(inp["cu_q"], inp["cu_kv"], inp["mask"])
        planned = _run(op, inp, t, o, m, l)
        op.plan(None, None, inp["mask"])  # dropped: the dense grid again
        again = _run(op, inp, t, o, m, l)
    for name, x, y, z in zip(("dq", "dk", "dv", "o", "m", "l"), dense, planned, again):
        assert torch.equal(x, y), f"{name}: planned run differs from the dense grid"
        assert torch.equal(x, z), f"{name}: run after dropping the plan differs"


def test_planned_matches_oracle():
    case = CASES[1]
    inp = I.make(case)
    dev = torch.device("cuda")
    t = _tensors(inp, dev)
    o, m, l = P.oracle_stats(inp)
    with _op(inp, case) as op:
        op.plan(inp["cu_q"], inp["cu_kv"], inp["mask"])
        dq, dk, dv = op.run(t["q"], t["k"], t["v"], o.to(dev), t["do"], m.to(dev), l.to(dev), t["cu_q"], t["cu_kv"],
                            inp["scale"], inp["mask"])
        torch.cuda.synchronize()
    P.check_full(inp, (dq.float().cpu(), dk.float().cpu(), dv.float().cpu()), P.oracle_backward(inp, o, m, l))


def test_plan_for_another_mask_is_not_used():
    case = CASES[1]
    inp = I.make(case)
    dev = torch.device("cuda")
    t = _tensors(inp, dev)
    o, m, l = (x.to(dev) for x in P.oracle_stats(inp))
    with _op(inp, case) as op:
        dense = _run(op, inp, t, o, m, l)
        op.plan(inp["cu_q"], inp["cu_kv"], NONE)  # the runs use CAUSAL: dense grid
        other = _run(op, inp, t, o, m, l)
    for x, y in zip(dense, other):
        assert torch.equal(x, y)


def test_plan_rejects_bad_offsets_and_keeps_the_previous_plan():
    case = CASES[0]
    inp = I.make(case)
    dev = torch.device("cuda")
    t = _tensors(inp, dev)
    o, m, l = (x.to(dev) for x in P.oracle_stats(inp))
    cu = inp["cu_q"].tolist()
    with _op(inp, case) as op:
        op.plan(inp["cu_q"], inp["cu_kv"], inp["mask"])
        planned = _run(op, inp, t, o, m, l)
        bad = [
            [1] + cu[1:],                                   # cu[0] != 0
            cu[:2] + [cu[1] - 1] + cu[3:],                  # decreasing
            cu[:-1] + [cu[-1] + 1],                         # past total_q
            [0] + [inp["max_seqlen_q"] + 1] * (len(cu) - 1),  # a length above max_seqlen_q
        ]
        for b in bad:
            with pytest.raises(ValueError):
                op.plan(b, inp["cu_kv"], inp["mask"])
        with pytest.raises(ValueError):
            op.plan(cu[:-1], inp["cu_kv"], inp["mask"])     # wrong count
        with pytest.raises(ValueError):
            op.plan(inp["cu_q"], None, inp["mask"])         # one array only
        after = _run(op, inp, t, o, m, l)
    for x, y in zip(planned, after):
        assert torch.equal(x, y)


@pytest.mark.parametrize("algo", [B.FA_BWD_ALGO_SINGLE_PASS, B.FA_BWD_ALGO_SPLIT_REDUCE])
def test_single_pass_handle_has_no_plan(algo):
    with B.FaBwd(1, 2, 128, 64, 64, 64, 64, algo) as op:
        with pytest.raises(NotImplementedError):
            op.plan([0, 64], [0, 64], NONE)
