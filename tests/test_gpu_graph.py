"""The backward captured in a HIP graph (torch.cuda.graph, whose capture records the work the library
enqueues on torch's current stream) and replayed: a handle's run allocates and memsets nothing per
call (its workspaces come from fa_bwd_create, and the row kernel clears what must start at zero), and
the allocation-free entry point allocates nothing at all. Each graph is replayed several times, with
the program's own eager work (the outputs filled with NaN) and a synchronisation between replays, and
every replay's dQ, dK, dV must equal the eager run's bitwise (every form here is deterministic).
"""
import pytest
import torch

from attention_backward_fa_amd import binding as B
from attention_backward_fa_amd import inputs as I
from tests import parity as P

pytestmark = pytest.mark.gpu

CASES = [
    # (case, algorithm): the stored-dS form on the 64-key layout (dS blocks), the recompute form, the
    # stored-dS form of the wide-head kernels (dS pieces), and the default's choice
    (I.custom_case("graph_storedds_causal", 4, 128, I.MASK_CAUSAL, 261, [700, 333]), B.FA_BWD_ALGO_STORED_DS),
    (I.custom_case("graph_recompute_padded", 2, 128, I.MASK_PADDING_CAUSAL, 262, [300, 131], padded_len=320),
     B.FA_BWD_ALGO_RECOMPUTE_DQ),
    (I.custom_case("graph_wide_storedds", 4, 192, I.MASK_CAUSAL, 263, [260, 111], head_dim_v=128),
     B.FA_BWD_ALGO_STORED_DS),
    (I.custom_case("graph_default_gqa_window", 4, 128, I.MASK_CAUSAL, 264, [500, 90], heads_kv=2, window=100),
     B.FA_BWD_ALGO_DEFAULT),
]
REPLAYS = 3


def _replay_and_check(graph, outs, want, label):
    for r in range(REPLAYS):
        for x in outs:  # the program's own eager work between replays
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, g, w in zip(("dq", "dk", "dv"), outs, want):
            assert torch.equal(g, w), f"{label}: {name} of replay {r} differs from the eager run"


@pytest.mark.parametrize("case,algo", CASES, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_backward_graph_replays_equal_eager(case, algo):
    inp = I.make(case)
    print(f"[graph] {case.name}: algorithm {algo}", flush=True)
    dev = torch.device("cuda:0")
    o, m, l = P.oracle_stats(inp)
    t = {k: inp[k].to(dev) for k in ("q", "k", "v", "do", "cu_q", "cu_kv")}
    od, md, ld = o.to(dev), m.to(dev), l.to(dev)
    tq, heads, d = inp["q"].shape
    with B.FaBwd(inp["batch"], heads, d, inp["max_seqlen_q"], inp["max_seqlen_kv"], tq, inp["k"].shape[0], algo,
                 num_heads_kv=inp["k"].shape[1], window=inp["window"], head_dim_v=inp["v"].shape[2]) as op:
        run = lambda *outs: op.run(t["q"], t["k"], t["v"], od, t["do"], md, ld, t["cu_q"], t["cu_kv"], inp["scale"],
                                   inp["mask"], *outs)
        want = tuple(x.clone() for x in run())
        torch.cuda.synchronize()
        outs = tuple(torch.empty_like(x) for x in want)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # a warm-up on a side stream before capture, as torch asks
            run(*outs)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run(*outs)
        torch.cuda.synchronize()
        _replay_and_check(graph, outs, want, case.name)
        del graph
    ref = P.oracle_backward(inp, o, m, l)
    P.check_full(inp, tuple(x.float().cpu() for x in want), ref)


def test_noalloc_graph_replays_equal_eager():
    """fa_bwd_run_noalloc captured: the callers it is for include code under graph capture."""
    case = I.custom_case("graph_noalloc", 4, 128, I.MASK_CAUSAL, 265, [900, 257])
    inp = I.make(case)
    print(f"[graph] {case.name}: fa_bwd_run_noalloc", flush=True)
    dev = torch.device("cuda:0")
    o, m, l = P.oracle_stats(inp)
    t = {k: inp[k].to(dev) for k in ("q", "k", "v", "do", "cu_q", "cu_kv")}
    od, md, ld = o.to(dev), m.to(dev), l.to(dev)
    tq, heads, d = inp["q"].shape
    desc = B.FaBwdDesc(inp["batch"], heads, d, inp["max_seqlen_q"], inp["max_seqlen_kv"], tq, inp["k"].shape[0],
                       B.FA_BWD_ALGO_DEFAULT, inp["k"].shape[1], inp["window"], inp["v"].shape[2])
    run = lambda *outs: B.fa_bwd_run_noalloc(desc, t["q"], t["k"], t["v"], od, t["do"], md, ld, t["cu_q"],
                                             t["cu_kv"], inp["scale"], inp["mask"], *outs)
    want = tuple(torch.empty_like(x) for x in (t["q"], t["k"], t["v"]))
    run(*want)
    torch.cuda.synchronize()
    outs = tuple(torch.empty_like(x) for x in want)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(*outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(*outs)
    torch.cuda.synchronize()
    _replay_and_check(graph, outs, want, case.name)
