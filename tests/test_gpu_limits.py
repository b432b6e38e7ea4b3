"""GPU parity at the largest row stride the library accepts.

fa_bwd_create requires 128 rows of any tensor to span less than 2^30 bytes (H * d * 2 * 128 < 2^30):
the kernels address a tile with 32-bit offsets, and a padded head-dim column reads zeros through an
offset of 2^30, past the end of any tile. These cases sit just under that limit, with tensors of
2.7-2.8 GB, so that every token offset past 2^31 bytes, the buffer bounds of a 128-row tile and the
out-of-range offset of padded columns (d = 248) are exercised at their edge.

Inputs are seeded normal bf16 tensors drawn on the GPU; O, m, l come from the plain fp32 torch forward
(input preparation, as for the full-size tests). A few heads -- the first, the middle and the last --
are copied to the host and compared in full with the fp64 oracle (each head is an independent
attention problem), with the tolerance of the other parity tests.
"""
import pytest
import torch

import bench
from attention_backward_fa_amd import binding as B
from tests import parity as P

pytestmark = pytest.mark.gpu

CAUSAL = 2
LENS = [190, 140]  # two sequences: several 64-row tiles and ragged tails


def _limit_heads(d: int) -> int:
    """The largest head count with 128 rows of a [T, H, d] bf16 tensor below 2^30 bytes, rounded down
    to a multiple of 8."""
    return ((1 << 30) - 1) // (d * 2 * 128) // 8 * 8


def _inputs(heads: int, d: int, seed: int):
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    tq = sum(LENS)
    q, k, v, do = (torch.randn((tq, heads, d), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
                   for _ in range(4))
    cu = torch.tensor([0, LENS[0], tq], dtype=torch.int32)
    inp = {"q": q, "k": k, "v": v, "do": do, "cu_q": cu, "cu_kv": cu, "scale": d ** -0.5, "mask": CAUSAL,
           "max_seqlen_q": max(LENS), "max_seqlen_kv": max(LENS), "batch": len(LENS), "window": 0,
           "padded_len": 0}
    return inp


def _head(inp, o, m, l, h):
    """Head h of every tensor on the host, as a one-head problem for the oracle."""
    small = {key: inp[key][:, h:h + 1].cpu() for key in ("q", "k", "v", "do")}
    small.update({key: inp[key] for key in ("cu_q", "cu_kv", "scale", "mask", "max_seqlen_q", "max_seqlen_kv")})
    small["window"] = 0
    return small, o[:, h:h + 1].cpu(), m[:, h:h + 1].cpu(), l[:, h:h + 1].cpu()


@pytest.mark.parametrize("d,algos", [
    (256, [B.FA_BWD_ALGO_DEFAULT]),
    (248, [B.FA_BWD_ALGO_DEFAULT]),
    (128, [B.FA_BWD_ALGO_RECOMPUTE_DQ_8W, B.FA_BWD_ALGO_RECOMPUTE_DQ_4W, B.FA_BWD_ALGO_SINGLE_PASS,
           B.FA_BWD_ALGO_SPLIT_REDUCE]),
])
def test_largest_row_stride(d, algos):
    heads = _limit_heads(d)
    assert heads * d * 2 * 128 < (1 << 30) <= (heads + 8) * d * 2 * 128
    print(f"[limits] d={d} H={heads}: row {heads * d * 2} B, tensors {sum(LENS) * heads * d * 2 / 1e9:.2f} GB",
          flush=True)
    inp = _inputs(heads, d, 7000 + d)
    o, m, l = bench.torch_forward_stats(inp, torch.device("cuda"), block=256)
    torch.cuda.synchronize()
    sample = [0, heads // 2, heads - 1]
    refs = {}
    for h in sample:
        small, oh, mh, lh = _head(inp, o, m, l, h)
        refs[h] = (small, P.oracle_backward(small, oh, mh, lh))
    tq = sum(LENS)
    for algo in algos:
        print(f"[limits] d={d} H={heads} algorithm {algo}", flush=True)
        with B.FaBwd(len(LENS), heads, d, max(LENS), max(LENS), tq, tq, algo) as op:
            dq, dk, dv = op.run(inp["q"], inp["k"], inp["v"], o, inp["do"], m, l, inp["cu_q"].cuda(),
                                inp["cu_kv"].cuda(), inp["scale"], CAUSAL)
            torch.cuda.synchronize()
        for nm, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            assert bool(torch.isfinite(t).all()), f"{nm}: non-finite values"
        for h in sample:
            small, ref = refs[h]
            got = tuple(t[:, h:h + 1].float().cpu() for t in (dq, dk, dv))
            res = P.check_full(small, got, ref)
            print(f"[limits] d={d} algorithm {algo} head {h}: "
                  + " ".join(f"{k}: rel_l2={v[0]:.2e} max={v[1]:.2e}" for k, v in res.items()), flush=True)
        del dq, dk, dv
        torch.cuda.empty_cache()
