"""GPU parity: the HIP backward against the fp64 oracle on the same seeded
inputs, every valid row compared, at sizes the oracle finishes in seconds.

Cases: the tiny workload (1 head, 128 tokens, d 64), the d in {64, 128} rows
of the PyPTO-Gym SK-16 test matrix (§七) as packed sequences (among them
test_02: 8 sequences of 2432 tokens, 8 heads, d 64, lengths that are not a
multiple of the 128-row tiles), and ragged
cases for every mask type (lengths that are not multiples of the 64-row q
step or the 128-row kv tile, a single-token sequence, an empty sequence,
Lq != Lk, padded slots with garbage in the padding rows).
"""
import numpy as np
import pytest
import torch

from attention_backward_fa_amd import binding as B
from attention_backward_fa_amd import inputs as I
from tests import parity as P

pytestmark = pytest.mark.gpu

NONE, PAD, CAUSAL, PADC = I.MASK_NONE, I.MASK_PADDING, I.MASK_CAUSAL, I.MASK_PADDING_CAUSAL

CASES = [
    I.CASES["tiny"],
    I.CASES["sk16_t01"],
    I.CASES["sk16_t02"],
    I.CASES["sk16_t05"],
    I.CASES["sk16_t06"],
    I.custom_case("ragged_none_d128", 3, 128, NONE, 201, [1, 77, 200, 333]),
    I.custom_case("ragged_causal_d128", 2, 128, CAUSAL, 202, [129, 300, 64, 1]),
    I.custom_case("ragged_causal_d64", 2, 64, CAUSAL, 203, [255, 257]),
    I.custom_case("kv_longer_none", 2, 128, NONE, 204, [100, 250], [180, 64]),
    I.custom_case("kv_longer_causal", 2, 128, CAUSAL, 205, [100, 250], [180, 64]),
    I.custom_case("empty_sequence", 2, 128, NONE, 206, [90, 0, 150]),
    I.custom_case("padded_d128", 2, 128, PAD, 207, [300, 131], padded_len=300),
    I.custom_case("padded_causal_d128", 2, 128, PADC, 208, [300, 131], padded_len=320, qk_mult=2.0),
    I.custom_case("padded_causal_d64", 2, 64, PADC, 209, [97, 200], [150, 64], padded_len=256),
]


ALGOS = {"recompute": B.FA_BWD_ALGO_RECOMPUTE_DQ, "recompute8w": B.FA_BWD_ALGO_RECOMPUTE_DQ_8W,
         "recompute4w": B.FA_BWD_ALGO_RECOMPUTE_DQ_4W, "singlepass": B.FA_BWD_ALGO_SINGLE_PASS,
         "splitreduce": B.FA_BWD_ALGO_SPLIT_REDUCE, "recompute64k": B.FA_BWD_ALGO_RECOMPUTE_DQ_64K,
         "storedds": B.FA_BWD_ALGO_STORED_DS}


def _supported(case, algo):
    # the 64-key dK/dV layout (and the stored-dS form on it) exists for head dims of 128
    return algo not in ("recompute64k", "storedds") or (case.head_dim == 128 and case.head_dim_v in (0, 128))


# (case, algorithm) pairs, case-major so that each case's oracle reference is computed once
PAIRS = [(c, a) for c in CASES for a in ALGOS if _supported(c, a)]
LAYOUTS = {"8w": B.FA_BWD_ALGO_RECOMPUTE_DQ_8W, "4w": B.FA_BWD_ALGO_RECOMPUTE_DQ_4W}


_held = {}


def _case_reference(case):
    """Inputs, oracle statistics and oracle gradients of one case, computed once for all algorithms
    (the cases run case-major)."""
    if case.name not in _held:
        _held.clear()
        inp = I.make(case)
        o, m, l = P.oracle_stats(inp)
        _held[case.name] = (inp, (o, m, l), P.oracle_backward(inp, o, m, l))
    inp, (o, m, l), ref = _held[case.name]
    clone = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    return clone, (o.clone(), m.clone(), l.clone()), ref


@pytest.mark.parametrize("case,algo", PAIRS, ids=[f"{c.name}-{a}" for c, a in PAIRS])
def test_parity_full(case, algo):
    print(f"[parity] {case.name} ({algo})", flush=True)
    inp, (o, m, l), ref = _case_reference(case)
    print(f"[parity] {case.name} ({algo}): T_q={inp['q'].shape[0]} H={case.heads} d={case.head_dim} "
          f"mask={case.mask}", flush=True)
    if I.is_padded_mask(case.mask):
        # the backward must not read padding rows: fill them with NaN
        vq = torch.from_numpy(P.oracle.valid_rows(inp["cu_q"], case.mask, inp["max_seqlen_q"], inp["q"].shape[0]))
        o[~vq] = float("nan")
        m[~vq] = float("nan")
        l[~vq] = float("nan")
        inp["do"][~vq] = float("nan")
        inp["q"][~vq] = float("nan")
        vk = torch.from_numpy(P.oracle.valid_rows(inp["cu_kv"], case.mask, inp["max_seqlen_kv"], inp["k"].shape[0]))
        inp["k"][~vk] = float("nan")
        inp["v"][~vk] = float("nan")
    gpu = P.run_gpu(inp, o, m, l, algorithm=ALGOS[algo])
    res = P.check_full(inp, gpu, ref)
    print(f"[parity] {case.name} ({algo}): " + " ".join(f"{k}: rel_l2={v[0]:.2e} max={v[1]:.2e}" for k, v in res.items()),
          flush=True)


def test_repeat_runs_agree_single_pass():
    """Atomic summation order may change between runs; results stay within tolerance of each other."""
    inp = I.make(I.CASES["sk16_t01"])
    o, m, l = P.oracle_stats(inp)
    a = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_SINGLE_PASS)
    b = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_SINGLE_PASS)
    for x, y in zip(a, b):
        P.assert_close("repeat", x.numpy(), y.numpy().astype(np.float64))


@pytest.mark.parametrize("layout", list(LAYOUTS))
def test_recompute_is_bitwise_reproducible(layout):
    """No atomics in the recompute form: repeated runs are bitwise identical, in either dK/dV layout."""
    inp = I.make(I.custom_case("repro", 4, 128, I.MASK_CAUSAL, 210, [700, 333]))
    o, m, l = P.oracle_stats(inp)
    a = P.run_gpu(inp, o, m, l, algorithm=LAYOUTS[layout])
    b = P.run_gpu(inp, o, m, l, algorithm=LAYOUTS[layout])
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("case", [I.custom_case("storedds_causal", 3, 128, I.MASK_CAUSAL, 216, [700, 333, 64, 1]),
                                  I.custom_case("storedds_padded", 2, 128, I.MASK_PADDING_CAUSAL, 217, [300, 131],
                                                padded_len=320),
                                  I.custom_case("storedds_kv_longer", 2, 128, I.MASK_NONE, 218, [100, 250],
                                                [600, 64]),
                                  # a window whose band starts at the last key of a 256-key block for the
                                  # q tile at row 384: the blocks of its later 32-row steps are not written
                                  I.custom_case("storedds_window_edge", 2, 128, I.MASK_CAUSAL, 219, [700, 450],
                                                window=130)], ids=lambda c: c.name)
def test_stored_ds_matches_recompute(case):
    """The stored-dS form runs the 64-key dK/dV kernel with dS stores added: its dK, dV equal the 64-key
    recompute form's bitwise; its dQ sums the same bf16 dS values in another kernel, so it agrees within
    the tolerance. Repeated runs are bitwise identical (every output row has one owner)."""
    inp = I.make(case)
    o, m, l = P.oracle_stats(inp)
    a = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_RECOMPUTE_DQ_64K)
    b = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_STORED_DS)
    c = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_STORED_DS)
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2]), "dk, dv differ from the 64-key recompute form"
    P.assert_close("dq", b[0].numpy(), a[0].numpy().astype(np.float64))
    for x, y in zip(b, c):
        assert torch.equal(x, y)


@pytest.mark.parametrize("case", [I.custom_case("layouts_causal", 3, 128, I.MASK_CAUSAL, 211, [700, 333, 64]),
                                  I.custom_case("layouts_padded", 2, 64, I.MASK_PADDING, 212, [250, 97],
                                                padded_len=256)], ids=lambda c: c.name)
def test_dkdv_layouts_agree(case):
    """The two dK/dV layouts share the dQ kernel (dQ bitwise equal); their dK, dV differ only in the
    order of the fp32 sums, so they agree within the tolerance."""
    inp = I.make(case)
    o, m, l = P.oracle_stats(inp)
    a = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_RECOMPUTE_DQ_8W)
    b = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_RECOMPUTE_DQ_4W)
    assert torch.equal(a[0], b[0]), "dq differs between the layouts"
    for name, x, y in zip(("dk", "dv"), a[1:], b[1:]):
        P.assert_close(name, y.numpy(), x.numpy().astype(np.float64))


@pytest.mark.parametrize("case,expect,form", [
    # causal, d 64 (no 64-key layout), 256 heads of 1024 tokens: the dK/dV work (128-key tiles, 64-row q
    # steps) totals 72 per head, 18432 in all; the largest workgroup has 16, and 2 * 16 * 256 CUs =
    # 8192 <= 18432: the four-wave layout
    (I.custom_case("layout_rule_4w", 256, 64, I.MASK_CAUSAL, 213, [1024]), B.FA_BWD_ALGO_RECOMPUTE_DQ_4W,
     B.FA_BWD_ALGO_RECOMPUTE_DQ),
    # no mask, 8 heads of 2 x 2048 tokens: 256-key tiles of 64 steps (32 rows) total 8192, and
    # 2 * 64 * 256 > 8192; 128-key tiles: 256 workgroups of 32 steps, 2 * 32 * 256 > 8192: eight waves
    (I.custom_case("layout_rule_8w", 8, 128, I.MASK_NONE, 214, [2048, 2048]), B.FA_BWD_ALGO_RECOMPUTE_DQ_8W,
     B.FA_BWD_ALGO_RECOMPUTE_DQ),
    # causal, d 128, 256 heads of 1024 tokens: 256-key tiles of 32, 24, 16 and 8 steps total 80 per
    # head, 20480 in all, and 2 * 32 * 256 = 16384 <= 20480: the 64-key layout, and with it the stored-dS
    # form (its dS workspace: 256 heads x 32 q steps x 4 kv tiles x 16 KiB = 512 MiB, within 8 GiB)
    (I.custom_case("layout_rule_64k", 256, 128, I.MASK_CAUSAL, 215, [1024]), B.FA_BWD_ALGO_RECOMPUTE_DQ_64K,
     B.FA_BWD_ALGO_STORED_DS),
    # causal, d 128, 64 query heads over 16 K/V heads of 2048 tokens: each workgroup runs the steps of 4
    # query heads; 256-key tiles: 288 steps per head, 18432 in all, largest workgroup 4 * 64, and
    # 2 * 256 * 256 > 18432; 128-key tiles: 17408 in all, largest 4 * 32, 2 * 128 * 256 > 17408: eight waves
    (I.custom_case("layout_rule_gqa", 64, 128, I.MASK_CAUSAL, 216, [2048], heads_kv=16),
     B.FA_BWD_ALGO_RECOMPUTE_DQ_8W, B.FA_BWD_ALGO_RECOMPUTE_DQ),
], ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_default_picks_the_balanced_dkdv_layout(case, expect, form):
    """The default form takes the dK/dV layout the load-balance rule names (figures for the 256
    compute units of an MI355X) and the dQ form its rule names: its dK, dV equal that layout's recompute
    form bitwise (the same kernel, with dS stores where it stores dS), and its dQ equals the recompute
    form's bitwise or, from stored dS, within the tolerance."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the expected layouts are worked out for 256 compute units")
    inp = I.make(case)
    tq, heads, d = inp["q"].shape
    with B.FaBwd(inp["batch"], heads, d, inp["max_seqlen_q"], inp["max_seqlen_kv"], tq, inp["k"].shape[0],
                 num_heads_kv=inp["k"].shape[1]) as op:
        assert op.dkdv_layout(case.mask) == expect
        assert op.dq_form(case.mask) == form
        assert op.dkdv_layout(-1) == -1 and op.dq_form(-1) == -1
    o, m, l = P.oracle_stats(inp)
    got = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_DEFAULT)
    ref = P.run_gpu(inp, o, m, l, algorithm=expect)
    assert torch.equal(got[1], ref[1]) and torch.equal(got[2], ref[2]), "dk, dv: not the expected layout"
    if form == B.FA_BWD_ALGO_STORED_DS:
        P.assert_close("dq", got[0].numpy(), ref[0].numpy().astype(np.float64))
    else:
        assert torch.equal(got[0], ref[0]), "dq: not the recompute form"


# sequences longer than 8 kv tiles of 128 keys: each split-reduce workgroup walks several tiles and
# adds into its own dQ buffer (the first tile stores, later ones load and add)
LONG_CASES = [
    I.custom_case("long_causal_d128", 2, 128, CAUSAL, 241, [2300, 1100]),
    I.custom_case("long_none_kv_longer_d64", 2, 64, NONE, 242, [700, 1500], [2200, 1030]),
    I.custom_case("long_padded_causal_d128", 1, 128, PADC, 243, [1900, 1024], padded_len=2048),
]


@pytest.mark.parametrize("case", LONG_CASES, ids=[c.name for c in LONG_CASES])
def test_parity_split_reduce_long(case):
    inp = I.make(case)
    print(f"[parity-long] {case.name}: lq {inp['seqlens_q']} lk {inp['seqlens_kv']}", flush=True)
    o, m, l = P.oracle_stats(inp)
    ref = P.oracle_backward(inp, o, m, l)
    gpu = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_SPLIT_REDUCE)
    res = P.check_full(inp, gpu, ref)
    again = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_SPLIT_REDUCE)
    for name, x, y in zip(("dq", "dk", "dv"), gpu, again):
        assert torch.equal(x, y), f"{name}: split-reduce runs differ"
    print(f"[parity-long] {case.name}: " + " ".join(f"{k}: rel_l2={v[0]:.2e} max={v[1]:.2e}" for k, v in res.items()),
          flush=True)


def test_split_reduce_is_bitwise_reproducible():
    """Each dQ element is summed in a fixed order (kv tiles of a split, then the splits): repeated runs
    are bitwise identical, and dK, dV are those of the single-pass form (no atomics touch them)."""
    inp = I.make(I.custom_case("repro_split", 4, 128, I.MASK_CAUSAL, 212, [1700, 333]))
    o, m, l = P.oracle_stats(inp)
    a = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_SPLIT_REDUCE)
    b = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_SPLIT_REDUCE)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    c = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_SINGLE_PASS)
    assert torch.equal(a[1], c[1]) and torch.equal(a[2], c[2])
    P.assert_close("dq", a[0].numpy(), c[0].numpy().astype(np.float64))


def test_algorithms_agree():
    inp = I.make(I.custom_case("agree", 2, 64, I.MASK_NONE, 211, [400, 129]))
    o, m, l = P.oracle_stats(inp)
    a = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_RECOMPUTE_DQ)
    b = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_SINGLE_PASS)
    # the two forms sum in different orders (dQ atomics vs owned rows; token order inside the MFMA
    # k-steps), so they agree to rounding, not bitwise
    for name, x, y in zip(("dq", "dk", "dv"), a, b):
        P.assert_close(name, x.numpy(), y.numpy().astype(np.float64))


# grouped K/V heads (query head h reads K/V head h // (H / H_kv)); recompute form only
GQA_CASES = [
    I.custom_case("gqa_none_d128", 4, 128, NONE, 221, [200, 129], heads_kv=2),
    I.custom_case("gqa_causal_d128", 8, 128, CAUSAL, 222, [300, 77], heads_kv=2),
    I.custom_case("mqa_causal_d64", 4, 64, CAUSAL, 223, [255], heads_kv=1),
    I.custom_case("gqa_padded_causal_d128", 6, 128, PADC, 224, [150, 97], padded_len=160, heads_kv=3),
]


# the default form, and the 64-key dK/dV layout (whose workgroups run every query head of a K/V head)
GQA_PAIRS = [(c, a) for c in GQA_CASES for a in ("recompute", "recompute64k", "storedds") if _supported(c, a)]


@pytest.mark.parametrize("case,algo", GQA_PAIRS, ids=[f"{c.name}-{a}" for c, a in GQA_PAIRS])
def test_parity_grouped_heads(case, algo):
    inp = I.make(case)
    print(f"[parity-gqa] {case.name} ({algo}): H={case.heads} H_kv={case.heads_kv} d={case.head_dim} "
          f"mask={case.mask}", flush=True)
    o, m, l = P.oracle_stats(inp)
    gpu = P.run_gpu(inp, o, m, l, algorithm=ALGOS[algo])
    ref = P.oracle_backward(inp, o, m, l)
    res = P.check_full(inp, gpu, ref)
    print(f"[parity-gqa] {case.name} ({algo}): " + " ".join(f"{k}: rel_l2={v[0]:.2e}" for k, v in res.items()),
          flush=True)


def test_grouped_heads_single_pass_unsupported():
    inp = I.make(GQA_CASES[0])
    o, m, l = P.oracle_stats(inp)
    with pytest.raises(NotImplementedError):
        P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_SINGLE_PASS)


# sliding window: each query i sees keys (i - w, i] only (recompute form)
WINDOW_CASES = [
    I.custom_case("window_causal_d128", 2, 128, CAUSAL, 231, [300, 129], window=64),
    I.custom_case("window_none_d64", 2, 64, NONE, 232, [257], window=40),
    I.custom_case("window_one_d128", 2, 128, CAUSAL, 233, [130], window=1),
    I.custom_case("window_wide_padded_d128", 2, 128, PADC, 234, [200, 90], padded_len=224, window=300),
    I.custom_case("window_gqa_causal_d128", 4, 128, CAUSAL, 235, [333], heads_kv=2, window=128),
    # windows far past every sequence (up to the int32 maximum): the causal bound alone
    I.custom_case("window_huge_none_d128", 2, 128, NONE, 236, [300, 129], window=2**31 - 1),
    I.custom_case("window_huge_padded_d64", 2, 64, PAD, 237, [200, 77], padded_len=256, window=2**30 + 5),
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=[c.name for c in WINDOW_CASES])
def test_parity_window(case):
    inp = I.make(case)
    print(f"[parity-window] {case.name}: window={case.window} mask={case.mask}", flush=True)
    o, m, l = P.oracle_stats(inp)
    gpu = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_DEFAULT)
    ref = P.oracle_backward(inp, o, m, l)
    res = P.check_full(inp, gpu, ref)
    print(f"[parity-window] {case.name}: " + " ".join(f"{k}: rel_l2={v[0]:.2e}" for k, v in res.items()),
          flush=True)


# the 64-key layout and the stored-dS form with a window: band edges inside and at the end of 256-key
# blocks, windows of 1 and wider than a block, grouped heads, padding
WINDOW_64K_CASES = [c for c in WINDOW_CASES if c.head_dim == 128] + [
    I.custom_case("window_edge_d128", 2, 128, CAUSAL, 238, [700, 450], window=130),
    I.custom_case("window_short_d128", 2, 128, CAUSAL, 239, [1100], window=40),
    I.custom_case("window_block_d128", 2, 128, PADC, 240, [600, 520], padded_len=640, window=256),
]


@pytest.mark.parametrize("case,algo", [(c, a) for c in WINDOW_64K_CASES for a in ("recompute64k", "storedds")],
                         ids=lambda x: x if isinstance(x, str) else x.name)
def test_parity_window_64k(case, algo):
    inp = I.make(case)
    print(f"[parity-window-64k] {case.name} {algo}: window={case.window} mask={case.mask}", flush=True)
    o, m, l = P.oracle_stats(inp)
    gpu = P.run_gpu(inp, o, m, l, algorithm=ALGOS[algo])
    ref = P.oracle_backward(inp, o, m, l)
    P.check_full(inp, gpu, ref)


def test_huge_window_is_the_causal_bound():
    """A window past every sequence gives the causal result, from the dense grid and from a host schedule."""
    case = next(c for c in WINDOW_CASES if c.name == "window_huge_none_d128")
    inp = I.make(case)
    o, m, l = P.oracle_stats(inp)
    huge = P.run_gpu(inp, o, m, l)
    causal = dict(inp, mask=CAUSAL, window=0)
    ref = P.oracle_backward(causal, o, m, l)
    P.check_full(causal, huge, ref)
    dev = torch.device("cuda")
    t = {k: inp[k].to(dev) for k in ("q", "k", "v", "do", "cu_q", "cu_kv")}
    with B.FaBwd(inp["batch"], case.heads, case.head_dim, inp["max_seqlen_q"], inp["max_seqlen_kv"],
                 inp["q"].shape[0], inp["k"].shape[0], window=inp["window"]) as op:
        op.plan(inp["cu_q"], inp["cu_kv"], inp["mask"])
        planned = op.run(t["q"], t["k"], t["v"], o.to(dev), t["do"], m.to(dev), l.to(dev), t["cu_q"], t["cu_kv"],
                         inp["scale"], inp["mask"])
        torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv"), huge, planned):
        assert torch.equal(x, y.float().cpu()), f"{name}: planned run differs from the dense grid"


def test_window_single_pass_unsupported():
    inp = I.make(WINDOW_CASES[0])
    o, m, l = P.oracle_stats(inp)
    with pytest.raises(NotImplementedError):
        P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_SINGLE_PASS)
