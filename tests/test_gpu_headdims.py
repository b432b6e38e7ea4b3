"""GPU parity of the recompute backward, of the stored-dS form where it applies (a head dim above 128,
no window) and of the forward over head dims other than 64 and 128:
any multiple of 8 up to 256, and a value head dim (V, O, dO, dV) that differs from the query/key
one (latent attention). Every valid row is compared with the fp64 oracle on the same seeded inputs,
with the tolerance of the other parity tests; rows outside every sequence must be exactly zero.

The kernels run on head dims padded to 64, 128, 192 or 256 with zero columns, so the cases cover each
pair of padded dims the library instantiates, with head dims both equal to and below the padded
one, ragged lengths, every mask type, grouped K/V heads and a window.
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

NONE, PAD, CAUSAL, PADC = I.MASK_NONE, I.MASK_PADDING, I.MASK_CAUSAL, I.MASK_PADDING_CAUSAL

CASES = [
    # padded (64, 64)
    I.custom_case("d8_none", 2, 8, NONE, 301, [70, 129]),
    I.custom_case("d40_causal", 3, 40, CAUSAL, 302, [200, 65]),
    # padded (128, 128)
    I.custom_case("d96_causal", 2, 96, CAUSAL, 303, [257, 100]),
    I.custom_case("d112_padded_causal", 2, 112, PADC, 304, [150, 77], padded_len=160),
    # padded (64, 128) and (128, 64): latent attention with small heads
    I.custom_case("mla_64_128_causal", 2, 64, CAUSAL, 305, [190, 64], head_dim_v=128),
    I.custom_case("mla_128_64_none", 2, 128, NONE, 306, [131, 200], head_dim_v=64),
    I.custom_case("mla_72_48_causal", 2, 72, CAUSAL, 307, [99, 140], head_dim_v=48),
    # padded (256, 256)
    I.custom_case("d256_causal", 2, 256, CAUSAL, 308, [300, 129]),
    I.custom_case("d256_none_kv_longer", 2, 256, NONE, 309, [100, 64], [170, 200]),
    I.custom_case("d232_causal", 2, 232, CAUSAL, 319, [150, 75]),
    # padded (192, 192)
    I.custom_case("d160_padded", 2, 160, PAD, 310, [200, 90], padded_len=224),
    I.custom_case("d192_causal", 2, 192, CAUSAL, 311, [257, 31]),
    # padded (192, 128), (128, 192), (256, 192), (192, 256)
    I.custom_case("mla_192_128_causal", 4, 192, CAUSAL, 312, [260, 111], head_dim_v=128),
    I.custom_case("mla_128_176_none", 2, 128, NONE, 320, [99, 180], head_dim_v=176),
    I.custom_case("mla_256_160_causal", 2, 256, CAUSAL, 321, [201], head_dim_v=160),
    I.custom_case("mla_184_256_padded", 2, 184, PAD, 322, [120, 64], padded_len=128, head_dim_v=256),
    # padded (256, 128) and (128, 256)
    I.custom_case("mla_256_64_none", 2, 256, NONE, 313, [140], head_dim_v=64),
    I.custom_case("mla_128_256_causal", 2, 128, CAUSAL, 314, [222, 70], head_dim_v=256),
    I.custom_case("mla_48_200_padded_causal", 2, 48, PADC, 315, [130, 60], padded_len=144, head_dim_v=200),
    # with grouped K/V heads and a window
    I.custom_case("d256_gqa_causal", 4, 256, CAUSAL, 316, [190], heads_kv=2),
    I.custom_case("mla_192_128_gqa_window", 4, 192, CAUSAL, 317, [300], heads_kv=1, window=70, head_dim_v=128),
    I.custom_case("d96_window", 2, 96, NONE, 318, [211], window=50),
]


def _wide_stored_ds(case):
    """The stored-dS form runs on the wide-head kernels: a head dim above 128 and no window."""
    return max(case.head_dim, case.head_dim_v or case.head_dim) > 128 and case.window == 0


@pytest.mark.parametrize("algo", [B.FA_BWD_ALGO_RECOMPUTE_DQ_8W, B.FA_BWD_ALGO_RECOMPUTE_DQ_4W,
                                  B.FA_BWD_ALGO_STORED_DS], ids=["8w", "4w", "storedds"])
@pytest.mark.parametrize("case", CASES, ids=[c.name for c in CASES])
def test_parity_head_dims(case, algo):
    if algo == B.FA_BWD_ALGO_STORED_DS and not _wide_stored_ds(case):
        pytest.skip("the stored-dS form at these head dims needs one above 128 and no window")
    inp = I.make(case)
    dv = case.head_dim_v or case.head_dim
    print(f"[headdim] {case.name}: d={case.head_dim} d_v={dv} H={case.heads} H_kv={inp['k'].shape[1]} "
          f"mask={case.mask} window={case.window}", flush=True)
    o, m, l = P.oracle_stats(inp)
    if I.is_padded_mask(case.mask):  # the backward must not read padding rows
        vq = torch.from_numpy(oracle.valid_rows(inp["cu_q"], case.mask, inp["max_seqlen_q"], inp["q"].shape[0]))
        for t in (o, m, l, inp["do"], inp["q"]):
            t[~vq] = float("nan")
        vk = torch.from_numpy(oracle.valid_rows(inp["cu_kv"], case.mask, inp["max_seqlen_kv"], inp["k"].shape[0]))
        inp["k"][~vk] = float("nan")
        inp["v"][~vk] = float("nan")
    gpu = P.run_gpu(inp, o, m, l, algorithm=algo)
    assert gpu[0].shape[2] == case.head_dim and gpu[2].shape[2] == dv
    ref = P.oracle_backward(inp, o, m, l)
    res = P.check_full(inp, gpu, ref)
    print(f"[headdim] {case.name}: " + " ".join(f"{k}: rel_l2={v[0]:.2e} max={v[1]:.2e}" for k, v in res.items()),
          flush=True)


@pytest.mark.parametrize("case", CASES, ids=[c.name for c in CASES])
def test_forward_head_dims(case):
    inp = I.make(case)
    print(f"[headdim-forward] {case.name}", flush=True)
    o, m, l = gpu_forward(inp)
    ro, rm, rl = oracle.forward(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_kv"], inp["scale"], inp["mask"],
                                inp["max_seqlen_q"], inp["max_seqlen_kv"], inp["window"])
    valid = oracle.valid_rows(inp["cu_q"], inp["mask"], inp["max_seqlen_q"], inp["q"].shape[0])
    assert o.shape[2] == (case.head_dim_v or case.head_dim)
    assert np.all(o[~valid] == 0) and np.all(m[~valid] == 0) and np.all(l[~valid] == 1)
    dm, dlse = check_forward(inp, (o[valid], m[valid], l[valid]), (ro[valid], rm[valid], rl[valid]))
    print(f"[headdim-forward] {case.name}: m err {dm:.2e} lse err {dlse:.2e}", flush=True)


@pytest.mark.parametrize("name", ["mla_192_128_causal", "d256_gqa_causal", "mla_184_256_padded", "d232_causal",
                                  "mla_128_176_none"])
def test_wide_stored_ds_matches_recompute(name):
    """The wide-head stored-dS form runs the recompute form's dK/dV kernel with the dS pieces stored: its dK,
    dV equal the recompute form's bitwise; its dQ sums the same bf16 dS values in another kernel, so it
    agrees within the tolerance. Repeated runs are bitwise identical."""
    inp = I.make(next(c for c in CASES if c.name == name))
    o, m, l = P.oracle_stats(inp)
    a = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_RECOMPUTE_DQ)
    b = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_STORED_DS)
    c = P.run_gpu(inp, o, m, l, algorithm=B.FA_BWD_ALGO_STORED_DS)
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2]), "dk, dv differ from the recompute form"
    P.assert_close("dq", b[0].numpy(), a[0].numpy().astype(np.float64))
    for x, y in zip(b, c):
        assert torch.equal(x, y)


def test_wide_head_dims_bitwise_reproducible():
    """The wide kernels swap P and dS through LDS and use no atomics: repeated runs agree bitwise."""
    inp = I.make(next(c for c in CASES if c.name == "mla_192_128_causal"))
    o, m, l = P.oracle_stats(inp)
    a = P.run_gpu(inp, o, m, l)
    b = P.run_gpu(inp, o, m, l)
    for x, y in zip(a, b):
        assert torch.equal(x, y)

