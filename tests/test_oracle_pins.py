"""Pins of the fp64 oracle against facts it does not derive from itself.

Every check here runs on the CPU. The backward's definition is the eight
per-tile steps of the PyPTO-Gym SK-16 article, §3.1; the mask codes are jax's
cuDNN ``MaskType``. The pins:

* a hand-derived closed form (two keys, rational softmax weights);
* central finite differences of sum(O * dO) w.r.t. Q, K, V on tiny shapes,
  every mask type, packed varlen and padded layouts;
* invariants: dS rows sum to 0 (so dK columns sum to 0), dV columns sum to dO
  columns, rowsum(O*dO) = rowsum(P*dP), causal zero patterns;
* closed forms: one key, all-equal V rows, Q = 0;
* torch fp64 autograd of softmax(scale*QK^T + mask) V, an independent library (with grouped
  K/V heads expanded by torch's repeat_interleave, so autograd sums the shared heads' gradients),
  also with a value head dim that differs from the query/key one;
* the forward on its own: O, the row max of the scaled logits and m + ln(l) against torch's
  softmax attention, max and logsumexp; the sampled-row forward against the full one;
* planted mistakes in the oracle's own source, each caught by one of the above.
"""
import inspect
import math
import textwrap

import numpy as np
import pytest
import torch

import oracle.attention as A
from oracle.attention import MASK_CAUSAL, MASK_NONE, MASK_PADDING, MASK_PADDING_CAUSAL


# ---------------------------------------------------------------- helpers

def _rand(shape, rng, mult=1.0):
    return rng.standard_normal(shape) * mult


def make_problem(mask, lens_q, lens_kv, heads=2, d=4, seed=0, padded_len=0, mult=1.0, heads_kv=None, window=0,
                 d_v=None):
    rng = np.random.default_rng(seed)
    if A.is_padded(mask):
        tq = tkv = len(lens_q) * padded_len
        msq = mskv = padded_len
    else:
        tq, tkv = sum(lens_q), sum(lens_kv)
        msq, mskv = max(lens_q), max(lens_kv)
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int64)
    cu_kv = np.concatenate([[0], np.cumsum(lens_kv)]).astype(np.int64)
    hkv = heads if heads_kv is None else heads_kv
    dv = d if d_v is None else d_v
    return dict(q=_rand((tq, heads, d), rng, mult), k=_rand((tkv, hkv, d), rng, mult),
                v=_rand((tkv, hkv, dv), rng), do=_rand((tq, heads, dv), rng),
                cu_q=cu_q, cu_kv=cu_kv, scale=1.0 / math.sqrt(d), mask=mask,
                max_seqlen_q=msq, max_seqlen_kv=mskv, window=window)


def exact_backward(p):
    """Backward fed with the unrounded fp64 forward (exact mode)."""
    o, m, l = A.forward(p["q"], p["k"], p["v"], p["cu_q"], p["cu_kv"], p["scale"], p["mask"],
                        p["max_seqlen_q"], p["max_seqlen_kv"], p.get("window", 0))
    dq, dk, dv = A.backward(p["q"], p["k"], p["v"], o, p["do"], m, l, p["cu_q"], p["cu_kv"],
                            p["scale"], p["mask"], p["max_seqlen_q"], p["max_seqlen_kv"], p.get("window", 0))
    return o, m, l, dq, dk, dv


def fd_grads(p, eps=1e-6):
    """Central differences of loss = sum(O * dO) for every element of Q, K, V."""
    out = {}
    for name in ("q", "k", "v"):
        x = p[name]
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = A.loss(p["q"], p["k"], p["v"], p["do"], p["cu_q"], p["cu_kv"], p["scale"], p["mask"],
                        p["max_seqlen_q"], p["max_seqlen_kv"], p.get("window", 0))
            x[idx] = keep - eps
            lm = A.loss(p["q"], p["k"], p["v"], p["do"], p["cu_q"], p["cu_kv"], p["scale"], p["mask"],
                        p["max_seqlen_q"], p["max_seqlen_kv"], p.get("window", 0))
            x[idx] = keep
            g[idx] = (lp - lm) / (2 * eps)
        out[name] = g
    return out


def fd_error(p):
    _, _, _, dq, dk, dv = exact_backward(p)
    fd = fd_grads(p)
    err = 0.0   # worst over Q, K, V of max|fd - analytic| / max|analytic|
    for name, an in (("q", dq), ("k", dk), ("v", dv)):
        if an.size:
            err = max(err, float(np.max(np.abs(fd[name] - an))) / max(float(np.max(np.abs(an))), 1e-30))
    return err


def torch_reference(p):
    """Independent gradients: torch fp64 autograd of softmax(scale*QK^T + bias) V per (b, h)."""
    q = torch.tensor(p["q"], requires_grad=True)
    k = torch.tensor(p["k"], requires_grad=True)
    v = torch.tensor(p["v"], requires_grad=True)
    do = torch.tensor(p["do"])
    nb = len(p["cu_q"]) - 1
    padded = p["mask"] in (MASK_PADDING, MASK_PADDING_CAUSAL)
    causal = p["mask"] in (MASK_CAUSAL, MASK_PADDING_CAUSAL)
    group = q.shape[1] // k.shape[1]
    ke, ve = k.repeat_interleave(group, dim=1), v.repeat_interleave(group, dim=1)  # shared K/V heads
    total = torch.zeros((), dtype=torch.float64)
    for b in range(nb):
        lq = int(p["cu_q"][b + 1] - p["cu_q"][b])
        lk = int(p["cu_kv"][b + 1] - p["cu_kv"][b])
        qs = b * p["max_seqlen_q"] if padded else int(p["cu_q"][b])
        ks = b * p["max_seqlen_kv"] if padded else int(p["cu_kv"][b])
        if lq == 0 or lk == 0:
            continue
        for h in range(q.shape[1]):
            qh, kh, vh = q[qs:qs + lq, h], ke[ks:ks + lk, h], ve[ks:ks + lk, h]
            logits = p["scale"] * qh @ kh.T
            if causal or p.get("window", 0):
                bias = torch.triu(torch.full((lq, lk), float("-inf"), dtype=torch.float64), diagonal=1)
                logits = logits + bias
            if p.get("window", 0):   # keys at or before i - window are outside the left local window
                logits = logits + torch.tril(torch.full((lq, lk), float("-inf"), dtype=torch.float64),
                                             diagonal=-p.get("window", 0))
            out = torch.softmax(logits, dim=-1) @ vh
            total = total + (out * do[qs:qs + lq, h]).sum()
    total.backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def torch_error(p):
    _, _, _, dq, dk, dv = exact_backward(p)
    tq, tk, tv = torch_reference(p)
    return max(float(np.max(np.abs(a - b))) / max(1.0, float(np.max(np.abs(b))))
               for a, b in ((dq, tq), (dk, tk), (dv, tv)))


FD_CASES = [
    # (mask, lens_q, lens_kv, d, padded_len)
    (MASK_NONE, [1], [1], 4, 0),
    (MASK_NONE, [3], [5], 4, 0),
    (MASK_NONE, [8], [2], 8, 0),
    (MASK_NONE, [3, 5], [2, 4], 4, 0),            # two packed sequences
    (MASK_CAUSAL, [5], [5], 4, 0),
    (MASK_CAUSAL, [8], [8], 8, 0),
    (MASK_CAUSAL, [2, 5], [3, 5], 4, 0),          # packed, Lq != Lk in the first sequence
    (MASK_PADDING, [5, 3], [5, 2], 4, 5),
    (MASK_PADDING_CAUSAL, [5, 3], [5, 3], 4, 5),
    (MASK_PADDING_CAUSAL, [2, 1], [3, 2], 4, 3),
]


# ---------------------------------------------------------------- closed form from a hand derivation

LN3 = math.log(3.0)


def _two_key(mask, cu_q):
    # scale 0.5, q = 1, keys (0, 2 ln 3) -> scaled logits (0, ln 3): P = (1/4, 3/4) when both keys are seen
    nq = cu_q[-1]
    return dict(q=np.ones((nq, 1, 1)), k=np.array([[[0.0]], [[2 * LN3]]]), v=np.array([[[1.0]], [[5.0]]]),
                do=np.full((nq, 1, 1), 2.0), cu_q=np.array(cu_q), cu_kv=np.array([0, 2]), scale=0.5,
                mask=mask, max_seqlen_q=nq, max_seqlen_kv=2)


def test_closed_form_two_keys_causal():
    # row 0 sees key 0 only: P=(1,0), O=1, D=2, dP=(2,10), dS=(0,0)
    # row 1 sees both: m=ln3, l=4/3, P=(1/4,3/4), O=4, D=8, dS=(-3/2, 3/2)
    p = _two_key(MASK_CAUSAL, [0, 2])
    o, m, l, dq, dk, dv = exact_backward(p)
    np.testing.assert_allclose(o[:, 0, 0], [1.0, 4.0], rtol=1e-15)
    np.testing.assert_allclose(m[:, 0], [0.0, LN3], rtol=1e-15)
    np.testing.assert_allclose(l[:, 0], [1.0, 4.0 / 3.0], rtol=1e-15)
    np.testing.assert_allclose(dq[:, 0, 0], [0.0, 1.5 * LN3], rtol=1e-14, atol=1e-15)   # 0.5 * 3/2 * 2 ln 3
    np.testing.assert_allclose(dk[:, 0, 0], [-0.75, 0.75], rtol=1e-14)                # 0.5 * (-3/2, 3/2)
    np.testing.assert_allclose(dv[:, 0, 0], [2.5, 1.5], rtol=1e-14)                   # (1*2 + 2/4, 3/4*2)


def test_closed_form_two_keys_one_query():
    p = _two_key(MASK_NONE, [0, 1])
    o, m, l, dq, dk, dv = exact_backward(p)
    np.testing.assert_allclose([o[0, 0, 0], m[0, 0], l[0, 0]], [4.0, LN3, 4.0 / 3.0], rtol=1e-15)
    np.testing.assert_allclose(dq[0, 0, 0], 1.5 * LN3, rtol=1e-14)
    np.testing.assert_allclose(dk[:, 0, 0], [-0.75, 0.75], rtol=1e-14)
    np.testing.assert_allclose(dv[:, 0, 0], [0.5, 1.5], rtol=1e-14)


# ---------------------------------------------------------------- finite differences

@pytest.mark.parametrize("mask,lq,lk,d,padded", FD_CASES)
def test_finite_differences(mask, lq, lk, d, padded):
    p = make_problem(mask, lq, lk, heads=2, d=d, seed=len(lq) * 7 + sum(lq) + mask, padded_len=padded)
    assert fd_error(p) < 2e-6


def test_padding_rows_get_zero_and_are_not_read():
    p = make_problem(MASK_PADDING_CAUSAL, [5, 3], [5, 2], heads=2, d=4, seed=3, padded_len=5)
    o, m, l, dq, dk, dv = exact_backward(p)
    vq = A.valid_rows(p["cu_q"], p["mask"], 5, 10)
    vk = A.valid_rows(p["cu_kv"], p["mask"], 5, 10)
    assert vq.tolist() == [True] * 5 + [True] * 3 + [False] * 2
    assert vk.tolist() == [True] * 5 + [True] * 2 + [False] * 3
    assert np.all(dq[~vq] == 0) and np.all(dk[~vk] == 0) and np.all(dv[~vk] == 0)
    # garbage (NaN) in the padding rows of every input leaves the valid outputs unchanged
    q2, k2, v2, o2, do2 = (x.copy() for x in (p["q"], p["k"], p["v"], o, p["do"]))
    m2, l2 = m.copy(), l.copy()
    for x, ok in ((q2, vq), (o2, vq), (do2, vq), (m2, vq), (l2, vq), (k2, vk), (v2, vk)):
        x[~ok] = np.nan
    dq2, dk2, dv2 = A.backward(q2, k2, v2, o2, do2, m2, l2, p["cu_q"], p["cu_kv"], p["scale"], p["mask"], 5, 5)
    assert np.array_equal(dq2[vq], dq[vq]) and np.array_equal(dk2[vk], dk[vk]) and np.array_equal(dv2[vk], dv[vk])


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("mask", [MASK_NONE, MASK_CAUSAL])
def test_ds_rows_sum_to_zero_and_dk_columns_vanish(mask):
    rng = np.random.default_rng(11)
    q, k, v, do = (rng.standard_normal((40, 16)) for _ in range(4))
    scale = 0.25
    o, m, l = A.forward_head(q, k, v, scale, mask == MASK_CAUSAL)
    r = A.backward_head(q, k, v, o, do, m, l, scale, mask == MASK_CAUSAL)
    assert np.max(np.abs(r["ds"].sum(axis=1))) < 1e-13
    assert np.max(np.abs(r["dk"].sum(axis=0))) < 1e-12


@pytest.mark.parametrize("mask", [MASK_NONE, MASK_CAUSAL])
def test_dv_column_sums_equal_do_column_sums(mask):
    rng = np.random.default_rng(12)
    q, k, v, do = (rng.standard_normal((33, 8)) for _ in range(4))
    o, m, l = A.forward_head(q, k, v, 0.3, mask == MASK_CAUSAL)
    r = A.backward_head(q, k, v, o, do, m, l, 0.3, mask == MASK_CAUSAL)
    np.testing.assert_allclose(r["dv"].sum(axis=0), do.sum(axis=0), atol=1e-13)


def test_d_identity_rowsum_o_do_equals_rowsum_p_dp():
    # ties the article's D = rowsum(O*dO) (step 4) to the softmax-backward form rowsum(P*dP)
    # used by the PyPTO block-attention-residual backward for its grad_logits
    rng = np.random.default_rng(13)
    q, k, v, do = (rng.standard_normal((25, 8)) for _ in range(4))
    for causal in (False, True):
        o, m, l = A.forward_head(q, k, v, 0.5, causal)
        r = A.backward_head(q, k, v, o, do, m, l, 0.5, causal)
        np.testing.assert_allclose(r["dvec"], np.sum(r["p"] * r["dp"], axis=1), atol=1e-13)


def test_causal_zero_patterns():
    rng = np.random.default_rng(14)
    n, d, scale = 12, 8, 0.35
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    o, m, l = A.forward_head(q, k, v, scale, True)
    r = A.backward_head(q, k, v, o, do, m, l, scale, True)
    assert np.all(np.triu(r["p"], 1) == 0)
    assert np.max(np.abs(r["dq"][0])) < 1e-14                 # row 0 sees key 0 only: P00 = 1, dS00 = 0
    last = n - 1                                              # key n-1 is seen by row n-1 only
    np.testing.assert_allclose(r["dv"][last], r["p"][last, last] * do[last], rtol=1e-14)
    np.testing.assert_allclose(r["dk"][last], scale * r["ds"][last, last] * q[last], rtol=1e-12, atol=1e-15)
    # keys/values after row i do not reach rows 0..i
    i = 5
    k2, v2 = k.copy(), v.copy()
    k2[i + 1:] = rng.standard_normal(k2[i + 1:].shape) * 3
    v2[i + 1:] = rng.standard_normal(v2[i + 1:].shape) * 3
    o2, m2, l2 = A.forward_head(q, k2, v2, scale, True)
    r2 = A.backward_head(q, k2, v2, o2, do, m2, l2, scale, True)
    assert np.array_equal(o2[:i + 1], o[:i + 1]) and np.array_equal(m2[:i + 1], m[:i + 1])
    assert np.array_equal(r2["dq"][:i + 1], r["dq"][:i + 1])


# ---------------------------------------------------------------- closed forms

def test_single_key():
    rng = np.random.default_rng(15)
    q, do = rng.standard_normal((7, 4)), rng.standard_normal((7, 4))
    k, v = rng.standard_normal((1, 4)), rng.standard_normal((1, 4))
    o, m, l = A.forward_head(q, k, v, 0.5, False)
    r = A.backward_head(q, k, v, o, do, m, l, 0.5, False)
    np.testing.assert_allclose(r["p"], 1.0, rtol=1e-15)
    assert np.max(np.abs(r["dq"])) < 1e-14 and np.max(np.abs(r["dk"])) < 1e-13
    np.testing.assert_allclose(r["dv"][0], do.sum(axis=0), rtol=1e-13)


def test_equal_value_rows_give_zero_dq_dk():
    rng = np.random.default_rng(16)
    q, k, do = (rng.standard_normal((9, 4)) for _ in range(3))
    v = np.tile(rng.standard_normal((1, 4)), (9, 1))
    for causal in (False, True):
        o, m, l = A.forward_head(q, k, v, 0.5, causal)
        r = A.backward_head(q, k, v, o, do, m, l, 0.5, causal)
        assert np.max(np.abs(r["dq"])) < 1e-13 and np.max(np.abs(r["dk"])) < 1e-13


def test_zero_queries_give_uniform_softmax():
    rng = np.random.default_rng(17)
    lq, lk = 6, 5
    q = np.zeros((lq, 4))
    k, v = rng.standard_normal((lk, 4)), rng.standard_normal((lk, 4))
    do = rng.standard_normal((lq, 4))
    o, m, l = A.forward_head(q, k, v, 0.5, False)
    r = A.backward_head(q, k, v, o, do, m, l, 0.5, False)
    np.testing.assert_allclose(r["p"], 1.0 / lk, rtol=1e-15)
    np.testing.assert_allclose(r["dv"], np.tile(do.sum(axis=0) / lk, (lk, 1)), rtol=1e-13)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (lq, 1)), rtol=1e-13)


# ---------------------------------------------------------------- independent library

@pytest.mark.parametrize("mask,lq,lk,d,padded", FD_CASES + [
    (MASK_NONE, [64, 37], [64, 37], 32, 0),
    (MASK_CAUSAL, [96], [96], 64, 0),
    (MASK_PADDING_CAUSAL, [80, 50], [80, 50], 16, 80),
])
def test_torch_fp64_autograd(mask, lq, lk, d, padded):
    p = make_problem(mask, lq, lk, heads=2, d=d, seed=99 + sum(lq), padded_len=padded, mult=2.0)
    assert torch_error(p) < 1e-12


# ---------------------------------------------------------------- the forward on its own

def torch_forward(p):
    """Independent forward: torch fp64 softmax attention per (b, h); O, row max of the scaled
    logits and their logsumexp (rows outside every sequence: O = 0, m = 0, lse = 0)."""
    q, k, v = (torch.tensor(p[x]) for x in ("q", "k", "v"))
    padded = p["mask"] in (MASK_PADDING, MASK_PADDING_CAUSAL)
    causal = p["mask"] in (MASK_CAUSAL, MASK_PADDING_CAUSAL)
    o = torch.zeros_like(q)
    m = torch.zeros(q.shape[:2], dtype=torch.float64)
    lse = torch.zeros(q.shape[:2], dtype=torch.float64)
    for b in range(len(p["cu_q"]) - 1):
        lq = int(p["cu_q"][b + 1] - p["cu_q"][b])
        lk = int(p["cu_kv"][b + 1] - p["cu_kv"][b])
        qs = b * p["max_seqlen_q"] if padded else int(p["cu_q"][b])
        ks = b * p["max_seqlen_kv"] if padded else int(p["cu_kv"][b])
        if lq == 0 or lk == 0:
            continue
        for h in range(q.shape[1]):
            logits = p["scale"] * q[qs:qs + lq, h] @ k[ks:ks + lk, h].T
            if causal:
                logits = logits + torch.triu(torch.full((lq, lk), float("-inf"), dtype=torch.float64), diagonal=1)
            o[qs:qs + lq, h] = torch.softmax(logits, dim=-1) @ v[ks:ks + lk, h]
            m[qs:qs + lq, h] = logits.max(dim=-1).values
            lse[qs:qs + lq, h] = torch.logsumexp(logits, dim=-1)
    return o.numpy(), m.numpy(), lse.numpy()


@pytest.mark.parametrize("mask,lq,lk,d,padded", FD_CASES + [
    (MASK_NONE, [64, 37], [64, 37], 32, 0),
    (MASK_CAUSAL, [96], [96], 64, 0),
    (MASK_PADDING_CAUSAL, [80, 50], [80, 50], 16, 80),
])
def test_forward_matches_torch(mask, lq, lk, d, padded):
    p = make_problem(mask, lq, lk, heads=2, d=d, seed=7 + sum(lq), padded_len=padded, mult=2.0)
    o, m, l = A.forward(p["q"], p["k"], p["v"], p["cu_q"], p["cu_kv"], p["scale"], p["mask"],
                        p["max_seqlen_q"], p["max_seqlen_kv"])
    to, tm, tlse = torch_forward(p)
    np.testing.assert_allclose(o, to, rtol=1e-12, atol=1e-13)
    valid = A.valid_rows(p["cu_q"], mask, p["max_seqlen_q"], p["q"].shape[0])
    np.testing.assert_allclose(m[valid], tm[valid], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose((m + np.log(l))[valid], tlse[valid], rtol=1e-12, atol=1e-12)
    assert np.all(o[~valid] == 0) and np.all(m[~valid] == 0) and np.all(l[~valid] == 1)


@pytest.mark.parametrize("mask", [MASK_NONE, MASK_CAUSAL, MASK_PADDING_CAUSAL])
def test_forward_rows_matches_forward(mask):
    padded = 40 if A.is_padded(mask) else 0
    p = make_problem(mask, [40, 23], [40, 23], heads=3, d=16, seed=6, padded_len=padded)
    o, m, l = A.forward(p["q"], p["k"], p["v"], p["cu_q"], p["cu_kv"], p["scale"], mask,
                        p["max_seqlen_q"], p["max_seqlen_kv"])
    for b, (qs, lq) in enumerate(A.segments(p["cu_q"], mask, p["max_seqlen_q"])):
        rows = [0, 1, lq // 2, lq - 1]
        ro, rm, rl = A.forward_rows(p["q"], p["k"], p["v"], p["cu_q"], p["cu_kv"], p["scale"], mask, b, 1, rows,
                                    p["max_seqlen_q"], p["max_seqlen_kv"])
        np.testing.assert_allclose(ro, o[[qs + r for r in rows], 1], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(rm, m[[qs + r for r in rows], 1], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(rl, l[[qs + r for r in rows], 1], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("mask", [MASK_NONE, MASK_CAUSAL, MASK_PADDING_CAUSAL])
def test_backward_from_lse_equals_backward_from_m_l(mask):
    """exp(s - m) / l = exp(s - (m + ln l)): the two statistic forms give the same gradients."""
    padded = 12 if A.is_padded(mask) else 0
    p = make_problem(mask, [12, 7], [12, 7], heads=2, d=8, seed=8, padded_len=padded, mult=2.0)
    o, m, l, dq, dk, dv = exact_backward(p)
    lq, lk, lv = A.backward_from_lse(p["q"], p["k"], p["v"], o, p["do"], m + np.log(l), p["cu_q"], p["cu_kv"],
                                     p["scale"], mask, p["max_seqlen_q"], p["max_seqlen_kv"])
    for a, b in ((lq, dq), (lk, dk), (lv, dv)):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- grouped K/V heads

GQA_CASES = [
    # (mask, lens_q, lens_kv, d, padded_len, heads, heads_kv)
    (MASK_NONE, [4], [5], 4, 0, 4, 2),
    (MASK_CAUSAL, [5, 3], [5, 3], 4, 0, 4, 1),
    (MASK_PADDING_CAUSAL, [4, 2], [4, 3], 4, 4, 6, 3),
]


@pytest.mark.parametrize("mask,lq,lk,d,padded,heads,heads_kv", GQA_CASES)
def test_grouped_heads_finite_differences(mask, lq, lk, d, padded, heads, heads_kv):
    p = make_problem(mask, lq, lk, heads=heads, d=d, seed=31 + heads_kv, padded_len=padded, heads_kv=heads_kv)
    assert fd_error(p) < 2e-6


@pytest.mark.parametrize("mask,lq,lk,d,padded,heads,heads_kv", GQA_CASES + [
    (MASK_CAUSAL, [64, 37], [64, 37], 16, 0, 8, 2),
])
def test_grouped_heads_torch_fp64_autograd(mask, lq, lk, d, padded, heads, heads_kv):
    p = make_problem(mask, lq, lk, heads=heads, d=d, seed=41 + heads_kv, padded_len=padded, mult=2.0,
                     heads_kv=heads_kv)
    assert torch_error(p) < 1e-12


def test_grouped_heads_backward_rows_matches_full():
    p = make_problem(MASK_CAUSAL, [30, 17], [30, 17], heads=4, d=8, seed=12, heads_kv=2)
    o, m, l, dq, dk, dv = exact_backward(p)
    for b, ((qs, lq), (ks, lk)) in enumerate(zip(A.segments(p["cu_q"], MASK_CAUSAL, 0),
                                                 A.segments(p["cu_kv"], MASK_CAUSAL, 0))):
        rows = [0, lq // 2, lq - 1]
        for h in range(4):
            sq, sk, sv = A.backward_rows(p["q"], p["k"], p["v"], o, p["do"], m, l, p["cu_q"], p["cu_kv"],
                                         p["scale"], MASK_CAUSAL, b, h, rows, rows)
            np.testing.assert_allclose(sq, dq[[qs + r for r in rows], h], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(sk, dk[[ks + r for r in rows], h // 2], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(sv, dv[[ks + r for r in rows], h // 2], rtol=1e-12, atol=1e-14)


def test_grouped_heads_reject_non_divisor():
    p = make_problem(MASK_NONE, [3], [3], heads=3, d=4, heads_kv=2)
    with pytest.raises(ValueError):
        A.forward(p["q"], p["k"], p["v"], p["cu_q"], p["cu_kv"], p["scale"], MASK_NONE)


# ---------------------------------------------------------------- sliding window

WINDOW_CASES = [
    # (mask, lens_q, lens_kv, d, padded_len, window)
    (MASK_CAUSAL, [8], [8], 4, 0, 3),
    (MASK_CAUSAL, [6, 5], [6, 5], 4, 0, 2),            # two packed sequences
    (MASK_NONE, [7], [7], 4, 0, 2),                    # the window implies the causal bound
    (MASK_PADDING_CAUSAL, [6, 4], [6, 4], 4, 6, 4),
]


@pytest.mark.parametrize("mask,lq,lk,d,padded,window", WINDOW_CASES)
def test_window_finite_differences(mask, lq, lk, d, padded, window):
    p = make_problem(mask, lq, lk, heads=2, d=d, seed=61 + window, padded_len=padded, window=window)
    assert fd_error(p) < 2e-6


@pytest.mark.parametrize("mask,lq,lk,d,padded,window", WINDOW_CASES + [(MASK_CAUSAL, [96, 40], [96, 40], 16, 0, 33)])
def test_window_torch_fp64_autograd(mask, lq, lk, d, padded, window):
    p = make_problem(mask, lq, lk, heads=2, d=d, seed=71 + window, padded_len=padded, mult=2.0, window=window)
    assert torch_error(p) < 1e-12


def test_window_one_gives_identity_attention():
    # window 1: every query sees only its own key, P = 1, O = V, dQ = dK = 0, dV = dO
    p = make_problem(MASK_CAUSAL, [6], [6], heads=1, d=4, seed=3, window=1)
    o, m, l, dq, dk, dv = exact_backward(p)
    np.testing.assert_allclose(o, p["v"], rtol=1e-14)
    np.testing.assert_allclose(dv, p["do"], rtol=1e-14)
    assert np.all(np.abs(dq) < 1e-14) and np.all(np.abs(dk) < 1e-14)


def test_planted_window_off_by_one_fails_torch_check(monkeypatch):
    p = make_problem(MASK_CAUSAL, [7], [7], heads=1, d=4, seed=81, window=3)
    assert torch_error(p) < 1e-12
    _mutant(monkeypatch, "visible_block", "(j > i - window)", "(j >= i - window)")
    assert torch_error(p) > 1e-3


# ---------------------------------------------------------------- sampled rows == full backward

@pytest.mark.parametrize("mask", [MASK_NONE, MASK_CAUSAL, MASK_PADDING_CAUSAL])
def test_backward_rows_matches_full(mask):
    padded = 40 if A.is_padded(mask) else 0
    p = make_problem(mask, [40, 23], [40, 23], heads=3, d=16, seed=5, padded_len=padded)
    o, m, l, dq, dk, dv = exact_backward(p)
    for b, (qs, lq) in enumerate(A.segments(p["cu_q"], mask, p["max_seqlen_q"])):
        ks = A.segments(p["cu_kv"], mask, p["max_seqlen_kv"])[b][0]
        rows = [0, 1, lq // 2, lq - 1]
        sq, sk, sv = A.backward_rows(p["q"], p["k"], p["v"], o, p["do"], m, l, p["cu_q"], p["cu_kv"],
                                     p["scale"], mask, b, 2, rows, rows, p["max_seqlen_q"], p["max_seqlen_kv"])
        np.testing.assert_allclose(sq, dq[[qs + r for r in rows], 2], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(sk, dk[[ks + r for r in rows], 2], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(sv, dv[[ks + r for r in rows], 2], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- planted mistakes are caught

# ---------------------------------------------------------------- value head dim != query/key head dim

MLA_CASES = [
    # (mask, lens_q, lens_kv, d, d_v, padded_len)
    (MASK_NONE, [3], [5], 4, 2, 0),
    (MASK_CAUSAL, [5], [5], 2, 6, 0),
    (MASK_PADDING_CAUSAL, [4, 2], [4, 3], 6, 3, 4),
]


@pytest.mark.parametrize("mask,lq,lk,d,d_v,padded", MLA_CASES)
def test_value_head_dim_finite_differences(mask, lq, lk, d, d_v, padded):
    p = make_problem(mask, lq, lk, heads=2, d=d, seed=71, padded_len=padded, d_v=d_v)
    assert fd_error(p) < 1e-6


@pytest.mark.parametrize("mask,lq,lk,d,d_v,padded", MLA_CASES + [(MASK_CAUSAL, [70, 33], [70, 50], 24, 8, 0)])
def test_value_head_dim_torch_fp64_autograd(mask, lq, lk, d, d_v, padded):
    p = make_problem(mask, lq, lk, heads=3, d=d, seed=72, padded_len=padded, mult=1.5, d_v=d_v)
    assert torch_error(p) < 1e-10


def test_value_head_dim_rows_match_full():
    p = make_problem(MASK_CAUSAL, [40, 17], [40, 30], heads=2, d=12, seed=73, d_v=20)
    o, m, l, dq, dk, dv = exact_backward(p)
    assert o.shape[2] == 20 and dq.shape[2] == 12 and dk.shape[2] == 12 and dv.shape[2] == 20
    rows = [0, 5, 39]
    ro, rm, rl = A.forward_rows(p["q"], p["k"], p["v"], p["cu_q"], p["cu_kv"], p["scale"], p["mask"], 0, 1, rows)
    assert np.allclose(ro, o[rows, 1]) and np.allclose(rm, m[rows, 1]) and np.allclose(rl, l[rows, 1])
    rq, rk, rv = A.backward_rows(p["q"], p["k"], p["v"], o, p["do"], m, l, p["cu_q"], p["cu_kv"], p["scale"],
                                 p["mask"], 0, 1, rows, [0, 7, 39])
    assert np.allclose(rq, dq[rows, 1]) and np.allclose(rk, dk[[0, 7, 39], 1]) and np.allclose(rv, dv[[0, 7, 39], 1])


def _mutant(monkeypatch, func_name, old, new):
    """Replace ``func_name`` in the oracle module by a copy of its source with one edit."""
    src = textwrap.dedent(inspect.getsource(getattr(A, func_name)))
    assert old in src, f"mutation target not found in {func_name}: {old!r}"
    ns = {}
    exec(compile(src.replace(old, new), f"<mutant {func_name}>", "exec"), A.__dict__, ns)
    monkeypatch.setattr(A, func_name, ns[func_name])


MUTANTS = [
    ("backward_head", "ds = p * (dp - dvec[:, None])", "ds = p * dp", "D dropped"),
    ("backward_head", "ds = p * (dp - dvec[:, None])", "ds = p * (dvec[:, None] - dp)", "sign of dS"),
    ("backward_head", "dk = scale * (ds.T @ q)", "dk = (ds.T @ q)", "scale dropped from dK"),
    ("backward_head", "dq = scale * (ds @ k)", "dq = (ds @ k)", "scale dropped from dQ"),
    ("backward_head", "dv = p.T @ do", "dv = p @ do", "transposed P in dV"),
    ("backward_head", "dq = scale * (ds @ k)", "dq = scale * (ds @ v)", "wrong operand in dQ"),
    ("backward_head", "p = softmax_probs(scale * s, m, l, vis)", "p = softmax_probs(s, m, l, vis)",
     "scale missing in the softmax"),
    ("softmax_probs", "np.exp(z) / np.where(ok, l[:, None], 1.0)", "np.exp(z)", "division by l dropped"),
    ("backward_head", "dvec = np.sum(o * do, axis=1)", "dvec = np.sum(o * do, axis=0)[:o.shape[0]]",
     "wrong reduction axis for D"),
]


@pytest.mark.parametrize("func,old,new,what", MUTANTS, ids=[m[3] for m in MUTANTS])
def test_planted_mistake_fails_finite_differences(monkeypatch, func, old, new, what):
    p = make_problem(MASK_CAUSAL, [5, 4], [5, 4], heads=1, d=4, seed=21)
    assert fd_error(p) < 2e-6
    _mutant(monkeypatch, func, old, new)
    try:
        err = fd_error(p)
    except ValueError:          # a shape error is also a caught mistake
        err = float("inf")
    assert err > 1e-3, what


@pytest.mark.parametrize("old,new,what", [
    ("return j <= i", "return j < i", "causal diagonal excluded"),
    ("return j <= i", "return j >= i", "causal mask flipped"),
])
def test_planted_mask_mistake_fails_torch_check(monkeypatch, old, new, what):
    p = make_problem(MASK_CAUSAL, [6, 5], [6, 5], heads=1, d=4, seed=22)
    assert torch_error(p) < 1e-12
    _mutant(monkeypatch, "visible_block", old, new)
    assert torch_error(p) > 1e-3, what


def test_planted_layout_mistake_fails_torch_check(monkeypatch):
    # padded slots must start at b * max_seqlen, not at the cumulative offset
    p = make_problem(MASK_PADDING, [5, 3], [5, 3], heads=1, d=4, seed=23, padded_len=6)
    assert torch_error(p) < 1e-12
    _mutant(monkeypatch, "segments", "start = b * max_seqlen if is_padded(mask) else cu[b]", "start = cu[b]")
    assert torch_error(p) > 1e-3


def test_planted_group_overwrite_fails_finite_differences(monkeypatch):
    # a shared K/V head must collect the gradients of all its query heads, not keep the last one
    p = make_problem(MASK_CAUSAL, [4], [4], heads=4, d=4, seed=51, heads_kv=2)
    assert fd_error(p) < 2e-6
    _mutant(monkeypatch, "backward", 'dk[ksl, hk] += r["dk"]', 'dk[ksl, hk] = r["dk"]')
    assert fd_error(p) > 1e-3


# ---------------------------------------------------------------- the query-row-block form

BLOCK_CASES = [
    (MASK_NONE, [13, 1, 40], [9, 30, 17], 0),
    (MASK_CAUSAL, [37, 5, 64], [37, 9, 64], 0),
    (MASK_PADDING, [20, 33], [20, 33], 0),
    (MASK_PADDING_CAUSAL, [29, 7], [25, 7], 0),
    (MASK_CAUSAL, [45, 19], [45, 19], 6),
    (MASK_NONE, [31, 0, 12], [31, 4, 12], 0),
]


@pytest.mark.parametrize("mask,lens_q,lens_kv,window", BLOCK_CASES)
@pytest.mark.parametrize("block", [1, 3, 8, 64])
def test_blocked_forward_backward_equal_whole_slice_form(mask, lens_q, lens_kv, window, block):
    """Row blocks split the sums over query rows (steps 6, 7) and leave every row's own computation
    unchanged, so both forms agree to rounding; blocks of one row, ragged last blocks and blocks that
    see no key are covered."""
    padded = max(max(lens_q), max(lens_kv)) + 3 if A.is_padded(mask) else 0
    p = make_problem(mask, lens_q, lens_kv, heads=3, d=8, seed=61, padded_len=padded, heads_kv=1, window=window)
    args = (p["cu_q"], p["cu_kv"], p["scale"], p["mask"], p["max_seqlen_q"], p["max_seqlen_kv"], window)
    o, m, l = A.forward(p["q"], p["k"], p["v"], *args)
    ob, mb, lb = A.forward_blocked(p["q"], p["k"], p["v"], *args, block=block, workers=2)
    assert np.allclose(ob, o, rtol=1e-12, atol=1e-13) and np.allclose(mb, m, rtol=1e-13, atol=1e-14)
    assert np.allclose(lb, l, rtol=1e-12)
    ref = A.backward(p["q"], p["k"], p["v"], o, p["do"], m, l, *args)
    got = A.backward_blocked(p["q"], p["k"], p["v"], o, p["do"], m, l, *args, block=block, workers=3)
    for r, g in zip(ref, got):
        assert np.allclose(g, r, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("mask", [MASK_NONE, MASK_CAUSAL])
def test_blocked_form_keeps_the_invariants(mask):
    """At a size the whole-slice pins do not reach (two 700-row sequences, blocks of 64): dK columns
    sum to zero and dV columns sum to the dO columns of the rows that see keys (rows of P sum to 1)."""
    p = make_problem(mask, [700, 333], [700, 333], heads=2, d=16, seed=62)
    args = (p["cu_q"], p["cu_kv"], p["scale"], p["mask"], p["max_seqlen_q"], p["max_seqlen_kv"])
    o, m, l = A.forward_blocked(p["q"], p["k"], p["v"], *args, block=64, workers=4)
    dq, dk, dv = A.backward_blocked(p["q"], p["k"], p["v"], o, p["do"], m, l, *args, block=64, workers=4)
    for (qs, lq), (ks, lk) in zip(A.segments(p["cu_q"], mask, 0), A.segments(p["cu_kv"], mask, 0)):
        for h in range(2):
            assert np.allclose(dk[ks:ks + lk, h].sum(axis=0), 0.0, atol=1e-9)
            assert np.allclose(dv[ks:ks + lk, h].sum(axis=0), p["do"][qs:qs + lq, h].sum(axis=0), atol=1e-9)
    if mask == MASK_CAUSAL:   # row 0 of a sequence sees only key 0 (P = 1): its dQ vanishes up to rounding
        assert np.allclose(dq[0], 0.0, atol=1e-12) and np.allclose(dq[700], 0.0, atol=1e-12)


def test_blocked_form_finite_differences():
    """Central differences through the blocked forward with blocks of two rows (every block boundary
    inside the sequences), against the blocked backward."""
    p = make_problem(MASK_CAUSAL, [5, 4], [5, 4], heads=1, d=4, seed=63)
    args = (p["cu_q"], p["cu_kv"], p["scale"], p["mask"], p["max_seqlen_q"], p["max_seqlen_kv"])

    def loss():
        o, _, _ = A.forward_blocked(p["q"], p["k"], p["v"], *args, block=2)
        return float(np.sum(o * p["do"]))

    o, m, l = A.forward_blocked(p["q"], p["k"], p["v"], *args, block=2)
    grads = dict(zip(("q", "k", "v"), A.backward_blocked(p["q"], p["k"], p["v"], o, p["do"], m, l, *args, block=2)))
    eps = 1e-6
    for name in ("q", "k", "v"):
        x = p[name]
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            lp = loss()
            x[idx] = keep - eps
            lm = loss()
            x[idx] = keep
            assert abs((lp - lm) / (2 * eps) - grads[name][idx]) < 2e-6, (name, idx)


BLOCK_MUTANTS = [
    ("backward_head_blocked", "dk[keys] += scale * (ds.T @ q[rows])", "dk[keys] = scale * (ds.T @ q[rows])",
     "dK keeps the last block only"),
    ("backward_head_blocked", "dq[rows] = scale * (ds @ k[keys])", "dq[rows] = scale * (ds @ k[rows])",
     "dQ contracted with the block's own rows"),
    ("key_range", "j1 = min(lk, i1) if (causal or window > 0) else lk", "j1 = min(lk, i1 - 1) if (causal or window > 0) else lk",
     "key range misses the block's diagonal key"),
]


@pytest.mark.parametrize("func,old,new,what", BLOCK_MUTANTS, ids=[m[3] for m in BLOCK_MUTANTS])
def test_planted_block_mistake_is_caught(monkeypatch, func, old, new, what):
    p = make_problem(MASK_CAUSAL, [9, 6], [9, 6], heads=1, d=4, seed=64)
    args = (p["cu_q"], p["cu_kv"], p["scale"], p["mask"], p["max_seqlen_q"], p["max_seqlen_kv"])
    o, m, l = A.forward(p["q"], p["k"], p["v"], *args)
    ref = A.backward(p["q"], p["k"], p["v"], o, p["do"], m, l, *args)
    _mutant(monkeypatch, func, old, new)
    try:
        got = A.backward_blocked(p["q"], p["k"], p["v"], o, p["do"], m, l, *args, block=4)
        err = max(float(np.max(np.abs(g - r))) for g, r in zip(got, ref))
    except ValueError:  # a shape error is also a caught mistake
        err = float("inf")
    assert err > 1e-3, what
