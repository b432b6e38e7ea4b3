"""Plain fp64 CPU oracle for the single-pass attention backward (and the forward
that produces its inputs O, m, l).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this
module: only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use it. It shares no code with the HIP library.

What it computes, and where the pages define it:

* Backward, per (sequence b, head h), following the eight per-tile steps of the
  PyPTO-Gym SK-16 article ("single-pass attention backward (FA Grad)"), §3.1,
  with the dtype discipline of its §4.2 reduced to exact fp64 arithmetic:
    1. S  = Q K^T                        (the scale is applied in step 2)
    2. P  = exp(S*scale - m) / l         (m, l are the caller's row statistics)
    3. dP = dO V^T
    4. D  = rowsum(O * dO)               (from the O the caller passes)
    5. dS = P * (dP - D)
    6. dK = scale * dS^T Q
    7. dV = P^T dO
    8. dQ = scale * dS K
  The article runs these per (q_tile, kv_tile) pair and accumulates; the sum
  over tiles equals the untiled matrix products written here, so the oracle
  uses the whole (b, h) slice at once and does no tiling of its own.
* Masks: the codes of ``MaskType`` in jax ``_src/cudnn/fused_attention_stablehlo.py``
  (NO_MASK=0, PADDING=1, CAUSAL=2, PADDING_CAUSAL=3). Causal visibility is
  top-left aligned in sequence-local coordinates (key j visible from query i
  iff j <= i); the pages do not fix the alignment when the two lengths differ.
* Sequence layout: packed modes (NO_MASK, CAUSAL) place sequence b at rows
  [cu[b], cu[b+1]) as in the article's ``actual_q``/``actual_kv`` offsets (§三).
  Padded modes (PADDING, PADDING_CAUSAL) place sequence b at rows
  [b*max_seqlen, b*max_seqlen + L_b) with L_b = cu[b+1] - cu[b], i.e. the
  BTNH padded layout of the jax page with per-batch valid lengths; the other
  rows of the slot are padding.
* Forward (input producer only): m = row max of the scaled visible logits,
  l = sum over visible keys of exp(scaled logit - m), O = P V; this is the
  reading under which step 2 above is the softmax.

* Sliding window (jax cuDNN wrapper, ``sliding_window_length``): with a window w > 0 each query
  i sees only its left local window of keys (i - w, i]; the window implies the causal bound
  whatever the mask code. w = 0 means no window.
* Grouped heads: K and V may have fewer heads than Q (a divisor of it). Query head h
  reads key/value head h // (H_q / H_kv), consecutive query heads sharing one K/V head
  (the grouping of the jax cuDNN wrapper's attention API); dK and dV of a shared head are
  the sums over its query heads.

* Query row blocks (``forward_blocked``, ``backward_blocked``): the same steps per block of query
  rows with the block's full key range, for sizes whose whole-slice matrices do not fit in memory;
  dK and dV add up the blocks' terms. Pinned against the whole-slice form, the invariants and
  finite differences in the tests.

Rows outside every sequence: forward gives O = 0, m = 0, l = 1 (finite filler
that the backward never reads); backward gives dQ = dK = dV = 0. A valid query
row with no visible key (only when its sequence has no keys) gets P = 0.
"""
from __future__ import annotations

import numpy as np

MASK_NONE = 0
MASK_PADDING = 1
MASK_CAUSAL = 2
MASK_PADDING_CAUSAL = 3


def is_causal(mask: int) -> bool:
    return mask in (MASK_CAUSAL, MASK_PADDING_CAUSAL)


def is_padded(mask: int) -> bool:
    return mask in (MASK_PADDING, MASK_PADDING_CAUSAL)


def segments(cu, mask: int, max_seqlen: int):
    """Return [(first_row, length)] per sequence (layout reading in the module docstring)."""
    cu = [int(x) for x in np.asarray(cu).reshape(-1)]
    out = []
    for b in range(len(cu) - 1):
        length = cu[b + 1] - cu[b]
        start = b * max_seqlen if is_padded(mask) else cu[b]
        out.append((start, length))
    return out


def kv_head(h: int, heads_q: int, heads_kv: int) -> int:
    """The K/V head that query head h reads (consecutive query heads share one)."""
    if heads_q % heads_kv:
        raise ValueError(f"{heads_q} query heads are not a multiple of {heads_kv} key/value heads")
    return h // (heads_q // heads_kv)


def visible_block(rows, cols, causal: bool, window: int = 0) -> np.ndarray:
    """Boolean [len(rows), len(cols)]: may query rows[a] attend to key cols[b]
    (sequence-local indices; causal: key j visible from query i iff j <= i; a window w > 0
    restricts every query to its left local window (i - w, i])."""
    i = np.asarray(rows)[:, None]
    j = np.asarray(cols)[None, :]
    if window > 0:
        return (j <= i) & (j > i - window)
    if causal:
        return j <= i
    return np.ones((i.shape[0], j.shape[1]), dtype=bool)


def visible(lq: int, lk: int, causal: bool, window: int = 0) -> np.ndarray:
    """Boolean [lq, lk]: visibility of every (query, key) pair of one sequence."""
    return visible_block(np.arange(lq), np.arange(lk), causal, window)


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor (any dtype) -> exact fp64 values
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def softmax_probs(s_scaled: np.ndarray, m: np.ndarray, l: np.ndarray, vis: np.ndarray) -> np.ndarray:
    """Step 2: P = exp(S*scale - m) / l on visible entries, 0 elsewhere.

    ``s_scaled`` already holds S*scale. Rows whose l is not positive (no
    visible key) give P = 0.
    """
    z = np.where(vis, s_scaled - m[:, None], -np.inf)
    ok = (l > 0)[:, None]
    return np.where(vis & ok, np.exp(z) / np.where(ok, l[:, None], 1.0), 0.0)


def forward_head(q, k, v, scale: float, causal: bool, window: int = 0):
    """Forward for one (b, h): returns O [Lq,d], m [Lq], l [Lq] in fp64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    lq, lk = q.shape[0], k.shape[0]
    vis = visible(lq, lk, causal, window)
    s = scale * (q @ k.T)
    has_key = vis.any(axis=1)
    m = np.where(has_key, np.max(np.where(vis, s, -np.inf), axis=1, initial=-np.inf), 0.0)
    e = np.where(vis, np.exp(np.where(vis, s - m[:, None], 0.0)), 0.0)
    l = np.where(has_key, e.sum(axis=1), 1.0)
    p = np.where(has_key[:, None], e / l[:, None], 0.0)
    o = p @ v
    return o, m, l


def backward_head(q, k, v, o, do, m, l, scale: float, causal: bool, window: int = 0):
    """Backward for one (b, h), steps 1-8 of the module docstring.

    Inputs are one sequence's rows of one head; everything is promoted to fp64.
    Returns a dict with dq, dk, dv and the intermediates p, dp, dvec, ds.
    """
    q, k, v, o, do = _f64(q), _f64(k), _f64(v), _f64(o), _f64(do)
    m, l = _f64(m), _f64(l)
    vis = visible(q.shape[0], k.shape[0], causal, window)
    s = q @ k.T                                   # 1
    p = softmax_probs(scale * s, m, l, vis)       # 2
    dp = do @ v.T                                 # 3
    dvec = np.sum(o * do, axis=1)                 # 4
    ds = p * (dp - dvec[:, None])                 # 5
    dk = scale * (ds.T @ q)                       # 6
    dv = p.T @ do                                 # 7
    dq = scale * (ds @ k)                         # 8
    return {"dq": dq, "dk": dk, "dv": dv, "p": p, "dp": dp, "dvec": dvec, "ds": ds}


def forward(q, k, v, cu_q, cu_kv, scale: float, mask: int, max_seqlen_q: int = 0, max_seqlen_kv: int = 0,
            window: int = 0):
    """Forward over [T, H, d] inputs. Returns fp64 O [Tq,H,d], m [Tq,H], l [Tq,H]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    tq, h_count, d = q.shape
    o = np.zeros((tq, h_count, v.shape[2]))
    m = np.zeros((tq, h_count))
    l = np.ones((tq, h_count))
    causal = is_causal(mask)
    for (qs, lq), (ks, lk) in zip(segments(cu_q, mask, max_seqlen_q), segments(cu_kv, mask, max_seqlen_kv)):
        if lq <= 0:
            continue
        for h in range(h_count):
            hk = kv_head(h, h_count, k.shape[1])
            ob, mb, lb = forward_head(q[qs:qs + lq, h], k[ks:ks + lk, hk], v[ks:ks + lk, hk], scale, causal, window)
            o[qs:qs + lq, h], m[qs:qs + lq, h], l[qs:qs + lq, h] = ob, mb, lb
    return o, m, l


def backward(q, k, v, o, do, m, l, cu_q, cu_kv, scale: float, mask: int,
             max_seqlen_q: int = 0, max_seqlen_kv: int = 0, window: int = 0):
    """Backward over [T, H, d] inputs. Returns fp64 dQ [Tq,H,d], dK, dV [Tkv,H,d]."""
    q, k, v, o, do = _f64(q), _f64(k), _f64(v), _f64(o), _f64(do)
    m, l = _f64(m), _f64(l)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    causal = is_causal(mask)
    for (qs, lq), (ks, lk) in zip(segments(cu_q, mask, max_seqlen_q), segments(cu_kv, mask, max_seqlen_kv)):
        if lq <= 0 and lk <= 0:
            continue
        qsl, ksl = slice(qs, qs + max(lq, 0)), slice(ks, ks + max(lk, 0))
        for h in range(q.shape[1]):
            hk = kv_head(h, q.shape[1], k.shape[1])
            r = backward_head(q[qsl, h], k[ksl, hk], v[ksl, hk], o[qsl, h], do[qsl, h],
                              m[qsl, h], l[qsl, h], scale, causal, window)
            dq[qsl, h] = r["dq"]
            dk[ksl, hk] += r["dk"]   # a shared K/V head collects the gradients of its query heads
            dv[ksl, hk] += r["dv"]
    return dq, dk, dv


def backward_from_lse(q, k, v, o, do, lse, cu_q, cu_kv, scale: float, mask: int,
                      max_seqlen_q: int = 0, max_seqlen_kv: int = 0, window: int = 0):
    """Backward from one log-sum-exp statistic per row (lse = m + ln l, the single softmax statistic
    of the jax cuDNN wrapper): step 2 reads P = exp(S*scale - lse), which is the step-2 formula with
    m = lse and l = 1."""
    lse = _f64(lse)
    return backward(q, k, v, o, do, lse, np.ones_like(lse), cu_q, cu_kv, scale, mask, max_seqlen_q, max_seqlen_kv,
                    window)


def forward_rows(q, k, v, cu_q, cu_kv, scale: float, mask: int, b: int, h: int, q_rows,
                 max_seqlen_q: int = 0, max_seqlen_kv: int = 0, window: int = 0):
    """O, m, l of selected query rows of one (b, h), each row computed on its own with the steps
    of ``forward_head``; indices are sequence-local. Returns fp64 O [n, d], m [n], l [n]."""
    qs, lq = segments(cu_q, mask, max_seqlen_q)[b]
    ks, lk = segments(cu_kv, mask, max_seqlen_kv)[b]
    causal = is_causal(mask)
    hk = kv_head(h, q.shape[1], k.shape[1])
    Q, K, V = _f64(q[qs:qs + lq, h]), _f64(k[ks:ks + lk, hk]), _f64(v[ks:ks + lk, hk])
    o_out, m_out, l_out = [], [], []
    for i in q_rows:
        vis = visible_block([i], np.arange(lk), causal, window)[0]
        s = scale * (Q[i] @ K.T)
        if not vis.any():
            o_out.append(np.zeros(V.shape[1]))
            m_out.append(0.0)
            l_out.append(1.0)
            continue
        m = np.max(s[vis])
        e = np.where(vis, np.exp(np.where(vis, s - m, 0.0)), 0.0)
        l = e.sum()
        o_out.append((e / l) @ V)
        m_out.append(m)
        l_out.append(l)
    return np.array(o_out).reshape(-1, V.shape[1]), np.array(m_out), np.array(l_out)


def backward_rows(q, k, v, o, do, m, l, cu_q, cu_kv, scale: float, mask: int, b: int, h: int,
                  q_rows, kv_rows, max_seqlen_q: int = 0, max_seqlen_kv: int = 0, window: int = 0):
    """Selected outputs of sequence b, each computed on its own: rows of dQ of query head h and
    rows of dK/dV of the K/V head that h reads (summed over the query heads sharing it).

    dQ row i needs row i of P and dS (all keys); dK/dV row j needs column j of
    P and dS (all queries). Indices are sequence-local. Returns
    (dq [len(q_rows), d], dk [len(kv_rows), d], dv [len(kv_rows), d]) in fp64.
    This is the same step list as ``backward_head``, restricted to the rows or
    columns asked for, so that full-size problems can be checked on samples.
    """
    qs, lq = segments(cu_q, mask, max_seqlen_q)[b]
    ks, lk = segments(cu_kv, mask, max_seqlen_kv)[b]
    causal = is_causal(mask)
    hq_count, hk_count = q.shape[1], k.shape[1]
    hk = kv_head(h, hq_count, hk_count)
    K, V = _f64(k[ks:ks + lk, hk]), _f64(v[ks:ks + lk, hk])
    d = q.shape[2]
    dv_d = v.shape[2]

    def head_slices(hq):
        return (_f64(q[qs:qs + lq, hq]), _f64(o[qs:qs + lq, hq]), _f64(do[qs:qs + lq, hq]),
                _f64(m[qs:qs + lq, hq]), _f64(l[qs:qs + lq, hq]))

    Q, O, dO, M, L = head_slices(h)
    dq_out = []
    for i in q_rows:
        vis = visible_block([i], np.arange(lk), causal, window)
        s = (Q[i:i + 1] @ K.T)
        p = softmax_probs(scale * s, M[i:i + 1], L[i:i + 1], vis)
        dp = dO[i:i + 1] @ V.T
        dvec = np.sum(O[i] * dO[i])
        ds = p * (dp - dvec)
        dq_out.append(scale * (ds @ K)[0])
    dk_out = np.zeros((len(kv_rows), d))
    dv_out = np.zeros((len(kv_rows), dv_d))
    group = [hq for hq in range(hq_count) if kv_head(hq, hq_count, hk_count) == hk]
    for hq in group if len(kv_rows) else []:
        Q, O, dO, M, L = head_slices(hq)
        dvec_all = np.sum(O * dO, axis=1)
        for n, j in enumerate(kv_rows):
            vis = visible_block(np.arange(lq), [j], causal, window)
            s = Q @ K[j:j + 1].T
            p = softmax_probs(scale * s, M, L, vis)
            dp = dO @ V[j:j + 1].T
            ds = p * (dp - dvec_all[:, None])
            dk_out[n] += scale * (ds.T @ Q)[0]
            dv_out[n] += (p.T @ dO)[0]
    return np.array(dq_out).reshape(-1, d), dk_out, dv_out


def loss(q, k, v, do, cu_q, cu_kv, scale: float, mask: int, max_seqlen_q: int = 0, max_seqlen_kv: int = 0,
         window: int = 0) -> float:
    """Scalar sum(O * dO) with dO a fixed cotangent; its gradient is (dQ, dK, dV)."""
    o, _, _ = forward(q, k, v, cu_q, cu_kv, scale, mask, max_seqlen_q, max_seqlen_kv, window)
    return float(np.sum(o * _f64(do)))


# ---------------------------------------------------------------- query row blocks
#
# Full-size problems (a 32768-token sequence) do not fit the whole-slice matrices above (8 GiB per
# fp64 matrix). The functions below take the same steps over blocks of query rows: each block holds
# its rows' full key range, so every row is computed exactly as in the whole-slice form (no online
# softmax), and dK, dV are sums over the blocks of the block's terms -- the sums over i in steps 6
# and 7 split into partial sums, as the SK-16 article itself accumulates dK/dV over q tiles (§3.1).
# A block looks only at the keys some row of it can see (keys past the block's last row under a
# causal bound, keys before its first row's window); the others have P = 0 and add nothing.


def key_range(i0: int, i1: int, lk: int, causal: bool, window: int = 0):
    """[j0, j1): the keys that some query row of [i0, i1) may see (sequence-local indices)."""
    j1 = min(lk, i1) if (causal or window > 0) else lk
    j0 = max(0, i0 - window + 1) if window > 0 else 0
    return j0, max(j0, j1)


def forward_head_blocked(q, k, v, scale: float, causal: bool, window: int = 0, block: int = 256):
    """``forward_head`` over blocks of ``block`` query rows. Returns O [Lq,d_v], m [Lq], l [Lq]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    lq, lk = q.shape[0], k.shape[0]
    o = np.zeros((lq, v.shape[1]))
    m = np.zeros(lq)
    l = np.ones(lq)
    for i0 in range(0, lq, block):
        i1 = min(lq, i0 + block)
        j0, j1 = key_range(i0, i1, lk, causal, window)
        if j1 <= j0:
            continue  # no row of the block sees a key: O = 0, m = 0, l = 1
        vis = visible_block(np.arange(i0, i1), np.arange(j0, j1), causal, window)
        s = scale * (q[i0:i1] @ k[j0:j1].T)
        has_key = vis.any(axis=1)
        mb = np.where(has_key, np.max(np.where(vis, s, -np.inf), axis=1, initial=-np.inf), 0.0)
        e = np.where(vis, np.exp(np.where(vis, s - mb[:, None], 0.0)), 0.0)
        lb = np.where(has_key, e.sum(axis=1), 1.0)
        p = np.where(has_key[:, None], e / lb[:, None], 0.0)
        o[i0:i1] = p @ v[j0:j1]
        m[i0:i1] = mb
        l[i0:i1] = lb
    return o, m, l


def backward_head_blocked(q, k, v, o, do, m, l, scale: float, causal: bool, window: int = 0, block: int = 256):
    """``backward_head`` (steps 1-8) over blocks of ``block`` query rows: dQ rows of a block come from
    that block alone, dK and dV add up the blocks' terms. Returns dq [Lq,d], dk [Lk,d], dv [Lk,d_v]."""
    q, k, v, o, do = _f64(q), _f64(k), _f64(v), _f64(o), _f64(do)
    m, l = _f64(m), _f64(l)
    lq, lk = q.shape[0], k.shape[0]
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for i0 in range(0, lq, block):
        i1 = min(lq, i0 + block)
        j0, j1 = key_range(i0, i1, lk, causal, window)
        if j1 <= j0:
            continue  # no visible key: P = 0, so the block adds nothing and its dQ rows stay 0
        rows, keys = slice(i0, i1), slice(j0, j1)
        vis = visible_block(np.arange(i0, i1), np.arange(j0, j1), causal, window)
        s = q[rows] @ k[keys].T                                   # 1
        p = softmax_probs(scale * s, m[rows], l[rows], vis)      # 2
        dp = do[rows] @ v[keys].T                                 # 3
        dvec = np.sum(o[rows] * do[rows], axis=1)                 # 4
        ds = p * (dp - dvec[:, None])                             # 5
        dk[keys] += scale * (ds.T @ q[rows])                      # 6 (this block's terms)
        dv[keys] += p.T @ do[rows]                                # 7 (this block's terms)
        dq[rows] = scale * (ds @ k[keys])                         # 8
    return dq, dk, dv


def _slices(cu_q, cu_kv, mask, max_seqlen_q, max_seqlen_kv, heads_q, heads_kv):
    """(query rows, key rows, query head, K/V head) of every (sequence, head) with rows on both sides."""
    out = []
    for (qs, lq), (ks, lk) in zip(segments(cu_q, mask, max_seqlen_q), segments(cu_kv, mask, max_seqlen_kv)):
        if lq <= 0 or lk <= 0:
            continue
        for h in range(heads_q):
            out.append((slice(qs, qs + lq), slice(ks, ks + lk), h, kv_head(h, heads_q, heads_kv)))
    return out


def _run_slices(fn, items, workers: int):
    """fn over items, in order; with workers > 1 on a thread pool (the BLAS calls and the large
    elementwise NumPy operations release the interpreter lock), BLAS held to one thread per call."""
    if workers <= 1 or len(items) <= 1:
        return [fn(it) for it in items]
    from concurrent.futures import ThreadPoolExecutor
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1, user_api="blas")
    except ImportError:  # pragma: no cover - BLAS then keeps its own thread count
        limit = None
    try:
        with ThreadPoolExecutor(max_workers=workers) as pool:
            return list(pool.map(fn, items))
    finally:
        if limit is not None:
            limit.restore_original_limits()


def forward_blocked(q, k, v, cu_q, cu_kv, scale: float, mask: int, max_seqlen_q: int = 0, max_seqlen_kv: int = 0,
                    window: int = 0, block: int = 256, workers: int = 1):
    """``forward`` computed per (sequence, head) by ``forward_head_blocked``. fp64 O, m, l."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    tq, h_count, _ = q.shape
    o = np.zeros((tq, h_count, v.shape[2]))
    m = np.zeros((tq, h_count))
    l = np.ones((tq, h_count))
    causal = is_causal(mask)
    items = _slices(cu_q, cu_kv, mask, max_seqlen_q, max_seqlen_kv, h_count, k.shape[1])

    def one(it):
        qsl, ksl, h, hk = it
        return forward_head_blocked(q[qsl, h], k[ksl, hk], v[ksl, hk], scale, causal, window, block)

    for (qsl, _, h, _), (ob, mb, lb) in zip(items, _run_slices(one, items, workers)):
        o[qsl, h], m[qsl, h], l[qsl, h] = ob, mb, lb
    return o, m, l


def backward_blocked(q, k, v, o, do, m, l, cu_q, cu_kv, scale: float, mask: int, max_seqlen_q: int = 0,
                     max_seqlen_kv: int = 0, window: int = 0, block: int = 256, workers: int = 1):
    """``backward`` computed per (sequence, head) by ``backward_head_blocked``; a shared K/V head
    collects the gradients of its query heads in query-head order. fp64 dQ, dK, dV."""
    q, k, v, o, do = _f64(q), _f64(k), _f64(v), _f64(o), _f64(do)
    m, l = _f64(m), _f64(l)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    causal = is_causal(mask)
    items = _slices(cu_q, cu_kv, mask, max_seqlen_q, max_seqlen_kv, q.shape[1], k.shape[1])

    def one(it):
        qsl, ksl, h, hk = it
        return backward_head_blocked(q[qsl, h], k[ksl, hk], v[ksl, hk], o[qsl, h], do[qsl, h], m[qsl, h], l[qsl, h],
                                     scale, causal, window, block)

    for (qsl, ksl, h, hk), (rq, rk, rv) in zip(items, _run_slices(one, items, workers)):
        dq[qsl, h] = rq
        dk[ksl, hk] += rk
        dv[ksl, hk] += rv
    return dq, dk, dv


def valid_rows(cu, mask: int, max_seqlen: int, total: int) -> np.ndarray:
    """Boolean [total]: rows that belong to some sequence."""
    ok = np.zeros(total, dtype=bool)
    for start, length in segments(cu, mask, max_seqlen):
        if length > 0:
            ok[max(start, 0):min(start + length, total)] = True
    return ok
