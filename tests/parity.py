"""Shared helpers of the GPU parity tests: feed the HIP library and the fp64
oracle the same seeded inputs and compare per gradient tensor.

Tolerance (per tensor, over the rows compared): relative L2 error
||gpu - ref||_2 / ||ref||_2 <= 1e-2 and max |gpu - ref| <= 3e-2 * max |ref|;
rows outside every sequence must be exactly zero.
"""
from __future__ import annotations

import hashlib
import os
import time

import numpy as np
import torch

import oracle
import oracle.attention
from attention_backward_fa_amd import binding, inputs

REL_L2_TOL = 1e-2
MAX_ABS_TOL = 3e-2


def cpu_workers() -> int:
    """Threads for the oracle: this process's CPUs, at most 16 (the host share of one GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_stats(inp, workers: int | None = None):
    """O (bf16), m, l (fp32) from the oracle's fp64 forward on the bf16 inputs (query row blocks)."""
    o, m, l = oracle.forward_blocked(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_kv"], inp["scale"],
                                     inp["mask"], inp["max_seqlen_q"], inp["max_seqlen_kv"], inp.get("window", 0),
                                     workers=workers or cpu_workers())
    return (torch.from_numpy(o).to(torch.bfloat16), torch.from_numpy(m).to(torch.float32),
            torch.from_numpy(l).to(torch.float32))


def run_gpu(inp, o, m, l, device="cuda", algorithm=binding.FA_BWD_ALGO_DEFAULT):
    """Run the HIP backward once; returns CPU fp32 dq, dk, dv."""
    dev = torch.device(device)
    t = {k: inp[k].to(dev) for k in ("q", "k", "v", "do", "cu_q", "cu_kv")}
    dq, dk, dv = binding.attention_backward(t["q"], t["k"], t["v"], o.to(dev), t["do"], m.to(dev), l.to(dev),
                                            t["cu_q"], t["cu_kv"], inp["scale"], inp["mask"],
                                            inp["max_seqlen_q"], inp["max_seqlen_kv"], algorithm, inp.get("window", 0))
    torch.cuda.synchronize()
    return dq.float().cpu(), dk.float().cpu(), dv.float().cpu()


def oracle_backward(inp, o, m, l, workers: int | None = None):
    """fp64 dQ, dK, dV of the oracle (query row blocks) on the inputs the GPU sees."""
    return oracle.backward_blocked(inp["q"], inp["k"], inp["v"], o, inp["do"], m, l, inp["cu_q"], inp["cu_kv"],
                                   inp["scale"], inp["mask"], inp["max_seqlen_q"], inp["max_seqlen_kv"],
                                   inp.get("window", 0), workers=workers or cpu_workers())


def _cache_path(name: str, seed: int):
    """File of the optional on-disk cache of oracle results (directory in FA_ORACLE_CACHE, unset = off),
    keyed by workload, seed and the source of the oracle and of the input generator."""
    root = os.environ.get("FA_ORACLE_CACHE")
    if not root:
        return None
    h = hashlib.sha256()
    for mod in (oracle.attention, inputs):
        with open(mod.__file__, "rb") as fh:
            h.update(fh.read())
    return os.path.join(root, f"{name}_seed{seed}_{h.hexdigest()[:16]}.npz")


def reference(inp, log=None):
    """Oracle forward statistics (O bf16, m, l fp32) and backward (dQ, dK, dV) of one workload. With
    FA_ORACLE_CACHE set, results are kept on disk (gradients as fp32, whose rounding is far below the
    tolerance) and reused for the same workload, seed and oracle source."""
    path = _cache_path(inp["name"], inp["seed"])
    if path and os.path.exists(path):
        z = np.load(path)
        return ((torch.from_numpy(z["o"]).to(torch.bfloat16), torch.from_numpy(z["m"]), torch.from_numpy(z["l"])),
                tuple(z[k].astype(np.float64) for k in ("dq", "dk", "dv")))
    t0 = time.perf_counter()
    o, m, l = oracle_stats(inp)
    if log:
        log(f"oracle forward {time.perf_counter() - t0:.1f} s")
    t0 = time.perf_counter()
    ref = oracle_backward(inp, o, m, l)
    if log:
        log(f"oracle backward {time.perf_counter() - t0:.1f} s")
    if path:
        os.makedirs(os.path.dirname(path), exist_ok=True)
        np.savez(path, o=o.float().numpy(), m=m.numpy(), l=l.numpy(),
                 **{k: r.astype(np.float32) for k, r in zip(("dq", "dk", "dv"), ref)})
    return (o, m, l), ref


def metrics(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ref_l2 = np.linalg.norm(ref)
    ref_max = np.max(np.abs(ref)) if ref.size else 0.0
    err = gpu - ref
    rel_l2 = np.linalg.norm(err) / ref_l2 if ref_l2 > 0 else np.linalg.norm(err)
    max_ratio = np.max(np.abs(err)) / ref_max if ref_max > 0 else (np.max(np.abs(err)) if err.size else 0.0)
    return float(rel_l2), float(max_ratio)


def assert_close(name, gpu, ref):
    assert np.all(np.isfinite(np.asarray(gpu))), f"{name}: non-finite values"
    rel_l2, max_ratio = metrics(gpu, ref)
    assert rel_l2 <= REL_L2_TOL and max_ratio <= MAX_ABS_TOL, \
        f"{name}: rel_l2={rel_l2:.3e} (tol {REL_L2_TOL}), max_abs/max_ref={max_ratio:.3e} (tol {MAX_ABS_TOL})"
    return rel_l2, max_ratio


def check_full(inp, gpu, ref):
    """Compare every valid row; rows outside every sequence must be exactly 0."""
    vq = oracle.valid_rows(inp["cu_q"], inp["mask"], inp["max_seqlen_q"], inp["q"].shape[0])
    vk = oracle.valid_rows(inp["cu_kv"], inp["mask"], inp["max_seqlen_kv"], inp["k"].shape[0])
    out = {}
    for name, g, r, ok in (("dq", gpu[0], ref[0], vq), ("dk", gpu[1], ref[1], vk), ("dv", gpu[2], ref[2], vk)):
        g = g.numpy() if hasattr(g, "numpy") else g
        assert np.all(g[~ok] == 0), f"{name}: rows outside every sequence are not zero"
        out[name] = assert_close(name, g[ok], r[ok])
    return out
