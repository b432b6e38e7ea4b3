#!/usr/bin/env python3
"""Benchmark of the attention backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload causal]

One step = one ``fa_bwd_run`` over the whole workload, inputs already
resident in HBM: the row preprocess, then (default) the dK/dV kernel with 64
keys per wave, which also writes dS, and the dQ = dS K pass (the stored-dS form,
where the workload takes the 64-key layout and its dS workspace fits 8 GiB; else
the recompute form: the dK/dV kernel and the dQ kernel that recomputes S and
dP), or (``--algorithm single-pass``) the single-pass
main kernel with dQ atomics and the dQ cast, or (``--algorithm split-reduce``)
the single-pass main kernel over 8 kv-tile splits with a fixed-order dQ sum. The default workload is
the causal one: batch 1, 32 heads, 8192 tokens, head_dim 128. Throughput is
algorithmic TFLOP/s, counting 10*Lq*Lk*d FLOPs per (sequence, head) -- the
five GEMMs of the backward -- halved for causal masks.

Inputs: seeded synthetic Q, K, V, dO (``attention_backward_fa_amd.inputs``);
O, m, l come from a plain fp32 torch forward on the GPU (input preparation,
outside the timed region).

Prints ONE JSON line with the metric, a ``roofline`` object for the longest
kernel (its duration taken from HIP events the library records around each
kernel on the launch stream during the timed steps; its work counted as the
GEMMs that kernel itself runs; ``traffic`` is the HBM bytes per launch measured
with rocprofv3 FETCH_SIZE/WRITE_SIZE counters and recorded in
profiles/fa_bwd_traffic_causal_s8192_h32_d128.md, reported only while the
kernel sources still hash to the recorded value, else null; ``clock_sustained_ghz`` is
that kernel's shader-cycle count per launch, recorded the same way from GRBM_GUI_ACTIVE in
profiles/fa_bwd_counters_causal_s8192_h32_d128.md, over its live time in this run) and a
``cpu_baseline`` object (the fp64 oracle's backward timed on this host's cores
over a bounded sample of the same workload).

Every timed step records HIP events around its kernels on the launch stream:
``ms_median`` and ``ms_min`` are the median and the fastest step, ``ms_per_step``
the mean over the timed region. The outputs of the timed run are compared with
the oracle's whole (sequence, head) slices that the CPU baseline computes on the
same inputs (``parity``: per-tensor relative L2 and max-abs error). The dense
bf16 peak is also re-derived from rocminfo (``peak_derived``: compute units x
maximum shader clock x 4096 FLOPs per clock per CU); ``pct_peak`` and the
roofline use the published 2.5 PFLOP/s.

``--path forward`` times the forward that produces O, m, l instead, under its
own metric; ``--plan`` launches from the host-side longest-first schedule
(``fa_bwd_plan``) instead of the dense grid; ``--calibrate-copy MIB`` first runs
a kernel of known traffic, for scaling the counters in a ``rocprofv3 --pmc`` run.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FA-bwd TFLOP/s + % bf16 MFMA peak, S=8192 H=32 D=128 causal, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
BF16_FLOP_PER_CLK_PER_CU = 4096  # 4 SIMDs, each one 32x32x16 bf16 MFMA (32768 FLOPs) per 32 clocks
MASK_NAMES = {0: "none", 1: "padding", 2: "causal", 3: "padding_causal"}
ALGORITHMS = {"default": 0, "single-pass": 1, "recompute": 2, "split-reduce": 3, "recompute-8w": 4, "recompute-4w": 5,
              "recompute-64k": 6, "stored-ds": 7}
ALGORITHM_NAMES = {1: "single-pass (dQ atomics)",
                   2: "recompute (dK/dV kernel + dQ kernel; dK/dV layout chosen by load balance)",
                   3: "split-reduce (single-pass main kernel over 8 kv-tile splits + fixed-order dQ sum)",
                   4: "recompute (dK/dV kernel in eight-wave workgroups + dQ kernel)",
                   5: "recompute (dK/dV kernel in four-wave workgroups + dQ kernel)",
                   6: "recompute (dK/dV kernel with 64 keys per wave + dQ kernel)",
                   7: "stored dS (the dK/dV kernel writes dS; dQ = dS K pass)"}
# the dK/dV layout a handle takes (fa_bwd_dkdv_layout's algorithm codes)
LAYOUT_NAMES = {1: "none (single-pass form)", 3: "none (single-pass form)",
                2: "one layout (heads wider than 128)",
                4: "eight-wave workgroups, 32 keys per wave",
                5: "four-wave workgroups (two per CU), 32 keys per wave",
                6: "one four-wave workgroup per CU, 64 keys per wave"}


def kernel_share(algorithm: int, d: int, dv: int, layout: int = 0) -> dict:
    """Share of the 5-GEMM algorithmic FLOPs each kernel runs itself. S = QK^T, dK, dQ contract or
    produce the query/key head dim d, dP, dV the value head dim dv (2 * pairs * dim FLOPs each).
    Keys are the kernels' function names (the 64-key dK/dV layout is its own kernel)."""
    total = 3 * d + 2 * dv
    if algorithm == 1:
        return {"fa_bwd_pre": 0.0, "fa_bwd_main": 1.0, "fa_bwd_dq_cast": 0.0}
    if algorithm == 3:
        return {"fa_bwd_pre": 0.0, "fa_bwd_main": 1.0, "fa_bwd_split_reduce": 0.0}
    dkdv = "fa_bwd_dkdv64" if layout == 6 else "fa_bwd_dkdv"
    if algorithm == 7:  # dK/dV kernel: S, dP, dV, dK (and dS stored); the dS pass: dQ
        return {"fa_bwd_pre": 0.0, dkdv: (2 * d + 2 * dv) / total, "fa_bwd_dq_ds": d / total}
    # dK/dV kernel: S, dP, dV, dK; dQ kernel: S and dP again, dQ
    return {"fa_bwd_pre": 0.0, dkdv: (2 * d + 2 * dv) / total, "fa_bwd_dq": (2 * d + dv) / total}


def visible_pairs(lq: int, lk: int, causal: bool, window: int) -> float:
    """(query, key) pairs a sequence's FLOPs count: Lq * Lk, halved under a causal mask (the metric's
    convention), counted exactly under a sliding window (query i sees keys (i - window, i])."""
    if window > 0:
        import numpy as np
        i = np.arange(lq)
        hi = np.minimum(i, lk - 1)
        lo = np.maximum(0, i - window + 1)
        return float(np.maximum(0, hi - lo + 1).sum())
    return lq * lk / 2 if causal else float(lq * lk)


def algorithmic_flops(inp) -> float:
    """The five GEMMs of the backward over the visible pairs: 2 * pairs * (3 d + 2 d_v) per head, which is
    10 * Lq * Lk * d (halved when causal) when d_v = d."""
    causal = inp["mask"] in (2, 3)
    d, dv, h = inp["q"].shape[2], inp["v"].shape[2], inp["q"].shape[1]
    return sum(2.0 * visible_pairs(lq, lk, causal, inp.get("window", 0)) * (3 * d + 2 * dv) * h
               for lq, lk in zip(inp["seqlens_q"], inp["seqlens_kv"]))


def forward_flops(inp) -> float:
    """The forward's two GEMMs (S = QK^T over d, O = PV over d_v) over the same pairs."""
    d, dv = inp["q"].shape[2], inp["v"].shape[2]
    return algorithmic_flops(inp) * (d + dv) / (3 * d + 2 * dv)


def segments(inp):
    padded = inp["mask"] in (1, 3)
    out = []
    cq, ck = inp["cu_q"].tolist(), inp["cu_kv"].tolist()
    for b in range(len(cq) - 1):
        qs = b * inp["max_seqlen_q"] if padded else cq[b]
        ks = b * inp["max_seqlen_kv"] if padded else ck[b]
        out.append((qs, cq[b + 1] - cq[b], ks, ck[b + 1] - ck[b]))
    return out


def torch_forward_stats(inp, device, block=4096):
    """Input preparation: O (bf16), m, l (fp32) from a plain fp32 softmax-attention
    forward in torch on the GPU, query rows in blocks (grouped K/V heads repeated per
    query head; the window, when set, masks keys at or before i - window). Rows outside
    every sequence get O = 0, m = 0, l = 1."""
    import torch
    q, k, v = inp["q"], inp["k"], inp["v"]
    tq, h, d = q.shape
    group = h // k.shape[1]
    scale = inp["scale"]
    window = inp.get("window", 0)
    causal = inp["mask"] in (2, 3) or window > 0
    o = torch.zeros((tq, h, v.shape[2]), dtype=torch.bfloat16, device=device)
    m = torch.zeros((tq, h), dtype=torch.float32, device=device)
    l = torch.ones((tq, h), dtype=torch.float32, device=device)
    for qs, lq, ks, lk in segments(inp):
        if lq <= 0 or lk <= 0:
            continue
        kt = k[ks:ks + lk].to(device).float().permute(1, 2, 0).repeat_interleave(group, 0).contiguous()  # [H, d, Lk]
        vb = v[ks:ks + lk].to(device).float().permute(1, 0, 2).repeat_interleave(group, 0).contiguous()  # [H, Lk, dv]
        for i0 in range(0, lq, block):
            i1 = min(lq, i0 + block)
            qb = q[qs + i0:qs + i1].to(device).float().permute(1, 0, 2).contiguous()  # [H, n, d]
            s = torch.bmm(qb, kt) * scale                                             # [H, n, Lk]
            if causal:
                rows = torch.arange(i0, i1, device=device)[:, None]
                cols = torch.arange(lk, device=device)[None, :]
                hidden = (cols > rows) | (cols <= rows - window) if window > 0 else cols > rows
                s.masked_fill_(hidden[None], float("-inf"))
            mb = s.amax(dim=-1)
            e = torch.exp(s - mb[..., None])
            del s
            lb = e.sum(dim=-1)
            ob = torch.bmm(e, vb) / lb[..., None]
            del e
            o[qs + i0:qs + i1] = ob.permute(1, 0, 2).to(torch.bfloat16)
            m[qs + i0:qs + i1] = mb.T
            l[qs + i0:qs + i1] = lb.T
    return o, m, l


def describe(name: str, inp) -> str:
    """The workload's name and sizes, with the variant settings that differ from the plain case."""
    seqlens = sorted(set(inp["seqlens_q"]))
    heads, d = inp["q"].shape[1], inp["q"].shape[2]
    text = (f"{name}: batch {inp['batch']}, {heads} heads, "
            f"seqlens {seqlens if len(seqlens) < 5 else str(len(inp['seqlens_q'])) + ' varlen'}, "
            f"head_dim {d}, mask {MASK_NAMES[inp['mask']]}")
    if inp["k"].shape[1] != heads:
        text += f", {inp['k'].shape[1]} K/V heads"
    if inp["v"].shape[2] != d:
        text += f", value head_dim {inp['v'].shape[2]}"
    if inp.get("window", 0):
        text += f", window {inp['window']}"
    return text


def make_workload(name: str, device):
    """Seeded inputs of a named workload on `device`, with O, m, l from the torch forward."""
    import torch
    from attention_backward_fa_amd import inputs
    inp = inputs.make(name)
    o, m, l = torch_forward_stats(inp, device)
    dev = {key: inp[key].to(device) for key in ("q", "k", "v", "do", "cu_q", "cu_kv")}
    dev.update(o=o, m=m, l=l)
    return inp, dev


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_bwd_traffic_causal_s8192_h32_d128.md")


def _code_only(text: str, python: bool) -> str:
    """Source text without comments and blank lines, so that edits of comments alone keep the hash."""
    import re
    if python:
        text = re.sub(r'(?m)^\s*#.*$', "", text)
        text = re.sub(r'(?s)""".*?"""', "", text)
    else:
        text = re.sub(r"(?s)/\*.*?\*/", "", text)
        text = re.sub(r"(?m)//.*$", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def kernel_source_hash() -> str:
    """sha256 over the code (comments dropped) of the HIP sources and the build script, sorted by name."""
    import hashlib
    csrc = os.path.join(ROOT, "attention_backward_fa_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".hpp", ".h")))
    files += [os.path.join(ROOT, "include", "fa_bwd.h"), os.path.join(ROOT, "attention_backward_fa_amd", "build.py")]
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f) as fh:
            h.update(_code_only(fh.read(), f.endswith(".py")).encode())
    return h.hexdigest()


COUNTERS_FILE = os.path.join(ROOT, "profiles", "fa_bwd_counters_causal_s8192_h32_d128.md")


def profile_record(path: str, field: str, kernel: str, workload: str, algorithm: int):
    """A number from the record of a committed profile summary, or None when the summary is absent,
    covers another kernel/workload/algorithm, or was taken on kernel sources other than the current
    ones."""
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].strip().split(": ", 1)
                rec[k.strip("`")] = v.strip().strip("`")
    try:
        ok = (rec["kernel"] == kernel and rec["workload"] == workload and int(rec["algorithm"]) == algorithm
              and rec["source_sha256"] == kernel_source_hash())
        return float(rec[field]) if ok else None
    except (KeyError, ValueError):
        return None


def recorded_traffic(kernel: str, workload: str, algorithm: int):
    """HBM bytes per launch of `kernel` from the committed counter summary (FETCH_SIZE + WRITE_SIZE,
    calibrated), or None."""
    return profile_record(TRAFFIC_FILE, "traffic_bytes_per_launch", kernel, workload, algorithm)


def sustained_clock_ghz(kernel: str, workload: str, algorithm: int, kernel_ms: float):
    """Shader clock while `kernel` ran in this process: its shader-cycle count per launch from the
    committed counter summary (GRBM_GUI_ACTIVE per XCD) over its live time, or None."""
    cycles = profile_record(COUNTERS_FILE, "cycles_per_launch", kernel, workload, algorithm)
    return None if cycles is None else round(cycles / (kernel_ms * 1e-3) / 1e9, 3)


def copy_calibration(mib: int, device) -> None:
    """Counter calibration for rocprofv3 --pmc runs: three launches of torch's
    elementwise negation over `mib` MiB of fp32 (reads and writes exactly mib MiB
    each), so FETCH_SIZE / WRITE_SIZE of a kernel of known traffic can be read."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: 3 x neg over {mib} MiB read + {mib} MiB written", file=sys.stderr, flush=True)
    del src, dst


def derived_peak():
    """The dense bf16 MFMA peak from this GPU's own figures: compute units x maximum shader clock x
    4096 FLOPs per clock per CU, read from rocminfo (run as a child process before the GPU is used)."""
    import re
    import subprocess
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    for agent in out.split("*******"):
        if "gfx950" not in agent:
            continue
        cu = re.search(r"Compute Unit:\s+(\d+)", agent)
        clk = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", agent)
        if cu and clk:
            cus, mhz = int(cu.group(1)), int(clk.group(1))
            return {"source": "rocminfo", "compute_units": cus, "max_sclk_mhz": mhz,
                    "flop_per_clk_per_cu": BF16_FLOP_PER_CLK_PER_CU,
                    "tflops": round(cus * mhz * 1e6 * BF16_FLOP_PER_CLK_PER_CU / 1e12, 1)}
    return None


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        info = [x for x in threadpool_info() if x.get("user_api") == "blas"]
        if info:
            return int(info[0]["num_threads"])
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(inp, dev, target_s: float = 15.0):
    """The fp64 oracle's backward, as it stands, on (sequence, head) slices of the
    same workload and the same inputs the GPU saw; sample grown until ~target_s."""
    import numpy as np
    import oracle
    o, m, l = dev["o"].float().cpu().numpy(), dev["m"].cpu().numpy(), dev["l"].cpu().numpy()
    q, k, v, do = (inp[x].float().numpy() for x in ("q", "k", "v", "do"))
    causal = inp["mask"] in (2, 3)
    window = inp.get("window", 0)
    d, dv, heads = q.shape[2], v.shape[2], q.shape[1]
    group = heads // k.shape[1]
    pairs = [(b, h) for b in range(len(inp["seqlens_q"])) for h in range(heads)]
    segs = segments(inp)
    done, flops, elapsed, slices = [], 0.0, 0.0, []
    for b, h in pairs:
        qs, lq, ks, lk = segs[b]
        if lq <= 0 or lk <= 0:
            continue
        hk = h // group
        t0 = time.perf_counter()
        r = oracle.backward_head(q[qs:qs + lq, h], k[ks:ks + lk, hk], v[ks:ks + lk, hk], o[qs:qs + lq, h],
                                 do[qs:qs + lq, h], m[qs:qs + lq, h], l[qs:qs + lq, h], inp["scale"], causal, window)
        elapsed += time.perf_counter() - t0
        flops += 2.0 * visible_pairs(lq, lk, causal, window) * (3 * d + 2 * dv)
        done.append((b, h))
        slices.append(((qs, lq, ks, lk, h, hk), r["dq"], r["dk"], r["dv"]))
        if elapsed >= target_s:
            break
    del np
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"fp64 oracle backward on {len(done)} of {len(pairs)} (sequence, head) slices of the same "
                      f"workload and inputs ({elapsed:.1f} s); same FLOP count as the metric",
            "seconds": elapsed}, slices


def timed_output_parity(inp, outs, slices):
    """The timed run's dQ, dK, dV against the oracle's whole (sequence, head) slices from the CPU
    baseline: relative L2 error and max |gpu - ref| / max |ref| per tensor over the sampled slices.
    dK, dV are compared only without grouped K/V heads (a slice of one query head is then the whole
    gradient of its K/V head)."""
    import numpy as np
    gq, gk, gv = (x.float().cpu().numpy() for x in outs)
    grouped = inp["k"].shape[1] != inp["q"].shape[1]
    got = {"dq": [], "dk": [], "dv": []}
    ref = {"dq": [], "dk": [], "dv": []}
    for (qs, lq, ks, lk, h, hk), rq, rk, rv in slices:
        got["dq"].append(gq[qs:qs + lq, h].ravel())
        ref["dq"].append(rq.ravel())
        if not grouped:
            got["dk"].append(gk[ks:ks + lk, hk].ravel())
            ref["dk"].append(rk.ravel())
            got["dv"].append(gv[ks:ks + lk, hk].ravel())
            ref["dv"].append(rv.ravel())
    out = {"slices": len(slices), "rel_l2_tol": 1e-2, "max_abs_tol": 3e-2}
    ok = bool(slices)
    for name in ("dq", "dk", "dv"):
        if not got[name]:
            continue
        g, r = np.concatenate(got[name]).astype(np.float64), np.concatenate(ref[name])
        rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
        mx = float(np.max(np.abs(g - r)) / max(np.max(np.abs(r)), 1e-300))
        out[name] = {"rel_l2": float(f"{rel:.3e}"), "max_abs_over_max_ref": float(f"{mx:.3e}")}
        ok = ok and np.isfinite(g).all() and rel <= 1e-2 and mx <= 3e-2
    out["ok"] = bool(ok)
    return out


def bench_forward(args, device):
    """The forward kernel (O, m, l for the backward) on the same workload: 4 * Lq * Lk * d FLOPs per
    (sequence, head) -- the two GEMMs S = Q K^T and O = P V -- halved under a causal mask."""
    import torch
    from attention_backward_fa_amd import binding, inputs
    print(f"[bench] forward, preparing workload {args.workload}", file=sys.stderr, flush=True)
    inp = inputs.make(args.workload)
    dev = {key: inp[key].to(device) for key in ("q", "k", "v", "cu_q", "cu_kv")}
    flops = forward_flops(inp)
    tq, heads, d = inp["q"].shape
    op = binding.FaBwd(inp["batch"], heads, d, inp["max_seqlen_q"], inp["max_seqlen_kv"], tq, inp["k"].shape[0],
                       num_heads_kv=inp["k"].shape[1], window=inp["window"], head_dim_v=inp["v"].shape[2])
    if args.plan:
        op.plan(inp["cu_q"], inp["cu_kv"], inp["mask"])
    o = torch.empty((tq, heads, inp["v"].shape[2]), dtype=torch.bfloat16, device=device)
    m = torch.empty((tq, heads), dtype=torch.float32, device=device)
    l = torch.empty((tq, heads), dtype=torch.float32, device=device)

    def step():
        op.forward(dev["q"], dev["k"], dev["v"], dev["cu_q"], dev["cu_kv"], inp["scale"], inp["mask"], o, m, l)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    binding.fa_bwd_profile_enable(op.handle, True)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    stages = binding.fa_bwd_profile_collect(op.handle)
    binding.fa_bwd_profile_enable(op.handle, False)
    finite = bool(torch.isfinite(o).all()) and bool(torch.isfinite(m).all())
    op.close()
    fill_ms = sum(s_[0] for s_ in stages) / len(stages)
    fwd_ms = sum(s_[1] for s_ in stages) / len(stages)
    tflops = flops / (ms * 1e-3) / 1e12
    achieved = flops / (fwd_ms * 1e-3) / 1e12
    seqlens = sorted(set(inp["seqlens_q"]))
    out = {
        "metric": "FA-fwd TFLOP/s (forward producing O, m, l), % bf16 MFMA peak", "value": round(tflops, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": describe(args.workload, inp), "path": "forward",
                   "algorithmic_flops": flops},
        "pct_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "kernels_ms": {"fa_fwd_fill": round(fill_ms, 5), "fa_fwd": round(fwd_ms, 5)},
        "roofline": {"bound": "mfma", "kernel": "fa_fwd", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "work_flops": flops},
        "outputs_finite": finite,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="causal")
    ap.add_argument("--plan", action="store_true",
                    help="launch from a host-side longest-first schedule (fa_bwd_plan) instead of the dense grid")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--algorithm", choices=list(ALGORITHMS), default="default")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run a known-traffic elementwise kernel over MIB MiB (for --pmc counter scaling)")
    ap.add_argument("--path", choices=("backward", "forward"), default="backward",
                    help="forward: time the forward that produces O, m, l instead (its own metric)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the backward shards by (sequence, head) with no exchange, so N GPUs run N independent copies)",
              file=sys.stderr)
        sys.exit(2)

    peak_info = derived_peak()  # child process, before this process touches the GPU
    import torch
    from attention_backward_fa_amd import binding
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    if args.calibrate_copy > 0:
        copy_calibration(args.calibrate_copy, device)
    if args.path == "forward":
        return bench_forward(args, device)
    print(f"[bench] preparing workload {args.workload}", file=sys.stderr, flush=True)
    inp, dev = make_workload(args.workload, device)
    flops = algorithmic_flops(inp)
    tq, heads, d = inp["q"].shape
    algo = ALGORITHMS[args.algorithm]
    op = binding.FaBwd(inp["batch"], heads, d, inp["max_seqlen_q"], inp["max_seqlen_kv"], tq, inp["k"].shape[0],
                       algo, num_heads_kv=inp["k"].shape[1], window=inp["window"], head_dim_v=inp["v"].shape[2])
    layout = op.dkdv_layout(inp["mask"])  # the dK/dV layout this workload takes
    algo_used = op.dq_form(inp["mask"]) if algo == 0 else algo  # the default: stored dS or recompute
    if args.plan:  # host-side longest-first schedule from the (host) sequence offsets
        op.plan(inp["cu_q"], inp["cu_kv"], inp["mask"])
    dq, dk, dv = (torch.empty_like(dev[x]) for x in ("q", "k", "v"))

    def step():
        op.run(dev["q"], dev["k"], dev["v"], dev["o"], dev["do"], dev["m"], dev["l"], dev["cu_q"], dev["cu_kv"],
               inp["scale"], inp["mask"], dq, dk, dv)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    binding.fa_bwd_profile_enable(op.handle, True)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    stages = binding.fa_bwd_profile_collect(op.handle)
    binding.fa_bwd_profile_enable(op.handle, False)
    finite = all(bool(torch.isfinite(x).all()) for x in (dq, dk, dv))
    op.close()
    print(f"[bench] {args.steps} steps: {ms:.4f} ms/step", file=sys.stderr, flush=True)
    shares = kernel_share(algo_used, d, inp["v"].shape[2], layout)
    names = list(shares)
    kern_ms = {n: sum(s[i] for s in stages) / len(stages) for i, n in enumerate(names)}
    step_ms = sorted(sum(s_) for s_ in stages)  # each timed step, first kernel start to last kernel end
    med_ms = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (step_ms[len(step_ms) // 2 - 1] +
                                                                         step_ms[len(step_ms) // 2])
    dom = max(kern_ms, key=kern_ms.get)
    tflops = flops / (ms * 1e-3) / 1e12
    dom_flops = flops * shares[dom]
    achieved = dom_flops / (kern_ms[dom] * 1e-3) / 1e12

    config = {"workload": describe(args.workload, inp),
              "batch": inp["batch"], "heads": heads, "head_dim": d, "seq_len": inp["max_seqlen_q"],
              "total_tokens": tq, "mask": MASK_NAMES[inp["mask"]], "seed": inp["seed"],
              "algorithmic_flops": flops,
              "algorithm": ALGORITHM_NAMES[algo_used],
              "dkdv_layout": LAYOUT_NAMES[layout] + (", dS stored" if algo_used == 7 else ""),
              "schedule": "host longest-first plan" if args.plan else "dense grid"}
    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": config,
        "pct_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "ms_median": round(med_ms, 5), "ms_min": round(step_ms[0], 5),
        "tflops_median": round(flops / (med_ms * 1e-3) / 1e12, 2),
        "kernels_ms": {n: round(v, 5) for n, v in kern_ms.items()},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(dom, args.workload, algo_used), "work_flops": dom_flops,
                     "clock_sustained_ghz": sustained_clock_ghz(dom, args.workload, algo_used, kern_ms[dom])},
        "peak_derived": peak_info,
        "outputs_finite": finite,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"], slices = cpu_baseline(inp, dev, args.cpu_seconds)
        out["parity"] = timed_output_parity(inp, (dq, dk, dv), slices)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
