"""Seeded synthetic inputs for the attention backward.

This module draws the random tensors only (Q, K, V, dO and the sequence
offsets); it holds none of the attention arithmetic, so the fp64 oracle and the
HIP path can both be fed from it. O, m and l are not drawn here: they are the
forward's outputs and come from whatever forward the caller uses.

Recipe (one CPU ``torch.Generator`` per case, seeded with the case's seed):
  1. varlen lengths first, when the case draws them (``torch.randint``);
  2. then Q, K, V, dO in that order as fp32 standard normals of shape [T, H, d]
     (V and dO with the value head dim d_v when it differs);
  3. Q and K are multiplied by ``qk_mult`` (2 sharpens the softmax: logit std
     about 4 at d = 128 with scale 1/sqrt(d));
  4. all four are cast to bf16 (round to nearest even).
Padding rows are part of the same draw (they hold N(0,1) values that the
backward must never read).

The five workloads are the ones the single-pass backward is measured on; the
extra ``sk16_*`` shapes are the d in {64, 128} rows of the PyPTO-Gym SK-16
article's test matrix (§七), run as 8 packed sequences of equal length.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

MASK_NONE = 0
MASK_PADDING = 1
MASK_CAUSAL = 2
MASK_PADDING_CAUSAL = 3


def is_padded_mask(mask: int) -> bool:
    """Padded layouts: each sequence sits in a fixed-length slot (see the C header)."""
    return mask in (MASK_PADDING, MASK_PADDING_CAUSAL)


@dataclass
class Case:
    name: str
    heads: int
    head_dim: int
    mask: int
    seed: int
    seqlens_q: list = field(default_factory=list)   # valid length per sequence
    seqlens_kv: list = field(default_factory=list)
    padded_len: int = 0        # slot length per sequence in padded modes (0 = packed)
    qk_mult: float = 1.0
    draw_lengths: tuple | None = None   # (count, lo, hi_inclusive): draw lengths from the generator
    heads_kv: int = 0          # K/V heads (0 = heads); query head h reads K/V head h // (heads / heads_kv)
    window: int = 0            # > 0: each query i sees only keys (i - window, i]
    head_dim_v: int = 0        # head dim of V and dO (0 = head_dim)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


CASES = {
    "tiny": Case("tiny", heads=1, head_dim=64, mask=MASK_NONE, seed=1, seqlens_q=[128], seqlens_kv=[128]),
    "dense": Case("dense", heads=8, head_dim=128, mask=MASK_NONE, seed=2,
                  seqlens_q=[2048, 2048], seqlens_kv=[2048, 2048]),
    "varlen": Case("varlen", heads=32, head_dim=128, mask=MASK_NONE, seed=3, draw_lengths=(8, 256, 4096)),
    "causal": Case("causal", heads=32, head_dim=128, mask=MASK_CAUSAL, seed=4,
                   seqlens_q=[8192], seqlens_kv=[8192]),
    "longpad": Case("longpad", heads=16, head_dim=128, mask=MASK_PADDING_CAUSAL, seed=5,
                    seqlens_q=[32768, 20000], seqlens_kv=[32768, 20000], padded_len=32768, qk_mult=2.0),
    # d in {64, 128} rows of the SK-16 test matrix (batch, heads, s1, s2, dim)
    "sk16_t01": Case("sk16_t01", heads=8, head_dim=64, mask=MASK_NONE, seed=101, seqlens_q=[320] * 8, seqlens_kv=[320] * 8),
    "sk16_t02": Case("sk16_t02", heads=8, head_dim=64, mask=MASK_NONE, seed=102, seqlens_q=[2432] * 8, seqlens_kv=[2432] * 8),
    "sk16_t05": Case("sk16_t05", heads=8, head_dim=64, mask=MASK_NONE, seed=105, seqlens_q=[32] * 8, seqlens_kv=[32] * 8),
    "sk16_t06": Case("sk16_t06", heads=4, head_dim=128, mask=MASK_NONE, seed=106, seqlens_q=[64] * 8, seqlens_kv=[64] * 8),
}

# the variants of the causal workload that the library also times (grouped K/V heads, a sliding
# window, head dims other than 128); each keeps one 8192-token sequence
CASES.update({
    "causal_gqa": Case("causal_gqa", heads=32, head_dim=128, mask=MASK_CAUSAL, seed=6,
                       seqlens_q=[8192], seqlens_kv=[8192], heads_kv=8),
    "causal_window": Case("causal_window", heads=32, head_dim=128, mask=MASK_CAUSAL, seed=7,
                          seqlens_q=[8192], seqlens_kv=[8192], window=1024),
    "causal_d256": Case("causal_d256", heads=16, head_dim=256, mask=MASK_CAUSAL, seed=8,
                        seqlens_q=[8192], seqlens_kv=[8192]),
    "causal_mla": Case("causal_mla", heads=32, head_dim=192, mask=MASK_CAUSAL, seed=9,
                       seqlens_q=[8192], seqlens_kv=[8192], head_dim_v=128),
})

# workload number -> case name, in the order the five synthetic workloads are listed
WORKLOADS = ["tiny", "dense", "varlen", "causal", "longpad"]
VARIANTS = ["causal_gqa", "causal_window", "causal_d256", "causal_mla"]


def custom_case(name: str, heads: int, head_dim: int, mask: int, seed: int, seqlens_q, seqlens_kv=None,
                padded_len: int = 0, qk_mult: float = 1.0, heads_kv: int = 0, window: int = 0,
                head_dim_v: int = 0) -> Case:
    return Case(name, heads=heads, head_dim=head_dim, mask=mask, seed=seed, seqlens_q=list(seqlens_q),
                seqlens_kv=list(seqlens_q if seqlens_kv is None else seqlens_kv), padded_len=padded_len,
                qk_mult=qk_mult, heads_kv=heads_kv, window=window, head_dim_v=head_dim_v)


def _cumsum(lengths) -> torch.Tensor:
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def make(case: Case | str) -> dict:
    """Draw one case. Returns CPU tensors and sizes:

    q: bf16 [T_q, H, d]; do: bf16 [T_q, H, d_v]; k: bf16 [T_kv, H_kv, d]; v: bf16 [T_kv, H_kv, d_v];
    cu_q, cu_kv: int32 [B+1]; and the ints/floats
    scale, mask, max_seqlen_q, max_seqlen_kv, batch.
    """
    if isinstance(case, str):
        case = CASES[case]
    g = torch.Generator().manual_seed(case.seed)
    lq, lkv = list(case.seqlens_q), list(case.seqlens_kv)
    if case.draw_lengths is not None:
        count, lo, hi = case.draw_lengths
        drawn = torch.randint(lo, hi + 1, (count,), generator=g).tolist()
        lq, lkv = drawn, list(drawn)
    batch = len(lq)
    if case.padded_len:
        tq = tkv = batch * case.padded_len
        msq = mskv = case.padded_len
    else:
        tq, tkv = sum(lq), sum(lkv)
        msq, mskv = max(lq, default=0), max(lkv, default=0)
    h, d = case.heads, case.head_dim
    dv = case.head_dim_v or d
    hkv = case.heads_kv or h
    q = torch.randn((tq, h, d), generator=g, dtype=torch.float32)
    k = torch.randn((tkv, hkv, d), generator=g, dtype=torch.float32)
    v = torch.randn((tkv, hkv, dv), generator=g, dtype=torch.float32)
    do = torch.randn((tq, h, dv), generator=g, dtype=torch.float32)
    if case.qk_mult != 1.0:
        q.mul_(case.qk_mult)
        k.mul_(case.qk_mult)
    return {
        "name": case.name,
        "q": q.to(torch.bfloat16), "k": k.to(torch.bfloat16), "v": v.to(torch.bfloat16),
        "do": do.to(torch.bfloat16),
        "cu_q": _cumsum(lq), "cu_kv": _cumsum(lkv),
        "scale": case.scale, "mask": case.mask, "batch": batch,
        "max_seqlen_q": msq, "max_seqlen_kv": mskv, "seed": case.seed,
        "seqlens_q": lq, "seqlens_kv": lkv, "window": case.window,
    }
