"""Workload table and seeded synthetic inputs.

This module holds no attention arithmetic: it only names the workloads and
draws their random inputs, so both the HIP-path tests and the oracle can be
fed the same tensors.

Values are N(0, 1) drawn in float32 and rounded to the workload dtype.  The
tiny ring simulation follows the ultralytics.com "Ring Attention" example
(seed 0, 4 devices x 8 tokens, dim 16, q, k, v = randn(3, 32, 16)); every
other workload draws q, then k, then v from a torch.Generator seeded with its
workload number.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    index: int          # 1-based workload number, also its seed
    name: str
    B: int
    Nq: int             # query rows handed to the call
    N: int              # key/value rows (the whole sequence)
    Hq: int
    Hkv: int
    d: int
    dtype: str
    causal: bool
    W: int              # simulated ring size
    zigzag: bool
    rank: int           # -1: all ranks in one launch
    sampled_rows: int   # 0: check every row against the oracle

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]


WORKLOADS = [
    Workload(1, "tiny_ring_sim_4x8_d16_f32", 1, 32, 32, 1, 1, 16, "f32", False, 4, False, -1, 0),
    Workload(2, "single_head_4k_d128_bf16", 1, 4096, 4096, 1, 1, 128, "bf16", False, 1, False,
             -1, 0),
    Workload(3, "mha_causal_b2_h32_4k_d128_f16", 2, 4096, 4096, 32, 32, 128, "f16", True, 1,
             False, -1, 0),
    Workload(4, "zigzag_rank2_of8_131k_h8_d128_bf16", 1, 16384, 131072, 8, 8, 128, "bf16", True,
             8, True, 2, 4096),
    Workload(5, "gqa_causal_512k_h32kv8_d128_bf16", 1, 524288, 524288, 32, 8, 128, "bf16", True,
             8, True, -1, 4096),
]


def workload(i: int) -> Workload:
    return WORKLOADS[i - 1]


def randn(shape, dtype, generator, device):
    """N(0,1) in float32, rounded to `dtype` (round-to-nearest-even)."""
    x = torch.randn(shape, generator=generator, dtype=torch.float32, device=device)
    return x.to(dtype)


def make_qkv(B, Nq, N, Hq, Hkv, d, dtype, seed, device="cpu"):
    """Seeded q [B,Nq,Hq,d], k and v [B,N,Hkv,d]; drawn in that order."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    q = randn((B, Nq, Hq, d), dtype, g, device)
    k = randn((B, N, Hkv, d), dtype, g, device)
    v = randn((B, N, Hkv, d), dtype, g, device)
    return q, k, v


def page_ring_sim_inputs():
    """The ultralytics page's inputs: seed 0, q, k, v = randn(3, 32, 16) (CPU)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(0)
    q, k, v = torch.randn(3, 32, 16, generator=g)
    return q, k, v


def make_inputs(w: Workload, device="cpu"):
    if w.index == 1:
        q, k, v = page_ring_sim_inputs()
        shape = (1, 32, 1, 16)
        return (q.reshape(shape).to(device), k.reshape(shape).to(device),
                v.reshape(shape).to(device))
    return make_qkv(w.B, w.Nq, w.N, w.Hq, w.Hkv, w.d, w.torch_dtype, w.index, device)


def sample_rows(B, Nq, Hq, n, seed, forced=()):
    """n distinct (b, i, h) rows drawn with numpy default_rng(seed), plus the
    forced (b, i, h) triples; returned sorted as an (m, 3) int64 array."""
    rng = np.random.default_rng(seed)
    total = B * Nq * Hq
    n = min(n, total)
    flat = rng.choice(total, size=n, replace=False)
    rows = np.stack([flat // (Nq * Hq), (flat // Hq) % Nq, flat % Hq], axis=1)
    if len(forced):
        rows = np.concatenate([rows, np.asarray(forced, dtype=np.int64).reshape(-1, 3)])
    rows = np.unique(rows.astype(np.int64), axis=0)
    return rows
