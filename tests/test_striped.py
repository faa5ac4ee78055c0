"""The Striped layout through the HIP step calls vs the fp64 oracle (needs a GPU).

Device r keeps positions r, r + W, ...; its ring steps are causal blocks in
local indices (ring.striped_key_offset).  The oracle gets the shard's real
positions against the whole natural-order key sequence.  Bars as in
test_parity.py (forward) and test_bwd_parity.py (gradients).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import layouts
from ring_attention_amd import ring, workloads

pytestmark = pytest.mark.gpu

TOL_O = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
TOL_G = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


CASES = [(torch.bfloat16, 128), (torch.float32, 64)]


@pytest.mark.parametrize("dtype,d", CASES, ids=["bf16_d128", "f32_d64"])
@pytest.mark.parametrize("rank", [0, 3])
@pytest.mark.parametrize("fused", [True, False], ids=["fused_merge", "merge_launch"])
def test_striped_forward_steps(gpu, dtype, d, rank, fused):
    W, N = 4, 512
    q, k, v = workloads.make_qkv(1, N, N, 4, 2, d, dtype, seed=300 + rank)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    ks = [ring.stripe(kd, W, r) for r in range(W)]
    vs = [ring.stripe(vd, W, r) for r in range(W)]
    out, lse = ring.striped_forward_steps(ring.stripe(qd, W, rank), ks, vs, W, rank,
                                          fused_merge=fused)
    torch.cuda.synchronize()
    pos = layouts.striped_shard_positions(N, W, rank)
    ro, rl = oracle.attention(q[:, torch.from_numpy(pos)], k, v, causal=True, q_pos=pos)
    err_o = float(np.abs(host(out) - ro).max())
    err_l = float(np.abs(host(lse) - rl).max())
    note(f"striped fwd {dtype} d={d} rank={rank} fused={fused}: max|dO|={err_o:.3e} "
         f"max|dLSE|={err_l:.3e}")
    assert err_o <= TOL_O[dtype] and err_l <= 1e-3


@pytest.mark.parametrize("dtype,d", CASES, ids=["bf16_d128", "f32_d64"])
@pytest.mark.parametrize("rank", [0, 2])
def test_striped_backward_steps(gpu, dtype, d, rank):
    W, N, B, Hq, Hkv = 4, 512, 2, 4, 2
    q, k, v = workloads.make_qkv(B, N, N, Hq, Hkv, d, dtype, seed=320 + rank)
    g = torch.Generator().manual_seed(330 + rank)
    pos = layouts.striped_shard_positions(N, W, rank)
    do = workloads.randn((B, N // W, Hq, d), dtype, g, "cpu")
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    qs = ring.stripe(qd, W, rank)
    ks = [ring.stripe(kd, W, r) for r in range(W)]
    vs = [ring.stripe(vd, W, r) for r in range(W)]
    out, lse = ring.striped_forward_steps(qs, ks, vs, W, rank)
    dq, dk_acc, dv_acc = ring.striped_backward_steps(qs, ks, vs, out.to(dtype), lse,
                                                     do.to(dev), W, rank)
    torch.cuda.synchronize()
    dk = np.zeros((B, N, Hkv, d))
    dv = np.zeros((B, N, Hkv, d))
    for src in range(W):
        dk[:, src::W] = host(dk_acc[src])
        dv[:, src::W] = host(dv_acc[src])
    qsh = q[:, torch.from_numpy(pos)]
    rq, rk, rv, _, _ = oracle.attention_bwd(qsh, k, v, do, causal=True, q_pos=pos)
    for name, a, b in (("dq", host(dq), rq), ("dk", dk, rk), ("dv", dv, rv)):
        err = float(np.abs(a - b).max())
        bar = TOL_G[dtype] * max(1.0, float(np.abs(b).max()))
        note(f"striped bwd {dtype} d={d} rank={rank} {name}: max|err|={err:.3e} "
             f"(bar {bar:.3e})")
        assert err <= bar
