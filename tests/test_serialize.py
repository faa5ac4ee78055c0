"""The 256-row d = 32/64/128 forward kernel under RATTN_SERIALIZE=1 against
its pipelined schedule, bit for bit (needs a GPU).

The serialized schedule keeps one key/value tile in flight, requested and
waited for by every wave right before the phase that reads it, with both wave
groups in lockstep and a workgroup barrier around every phase; each wave does
the same arithmetic in the same order as in the pipelined schedule (a ring of
four direct-to-LDS buffers, two tiles ahead, two wave groups one phase apart).
Equal outputs show that the pipelined schedule reads no LDS buffer before its
DMA has landed and overwrites none that a wave still reads.
"""
import numpy as np
import pytest
import torch

from ring_attention_amd import binding, ring, workloads

pytestmark = pytest.mark.gpu


def both_modes(monkeypatch, fn):
    """fn() with the pipelined schedule, then with the serialized one."""
    monkeypatch.delenv("RATTN_SERIALIZE", raising=False)
    a = fn()
    torch.cuda.synchronize()
    monkeypatch.setenv("RATTN_SERIALIZE", "1")
    b = fn()
    torch.cuda.synchronize()
    monkeypatch.delenv("RATTN_SERIALIZE", raising=False)
    return a, b


def assert_same(a, b, what):
    for x, y in zip(a, b):
        assert torch.equal(x, y), f"{what}: serialized and pipelined schedules differ"


@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (128, torch.float16),
                                     (64, torch.float16), (32, torch.bfloat16)])
@pytest.mark.parametrize("causal", [False, True])
def test_fused_call(gpu, monkeypatch, d, dtype, causal):
    # three query tiles of 256 rows (the last ragged), ragged key tiles, GQA
    N = 2 * 256 + 37
    q, k, v = workloads.make_qkv(2, N, N, 4, 2, d, dtype, seed=d + causal, device=gpu)
    a, b = both_modes(monkeypatch, lambda: binding.fwd(q, k, v, causal=causal))
    assert_same(a, b, f"fwd d={d} {dtype} causal={causal}")


@pytest.mark.parametrize("fused_merge", [True, False])
def test_ring_steps(gpu, monkeypatch, fused_merge):
    """ZigZag ring steps into a float32 running result (merge in the kernel
    epilogue, or separate merges), every device of a 4-device ring."""
    W, N = 4, 2 * 4 * 200
    q, k, v = workloads.make_qkv(1, N, N, 4, 2, 128, torch.bfloat16, seed=7, device=gpu)
    ks = [ring.shard(k, W, True, r) for r in range(W)]
    vs = [ring.shard(v, W, True, r) for r in range(W)]
    for r in range(W):
        qs = ring.shard(q, W, True, r)
        a, b = both_modes(monkeypatch, lambda: ring.ring_forward_steps(
            qs, ks, vs, W, True, r, causal=True, fused_merge=fused_merge))
        assert_same(a, b, f"ring steps rank={r} fused={fused_merge}")


def test_rescaling_and_large_scores(gpu, monkeypatch):
    """Scores that move the running max on every key tile, and q, k ~ N(0, 10^2)."""
    g = torch.Generator().manual_seed(3)
    N, d = 640, 128
    q = torch.zeros(1, N, 2, d)
    q[..., 0] = 1.0
    q[..., 1:] = torch.randn(1, N, 2, d - 1, generator=g) * 0.05
    k = torch.randn(1, N, 1, d, generator=g) * 0.05
    k[0, :, 0, 0] = 0.1 * torch.arange(N, dtype=torch.float32) * d ** 0.5
    v = torch.randn(1, N, 1, d, generator=g)
    qd, kd, vd = (x.to(torch.bfloat16).to(gpu) for x in (q, k, v))
    for causal in (False, True):
        a, b = both_modes(monkeypatch, lambda: binding.fwd(qd, kd, vd, causal=causal))
        assert_same(a, b, f"ramp causal={causal}")
    q2 = (torch.randn(1, 700, 4, d, generator=g) * 10).to(torch.float16).to(gpu)
    k2 = (torch.randn(1, 700, 2, d, generator=g) * 10).to(torch.float16).to(gpu)
    v2 = torch.randn(1, 700, 2, d, generator=g).to(torch.float16).to(gpu)
    a, b = both_modes(monkeypatch, lambda: binding.fwd(q2, k2, v2, causal=True))
    assert_same(a, b, "large scores")


def test_workload3_shape(gpu, monkeypatch):
    """The batched causal workload (B=2, 32 heads, 4096 tokens, fp16): 1024
    work items of every length from 4 to 64 key tiles."""
    w = workloads.workload(3)
    q, k, v = workloads.make_inputs(w, device=gpu)
    a, b = both_modes(monkeypatch, lambda: binding.fwd(q, k, v, causal=True))
    assert_same(a, b, "workload 3")


def test_kv_rows_over_4gb(gpu, monkeypatch):
    """The 64-bit-address DMA form (key/value rows past 4 GB), 256 query rows
    over 1,048,600 keys x 16 heads, one step."""
    Nq, Nk, H, d = 256, 1_048_600, 16, 128
    q, k, v = workloads.make_qkv(1, Nq, Nk, H, H, d, torch.bfloat16, seed=21, device=gpu)
    a, b = both_modes(monkeypatch, lambda: binding.fwd_step(q, k, v, False, [(0, Nq)], [(0, Nk)]))
    assert_same(a, b, "kv rows over 4 GB")
