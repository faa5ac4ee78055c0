"""rattn_fwd_queued (query tiles handed out from per-XCD queues) against
rattn_fwd and the fp64 oracle (needs a GPU).

Every work item is computed by the same code in both launches, so the queued
results must equal rattn_fwd's bit for bit; sampled rows are also checked
against the oracle with the bars of the parity tests (max |dO| <= 2e-2 for
16-bit inputs, |dLSE| <= 1e-3).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import layouts
from ring_attention_amd import binding, workloads

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def same(a, b):
    return torch.equal(a, b)


def oracle_rows(q, k, v, out, lse, rows, qpos, causal, what):
    """Sampled (batch, row, head) triples against the oracle."""
    ridx = torch.as_tensor(rows, device=q.device)
    o = out[ridx[:, 0], ridx[:, 1], ridx[:, 2]].float().cpu().numpy().astype(np.float64)
    l = lse[ridx[:, 0], ridx[:, 1], ridx[:, 2]].cpu().numpy().astype(np.float64)
    Hq, Hkv, d = q.shape[2], k.shape[2], q.shape[3]
    group = Hq // Hkv
    ref_o = np.zeros((len(rows), d))
    ref_l = np.zeros(len(rows))
    for i, (b, r, h) in enumerate(rows):
        qi = q[b:b + 1, r:r + 1, h:h + 1].cpu().contiguous()
        kh = k[b:b + 1, :, h // group:h // group + 1].cpu().contiguous()
        vh = v[b:b + 1, :, h // group:h // group + 1].cpu().contiguous()
        ro, rl = oracle.attention(qi, kh, vh, causal=causal, q_pos=np.array([qpos[r]]))
        ref_o[i], ref_l[i] = ro[0, 0, 0], rl[0, 0, 0]
    err_o = np.max(np.abs(o - ref_o))
    fin = ~(np.isneginf(l) & np.isneginf(ref_l))
    err_l = np.max(np.abs(l[fin] - ref_l[fin])) if fin.any() else 0.0
    note(f"{what}: oracle rows {len(rows)} max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
    assert np.all(np.isfinite(o)) and err_o <= 2e-2 and err_l <= 1e-3


def rows_of(B, Nq, Hq, n, seed):
    rng = np.random.default_rng(seed)
    rows = np.stack([rng.integers(0, B, n), rng.integers(0, Nq, n), rng.integers(0, Hq, n)], 1)
    edge = np.array([[0, 0, 0], [B - 1, Nq - 1, Hq - 1], [0, Nq - 1, 0], [B - 1, 0, Hq - 1]])
    return np.concatenate([rows, edge])


CASES = [
    # name, B, N, Hq, Hkv, dtype, causal, W, zigzag  (all with >= 1024 query tiles of 256 rows)
    ("mha_causal_b2_h32_4k_f16", 2, 4096, 32, 32, torch.float16, True, 1, False),
    ("gqa_causal_zigzag8_16k_h32kv8_bf16", 1, 16384, 32, 8, torch.bfloat16, True, 8, True),
    ("noncausal_32k_h8_bf16", 1, 32768, 8, 8, torch.bfloat16, False, 1, False),
    ("causal_contiguous4_ragged_b3_h12_f16", 3, 12000, 12, 4, torch.float16, True, 4, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_queued_equals_fwd(gpu, case):
    name, B, N, Hq, Hkv, dtype, causal, W, zigzag = case
    note(f"case queued {name}")
    q, k, v = workloads.make_qkv(B, N, N, Hq, Hkv, 128, dtype, seed=31, device=gpu)
    ref_o, ref_l = binding.fwd(q, k, v, causal=causal, n_ring_steps=W, zigzag=zigzag, rank=-1)
    ws = binding.queue_workspace(gpu)
    for call in range(2):  # the second call reuses the workspace its predecessor left
        out, lse = binding.fwd_queued(q, k, v, causal=causal, n_ring_steps=W, zigzag=zigzag,
                                      rank=-1, queue_ws=ws)
        torch.cuda.synchronize()
        assert same(out, ref_o) and same(lse, ref_l), f"{name}: call {call} differs from rattn_fwd"
    oracle_rows(q, k, v, out, lse, rows_of(B, N, Hq, 24, seed=5), np.arange(N), causal, name)


def test_queued_workspace_contents_do_not_matter(gpu):
    note("case queued workspace garbage")
    q, k, v = workloads.make_qkv(2, 4096, 4096, 32, 32, 128, torch.bfloat16, seed=32, device=gpu)
    ref_o, ref_l = binding.fwd(q, k, v, causal=True)
    for fill in (0x7fffffff, -1, 12345):
        ws = torch.full((binding.QUEUE_WS_BYTES // 4,), fill, dtype=torch.int32, device=gpu)
        out, lse = binding.fwd_queued(q, k, v, causal=True, queue_ws=ws)
        torch.cuda.synchronize()
        assert same(out, ref_o) and same(lse, ref_l), f"workspace filled with {fill}"


@pytest.mark.parametrize("d,dtype,B,N,H", [(128, torch.bfloat16, 1, 1000, 4),
                                           (64, torch.float16, 2, 4096, 32),
                                           (32, torch.bfloat16, 1, 2048, 8),
                                           (16, torch.float16, 1, 512, 2),
                                           (64, torch.float32, 1, 256, 2)])
def test_queued_small_or_other_d_runs_as_fwd(gpu, d, dtype, B, N, H):
    """Calls below the queue threshold, and d != 128, run the plain launch."""
    note(f"case queued fallback d={d} {dtype} N={N}")
    q, k, v = workloads.make_qkv(B, N, N, H, H, d, dtype, seed=33, device=gpu)
    ref_o, ref_l = binding.fwd(q, k, v, causal=True, n_ring_steps=2, zigzag=False, rank=-1)
    out, lse = binding.fwd_queued(q, k, v, causal=True, n_ring_steps=2, zigzag=False, rank=-1)
    torch.cuda.synchronize()
    assert same(out, ref_o) and same(lse, ref_l)


def test_queued_rank_shard(gpu):
    """One device's ZigZag shard (rank = 5 of 8): 2 x 2048 query rows."""
    note("case queued rank shard")
    B, N, Hq, Hkv, W, rank = 1, 32768, 32, 8, 8, 5
    q_all, k, v = workloads.make_qkv(B, N, N, Hq, Hkv, 128, torch.bfloat16, seed=34, device=gpu)
    pos = layouts.zigzag_shard_positions(N, W, rank)
    q = q_all[:, torch.as_tensor(pos, device=gpu)].contiguous()
    ref_o, ref_l = binding.fwd(q, k, v, causal=True, n_ring_steps=W, zigzag=True, rank=rank)
    out, lse = binding.fwd_queued(q, k, v, causal=True, n_ring_steps=W, zigzag=True, rank=rank)
    torch.cuda.synchronize()
    assert same(out, ref_o) and same(lse, ref_l)
    oracle_rows(q, k, v, out, lse, rows_of(B, q.shape[1], Hq, 16, seed=6), pos, True,
                "queued rank shard")


def test_queued_kv_over_4gb(gpu):
    """The queued kernel's 64-bit-address DMA form: key/value rows of 16
    heads past 4 GB (N = 32 x 32769 rows, 4.295e9 bytes each for k and v),
    one contiguous ring rank's 32769 query rows (2064 work items, ragged last
    tile), causal.  Equal to rattn_fwd bit for bit; sampled rows against the
    oracle."""
    W, rank, H, d = 32, 5, 16, 128
    N = W * 32769
    assert N * H * d * 2 > 0xFFFF0000
    note("case queued kv over 4 GB: generating inputs on the GPU")
    q_all, k, v = workloads.make_qkv(1, 32769, N, H, H, d, torch.bfloat16, seed=35, device=gpu)
    q = q_all.contiguous()
    ref_o, ref_l = binding.fwd(q, k, v, causal=True, n_ring_steps=W, zigzag=False, rank=rank)
    out, lse = binding.fwd_queued(q, k, v, causal=True, n_ring_steps=W, zigzag=False, rank=rank)
    torch.cuda.synchronize()
    assert same(out, ref_o) and same(lse, ref_l)
    pos = np.arange(rank * 32769, (rank + 1) * 32769)
    oracle_rows(q, k, v, out, lse, rows_of(1, 32769, H, 6, seed=7), pos, True,
                "queued kv over 4 GB")
