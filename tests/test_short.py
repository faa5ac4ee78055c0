"""The key-split forward (fwd_short.hip; 16-bit, d = 128, 64, 32) vs the fp64
oracle (needs a GPU).

Launches whose 256-row work items would occupy at most half of the compute
units (a single head of 4096 queries: 16 items) run on a kernel that gives
each workgroup 32 query rows and divides their key tiles among its 8 waves,
whose partial results are merged in LDS by the log-sum-exp rule.  rattn_fwd
and the ring-step calls choose it by themselves ("auto"); RATTN_FWD_SHORT=1
sends every eligible launch to it, which these tests use to run it on the
same cases as the 256-row kernel: ragged query and key tails, waves left
without key tiles, GQA, ring layouts and steps with fused and separate
merges, large scores, the running-max thresholds, and key/value tensors at
and past 4 GB (both DMA address forms).

Tolerances as for every 16-bit case: max |dO| <= 2e-2, |dLSE| <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import test_parity as tp
import test_rescale_edges as tre
from ring_attention_amd import binding, workloads

pytestmark = pytest.mark.gpu


@pytest.mark.fwd_short("auto")
def test_workload2_single_head_auto(gpu):
    """Single head, 4096 queries and keys, bf16, non-causal: chosen by itself."""
    w = workloads.workload(2)
    q, k, v = workloads.make_inputs(w)
    tp.note(f"case {w.name} (key-split kernel, automatic)")
    tp.run_full_check(q, k, v, w.causal, w.W, w.zigzag, w.rank, w.name + " short")


@pytest.mark.fwd_short("auto")
def test_single_head_causal_auto(gpu):
    q, k, v = workloads.make_qkv(1, 4096, 4096, 1, 1, 128, torch.bfloat16, seed=81)
    tp.note("case single head causal 4096 (key-split kernel, automatic)")
    tp.run_full_check(q, k, v, True, 1, False, -1, "single head causal 4096 short")


# (B, N, Hq, Hkv): N = 1 and 31 leave most waves without a key tile; 100 gives
# 4 tiles for 8 waves; 1000 ends on a ragged query tile and a ragged key tile
SHAPES = [(1, 1, 1, 1), (1, 31, 2, 2), (1, 33, 2, 1), (1, 100, 1, 1), (1, 64, 3, 3),
          (2, 1000, 4, 2), (1, 1500, 8, 2)]


@pytest.mark.fwd_short("1")
@pytest.mark.parametrize("B,N,Hq,Hkv", SHAPES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("causal", [False, True])
def test_shapes(gpu, B, N, Hq, Hkv, dtype, causal):
    q, k, v = workloads.make_qkv(B, N, N, Hq, Hkv, 128, dtype, seed=N + 7 * Hq + causal)
    tp.run_full_check(q, k, v, causal, 1, False, -1,
                      f"short B={B} N={N} H={Hq}/{Hkv} {dtype} causal={causal}")


# d = 64 and 32: the same kernel with narrower rows (other swizzles, 4 or 2
# DMA requests per K or V tile, fewer MFMA steps)
SHAPES_SMALL_D = [(1, 1, 1, 1), (1, 33, 2, 1), (1, 100, 1, 1), (2, 1000, 4, 2), (1, 1500, 8, 2)]


@pytest.mark.fwd_short("1")
@pytest.mark.parametrize("B,N,Hq,Hkv", SHAPES_SMALL_D)
@pytest.mark.parametrize("d", [64, 32])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("causal", [False, True])
def test_shapes_small_d(gpu, B, N, Hq, Hkv, d, dtype, causal):
    q, k, v = workloads.make_qkv(B, N, N, Hq, Hkv, d, dtype, seed=N + 3 * d + causal)
    tp.run_full_check(q, k, v, causal, 1, False, -1,
                      f"short d={d} B={B} N={N} H={Hq}/{Hkv} {dtype} causal={causal}")


@pytest.mark.fwd_short("1")
@pytest.mark.parametrize("d", [64, 32])
def test_small_d_steps_and_rescaling(gpu, d):
    """Ring steps (fused and separate merges), large scores and the running-max
    thresholds at d = 64 and 32."""
    tp.test_ring_steps_batched_read_shards_in_place(gpu, torch.float16, d, True)
    tp.test_ring_steps_batched_read_shards_in_place(gpu, torch.bfloat16, d, False)
    for dtype in (torch.bfloat16, torch.float16):
        tre.test_large_magnitude_scores(gpu, dtype, d)
        tre.test_max_moves_every_key_tile(gpu, dtype, d)
        tre.test_thresholds_of_lazy_rescaling(gpu, dtype, d)


@pytest.mark.fwd_short("1")
@pytest.mark.parametrize("W,zigzag", [(3, False), (4, True)])
def test_ring_layouts(gpu, W, zigzag):
    N = 2 * W * 72 if zigzag else W * 150
    q, k, v = workloads.make_qkv(1, N, N, 4, 2, 128, torch.bfloat16, seed=90 + W)
    tp.run_full_check(q, k, v, True, W, zigzag, -1, f"short W={W} zigzag={zigzag} all ranks")
    from ring_attention_amd import ring
    for r in range(W):
        qs = ring.shard(q, W, zigzag, r)
        tp.run_full_check(qs, k, v, True, W, zigzag, r, f"short W={W} zigzag={zigzag} rank={r}")


@pytest.mark.fwd_short("1")
@pytest.mark.parametrize("fused_merge", [True, False])
@pytest.mark.parametrize("W,zigzag", [(2, False), (4, True)])
def test_ring_steps(gpu, W, zigzag, fused_merge):
    """Ring steps into a float32 running result: the kernel's merge epilogue
    (fused) and its plain partial output followed by rattn_merge."""
    tp.test_ring_steps_equal_oracle(gpu, W, zigzag, fused_merge)


@pytest.mark.fwd_short("1")
def test_steps_offsets_and_empty_rows(gpu):
    tp.test_d128_step_offset_diagonal(gpu)
    tp.test_d128_step_query_tiles_without_keys(gpu)
    tp.test_step_two_key_segments(gpu)
    tp.test_step_row_offsets_match_copies(gpu)


@pytest.mark.fwd_short("1")
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_large_scores_and_max_thresholds(gpu, dtype):
    tre.test_large_magnitude_scores(gpu, dtype, 128)
    tre.test_max_moves_every_key_tile(gpu, dtype, 128)
    tre.test_thresholds_of_lazy_rescaling(gpu, dtype, 128)


@pytest.mark.fwd_short("1")
def test_tile_sums_at_the_slow_path_bound(gpu):
    """This kernel's lanes hold 16 keys of a 32-key tile: tiles of equal p
    whose lane sums are 127, 128 and 129 (the exact-max bound is 128), and
    64 and 200, after a first tile of p = 1 (base-2 score 0)."""
    g = torch.Generator().manual_seed(65)
    J = [np.zeros(32)]
    for target in (127.0, 128.0, 129.0, 64.0, 200.0):
        J.append(np.full(32, math.log2(target / 16.0)))
    J = np.concatenate(J)
    N, d = J.size, 128
    q = torch.zeros(1, N, 2, d)
    q[..., 0] = 1.0
    k = torch.zeros(1, N, 1, d)
    k[0, :, 0, 0] = torch.from_numpy(16.0 * J).float()
    k[..., 1:] = torch.randn(1, N, 1, d - 1, generator=g)
    v = torch.randn(1, N, 1, d, generator=g)
    for dtype in (torch.bfloat16, torch.float16):
        tre.run_all_paths(q.to(dtype), k.to(dtype), v.to(dtype), tre.LN2 / 16,
                          f"short tile sums {dtype}")


@pytest.mark.fwd_short("1")
@pytest.mark.parametrize("Nk", tp.BIG_NK)
def test_kv_rows_at_and_over_4gb(gpu, Nk):
    """256 query rows over 1M keys x 16 heads: the buffer-form DMA at its
    limit and the 64-bit-address form past 4 GB, on planted dominant keys."""
    tp.test_kv_rows_at_and_over_4gb(gpu, Nk)


@pytest.mark.fwd_short("auto")
def test_auto_choice_matches_forced(gpu):
    """The automatic choice for a small launch gives what forcing the key-split
    kernel gives, bit for bit (same kernel), and both match the oracle."""
    import os
    q, k, v = workloads.make_qkv(1, 2048, 2048, 2, 1, 128, torch.bfloat16, seed=95, device=gpu)
    a_o, a_l = binding.fwd(q, k, v, causal=True)
    os.environ["RATTN_FWD_SHORT"] = "1"
    try:
        f_o, f_l = binding.fwd(q, k, v, causal=True)
    finally:
        del os.environ["RATTN_FWD_SHORT"]
    torch.cuda.synchronize()
    assert torch.equal(a_o, f_o) and torch.equal(a_l, f_l)
    ref_o, ref_l = oracle.attention(q.cpu(), k.cpu(), v.cpu(), causal=True)
    tp.compare(tp.host(a_o), tp.host(a_l), ref_o, ref_l, torch.bfloat16, what="auto 2048 causal")


@pytest.mark.fwd_short("auto")
def test_queued_small_launch_matches_fwd(gpu):
    """rattn_fwd_queued on a launch this small takes the same kernel as
    rattn_fwd (the queues serve only large launches): equal bit for bit."""
    q, k, v = workloads.make_qkv(1, 4096, 4096, 2, 2, 128, torch.bfloat16, seed=96, device=gpu)
    ws = binding.queue_workspace(gpu)
    a_o, a_l = binding.fwd(q, k, v, causal=True)
    b_o, b_l = binding.fwd_queued(q, k, v, causal=True, queue_ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(a_o, b_o) and torch.equal(a_l, b_l)


# split-KV on the key-split kernel: each split of a 32-row query tile is one
# workgroup (its 8 waves divide the split's key tiles), partials in the
# workspace, then the n-way log-sum-exp combine


@pytest.mark.fwd_short("1")
@pytest.mark.parametrize("d", [128, 64, 32])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n_splits", [2, 3, 8])
def test_split_kv(gpu, d, causal, n_splits):
    q, k, v = workloads.make_qkv(2, 1000, 1000, 4, 2, d, torch.bfloat16, seed=d + n_splits)
    tp.run_split_check(q, k, v, causal, 1, False, -1, n_splits,
                       f"short split d={d} causal={causal} n={n_splits}")


@pytest.mark.fwd_short("1")
@pytest.mark.parametrize("W,zigzag,rank", [(4, True, 1), (4, True, -1), (3, False, 2)])
def test_split_kv_ring_layouts(gpu, W, zigzag, rank):
    N = 2 * W * 100 if zigzag else W * 160
    q, k, v = workloads.make_qkv(1, N, N, 2, 1, 128, torch.float16, seed=W + rank)
    if rank >= 0:
        from ring_attention_amd import ring
        q = ring.shard(q, W, zigzag, rank)
    tp.run_split_check(q, k, v, True, W, zigzag, rank, 3,
                       f"short split W={W} zigzag={zigzag} rank={rank}")


@pytest.mark.fwd_short("auto")
def test_split_kv_workload2_auto(gpu):
    """Workload 2 with the split count the hint gives for the key-split
    kernel (2 on a 256-CU GPU), against the oracle; the allocation-free entry
    point gives the same bits."""
    w = workloads.workload(2)
    q, k, v = workloads.make_inputs(w)
    ns = binding.split_hint(q.to(gpu), k.to(gpu))
    tp.note(f"case {w.name}: key-split kernel with {ns} splits")
    assert ns >= 1
    tp.run_split_check(q, k, v, False, 1, False, -1, ns, w.name + f" short split {ns}")
    qd, kd, vd = q.to(gpu), k.to(gpu), v.to(gpu)
    a_o, a_l = binding.fwd_split(qd, kd, vd, n_splits=ns)
    b_o, b_l = binding.fwd_split_noalloc(qd, kd, vd, n_splits=ns)
    torch.cuda.synchronize()
    assert torch.equal(a_o, b_o) and torch.equal(a_l, b_l)
