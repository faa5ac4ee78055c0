"""Backward (dQ, dK, dV) of the HIP path vs the fp64 oracle (needs a GPU).

Bar: max |error| <= tol * max(1, max |reference|) per gradient tensor, with
tol = 1e-4 for float32 inputs and 2e-2 for bfloat16/float16 inputs (the
gradients are not bounded by the values the way the forward output is, so
the bar scales with their magnitude).  The oracle computes the gradients of
the definition from q, k, v and dO alone; the HIP path gets the forward's
own (out, lse) as a caller would.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import layouts
from ring_attention_amd import binding, ring, workloads

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.float16: 2e-2, torch.bfloat16: 2e-2}


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare(name, got, ref, dtype, what, rel=None):
    """max |got - ref| <= TOL * max(1, max|ref|); with rel, also
    <= rel * max|ref| (for gradients far below 1, where the first bar says
    little)."""
    got = np.asarray(got, np.float64)
    mref = float(np.abs(ref).max()) if ref.size else 0.0
    scale = max(1.0, mref)
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    tol = TOL[dtype] * scale
    if rel is not None:
        tol = min(tol, rel * mref)
    note(f"{what} {name}: max|err|={err:.3e} (bar {tol:.3e}, max|ref|={mref:.3g})")
    assert np.all(np.isfinite(got)), f"{what}: non-finite {name}"
    assert err <= tol, f"{what}: {name} max|err| {err} > {tol}"


def inputs(B, Nq, N, Hq, Hkv, d, dtype, seed):
    q, k, v = workloads.make_qkv(B, Nq, N, Hq, Hkv, d, dtype, seed=seed)
    g = torch.Generator().manual_seed(seed + 1000)
    do = workloads.randn((B, Nq, Hq, d), dtype, g, "cpu")
    return q, k, v, do


def q_positions(N, W, zigzag, rank):
    return np.arange(N) if rank < 0 else layouts.shard_positions(N, W, rank, zigzag)


def gpu_bwd(q, k, v, do, causal, W=1, zigzag=False, rank=-1):
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    out, lse = binding.fwd(qd, kd, vd, causal=causal, n_ring_steps=W, zigzag=zigzag, rank=rank)
    dq, dk, dv = binding.bwd(qd, kd, vd, out, lse, dod, causal=causal, n_ring_steps=W,
                             zigzag=zigzag, rank=rank)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv)


def check_full(q, k, v, do, causal, W=1, zigzag=False, rank=-1, what=""):
    dq, dk, dv = gpu_bwd(q, k, v, do, causal, W, zigzag, rank)
    rq, rk, rv, _, _ = oracle.attention_bwd(q, k, v, do, causal=causal,
                                            q_pos=q_positions(k.shape[1], W, zigzag, rank))
    for name, a, b in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        compare(name, a, b, q.dtype, what)


DTYPES = [torch.float32, torch.float16, torch.bfloat16]


@pytest.mark.parametrize("dtype", DTYPES, ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_bwd_small_ragged(gpu, dtype, d, causal):
    """Several tiles of every kernel plus a ragged tail (200 rows), GQA 4:2."""
    q, k, v, do = inputs(2, 200, 200, 4, 2, d, dtype, seed=d + (1 if causal else 0))
    what = f"bwd {dtype} d={d} causal={causal}"
    note(f"case {what}")
    check_full(q, k, v, do, causal, what=what)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("zigzag", [False, True], ids=["contig", "zigzag"])
@pytest.mark.parametrize("rank", [-1, 0, 3])
def test_bwd_ring_layouts(gpu, dtype, zigzag, rank):
    W, N = 4, 512
    Nq = N if rank < 0 else N // W
    q, k, v, do = inputs(1, Nq, N, 2, 1, 64, dtype, seed=70 + rank)
    what = f"bwd ring W={W} zigzag={zigzag} rank={rank} {dtype}"
    note(f"case {what}")
    check_full(q, k, v, do, True, W, zigzag, rank, what=what)


def test_bwd_mha_no_gqa_d128_multi_tile(gpu):
    q, k, v, do = inputs(1, 700, 700, 3, 3, 128, torch.bfloat16, seed=90)
    note("case bwd mha d=128 700 rows")
    check_full(q, k, v, do, True, what="bwd mha 700")


def test_bwd_custom_scale(gpu):
    dev = torch.device("cuda:0")
    q, k, v, do = inputs(1, 96, 96, 2, 2, 64, torch.bfloat16, seed=91)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    out, lse = binding.fwd(qd, kd, vd, causal=True, scale=0.3)
    dq, dk, dv = binding.bwd(qd, kd, vd, out, lse, dod, causal=True, scale=0.3)
    torch.cuda.synchronize()
    rq, rk, rv, _, _ = oracle.attention_bwd(q, k, v, do, causal=True, scale=0.3)
    for name, a, b in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        compare(name, host(a), b, q.dtype, "bwd scale 0.3")


def test_bwd_delta_matches_rowsum(gpu):
    dev = torch.device("cuda:0")
    for dtype in DTYPES:
        for d in (16, 32, 64, 128):
            o = workloads.randn((3, 37, 2, d), dtype, torch.Generator().manual_seed(d), "cpu")
            g = workloads.randn((3, 37, 2, d), dtype, torch.Generator().manual_seed(d + 1), "cpu")
            delta = binding.bwd_delta(o.to(dev), g.to(dev))
            torch.cuda.synchronize()
            ref = (o.double() * g.double()).sum(-1).numpy()
            err = np.abs(host(delta) - ref).max()
            assert err <= 1e-5 * max(1.0, np.abs(ref).max()), (dtype, d, err)


# --------------------------------------------------------------------------
# ring steps: the sum of the steps is the whole backward


@pytest.mark.parametrize("zigzag", [False, True], ids=["contig", "zigzag"])
@pytest.mark.parametrize("rank", [0, 1, 3])
def test_bwd_ring_steps_sum_to_whole(gpu, zigzag, rank):
    dev = torch.device("cuda:0")
    W, N, dtype = 4, 512, torch.bfloat16
    q, k, v, do = inputs(2, N // W, N, 4, 2, 128, dtype, seed=100 + rank)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    out, lse = binding.fwd(qd, kd, vd, causal=True, n_ring_steps=W, zigzag=zigzag, rank=rank)
    k_sh = [ring.shard(kd, W, zigzag, r) for r in range(W)]
    v_sh = [ring.shard(vd, W, zigzag, r) for r in range(W)]
    dq, dk_acc, dv_acc = ring.ring_backward_steps(qd, k_sh, v_sh, out, lse, dod, W, zigzag,
                                                  rank, causal=True)
    torch.cuda.synchronize()
    # back to natural key order
    dk = np.zeros((2, N, 2, 128))
    dv = np.zeros((2, N, 2, 128))
    for src in range(W):
        pos = np.concatenate([np.arange(a, a + n) for a, n in ring.shard_rows(N, W, zigzag, src)])
        dk[:, pos] = host(dk_acc[src])
        dv[:, pos] = host(dv_acc[src])
    what = f"bwd ring steps zigzag={zigzag} rank={rank}"
    note(f"case {what}")
    rq, rk, rv, _, _ = oracle.attention_bwd(q, k, v, do, causal=True,
                                            q_pos=q_positions(N, W, zigzag, rank))
    for name, a, b in (("dq", host(dq), rq), ("dk", dk, rk), ("dv", dv, rv)):
        compare(name, a, b, dtype, what)


def test_bwd_step_offsets_and_accumulation(gpu):
    """A step over rows [q_off, q_off+Nq) x [k_off, k_off+Nk) adds exactly its
    pairs: two steps splitting the keys add up to one step over all of them,
    and rows outside the ranges stay untouched."""
    dev = torch.device("cuda:0")
    dtype = torch.float16
    q, k, v, do = inputs(1, 300, 260, 2, 1, 64, dtype, seed=120)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    qpos = np.arange(300) + 40     # queries at 40..339 over keys 0..259
    out32, lse = binding.fwd_step(qd, kd, vd, True, [(40, 300)], [(0, 260)])
    delta = binding.bwd_delta(out32.to(dtype), dod)
    acc = [torch.zeros(t.shape, dtype=torch.float32, device=dev) for t in (qd, kd, vd)]
    for k0, k1 in ((0, 100), (100, 260)):
        binding.bwd_step(qd, kd, vd, dod, lse, delta, *acc, True, [(40, 300)], [(k0, k1 - k0)],
                         q_off=0, Nq=300, k_off=k0, Nk=k1 - k0)
    one = [torch.zeros(t.shape, dtype=torch.float32, device=dev) for t in (qd, kd, vd)]
    binding.bwd_step(qd, kd, vd, dod, lse, delta, *one, True, [(40, 120), (160, 180)],
                     [(0, 260)], q_off=0, Nq=300)
    # a step over query rows 50..149 only
    part = [torch.zeros(t.shape, dtype=torch.float32, device=dev) for t in (qd, kd, vd)]
    binding.bwd_step(qd, kd, vd, dod, lse, delta, *part, True, [(90, 100)], [(0, 260)],
                     q_off=50, Nq=100)
    torch.cuda.synchronize()
    rq, rk, rv, _, _ = oracle.attention_bwd(q, k, v, do, causal=True, q_pos=qpos)
    for name, a, b in zip(("dq", "dk", "dv"), acc, (rq, rk, rv)):
        compare(name, host(a), b, dtype, "two key steps")
    for name, a, b in zip(("dq", "dk", "dv"), one, (rq, rk, rv)):
        compare(name, host(a), b, dtype, "one step, two query runs")
    pq = host(part[0])
    assert np.all(pq[:, :50] == 0) and np.all(pq[:, 150:] == 0)
    compare("dq rows 50..149", pq[:, 50:150], rq[:, 50:150], dtype, "query-range step")
    # dK of the query-range step: the oracle over those query rows only
    lse_s, dl_s = oracle.bwd_stats(q, k, v, do, causal=True, q_pos=qpos)
    sk, sv = oracle.bwd_dkv(q[:, 50:150], k, v, do[:, 50:150], lse_s[:, 50:150],
                            dl_s[:, 50:150], causal=True, q_pos=qpos[50:150])
    compare("dk", host(part[1]), sk, dtype, "query-range step")
    compare("dv", host(part[2]), sv, dtype, "query-range step")


def test_bwd_empty_and_unseen_rows(gpu):
    dev = torch.device("cuda:0")
    q = torch.zeros((1, 0, 2, 64), dtype=torch.bfloat16, device=dev)
    dq, dk, dv = binding.bwd(q, q, q, q, torch.zeros((1, 0, 2), device=dev), q)
    assert dq.numel() == 0
    # queries that precede every key: lse = -inf, no gradient anywhere
    dtype = torch.bfloat16
    q, k, v, do = inputs(1, 64, 64, 1, 1, 64, dtype, seed=130)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    lse = torch.full((1, 64, 1), float("-inf"), device=dev)
    out = torch.zeros_like(qd)
    delta = binding.bwd_delta(out, dod)
    acc = [torch.zeros(t.shape, dtype=torch.float32, device=dev) for t in (qd, kd, vd)]
    binding.bwd_step(qd, kd, vd, dod, lse, delta, *acc, True, [(0, 64)], [(100, 64)])
    torch.cuda.synchronize()
    assert all(float(a.abs().max()) == 0.0 for a in acc)


# --------------------------------------------------------------------------
# the batched causal workload at full size, on sampled rows


def test_bwd_workload3_sampled(gpu):
    w = workloads.workload(3)
    q, k, v = workloads.make_inputs(w)
    g = torch.Generator().manual_seed(3000)
    do = workloads.randn(q.shape, q.dtype, g, "cpu")
    note(f"case bwd {w.name}")
    dq, dk, dv = gpu_bwd(q, k, v, do, True)
    rng = np.random.default_rng(3)
    B, N, H = w.B, w.N, w.Hq
    qrows = np.stack([rng.integers(0, B, 256), rng.integers(0, N, 256),
                      rng.integers(0, H, 256)], 1)
    qrows = np.concatenate([qrows, [[0, 0, 0], [B - 1, N - 1, H - 1], [1, 63, 5]]])
    lse_r, dl_r = oracle.bwd_stats(q, k, v, do, causal=True, rows=qrows)
    lse_all = np.full((B, N, H), np.nan)
    dl_all = np.full((B, N, H), np.nan)
    lse_all[qrows[:, 0], qrows[:, 1], qrows[:, 2]] = lse_r
    dl_all[qrows[:, 0], qrows[:, 1], qrows[:, 2]] = dl_r
    rq = oracle.bwd_dq(q, k, v, do, lse_all, dl_all, causal=True, rows=qrows)
    compare("dq", dq[qrows[:, 0], qrows[:, 1], qrows[:, 2]], rq, q.dtype, w.name)
    # dK, dV rows of two heads: their statistics over every query row
    heads = [(0, 7), (1, 30)]
    allrows = np.array([[b, i, h] for b, h in heads for i in range(N)])
    lse_r, dl_r = oracle.bwd_stats(q, k, v, do, causal=True, rows=allrows)
    lse_all[allrows[:, 0], allrows[:, 1], allrows[:, 2]] = lse_r
    dl_all[allrows[:, 0], allrows[:, 1], allrows[:, 2]] = dl_r
    krows = np.array([[b, j, h] for b, h in heads
                      for j in list(rng.integers(0, N, 48)) + [0, N - 1, 64, 4031]])
    rk, rv = oracle.bwd_dkv(q, k, v, do, lse_all, dl_all, causal=True, rows=krows)
    compare("dk", dk[krows[:, 0], krows[:, 1], krows[:, 2]], rk, q.dtype, w.name)
    compare("dv", dv[krows[:, 0], krows[:, 1], krows[:, 2]], rv, q.dtype, w.name)


# --------------------------------------------------------------------------
# the ZigZag ring share at full size (131072 tokens, rank 2 of 8), sampled


def test_bwd_workload4_sampled(gpu):
    """rattn_bwd and the 8 backward ring steps at the ring share's full size,
    checked on sampled rows: dQ on seeded query rows; dK, dV on key rows near
    the end of chunk 13, whose visible queries are few enough for the oracle
    to sum over (their statistics need every key of each such query).  These
    gradients are far below 1 (each query spreads its weight over ~10^5
    keys), so the bar is also taken relative to their own size: 5e-2 of
    max|ref| (P and dS are rounded to bf16, 2^-8 relative, before their
    products)."""
    w = workloads.workload(4)
    dev = torch.device("cuda:0")
    q, k, v = workloads.make_inputs(w, device=dev)
    g = torch.Generator(device=dev).manual_seed(4000)
    do = workloads.randn(q.shape, q.dtype, g, dev)
    note(f"case bwd {w.name}")
    out, lse = binding.fwd(q, k, v, causal=True, n_ring_steps=w.W, zigzag=True, rank=w.rank)
    dq, dk, dv = binding.bwd(q, k, v, out, lse, do, causal=True, n_ring_steps=w.W, zigzag=True,
                             rank=w.rank)
    ks = [ring.shard(k, w.W, True, r) for r in range(w.W)]
    vs = [ring.shard(v, w.W, True, r) for r in range(w.W)]
    sq, sk_acc, sv_acc = ring.ring_backward_steps(q, ks, vs, out, lse, do, w.W, True, w.rank)
    torch.cuda.synchronize()
    qc, kc, vc, doc = (t.cpu() for t in (q, k, v, do))
    qpos = q_positions(w.N, w.W, True, w.rank)
    H, Nq, c = w.Hq, w.Nq, w.N // (2 * w.W)
    rng = np.random.default_rng(4)
    qrows = np.stack([np.zeros(48, int), rng.integers(0, Nq, 48), rng.integers(0, H, 48)], 1)
    qrows = np.concatenate([qrows, [[0, 0, 0], [0, Nq - 1, H - 1], [0, c - 1, 3], [0, c, 5]]])
    lse_all = np.full((1, Nq, H), np.nan)
    dl_all = np.full((1, Nq, H), np.nan)
    lr, dr = oracle.bwd_stats(qc, kc, vc, doc, causal=True, q_pos=qpos, rows=qrows)
    lse_all[0, qrows[:, 1], qrows[:, 2]] = lr
    dl_all[0, qrows[:, 1], qrows[:, 2]] = dr
    rq = oracle.bwd_dq(qc, kc, vc, doc, lse_all, dl_all, causal=True, q_pos=qpos, rows=qrows)
    compare("dq", host(dq)[0, qrows[:, 1], qrows[:, 2]], rq, q.dtype, w.name, rel=5e-2)
    compare("dq (ring steps)", host(sq)[0, qrows[:, 1], qrows[:, 2]], rq, q.dtype, w.name, rel=5e-2)
    # key rows at positions end-of-chunk-13 - {0, 1, 7, 100}: visible to the
    # few chunk-13 queries at or after them; their statistics on two heads
    end13 = (2 * w.W - 1 - w.rank) * c + c   # one past the last position of chunk 13
    kpos = [end13 - 1, end13 - 2, end13 - 8, end13 - 101]
    heads = [0, 6]
    need_q = [i for i in range(Nq) if qpos[i] >= min(kpos)]
    allrows = np.array([[0, i, h] for h in heads for i in need_q])
    lr, dr = oracle.bwd_stats(qc, kc, vc, doc, causal=True, q_pos=qpos, rows=allrows)
    lse_all[0, allrows[:, 1], allrows[:, 2]] = lr
    dl_all[0, allrows[:, 1], allrows[:, 2]] = dr
    # the other query rows see none of these keys; the oracle skips them by
    # position and never reads their (unset) statistics
    krows = np.array([[0, j, h] for h in heads for j in kpos])
    rk, rv = oracle.bwd_dkv(qc, kc, vc, doc, lse_all, dl_all, causal=True, q_pos=qpos,
                            rows=krows)
    compare("dk", host(dk)[0, krows[:, 1], krows[:, 2]], rk, q.dtype, w.name, rel=5e-2)
    compare("dv", host(dv)[0, krows[:, 1], krows[:, 2]], rv, q.dtype, w.name, rel=5e-2)
    # the ring steps' accumulators hold those rows in the shard of chunk 13's owner
    owner = w.rank  # chunk 2W-1-rank is the back chunk of device `rank`
    rows_in_shard = [c + (j - (end13 - c)) for j in kpos]
    gk = host(sk_acc[owner])[0][rows_in_shard][:, heads]
    gv = host(sv_acc[owner])[0][rows_in_shard][:, heads]
    compare("dk (ring steps)", np.transpose(gk, (1, 0, 2)).reshape(-1, w.d), rk, q.dtype,
            w.name, rel=5e-2)
    compare("dv (ring steps)", np.transpose(gv, (1, 0, 2)).reshape(-1, w.d), rv, q.dtype,
            w.name, rel=5e-2)


@pytest.mark.parametrize("Nk", [1_048_560, 1_048_600],
                         ids=["buffer_offsets_at_limit", "over_4gb_64bit_addresses"])
def test_bwd_kv_rows_at_and_over_4gb(gpu, Nk):
    """One backward ring step whose key/value tensors (Nk rows x 16 heads x
    128 x 2 bytes) fill 0xFFFF0000 bytes exactly -- the largest the backward
    kernels still read through 32-bit buffer offsets -- or exceed 4 GB, where
    they take their 64-bit-address DMA.  Both end in a ragged key tile.
    Non-causal: every query sees all 1M keys, so the gradients are tiny and
    the bar is relative (as for the ring share).  dQ on sampled query rows;
    dK, dV on key rows of one head at the first and last row, byte offset
    2**31, the first row of the last 64-row tile and (over 4 GB) byte offset
    2**32."""
    Nq, H, d = 256, 16, 128
    dev = torch.device("cuda:0")
    note(f"case bwd kv rows Nk={Nk}: generating inputs on the GPU")
    q, k, v = workloads.make_qkv(1, Nq, Nk, H, H, d, torch.bfloat16, seed=22, device=dev)
    assert (Nk * H * d * 2 <= 0xFFFF0000) == (Nk == 1_048_560)
    g = torch.Generator(device=dev).manual_seed(23)
    do = workloads.randn(q.shape, q.dtype, g, dev)
    out, lse = binding.fwd_step(q, k, v, False, [(0, Nq)], [(0, Nk)])  # all keys: final out
    delta = (out * do.float()).sum(-1).contiguous()                    # D = rowsum(dO o O)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=dev)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=dev)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=dev)
    binding.bwd_step(q, k, v, do, lse, delta, dq, dk, dv, False, [(0, Nq)], [(0, Nk)])
    torch.cuda.synchronize()
    head = 4
    krows = np.array([[0, 0, head], [0, Nk - 1, head], [0, 524_288, head],
                      [0, Nk - Nk % 64, head], [0, min(1_048_576, Nk - 30), head]])
    kidx = torch.as_tensor(krows, device=dev)
    gk = dk[kidx[:, 0], kidx[:, 1], kidx[:, 2]].cpu().numpy().astype(np.float64)
    gv = dv[kidx[:, 0], kidx[:, 1], kidx[:, 2]].cpu().numpy().astype(np.float64)
    del dk, dv, out, lse, delta
    qc, kc, vc, doc = (t.cpu() for t in (q, k, v, do))
    qrows = np.array([[0, 0, 0], [0, Nq - 1, H - 1], [0, 77, 9]])
    allrows = np.concatenate([qrows, [[0, i, head] for i in range(Nq)]])
    lse_all = np.full((1, Nq, H), np.nan)
    dl_all = np.full((1, Nq, H), np.nan)
    lr, dr = oracle.bwd_stats(qc, kc, vc, doc, causal=False, rows=allrows)
    lse_all[0, allrows[:, 1], allrows[:, 2]] = lr
    dl_all[0, allrows[:, 1], allrows[:, 2]] = dr
    rq = oracle.bwd_dq(qc, kc, vc, doc, lse_all, dl_all, causal=False, rows=qrows)
    compare("dq", host(dq)[0, qrows[:, 1], qrows[:, 2]], rq, q.dtype, f"kv rows Nk={Nk}",
            rel=5e-2)
    rk, rv = oracle.bwd_dkv(qc, kc, vc, doc, lse_all, dl_all, causal=False, rows=krows)
    compare("dk", gk, rk, q.dtype, f"kv rows Nk={Nk}", rel=5e-2)
    compare("dv", gv, rv, q.dtype, f"kv rows Nk={Nk}", rel=5e-2)
