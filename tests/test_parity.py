"""HIP path vs the fp64 oracle on identical seeded inputs (needs a GPU).

Tolerances (stated for this method): max |dO| <= 1e-5 for float32 inputs and
<= 2e-2 for bfloat16/float16 inputs, |dLSE| <= 1e-3.  Small workloads compare
every output element; the long workloads compare seeded sampled rows plus
forced edge rows (the first and last row of every chunk, the first and last
position).
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import layouts
from ring_attention_amd import binding, ring, workloads

pytestmark = pytest.mark.gpu

TOL_O = {torch.float32: 1e-5, torch.float16: 2e-2, torch.bfloat16: 2e-2}
TOL_LSE = 1e-3


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def compare(out, lse, ref_o, ref_l, dtype, tol_o=None, what=""):
    out = np.asarray(out, np.float64)
    lse = np.asarray(lse, np.float64)
    tol_o = TOL_O[dtype] if tol_o is None else tol_o
    both_empty = np.isneginf(lse) & np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref_l)), f"{what}: empty rows differ"
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err_o = np.max(np.abs(out - ref_o)) if out.size else 0.0
    fin = ~both_empty
    err_l = np.max(np.abs(lse[fin] - ref_l[fin])) if fin.any() else 0.0
    note(f"{what}: max|dO|={err_o:.3e} (tol {tol_o:g}) max|dLSE|={err_l:.3e}")
    assert err_o <= tol_o, f"{what}: max|dO| {err_o} > {tol_o}"
    assert err_l <= TOL_LSE, f"{what}: max|dLSE| {err_l} > {TOL_LSE}"
    return err_o, err_l


def host(t):
    return t.detach().float().cpu().numpy() if t.dtype != torch.float32 else t.detach().cpu().numpy()


def q_positions(N, W, zigzag, rank):
    return np.arange(N) if rank < 0 else layouts.shard_positions(N, W, rank, zigzag)


def run_full_check(q, k, v, causal, W, zigzag, rank, what, tol_o=None):
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out, lse = binding.fwd(qd, kd, vd, causal=causal, n_ring_steps=W, zigzag=zigzag, rank=rank)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention(q, k, v, causal=causal,
                                    q_pos=q_positions(k.shape[1], W, zigzag, rank))
    return compare(host(out), host(lse), ref_o, ref_l, q.dtype, tol_o, what)


# --------------------------------------------------------------------------
# the five workloads


def test_workload1_tiny_ring_simulation(gpu):
    w = workloads.workload(1)
    q, k, v = workloads.make_inputs(w)
    note(f"case {w.name}")
    run_full_check(q, k, v, w.causal, w.W, w.zigzag, w.rank, w.name)


def test_workload2_single_head(gpu):
    w = workloads.workload(2)
    q, k, v = workloads.make_inputs(w)
    note(f"case {w.name}")
    run_full_check(q, k, v, w.causal, w.W, w.zigzag, w.rank, w.name)


def test_workload3_batched_multihead_causal(gpu):
    w = workloads.workload(3)
    q, k, v = workloads.make_inputs(w)
    note(f"case {w.name}")
    run_full_check(q, k, v, w.causal, w.W, w.zigzag, w.rank, w.name)


def forced_rows_zigzag(w, c):
    """First/last row of every chunk the query tensor holds, first/last head."""
    idx = set()
    for start in range(0, w.Nq, c):
        idx.update({start, start + c - 1})
    idx.update({0, w.Nq - 1})
    return [(0, i, h) for i in sorted(idx) for h in (0, w.Hq - 1)]


def sampled_rows(w):
    c = w.N // (2 * w.W)
    rows = workloads.sample_rows(w.B, w.Nq, w.Hq, w.sampled_rows, seed=100 + w.index,
                                 forced=forced_rows_zigzag(w, c))
    # group rows of one key/value head, in position order, so concurrent oracle
    # threads stream the same keys
    order = np.lexsort((rows[:, 1], rows[:, 2] // (w.Hq // w.Hkv), rows[:, 0]))
    return rows[order]


def check_sampled(out, lse, q_host, k_host, v_host, rows, qpos, w, what):
    o = out[rows[:, 0], rows[:, 1], rows[:, 2]]
    l = lse[rows[:, 0], rows[:, 1], rows[:, 2]]
    ref_o, ref_l = oracle.attention(q_host, k_host, v_host, causal=w.causal, q_pos=qpos,
                                    rows=rows)
    return compare(host(o), host(l), ref_o, ref_l, q_host.dtype, what=what)


@pytest.fixture(scope="module")
def workload4_inputs(gpu):
    w = workloads.workload(4)
    q, k, v = workloads.make_inputs(w, device=gpu)
    return w, q, k, v


def test_workload4_fused(workload4_inputs):
    w, q, k, v = workload4_inputs
    note(f"case {w.name} fused")
    out, lse = binding.fwd(q, k, v, causal=True, n_ring_steps=w.W, zigzag=True, rank=w.rank)
    torch.cuda.synchronize()
    rows = sampled_rows(w)
    check_sampled(out.cpu(), lse.cpu(), q.cpu(), k.cpu(), v.cpu(), rows,
                  layouts.zigzag_shard_positions(w.N, w.W, w.rank), w, w.name + " fused")


def test_workload4_ring_steps_and_merge(workload4_inputs):
    w, q, k, v = workload4_inputs
    note(f"case {w.name} steps+merge")
    ks = [ring.shard(k, w.W, True, r) for r in range(w.W)]
    vs = [ring.shard(v, w.W, True, r) for r in range(w.W)]
    out, lse = ring.ring_forward_steps(q, ks, vs, w.W, True, w.rank, causal=True)
    torch.cuda.synchronize()
    rows = sampled_rows(w)
    check_sampled(out.cpu(), lse.cpu(), q.cpu(), k.cpu(), v.cpu(), rows,
                  layouts.zigzag_shard_positions(w.N, w.W, w.rank), w, w.name + " steps")
    # merges as their own launches: the same result up to rounding order
    so, sl = ring.ring_forward_steps(q, ks, vs, w.W, True, w.rank, causal=True,
                                     fused_merge=False)
    torch.cuda.synchronize()
    assert (so - out).abs().max().item() <= 1e-5 and (sl - lse).abs().max().item() <= 1e-5
    # fused and step-by-step agree closely on every row
    fo, fl = binding.fwd(q, k, v, causal=True, n_ring_steps=w.W, zigzag=True, rank=w.rank)
    torch.cuda.synchronize()
    d_o = (fo.float() - out).abs().max().item()
    d_l = (fl - lse).abs().max().item()
    note(f"fused vs steps: max|dO|={d_o:.3e} max|dLSE|={d_l:.3e}")
    assert d_o <= 2e-2 and d_l <= 1e-3


def test_workload5_long_context_gqa(gpu):
    w = workloads.workload(5)
    note(f"case {w.name}: generating inputs on the GPU")
    q, k, v = workloads.make_inputs(w, device=gpu)
    out, lse = binding.fwd(q, k, v, causal=True, n_ring_steps=w.W, zigzag=True, rank=-1)
    torch.cuda.synchronize()
    rows = sampled_rows(w)
    ridx = torch.as_tensor(rows, device=gpu)
    o = out[ridx[:, 0], ridx[:, 1], ridx[:, 2]].cpu()
    l = lse[ridx[:, 0], ridx[:, 1], ridx[:, 2]].cpu()
    q_sel = q[ridx[:, 0], ridx[:, 1], ridx[:, 2]].cpu()  # [n, d]
    del out, lse, q
    note(f"{w.name}: oracle on {len(rows)} rows")
    k_host, v_host = k.cpu(), v.cpu()
    group = w.Hq // w.Hkv
    ref_o = np.zeros((len(rows), w.d))
    ref_l = np.zeros(len(rows))
    for g in range(w.Hkv):
        sel = np.nonzero(rows[:, 2] // group == g)[0]
        if len(sel) == 0:
            continue
        qg = q_sel[sel].reshape(1, len(sel), 1, w.d).contiguous()
        kg = k_host[:, :, g:g + 1].contiguous()
        vg = v_host[:, :, g:g + 1].contiguous()
        ro, rl = oracle.attention(qg, kg, vg, causal=True, q_pos=rows[sel, 1])
        ref_o[sel] = ro[0, :, 0]
        ref_l[sel] = rl[0, :, 0]
    compare(host(o), host(l), ref_o, ref_l, torch.bfloat16, what=w.name)


# Key/value rows of 16 heads x 128 x 2 bytes.  1,048,560 rows fill
# 0xFFFF0000 bytes exactly: the largest tensor the d = 128 kernel still reads
# through 32-bit buffer offsets.  1,048,600 rows (4.29 GB + 160 KB) take its
# 64-bit-address DMA.  Both end in a ragged key tile (48 and 24 rows).
BIG_NK = [pytest.param(1_048_560, id="buffer_offsets_at_limit"),
          pytest.param(1_048_600, id="over_4gb_64bit_addresses")]


def far_key_spikes(Nk):
    """(query row, head, key row) triples: the key row gets the query's own
    direction, scaled to a score of 18, so that it carries about 97% of that
    row's softmax weight against 1M N(0,1) keys.  An output that read the
    wrong bytes for that key row then misses by O(1).  The rows sit where
    address arithmetic can break: the last row of the last head (the largest
    offset), byte offset 2**31 and 2**32 of head 0 and head 8 (the latter
    clamped into the tensor), the first row of the ragged last tile, and row 0."""
    return np.array([(0, 15, Nk - 1), (255, 0, 524_288), (31, 8, min(1_048_576, Nk - 30)),
                     (100, 7, Nk - Nk % 64), (32, 3, 0)])


@pytest.mark.parametrize("Nk", BIG_NK)
def test_kv_rows_at_and_over_4gb(gpu, Nk):
    # One ring step, non-causal: each of 256 query rows sees all 1M keys;
    # checked on the spiked (row, head) pairs, each against the oracle.
    Nq, H, d = 256, 16, 128
    note(f"case kv rows Nk={Nk}: generating inputs on the GPU")
    q, k, v = workloads.make_qkv(1, Nq, Nk, H, H, d, torch.bfloat16, seed=21, device=gpu)
    assert (Nk * H * d * 2 <= 0xFFFF0000) == (Nk == 1_048_560)
    spikes = far_key_spikes(Nk)
    for r, h, kp in spikes:
        qr = q[0, r, h].float()
        k[0, kp, h] = (qr * (18.0 * d ** 0.5 / float(qr @ qr))).to(k.dtype)
    out, lse = binding.fwd_step(q, k, v, False, [(0, Nq)], [(0, Nk)])
    torch.cuda.synchronize()
    ridx = torch.as_tensor(np.stack([np.zeros(len(spikes), np.int64), spikes[:, 0],
                                     spikes[:, 1]], 1), device=gpu)
    o = out[ridx[:, 0], ridx[:, 1], ridx[:, 2]].cpu().numpy().astype(np.float64)
    l = lse[ridx[:, 0], ridx[:, 1], ridx[:, 2]].cpu().numpy().astype(np.float64)
    q_sel = q[ridx[:, 0], ridx[:, 1], ridx[:, 2]].cpu()
    del out, lse, q
    ref_o = np.zeros((len(spikes), d))
    ref_l = np.zeros(len(spikes))
    for i, (_, h, kp) in enumerate(spikes):
        kh = k[:, :, h:h + 1].cpu().contiguous()
        vh = v[:, :, h:h + 1].cpu().contiguous()
        ro, rl = oracle.attention(q_sel[i].reshape(1, 1, 1, d).contiguous(), kh, vh,
                                  causal=False)
        ref_o[i] = ro[0, 0, 0]
        ref_l[i] = rl[0, 0, 0]
        # the spike dominates: the exact output is close to that key's value
        vp = vh[0, kp, 0].double().numpy()
        assert np.linalg.norm(ref_o[i] - vp) < 0.2 * np.linalg.norm(vp)
    compare(o, l, ref_o, ref_l, torch.bfloat16, what=f"kv rows Nk={Nk}")


# --------------------------------------------------------------------------
# edge cases and variants at sizes the oracle checks in full


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_dtypes_and_head_dims_ragged(gpu, dtype, d, causal):
    # 200 rows: not a multiple of any tile size
    q, k, v = workloads.make_qkv(2, 200, 200, 4, 2, d, dtype, seed=7 + d)
    run_full_check(q, k, v, causal, 1, False, -1, f"dtype={dtype} d={d} causal={causal}")


@pytest.mark.parametrize("W,zigzag", [(1, False), (2, False), (3, False), (4, False), (1, True),
                                      (2, True), (3, True), (4, True)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_ring_layouts_all_ranks(gpu, W, zigzag, dtype):
    N = 2 * W * 40 if zigzag else W * 70  # chunks shorter than a tile, ragged
    q, k, v = workloads.make_qkv(1, N, N, 2, 1, 64, dtype, seed=11 * W + zigzag)
    run_full_check(q, k, v, True, W, zigzag, -1, f"W={W} zigzag={zigzag} all ranks")
    for r in range(W):
        qs = ring.shard(q, W, zigzag, r)
        run_full_check(qs, k, v, True, W, zigzag, r, f"W={W} zigzag={zigzag} rank={r}")


@pytest.mark.parametrize("fused_merge", [True, False])
@pytest.mark.parametrize("W,zigzag", [(2, False), (3, True), (4, True)])
def test_ring_steps_equal_oracle(gpu, W, zigzag, fused_merge):
    N = 2 * W * 96 if zigzag else W * 160
    q, k, v = workloads.make_qkv(1, N, N, 4, 2, 128, torch.bfloat16, seed=5 + W)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    ks = [ring.shard(kd, W, zigzag, r) for r in range(W)]
    vs = [ring.shard(vd, W, zigzag, r) for r in range(W)]
    for r in range(W):
        out, lse = ring.ring_forward_steps(ring.shard(qd, W, zigzag, r), ks, vs, W, zigzag, r,
                                           fused_merge=fused_merge)
        torch.cuda.synchronize()
        qs = ring.shard(q, W, zigzag, r)
        ref_o, ref_l = oracle.attention(qs, k, v, causal=True,
                                        q_pos=layouts.shard_positions(N, W, r, zigzag))
        compare(host(out), host(lse), ref_o, ref_l, torch.bfloat16,
                what=f"steps W={W} zigzag={zigzag} rank={r}")


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float16, 64),
                                     (torch.float32, 32)])
@pytest.mark.parametrize("fused_merge", [True, False])
def test_ring_steps_batched_read_shards_in_place(gpu, dtype, d, fused_merge):
    """B = 2: the ZigZag ring steps read the back query half and the front key
    chunk of each shard through row offsets (no per-step copies); every
    device's result against the oracle, and the shards are left untouched."""
    W, N = 4, 2 * 4 * 72  # chunks of 72 rows: ragged tiles on every kernel
    q, k, v = workloads.make_qkv(2, N, N, 4, 2, d, dtype, seed=70 + d)
    dev = torch.device("cuda:0")
    kd, vd = k.to(dev), v.to(dev)
    ks = [ring.shard(kd, W, True, r) for r in range(W)]
    vs = [ring.shard(vd, W, True, r) for r in range(W)]
    ks_before = [x.clone() for x in ks]
    for r in range(W):
        qs = ring.shard(q, W, True, r)
        qd = qs.to(dev)
        out, lse = ring.ring_forward_steps(qd, ks, vs, W, True, r, fused_merge=fused_merge)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.attention(qs, k, v, causal=True,
                                        q_pos=layouts.shard_positions(N, W, r, True))
        compare(host(out), host(lse), ref_o, ref_l, dtype,
                what=f"B=2 steps {dtype} d={d} rank={r} fused={fused_merge}")
        assert torch.equal(qd, qs.to(dev))
    assert all(torch.equal(a, b) for a, b in zip(ks, ks_before))


def test_step_row_offsets_match_copies(gpu):
    """rattn_fwd_step on rows [q_off, q_off + Nq) x [k_off, k_off + Nk) of
    larger tensors equals the same step on copies of those rows, bit for bit
    (B = 3, GQA, d = 128 and d = 64)."""
    dev = torch.device("cuda:0")
    for d in (128, 64):
        q, k, v = workloads.make_qkv(3, 700, 900, 4, 2, d, torch.bfloat16, seed=80 + d,
                                     device=dev)
        q_off, Nq, k_off, Nk = 133, 400, 257, 520
        q_segs, k_segs = [(1000, 150), (5000, 250)], [(900, 300), (4800, 220)]
        a_o, a_l = binding.fwd_step(q, k, v, True, q_segs, k_segs, q_off=q_off, k_off=k_off)
        b_o, b_l = binding.fwd_step(q[:, q_off:q_off + Nq].contiguous(),
                                    k[:, k_off:k_off + Nk].contiguous(),
                                    v[:, k_off:k_off + Nk].contiguous(), True, q_segs, k_segs)
        torch.cuda.synchronize()
        assert torch.equal(a_o, b_o) and torch.equal(a_l, b_l), d
        ref_o, ref_l = oracle.attention(
            q[:, q_off:q_off + Nq].cpu(), k[:, k_off:k_off + Nk].cpu(),
            v[:, k_off:k_off + Nk].cpu(), causal=True,
            q_pos=np.concatenate([np.arange(1000, 1150), np.arange(5000, 5250)]),
            k_pos=np.concatenate([np.arange(900, 1200), np.arange(4800, 5020)]))
        compare(host(a_o), host(a_l), ref_o, ref_l, torch.bfloat16, what=f"offsets d={d}")


def test_noncausal_result_independent_of_schedule(gpu):
    q, k, v = workloads.make_qkv(1, 512, 512, 2, 2, 128, torch.float16, seed=3, device=gpu)
    base, base_l = binding.fwd(q, k, v)
    for W, zz in ((2, False), (4, True), (8, True)):
        o, l = binding.fwd(q, k, v, n_ring_steps=W, zigzag=zz)
        assert (o.float() - base.float()).abs().max().item() <= 2e-3
        assert (l - base_l).abs().max().item() <= 1e-5


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
def test_large_magnitude_scores(gpu, dtype):
    g = torch.Generator().manual_seed(21)
    q = (torch.randn(1, 300, 2, 64, generator=g) * 10).to(dtype)
    k = (torch.randn(1, 300, 2, 64, generator=g) * 10).to(dtype)
    v = torch.randn(1, 300, 2, 64, generator=g).to(dtype)
    # float32: the score error grows with |s| (~1e3 here), so allow 1e-4
    tol = 1e-4 if dtype == torch.float32 else None
    run_full_check(q, k, v, True, 1, False, -1, f"large scores {dtype}", tol_o=tol)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (8, 1), (6, 6)])
def test_gqa_head_mapping(gpu, Hq, Hkv):
    q, k, v = workloads.make_qkv(1, 256, 256, Hq, Hkv, 128, torch.bfloat16, seed=Hq * 10 + Hkv)
    run_full_check(q, k, v, True, 1, False, -1, f"GQA {Hq}/{Hkv}")


def test_single_row_and_single_key(gpu):
    for dtype in (torch.float32, torch.bfloat16):
        q, k, v = workloads.make_qkv(1, 1, 1, 1, 1, 128, dtype, seed=2)
        run_full_check(q, k, v, True, 1, False, -1, f"N=1 {dtype}")


def test_page_triton_test_shape(gpu):
    """The yz520gzy chapter's kernel test: seed 42, (B,H,N,D) = (2,4,1024,64)
    fp16, non-causal, gate max|diff| < 1e-2 against softmax attention."""
    torch.manual_seed(42)
    B, H, N, D = 2, 4, 1024, 64
    q = torch.randn(B, H, N, D, device="cuda", dtype=torch.float16)
    k = torch.randn(B, H, N, D, device="cuda", dtype=torch.float16)
    v = torch.randn(B, H, N, D, device="cuda", dtype=torch.float16)
    qs, ks, vs = (x.transpose(1, 2).contiguous() for x in (q, k, v))  # to (B, N, H, D)
    out, lse = binding.fwd(qs, ks, vs)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention(qs.cpu(), ks.cpu(), vs.cpu())
    err = compare(host(out), host(lse), ref_o, ref_l, torch.float16, tol_o=1e-2,
                  what="page Triton-test shape")[0]
    assert err < 1e-2


# --------------------------------------------------------------------------
# step kernel and merge kernel on their own


def test_step_rows_without_visible_keys(gpu):
    dev = torch.device("cuda:0")
    q, k, v = workloads.make_qkv(1, 130, 70, 2, 2, 64, torch.bfloat16, seed=9)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    # queries at positions 0..64 and 1000..1064; keys at 30..99
    q_segs, k_segs = [(0, 65), (1000, 65)], [(30, 70)]
    out, lse = binding.fwd_step(qd, kd, vd, True, q_segs, k_segs)
    torch.cuda.synchronize()
    qpos = np.concatenate([np.arange(0, 65), np.arange(1000, 1065)])
    ref_o, ref_l = oracle.attention(q, k, v, causal=True, q_pos=qpos, k_pos=np.arange(30, 100))
    compare(host(out), host(lse), ref_o, ref_l, torch.bfloat16, what="step, empty rows")
    assert np.isneginf(host(lse)[0, :30]).all() and (host(out)[0, :30] == 0).all()


def test_step_with_no_keys(gpu):
    dev = torch.device("cuda:0")
    q, k, v = workloads.make_qkv(1, 40, 0, 1, 1, 32, torch.float16, seed=1, device=dev)
    out, lse = binding.fwd_step(q, k, v, False, [(0, 40)], [(0, 0)])
    torch.cuda.synchronize()
    assert (out == 0).all() and torch.isneginf(lse).all()


def test_step_two_key_segments(gpu):
    dev = torch.device("cuda:0")
    q, k, v = workloads.make_qkv(2, 150, 190, 4, 4, 128, torch.float16, seed=31)
    q_segs, k_segs = [(500, 150)], [(0, 90), (600, 100)]
    out, lse = binding.fwd_step(q.to(dev), k.to(dev), v.to(dev), True, q_segs, k_segs)
    torch.cuda.synchronize()
    kpos = np.concatenate([np.arange(0, 90), np.arange(600, 700)])
    ref_o, ref_l = oracle.attention(q, k, v, causal=True, q_pos=np.arange(500, 650), k_pos=kpos)
    compare(host(out), host(lse), ref_o, ref_l, torch.float16, what="step, two key runs")


# The d = 128 16-bit kernel works on 256-row query tiles (8 waves of 32
# rows) and 64-key tiles; these cases cross several of both, end on ragged
# tails (inactive waves, partial key tiles) and put the causal diagonal off
# every tile boundary.


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("causal", [False, True])
def test_d128_several_query_and_key_tiles_ragged(gpu, dtype, causal):
    N = 2 * 256 + 37  # three query tiles, the last with 37 rows; 8 key tiles + 37
    q, k, v = workloads.make_qkv(1, N, N, 4, 2, 128, dtype, seed=41 + causal)
    run_full_check(q, k, v, causal, 1, False, -1, f"d=128 N={N} {dtype} causal={causal}")


def test_d128_step_offset_diagonal(gpu):
    dev = torch.device("cuda:0")
    q, k, v = workloads.make_qkv(1, 300, 400, 2, 2, 128, torch.bfloat16, seed=43)
    q_segs, k_segs = [(100, 300)], [(0, 400)]
    out, lse = binding.fwd_step(q.to(dev), k.to(dev), v.to(dev), True, q_segs, k_segs)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention(q, k, v, causal=True, q_pos=np.arange(100, 400),
                                    k_pos=np.arange(0, 400))
    compare(host(out), host(lse), ref_o, ref_l, torch.bfloat16, what="d=128 step, diagonal")


def test_d128_step_query_tiles_without_keys(gpu):
    dev = torch.device("cuda:0")
    q, k, v = workloads.make_qkv(1, 600, 200, 2, 1, 128, torch.float16, seed=47)
    # 300 queries before every key (whole 256-row tiles with no live key tile),
    # then 300 queries after them
    q_segs, k_segs = [(0, 300), (5000, 300)], [(1000, 200)]
    out, lse = binding.fwd_step(q.to(dev), k.to(dev), v.to(dev), True, q_segs, k_segs)
    torch.cuda.synchronize()
    qpos = np.concatenate([np.arange(0, 300), np.arange(5000, 5300)])
    ref_o, ref_l = oracle.attention(q, k, v, causal=True, q_pos=qpos,
                                    k_pos=np.arange(1000, 1200))
    compare(host(out), host(lse), ref_o, ref_l, torch.float16, what="d=128 step, no keys")
    assert np.isneginf(host(lse)[0, :300]).all() and (host(out)[0, :300] == 0).all()


# --------------------------------------------------------------------------
# split-KV: the key tiles of every query tile over n_splits workgroups, then
# the n-way log-sum-exp merge


def run_split_check(q, k, v, causal, W, zigzag, rank, n_splits, what, tol_o=None):
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out, lse = binding.fwd_split(qd, kd, vd, causal=causal, n_ring_steps=W, zigzag=zigzag,
                                 rank=rank, n_splits=n_splits)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention(q, k, v, causal=causal,
                                    q_pos=q_positions(k.shape[1], W, zigzag, rank))
    return compare(host(out), host(lse), ref_o, ref_l, q.dtype, tol_o, what)


@pytest.mark.parametrize("dtype,d", [(torch.float32, 16), (torch.float16, 32),
                                     (torch.bfloat16, 64), (torch.bfloat16, 128),
                                     (torch.float16, 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n_splits", [2, 5, 64])
def test_split_kv(gpu, dtype, d, causal, n_splits):
    # 600 rows: ragged in every tile size; 64 splits leave some splits empty
    q, k, v = workloads.make_qkv(1, 600, 600, 2, 1, d, dtype, seed=50 + d + n_splits)
    run_split_check(q, k, v, causal, 1, False, -1, n_splits,
                    f"split-KV {dtype} d={d} causal={causal} splits={n_splits}")


@pytest.mark.parametrize("W,zigzag,rank", [(4, True, 1), (4, True, -1), (3, False, 2)])
def test_split_kv_ring_layouts(gpu, W, zigzag, rank):
    N = 2 * W * 96 if zigzag else W * 128
    q, k, v = workloads.make_qkv(1, N, N, 2, 2, 128, torch.bfloat16, seed=60 + W)
    if rank >= 0:
        q = ring.shard(q, W, zigzag, rank)
    run_split_check(q, k, v, True, W, zigzag, rank, 3, f"split-KV W={W} zz={zigzag} r={rank}")


def test_split_kv_workload2_with_hint(gpu):
    w = workloads.workload(2)
    q, k, v = workloads.make_inputs(w)
    qd = q.to("cuda:0")
    n = binding.split_hint(qd, k.to("cuda:0"))
    note(f"case {w.name}, {n} splits")
    assert n > 1
    run_split_check(q, k, v, w.causal, w.W, w.zigzag, w.rank, n, f"{w.name} split {n}")


def test_split_kv_one_split_is_fwd(gpu):
    q, k, v = workloads.make_qkv(1, 300, 300, 2, 2, 128, torch.bfloat16, seed=70, device=gpu)
    a, la = binding.fwd(q, k, v, causal=True)
    b, lb = binding.fwd_split(q, k, v, causal=True, n_splits=1)
    assert torch.equal(a, b) and torch.equal(la, lb)


@pytest.mark.parametrize("dtype,d", [(torch.float32, 16), (torch.float16, 64),
                                     (torch.bfloat16, 128)])
def test_step_merge_into_rows(gpu, dtype, d):
    """rattn_fwd_step_merge on a row range of a batched output: rows of batch
    b sit Nq_out apart, so the kernel addresses them from out_rows/row_off."""
    dev = torch.device("cuda:0")
    B, Nq_out, off, Nq, Nk = 2, 400, 150, 200, 300
    q, k, v = workloads.make_qkv(B, Nq, Nk, 4, 2, d, dtype, seed=80 + d)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    # running result: the first 100 keys as a step of its own, written into
    # rows [off, off + Nq) of a larger float32 output that starts out garbage
    # elsewhere; queries at positions 1000.. see every key (causal passes)
    out = torch.full((B, Nq_out, 4, d), 7.0, device=dev)
    lse = torch.full((B, Nq_out, 4), 3.0, device=dev)
    o1, l1 = binding.fwd_step(qd, kd[:, :100].contiguous(), vd[:, :100].contiguous(), True,
                              [(1000, Nq)], [(0, 100)])
    out[:, off:off + Nq] = o1
    lse[:, off:off + Nq] = l1
    binding.fwd_step_merge(qd, kd[:, 100:].contiguous(), vd[:, 100:].contiguous(), True,
                           [(1000, Nq)], [(100, Nk - 100)], out, lse, row_off=off)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention(q, k, v, causal=True, q_pos=np.arange(1000, 1000 + Nq),
                                    k_pos=np.arange(Nk))
    compare(host(out[:, off:off + Nq]), host(lse[:, off:off + Nq]), ref_o, ref_l, dtype,
            what=f"step merge {dtype} d={d}")
    # rows outside the range are untouched
    assert (out[:, :off] == 7.0).all() and (out[:, off + Nq:] == 7.0).all()
    assert (lse[:, :off] == 3.0).all() and (lse[:, off + Nq:] == 3.0).all()


@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_merge_kernel(gpu, d):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(d)
    B, Nq, H, Nb, off = 2, 50, 3, 20, 17
    o = rng.standard_normal((B, Nq, H, d)).astype(np.float32)
    l = (rng.standard_normal((B, Nq, H)) * 5).astype(np.float32)
    bo = rng.standard_normal((B, Nb, H, d)).astype(np.float32)
    bl = (rng.standard_normal((B, Nb, H)) * 5).astype(np.float32)
    l[0, off:off + 3] = -np.inf          # empty running rows
    o[0, off:off + 3] = 0
    bl[0, 2:5] = -np.inf                 # empty block rows (2 overlap the above)
    bo[0, 2:5] = 0
    od, ld = torch.from_numpy(o).to(dev), torch.from_numpy(l).to(dev)
    binding.merge(od, ld, torch.from_numpy(bo).to(dev), torch.from_numpy(bl).to(dev), row_off=off)
    torch.cuda.synchronize()
    ref_o, ref_l = o.astype(np.float64).copy(), l.astype(np.float64).copy()
    mo, ml = oracle.merge(ref_o[:, off:off + Nb], ref_l[:, off:off + Nb], bo, bl)
    ref_o[:, off:off + Nb], ref_l[:, off:off + Nb] = mo, ml
    got_o, got_l = od.cpu().numpy(), ld.cpu().numpy()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(ref_l))
    fin = ~np.isneginf(ref_l)
    assert np.max(np.abs(got_o - ref_o)) <= 1e-5
    assert np.max(np.abs(got_l[fin] - ref_l[fin])) <= 1e-5
    # rows outside [off, off+Nb) are untouched, bit for bit
    assert np.array_equal(got_o[:, :off], o[:, :off]) and np.array_equal(got_l[:, :off], l[:, :off])


def test_runs_on_a_side_stream_and_is_deterministic(gpu):
    q, k, v = workloads.make_qkv(1, 1000, 1000, 4, 4, 128, torch.bfloat16, seed=4, device=gpu)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o1, l1 = binding.fwd(q, k, v, causal=True, n_ring_steps=4, zigzag=True)
        o2, l2 = binding.fwd(q, k, v, causal=True, n_ring_steps=4, zigzag=True)
    s.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
