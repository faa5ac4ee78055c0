"""Variable-length batches (rattn_fwd_varlen, rattn_bwd_varlen) vs the fp64
oracle (needs a GPU).

Each sequence is checked on its own against the oracle, with the positions
the boundary documents (key j at j, query i at k_len - q_len + i); rows
outside every sequence must keep what the output held.  Bars as in
test_parity.py.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from ring_attention_amd import binding, workloads

pytestmark = pytest.mark.gpu

TOL_O = {torch.float32: 1e-5, torch.float16: 2e-2, torch.bfloat16: 2e-2}


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(q, k, v, out, lse, qs, ql, ks, kl, causal, dtype, what):
    o, l = host(out), host(lse)
    worst_o = worst_l = 0.0
    for i, (a, n, b, m) in enumerate(zip(qs, ql, ks, kl)):
        if n == 0:
            continue
        qpos = np.arange(n) + (m - n)
        ro, rl = oracle.attention(q[None, a:a + n], k[None, b:b + m], v[None, b:b + m],
                                  causal=causal, q_pos=qpos, k_pos=np.arange(m))
        got_o, got_l = o[a:a + n], l[a:a + n]
        assert np.array_equal(np.isneginf(got_l), np.isneginf(rl[0])), f"{what} seq {i}"
        fin = np.isfinite(rl[0])
        worst_o = max(worst_o, float(np.abs(got_o - ro[0]).max()))
        if fin.any():
            worst_l = max(worst_l, float(np.abs(got_l[fin] - rl[0][fin]).max()))
    note(f"{what}: max|dO|={worst_o:.3e} max|dLSE|={worst_l:.3e}")
    assert worst_o <= TOL_O[dtype] and worst_l <= 1e-3


def packed_inputs(lens, H, Hkv, d, dtype, seed):
    N = sum(lens)
    q, k, v = workloads.make_qkv(1, N, N, H, Hkv, d, dtype, seed=seed)
    return q[0], k[0], v[0]


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float16, 64),
                                     (torch.float32, 32)], ids=["bf16_d128", "f16_d64", "f32_d32"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_varlen_packed(gpu, dtype, d, causal):
    lens = [1, 7, 64, 200, 513, 0, 1000, 255]
    q, k, v = packed_inputs(lens, 4, 2, d, dtype, seed=400 + d)
    starts, ls = binding.varlen_from_cu_seqlens(np.concatenate([[0], np.cumsum(lens)]))
    dev = torch.device("cuda:0")
    out, lse = binding.fwd_varlen(q.to(dev), k.to(dev), v.to(dev), starts, ls, starts, ls,
                                  causal=causal)
    torch.cuda.synchronize()
    check(q, k, v, out, lse, starts, ls, starts, ls, causal, dtype,
          f"varlen packed {dtype} d={d} causal={causal}")


def test_varlen_padded_rows_untouched(gpu):
    """Three sequences in blocks of 600 rows with true lengths 600, 17, 333:
    the pad rows are neither keys nor written."""
    dtype, d, S = torch.bfloat16, 128, 600
    q, k, v = packed_inputs([3 * S], 4, 4, d, dtype, seed=420)
    lens = [600, 17, 333]
    starts = [0, S, 2 * S]
    dev = torch.device("cuda:0")
    out = torch.full(q.shape, 7.0, dtype=dtype, device=dev)
    lse = torch.full(q.shape[:2], 7.0, dtype=torch.float32, device=dev)
    binding.fwd_varlen(q.to(dev), k.to(dev), v.to(dev), starts, lens, starts, lens,
                       causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    check(q, k, v, out, lse, starts, lens, starts, lens, True, dtype, "varlen padded")
    o, l = host(out), host(lse)
    for s0, n in zip(starts, lens):
        assert np.all(o[s0 + n:s0 + S] == 7.0) and np.all(l[s0 + n:s0 + S] == 7.0)


def test_varlen_query_and_key_lengths_differ(gpu):
    """q_len != k_len: the last query is aligned with the last key."""
    dtype, d = torch.bfloat16, 128
    ql, kl = [5, 300, 64, 1], [100, 50, 64, 1]
    qs = list(np.concatenate([[0], np.cumsum(ql)[:-1]]))
    ks = list(np.concatenate([[0], np.cumsum(kl)[:-1]]))
    q, _, _ = packed_inputs([sum(ql)], 2, 2, d, dtype, seed=430)
    _, k, v = packed_inputs([sum(kl)], 2, 2, d, dtype, seed=431)
    dev = torch.device("cuda:0")
    for causal in (False, True):
        out, lse = binding.fwd_varlen(q.to(dev), k.to(dev), v.to(dev), qs, ql, ks, kl,
                                      causal=causal)
        torch.cuda.synchronize()
        check(q, k, v, out, lse, qs, ql, ks, kl, causal, dtype,
              f"varlen cross lengths causal={causal}")


def test_varlen_one_sequence_equals_fwd(gpu):
    dtype, d, N = torch.bfloat16, 128, 777
    q, k, v = packed_inputs([N], 4, 2, d, dtype, seed=440)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o1, l1 = binding.fwd_varlen(qd, kd, vd, [0], [N], [0], [N], causal=True)
    o2, l2 = binding.fwd(qd[None], kd[None], vd[None], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2[0]) and torch.equal(l1, l2[0])


# --------------------------------------------------------------------------
# backward (rattn_bwd_varlen)

TOL_G = {torch.float32: 1e-4, torch.float16: 2e-2, torch.bfloat16: 2e-2}


def check_bwd(q, k, v, do, grads, qs, ql, ks, kl, causal, dtype, what):
    dq, dk, dv = (host(t) for t in grads)
    for i, (a, n, b, m) in enumerate(zip(qs, ql, ks, kl)):
        if n == 0 and m == 0:
            continue
        qpos = np.arange(n) + (m - n)
        rq, rk, rv, _, _ = oracle.attention_bwd(q[None, a:a + n], k[None, b:b + m],
                                                v[None, b:b + m], do[None, a:a + n],
                                                causal=causal, q_pos=qpos, k_pos=np.arange(m))
        for name, got, ref in (("dq", dq[a:a + n], rq[0]), ("dk", dk[b:b + m], rk[0]),
                               ("dv", dv[b:b + m], rv[0])):
            if ref.size == 0:
                continue
            err = float(np.abs(got - ref).max())
            bar = TOL_G[dtype] * max(1.0, float(np.abs(ref).max()))
            assert err <= bar, f"{what} seq {i} {name}: {err} > {bar}"
    note(f"{what}: every sequence within its bar")


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)],
                         ids=["bf16_d128", "f32_d64"])
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_varlen_backward_packed(gpu, dtype, d, causal):
    lens = [1, 70, 300, 0, 129, 511]
    q, k, v = packed_inputs(lens, 4, 2, d, dtype, seed=450 + d)
    N = sum(lens)
    do = workloads.randn((N, 4, d), dtype, torch.Generator().manual_seed(451), "cpu")
    starts, ls = binding.varlen_from_cu_seqlens(np.concatenate([[0], np.cumsum(lens)]))
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    out, lse = binding.fwd_varlen(qd, kd, vd, starts, ls, starts, ls, causal=causal)
    grads = binding.bwd_varlen(qd, kd, vd, out, lse, dod, starts, ls, starts, ls, causal=causal)
    torch.cuda.synchronize()
    check_bwd(q, k, v, do, grads, starts, ls, starts, ls, causal, dtype,
              f"varlen bwd {dtype} d={d} causal={causal}")


def test_varlen_backward_padded_and_cross_lengths(gpu):
    """Padded blocks (pad rows get no gradient) and q_len != k_len."""
    dtype, d = torch.bfloat16, 128
    S = 256
    ql, kl = [256, 17, 100], [256, 40, 7]
    qs, ks = [0, S, 2 * S], [0, S, 2 * S]
    q, k, v = packed_inputs([3 * S], 2, 2, d, dtype, seed=460)
    do = workloads.randn((3 * S, 2, d), dtype, torch.Generator().manual_seed(461), "cpu")
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    out, lse = binding.fwd_varlen(qd, kd, vd, qs, ql, ks, kl, causal=True)
    grads = binding.bwd_varlen(qd, kd, vd, out, lse, dod, qs, ql, ks, kl, causal=True)
    torch.cuda.synchronize()
    check_bwd(q, k, v, do, grads, qs, ql, ks, kl, True, dtype, "varlen bwd padded")
    dq, dk, dv = (host(t) for t in grads)
    for s0, n, m in zip(qs, ql, kl):
        assert np.all(dq[s0 + n:s0 + S] == 0)
        assert np.all(dk[s0 + m:s0 + S] == 0) and np.all(dv[s0 + m:s0 + S] == 0)
