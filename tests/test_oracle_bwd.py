"""Pins of the fp64 oracle's backward pass (dQ, dK, dV) against mathematics.

The forward oracle is pinned in test_oracle.py.  Here its gradients are
checked against things other than their own formulas: central finite
differences of the pinned forward oracle, torch autograd through a float64
textbook attention, invariants the softmax forces (shift invariance in the
keys, weights summing to one), closed forms of degenerate cases, and the
youngju.dev ring backward simulated over W blocks.  Planted mistakes in the
backward code must each fail one of these pins.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle
from oracle import recurrences


def rnd(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def loss(q, k, v, do, lib_path=None, **kw):
    """sum(dO * O) with O from the forward oracle (float64)."""
    out, _ = oracle.attention(q, k, v, lib_path=lib_path, **kw)
    return float((out * np.asarray(do, np.float64)).sum())


def finite_difference(q, k, v, do, h=2.0 ** -10, lib_path=None, **kw):
    """Central differences of sum(dO * O) in every entry of q, k and v.

    The step is a power of two, so x +- h is exact in float32 for |x| < 2^13
    and the denominator is exactly 2h."""
    grads = []
    arrs = [q, k, v]
    for which in range(3):
        base = arrs[which]
        g = np.zeros(base.shape, np.float64)
        for idx in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[idx] += np.float32(h)
            minus[idx] -= np.float32(h)
            denom = float(plus[idx]) - float(minus[idx])
            assert denom == 2 * h
            ap = list(arrs); ap[which] = plus
            am = list(arrs); am[which] = minus
            g[idx] = (loss(*ap, do, lib_path=lib_path, **kw) -
                      loss(*am, do, lib_path=lib_path, **kw)) / denom
        grads.append(g)
    return grads


def autograd_reference(q, k, v, do, causal=False, scale=None, q_pos=None, k_pos=None):
    """torch autograd (float64, CPU) through softmax(scale QK^T)V with GQA heads
    expanded in contiguous groups and the causal rule by position."""
    q = torch.tensor(np.asarray(q, np.float64), requires_grad=True)
    k = torch.tensor(np.asarray(k, np.float64), requires_grad=True)
    v = torch.tensor(np.asarray(v, np.float64), requires_grad=True)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    ke = k.repeat_interleave(g, dim=2)
    ve = v.repeat_interleave(g, dim=2)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    s = torch.matmul(q.permute(0, 2, 1, 3), ke.permute(0, 2, 3, 1).contiguous()) * scale
    if causal:
        qp = torch.arange(Nq) if q_pos is None else torch.as_tensor(q_pos)
        kp = torch.arange(Nk) if k_pos is None else torch.as_tensor(k_pos)
        s = s.masked_fill(kp[None, :] > qp[:, None], float("-inf"))
    w = torch.nan_to_num(torch.softmax(s, dim=-1), nan=0.0)
    out = torch.matmul(w, ve.permute(0, 2, 1, 3).contiguous()).permute(0, 2, 1, 3)
    (out * torch.as_tensor(np.asarray(do, np.float64))).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


FD_CASES = {
    # name: (shapes, causal, q_pos, k_pos)
    "plain": (((1, 5, 1, 3), (1, 5, 1, 3)), False, None, None),
    "causal_gqa_positions": (((1, 5, 2, 3), (1, 6, 1, 3)), True,
                             [3, -1, 7, 5, 1], [2, 6, 0, 4, 8, 3]),
    "batch_gqa_noncausal": (((2, 3, 4, 2), (2, 4, 2, 2)), False, None, None),
}


@pytest.mark.parametrize("name", sorted(FD_CASES))
def test_bwd_matches_finite_differences(name):
    (qs, ks), causal, qp, kp = FD_CASES[name]
    q, k, v, do = rnd(qs, 1), rnd(ks, 2), rnd(ks, 3), rnd(qs, 4)
    kw = dict(causal=causal, q_pos=qp, k_pos=kp)
    dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, do, **kw)
    fq, fk, fv = finite_difference(q, k, v, do, **kw)
    for got, ref in ((dq, fq), (dk, fk), (dv, fv)):
        assert np.abs(got - ref).max() <= 2e-6 * max(1.0, np.abs(ref).max())


def test_bwd_matches_autograd_float64():
    q, k, v, do = rnd((2, 33, 4, 16), 5), rnd((2, 40, 2, 16), 6), rnd((2, 40, 2, 16), 7), \
        rnd((2, 33, 4, 16), 8)
    qp = np.arange(33) + 5   # queries 5..37 over keys 0..39: some keys never seen
    dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, do, causal=True, q_pos=qp)
    rq, rk, rv = autograd_reference(q, k, v, do, causal=True, q_pos=qp)
    assert np.allclose(dq, rq, atol=1e-12, rtol=0)
    assert np.allclose(dk, rk, atol=1e-12, rtol=0)
    assert np.allclose(dv, rv, atol=1e-12, rtol=0)


def test_bwd_custom_scale_matches_autograd():
    q, k, v, do = rnd((1, 9, 2, 8), 9), rnd((1, 9, 2, 8), 10), rnd((1, 9, 2, 8), 11), \
        rnd((1, 9, 2, 8), 12)
    dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, do, scale=0.7)
    rq, rk, rv = autograd_reference(q, k, v, do, scale=0.7)
    for a, b in ((dq, rq), (dk, rk), (dv, rv)):
        assert np.allclose(a, b, atol=1e-12, rtol=0)


def test_bwd_key_shift_invariance():
    """Adding one vector to every key changes each row's scores by a constant,
    which the softmax ignores: the gradient along that shift, sum_j dK_j, is 0."""
    q, k, v, do = rnd((2, 20, 4, 8), 13), rnd((2, 24, 2, 8), 14), rnd((2, 24, 2, 8), 15), \
        rnd((2, 20, 4, 8), 16)
    dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, do, causal=True, q_pos=np.arange(20) + 4)
    assert np.abs(dk.sum(axis=1)).max() < 1e-12 * np.abs(dk).max() * 24


def test_bwd_value_gradient_sums_to_upstream():
    """The weights of a row sum to one, so sum_j dV_j = sum over the group's
    rows (with something visible) of dO_i."""
    q, k, v, do = rnd((1, 12, 4, 8), 17), rnd((1, 12, 2, 8), 18), rnd((1, 12, 2, 8), 19), \
        rnd((1, 12, 4, 8), 20)
    qp = np.arange(12) - 3   # rows at positions -3..-1 see no key
    dq, dk, dv, lse, _ = oracle.attention_bwd(q, k, v, do, causal=True, q_pos=qp)
    seen = (qp >= 0)
    want = do.astype(np.float64)[:, seen].sum(axis=1).reshape(1, 2, 2, 8).sum(axis=2)
    assert np.allclose(dv.sum(axis=1), want, atol=1e-12)
    assert np.all(np.isneginf(lse[0, ~seen]))
    assert np.all(dq[0, ~seen] == 0.0)


def test_bwd_single_key_closed_form():
    """One visible key: O = v, so dV = sum dO, dQ = 0, dK = 0."""
    q, k, v, do = rnd((1, 3, 1, 4), 21), rnd((1, 1, 1, 4), 22), rnd((1, 1, 1, 4), 23), \
        rnd((1, 3, 1, 4), 24)
    dq, dk, dv, _, delta = oracle.attention_bwd(q, k, v, do)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    assert np.allclose(dv[0, 0, 0], do.astype(np.float64).sum(axis=(0, 1, 2)), atol=1e-14)
    assert np.allclose(delta[0, :, 0], do.astype(np.float64)[0, :, 0] @ v[0, 0, 0].astype(
        np.float64), atol=1e-14)


def test_bwd_two_equal_keys_closed_form():
    """Two identical keys get weight 1/2 each: dV_j = dO/2; dS_0 = -dS_1 =
    (dO.(v0 - v1))/4, so dQ = scale (dS_0 + dS_1) k = 0 and
    dK_0 = -dK_1 = scale/4 (dO.(v0 - v1)) q."""
    q = rnd((1, 1, 1, 4), 25)
    k1 = rnd((1, 1, 1, 4), 26)
    k = np.concatenate([k1, k1], axis=1)
    v, do = rnd((1, 2, 1, 4), 27), rnd((1, 1, 1, 4), 28)
    dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, do, scale=0.5)
    q64, v64, do64 = (x.astype(np.float64) for x in (q, v, do))
    assert np.allclose(dv[0, :, 0], np.stack([do64[0, 0, 0] / 2] * 2), atol=1e-15)
    assert np.abs(dq).max() < 1e-15
    c = 0.5 / 4 * float(do64[0, 0, 0] @ (v64[0, 0, 0] - v64[0, 1, 0]))
    assert np.allclose(dk[0, 0, 0], c * q64[0, 0, 0], atol=1e-14)
    assert np.allclose(dk[0, 1, 0], -c * q64[0, 0, 0], atol=1e-14)


@pytest.mark.parametrize("W,rank", [(4, 0), (4, 3), (3, 1)])
def test_bwd_equals_page_ring_backward(W, rank):
    """The youngju.dev ring backward, simulated over W key/value blocks from
    one device's saved output and LSE, reaches the definition's gradients
    for that device's query block (non-causal, as on the page)."""
    N, d = 24, 8
    S = N // W
    qa, k, v, doa = rnd((N, d), 30), rnd((N, d), 31), rnd((N, d), 32), rnd((N, d), 33)
    rows = slice(rank * S, (rank + 1) * S)
    q, do = qa[rows], doa[rows]
    o, lse = oracle.attention(q[None, :, None], k[None, :, None], v[None, :, None])
    rq, rk, rv = recurrences.ring_backward(q, k, v, o[0, :, 0], lse[0, :, 0], do, W, rank)
    dq, dk, dv, _, _ = oracle.attention_bwd(q[None, :, None], k[None, :, None],
                                            v[None, :, None], do[None, :, None])
    assert np.allclose(dq[0, :, 0], rq, atol=1e-12)
    assert np.allclose(dk[0, :, 0], rk, atol=1e-12)
    assert np.allclose(dv[0, :, 0], rv, atol=1e-12)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_bwd_16bit_storage_equals_widened_float32(dtype):
    """16-bit inputs decode exactly; their gradients equal those of the same
    values stored as float32."""
    t = [torch.from_numpy(rnd(s, 40 + i)).to(dtype) for i, s in
         enumerate([(1, 10, 2, 8), (1, 10, 1, 8), (1, 10, 1, 8), (1, 10, 2, 8)])]
    g16 = oracle.attention_bwd(*t, causal=True)
    g32 = oracle.attention_bwd(*[x.float() for x in t], causal=True)
    for a, b in zip(g16, g32):
        assert np.array_equal(a, b)


def test_bwd_sampled_rows_match_full():
    q, k, v, do = rnd((2, 14, 4, 8), 50), rnd((2, 14, 2, 8), 51), rnd((2, 14, 2, 8), 52), \
        rnd((2, 14, 4, 8), 53)
    dq, dk, dv, lse, delta = oracle.attention_bwd(q, k, v, do, causal=True)
    qrows = np.array([[0, 0, 0], [1, 13, 3], [0, 7, 2]])
    krows = np.array([[1, 0, 1], [0, 13, 0], [1, 6, 0]])
    sl, sd = oracle.bwd_stats(q, k, v, do, causal=True, rows=qrows)
    assert np.array_equal(sl, lse[qrows[:, 0], qrows[:, 1], qrows[:, 2]])
    assert np.array_equal(sd, delta[qrows[:, 0], qrows[:, 1], qrows[:, 2]])
    sq = oracle.bwd_dq(q, k, v, do, lse, delta, causal=True, rows=qrows)
    assert np.array_equal(sq, dq[qrows[:, 0], qrows[:, 1], qrows[:, 2]])
    sk, sv = oracle.bwd_dkv(q, k, v, do, lse, delta, causal=True, rows=krows)
    assert np.array_equal(sk, dk[krows[:, 0], krows[:, 1], krows[:, 2]])
    assert np.array_equal(sv, dv[krows[:, 0], krows[:, 1], krows[:, 2]])


def test_bwd_rejects_bad_arguments():
    q, k = rnd((1, 4, 3, 4), 60), rnd((1, 4, 2, 4), 61)
    with pytest.raises(ValueError):
        oracle.attention_bwd(q, k, k, q)        # Hq % Hkv != 0
    with pytest.raises(ValueError):
        oracle.bwd_dq(q[:, :, :2], k, k, q[:, :, :2], np.zeros((1, 3, 2)), np.zeros((1, 3, 2)))


# --------------------------------------------------------------------------
# planted mistakes in the backward code: each must fail at least one pin


def _bwd_pin_battery(lib_path):
    failed = []

    def check(name, fn):
        try:
            if not fn():
                failed.append(name)
        except Exception:
            failed.append(name)

    def fd_pin():
        (qs, ks), causal, qp, kp = FD_CASES["causal_gqa_positions"]
        q, k, v, do = rnd(qs, 1), rnd(ks, 2), rnd(ks, 3), rnd(qs, 4)
        kw = dict(causal=causal, q_pos=qp, k_pos=kp)
        got = oracle.attention_bwd(q, k, v, do, lib_path=lib_path, **kw)[:3]
        # the finite differences use the pinned forward of the same build:
        # the forward code is not mutated here
        ref = finite_difference(q, k, v, do, lib_path=lib_path, **kw)
        return all(np.abs(a - b).max() <= 2e-6 * max(1.0, np.abs(b).max())
                   for a, b in zip(got, ref))

    def autograd_pin():
        q, k, v, do = rnd((1, 12, 4, 8), 5), rnd((1, 12, 2, 8), 6), rnd((1, 12, 2, 8), 7), \
            rnd((1, 12, 4, 8), 8)
        got = oracle.attention_bwd(q, k, v, do, causal=True, scale=0.3, lib_path=lib_path)[:3]
        ref = autograd_reference(q, k, v, do, causal=True, scale=0.3)
        return all(np.allclose(a, b, atol=1e-12, rtol=0) for a, b in zip(got, ref))

    check("finite_differences", fd_pin)
    check("autograd", autograd_pin)
    return failed


def test_bwd_pin_battery_passes_on_the_oracle():
    assert _bwd_pin_battery(None) == []


BWD_MUTATIONS = {
    "dropped_delta": ("const double dS = P * (dp - Dl);\n                    for (int t = 0; t < d; ++t) g_out",
                      "const double dS = P * dp;\n                    for (int t = 0; t < d; ++t) g_out"),
    "dq_without_scale": ("for (int t = 0; t < d; ++t) g_out[t] *= scale;", ""),
    "dk_from_k": ("gk[t] += dS * load(q, row * d + t, dtype);", "gk[t] += dS * krow[t];"),
    "dv_weighted_by_ds": ("gv[t] += P * load(dout, row * d + t, dtype);",
                          "gv[t] += dS * load(dout, row * d + t, dtype);"),
    "dkv_one_head_of_group": ("for (int64_t hq = g * group; hq < (g + 1) * group; ++hq)",
                              "for (int64_t hq = g * group; hq < g * group + 1; ++hq)"),
    "dkv_mask_flipped": ("if (causal && k_pos[j] > q_pos[i]) continue;\n                        const int64_t row",
                         "if (causal && k_pos[j] < q_pos[i]) continue;\n                        const int64_t row"),
    "delta_sign": ("dsum += load(dout, ((b * Nq + i) * Hq + hq) * d + t, dtype) * o[t];",
                   "dsum -= load(dout, ((b * Nq + i) * Hq + hq) * d + t, dtype) * o[t];"),
    "dq_p_without_lse": ("const double P = exp(scale * dot - L);\n                    const double dS = P * (dp - Dl);\n                    for (int t = 0; t < d; ++t) g_out",
                         "const double P = exp(scale * dot);\n                    const double dS = P * (dp - Dl);\n                    for (int t = 0; t < d; ++t) g_out"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTATIONS))
def test_bwd_planted_mistake_is_caught(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = BWD_MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found once"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = str(tmp_path / "liboracle_mut.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", str(mutated), "-o", lib, "-lm"],
                   check=True)
    assert _bwd_pin_battery(lib), f"planted mistake {name} went unnoticed"
