"""Pins of the fp64 oracle against what the pages and the mathematics fix.

No test here compares the oracle with itself: each one checks it against a
closed form, a hand-worked example, a textbook/library routine (torch softmax
and logsumexp in float64), brute force in pure Python, a fact the pages print,
or one of the pages' own algorithms (blockwise online softmax, the ring
simulation, the ZigZag step rules with the sigmoid merge).
"""
import itertools
import json
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle
from oracle import layouts, recurrences
from ring_attention_amd import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rnd(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def textbook(q, k, v, causal=False, scale=None, q_pos=None, k_pos=None):
    """torch.softmax / torch.logsumexp in float64 on the CPU, heads expanded
    for GQA with contiguous groups."""
    q = torch.as_tensor(np.asarray(q, np.float64))
    k = torch.as_tensor(np.asarray(k, np.float64))
    v = torch.as_tensor(np.asarray(v, np.float64))
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    k = k.repeat_interleave(g, dim=2)
    v = v.repeat_interleave(g, dim=2)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    s = torch.einsum("bihd,bjhd->bhij", q, k) * scale
    if causal:
        qp = torch.arange(Nq) if q_pos is None else torch.as_tensor(q_pos)
        kp = torch.arange(Nk) if k_pos is None else torch.as_tensor(k_pos)
        s = s.masked_fill(kp[None, :] > qp[:, None], float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    w = torch.softmax(s, dim=-1)
    w = torch.nan_to_num(w, nan=0.0)  # rows with nothing visible
    out = torch.einsum("bhij,bjhd->bihd", w, v)
    return out.numpy(), lse.permute(0, 2, 1).numpy()


# --------------------------------------------------------------------------
# storage decoders


def test_f16_decoder_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.decode_f16(int(b)) for b in bits])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_bf16_decoder_exhaustive():
    bits = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.decode_bf16(int(b) & 0xFFFF) for b in bits.numpy()])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


# --------------------------------------------------------------------------
# closed forms


def test_single_key_gives_its_value_and_score():
    q, k, v = rnd((2, 3, 2, 8), 1), rnd((2, 1, 2, 8), 2), rnd((2, 1, 2, 8), 3)
    out, lse = oracle.attention(q, k, v)
    assert np.allclose(out, np.broadcast_to(v.astype(np.float64), out.shape), rtol=0, atol=1e-15)
    s = np.einsum("bihd,bjhd->bih", q.astype(np.float64), k.astype(np.float64)) / math.sqrt(8)
    assert np.allclose(lse, s, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_averages_visible_values(causal):
    N, d = 9, 4
    q = np.zeros((1, N, 1, d), np.float32)
    k, v = rnd((1, N, 1, d), 4), rnd((1, N, 1, d), 5)
    out, lse = oracle.attention(q, k, v, causal=causal)
    v64 = v[0, :, 0].astype(np.float64)
    for i in range(N):
        n_vis = i + 1 if causal else N
        assert abs(lse[0, i, 0] - math.log(n_vis)) < 1e-13
        assert np.allclose(out[0, i, 0], v64[:n_vis].mean(axis=0), rtol=0, atol=1e-13)
    # the number of computed pairs under the causal rule is N(N+1)/2
    total = sum(round(math.exp(x)) for x in lse[0, :, 0])
    assert total == (N * (N + 1) // 2 if causal else N * N)


def test_equal_keys_give_uniform_weights():
    N, d = 7, 8
    q = rnd((1, 5, 1, d), 6)
    k = np.repeat(rnd((1, 1, 1, d), 7), N, axis=1)
    v = rnd((1, N, 1, d), 8)
    out, lse = oracle.attention(q, k, v)
    s = (q[0, :, 0].astype(np.float64) @ k[0, 0, 0].astype(np.float64)) / math.sqrt(d)
    assert np.allclose(lse[0, :, 0], s + math.log(N), rtol=0, atol=1e-12)
    assert np.allclose(out[0, :, 0], v[0, :, 0].astype(np.float64).mean(0), rtol=0, atol=1e-13)


def test_causal_first_query_sees_only_first_key():
    q, k, v = rnd((1, 6, 3, 8), 9), rnd((1, 6, 3, 8), 10), rnd((1, 6, 3, 8), 11)
    out, lse = oracle.attention(q, k, v, causal=True)
    assert np.array_equal(out[0, 0], v[0, 0].astype(np.float64))
    s00 = (q[0, 0].astype(np.float64) * k[0, 0].astype(np.float64)).sum(-1) / math.sqrt(8)
    assert np.allclose(lse[0, 0], s00, rtol=0, atol=1e-12)


def test_hand_worked_example():
    g = golden("hand_d1_n2.json")
    q = np.array(g["q"], np.float32).reshape(1, 1, 1, 1)
    k = np.array(g["k"], np.float32).reshape(1, 2, 1, 1)
    v = np.array(g["v"], np.float32).reshape(1, 2, 1, 1)
    out, lse = oracle.attention(q, k, v, scale=g["scale"])
    assert abs(out[0, 0, 0, 0] - g["out"]) < 1e-13
    assert abs(lse[0, 0, 0] - g["lse"]) < 1e-13
    out, lse = oracle.attention(q, k, v, scale=g["scale"], causal=True,
                                q_pos=[0], k_pos=[0, 1])
    assert abs(out[0, 0, 0, 0] - g["causal_q_pos0"]["out"]) < 1e-13
    assert abs(lse[0, 0, 0] - g["causal_q_pos0"]["lse"]) < 1e-13


def test_dominant_key_wins():
    d, N, star = 16, 10, 6
    k, v = rnd((1, N, 1, d), 12), rnd((1, N, 1, d), 13)
    q = (k[:, star:star + 1] * 60.0).astype(np.float32)
    out, _ = oracle.attention(q, k, v)
    assert np.allclose(out[0, 0, 0], v[0, star, 0].astype(np.float64), atol=1e-6)


def test_no_visible_key_is_empty():
    q, k, v = rnd((1, 2, 1, 4), 14), rnd((1, 3, 1, 4), 15), rnd((1, 3, 1, 4), 16)
    out, lse = oracle.attention(q, k, v, causal=True, q_pos=[0, 10], k_pos=[5, 6, 7])
    assert np.all(out[0, 0] == 0) and np.isneginf(lse[0, 0, 0])
    assert np.isfinite(lse[0, 1, 0])
    out, lse = oracle.attention(q, k[:, :0], v[:, :0])
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# --------------------------------------------------------------------------
# textbook routine and brute force


@pytest.mark.parametrize("B,Nq,Nk,Hq,Hkv,d,causal", [
    (1, 33, 33, 1, 1, 16, False), (2, 40, 40, 4, 2, 32, True), (1, 65, 65, 8, 1, 64, True),
    (2, 17, 50, 6, 3, 8, False), (1, 128, 128, 2, 2, 128, True)])
def test_matches_textbook_softmax(B, Nq, Nk, Hq, Hkv, d, causal):
    q, k, v = rnd((B, Nq, Hq, d), 20), rnd((B, Nk, Hkv, d), 21), rnd((B, Nk, Hkv, d), 22)
    qp = np.arange(Nk - Nq, Nk)  # queries are the last Nq positions
    out, lse = oracle.attention(q, k, v, causal=causal, q_pos=qp)
    ro, rl = textbook(q, k, v, causal=causal, q_pos=qp)
    assert np.allclose(out, ro, rtol=0, atol=1e-12)
    assert np.allclose(lse, rl, rtol=0, atol=1e-12)


def test_matches_textbook_on_large_scores():
    # scores of several hundred: an unshifted exp would overflow
    q, k, v = rnd((1, 20, 2, 128), 23, 10.0), rnd((1, 20, 2, 128), 24, 10.0), rnd((1, 20, 2, 128), 25)
    out, lse = oracle.attention(q, k, v, causal=True)
    ro, rl = textbook(q, k, v, causal=True)
    assert np.all(np.isfinite(out)) and np.max(np.abs(lse)) > 100
    assert np.allclose(out, ro, rtol=0, atol=1e-10)
    assert np.allclose(lse, rl, rtol=1e-13, atol=0)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_16bit_storage_decoded_exactly(dtype):
    q, k, v = (torch.from_numpy(rnd((1, 24, 2, 32), s)).to(dtype) for s in (26, 27, 28))
    out, lse = oracle.attention(q, k, v, causal=True)
    ro, rl = textbook(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal=True)
    assert np.allclose(out, ro, rtol=0, atol=1e-12)
    assert np.allclose(lse, rl, rtol=0, atol=1e-12)


def test_matches_sdpa_float64():
    q, k, v = (torch.from_numpy(rnd((2, 31, 3, 16), s)).double() for s in (29, 30, 31))
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), is_causal=True).transpose(1, 2)
    out, _ = oracle.attention(q.float(), k.float(), v.float(), causal=True)
    # inputs were rounded to float32 for the oracle; compare on those values
    ref32 = torch.nn.functional.scaled_dot_product_attention(
        q.float().double().transpose(1, 2), k.float().double().transpose(1, 2),
        v.float().double().transpose(1, 2), is_causal=True).transpose(1, 2)
    assert np.allclose(out, ref32.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(out, ref.numpy(), atol=1e-5)


def brute_force(q, k, v, causal, scale):
    """Pure-Python loops; weights exp(s_j)/sum exp(s_i) without any shift."""
    Nq, d = len(q), len(q[0])
    Nk = len(k)
    out, lse = [], []
    for i in range(Nq):
        vis = [j for j in range(Nk) if not causal or j <= i]
        e = {j: math.exp(scale * sum(q[i][t] * k[j][t] for t in range(d))) for j in vis}
        z = sum(e.values())
        out.append([sum(e[j] * v[j][t] for j in vis) / z for t in range(d)])
        lse.append(math.log(z))
    return out, lse


@pytest.mark.parametrize("N,d,causal", [(1, 1, False), (2, 3, True), (5, 4, False), (6, 2, True)])
def test_brute_force_tiny(N, d, causal):
    q, k, v = rnd((1, N, 1, d), 40 + N), rnd((1, N, 1, d), 50 + N), rnd((1, N, 1, d), 60 + N)
    scale = 0.7
    out, lse = oracle.attention(q, k, v, causal=causal, scale=scale)
    bo, bl = brute_force(q[0, :, 0].tolist(), k[0, :, 0].tolist(), v[0, :, 0].tolist(),
                         causal, scale)
    assert np.allclose(out[0, :, 0], np.array(bo), rtol=0, atol=1e-13)
    assert np.allclose(lse[0, :, 0], np.array(bl), rtol=0, atol=1e-13)


def test_default_scale_is_inverse_sqrt_d():
    q, k, v = rnd((1, 5, 1, 9), 70), rnd((1, 6, 1, 9), 71), rnd((1, 6, 1, 9), 72)
    a = oracle.attention(q, k, v)
    b = oracle.attention(q, k, v, scale=1 / 3)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_sampled_rows_match_full():
    q, k, v = rnd((2, 20, 4, 8), 73), rnd((2, 20, 2, 8), 74), rnd((2, 20, 2, 8), 75)
    full_o, full_l = oracle.attention(q, k, v, causal=True)
    rows = workloads.sample_rows(2, 20, 4, 30, seed=3, forced=[(1, 19, 3)])
    o, l = oracle.attention(q, k, v, causal=True, rows=rows)
    for n, (b, i, h) in enumerate(rows):
        assert np.array_equal(o[n], full_o[b, i, h]) and l[n] == full_l[b, i, h]


# --------------------------------------------------------------------------
# the pages' claims


def test_page_ring_simulation_reproduced():
    """ultralytics.com: the 4-device simulation matches full attention (True)."""
    g = golden("ultralytics_ring_sim.json")
    r = g["recipe"]
    q, k, v = workloads.page_ring_sim_inputs()
    torch.manual_seed(r["seed"])
    q2, k2, v2 = torch.randn(3, r["n_devices"] * r["block"], r["dim"])
    assert torch.equal(q, q2) and torch.equal(k, k2) and torch.equal(v, v2)
    # the page's loop, in float32 as on the page
    n, blk, dim = r["n_devices"], r["block"], r["dim"]
    qb, kb, vb = q.chunk(n), k.chunk(n), v.chunk(n)
    outs = []
    largest = 0
    for i in range(n):
        num, den = torch.zeros(blk, dim), torch.zeros(blk, 1)
        for step in range(n):
            j = (i - step) % n
            p = torch.exp(qb[i] @ kb[j].T / dim ** 0.5)
            largest = max(largest, p.shape[0] * p.shape[1])
            num += p @ vb[j]
            den += p.sum(dim=-1, keepdim=True)
        outs.append(num / den)
    full = torch.softmax(q @ k.T / dim ** 0.5, dim=-1) @ v
    assert torch.allclose(torch.cat(outs), full, atol=1e-5) == g["printed"]["matches_full_attention"]
    assert f"{blk}x{blk}" == g["printed"]["largest_block"] and largest == blk * blk
    assert f"{len(q)}x{len(k)}" == g["printed"]["full_matrix"]
    # the oracle on the same inputs agrees with that loop and with its fp64 restatement
    out, lse = oracle.attention(q.reshape(1, 32, 1, 16), k.reshape(1, 32, 1, 16),
                                v.reshape(1, 32, 1, 16))
    assert np.allclose(out[0, :, 0], torch.cat(outs).numpy(), atol=1e-5)
    sim = recurrences.ring_simulation(q.numpy(), k.numpy(), v.numpy(), n)
    assert np.allclose(out[0, :, 0], sim, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_block_size_invariance(causal):
    N, d = 37, 8
    q, k, v = rnd((N, d), 80), rnd((N, d), 81), rnd((N, d), 82)
    out, lse = oracle.attention(q[None, :, None], k[None, :, None], v[None, :, None],
                                causal=causal)
    for Br, Bc in itertools.product([1, 3, 5, 8, 16, 32], repeat=2):
        bo, bl = recurrences.tiled_online_softmax(q, k, v, Br, Bc, causal=causal)
        assert np.allclose(bo, out[0, :, 0], rtol=0, atol=1e-12), (Br, Bc)
        assert np.allclose(bl, lse[0, :, 0], rtol=0, atol=1e-12), (Br, Bc)


def test_ring_order_invariance():
    q, k, v = workloads.page_ring_sim_inputs()
    q, k, v = q.numpy(), k.numpy(), v.numpy()
    out, lse = oracle.attention(q[None, :, None], k[None, :, None], v[None, :, None])
    kb, vb = np.split(k, 4), np.split(v, 4)
    for perm in itertools.permutations(range(4)):
        o, l = recurrences.online_softmax_over_blocks(q, [kb[j] for j in perm],
                                                      [vb[j] for j in perm])
        assert np.allclose(o, out[0, :, 0], rtol=0, atol=1e-12)
        assert np.allclose(l, lse[0, :, 0], rtol=0, atol=1e-12)
    for direction in (-1, +1):
        sim = recurrences.ring_simulation(q, k, v, 4, direction=direction)
        assert np.allclose(sim, out[0, :, 0], rtol=0, atol=1e-12)


def test_zigzag_layout_matches_page_example():
    g = golden("twinkle_zigzag_layout.json")
    W, n_chunks = g["n_devices"], g["n_chunks"]
    c = 3
    N = n_chunks * c
    for r, chunks in enumerate(g["device_chunks"]):
        pos = layouts.zigzag_shard_positions(N, W, r)
        expect = np.concatenate([np.arange(ch * c, (ch + 1) * c) for ch in chunks])
        assert np.array_equal(pos, expect)
    # every position is held by exactly one device
    allpos = np.concatenate([layouts.zigzag_shard_positions(N, W, r) for r in range(W)])
    assert np.array_equal(np.sort(allpos), np.arange(N))


@pytest.mark.parametrize("W", [1, 2, 3, 4, 8])
def test_zigzag_ring_equals_causal_attention(W):
    c, d = 5, 8
    N = 2 * W * c
    q, k, v = rnd((N, d), 90 + W), rnd((N, d), 100 + W), rnd((N, d), 110 + W)
    shards = [layouts.zigzag_shard_positions(N, W, r) for r in range(W)]
    full_o, full_l = oracle.attention(q[None, :, None], k[None, :, None], v[None, :, None],
                                      causal=True)
    for r in range(W):
        o, l = recurrences.zigzag_ring_forward([q[s] for s in shards], [k[s] for s in shards],
                                               [v[s] for s in shards], W, r)
        assert np.allclose(o, full_o[0, shards[r], 0], rtol=0, atol=1e-12)
        assert np.allclose(l, full_l[0, shards[r], 0], rtol=0, atol=1e-12)
        # and the oracle fed the shard with its positions directly agrees too
        so, sl = oracle.attention(q[None, shards[r], None], k[None, :, None], v[None, :, None],
                                  causal=True, q_pos=shards[r])
        assert np.allclose(so[0, :, 0], o, rtol=0, atol=1e-12)


@pytest.mark.parametrize("N,W", [(32, 4), (24, 3), (64, 8)])
def test_striped_layout_spreads_tokens_evenly(N, W):
    """Every position belongs to exactly one device, and each device's
    positions are spaced W apart (the ultralytics page's even spread)."""
    allpos = np.concatenate([layouts.striped_shard_positions(N, W, r) for r in range(W)])
    assert np.array_equal(np.sort(allpos), np.arange(N))
    for r in range(W):
        p = layouts.striped_shard_positions(N, W, r)
        assert p[0] == r and np.all(np.diff(p) == W)


def test_striped_step_rule_is_the_causal_rule():
    """Brute force: the local rule j + offset <= i is the position rule
    src + W j <= rank + W i, for every pair of devices and rows."""
    for W in (1, 2, 3, 5, 8):
        for rank in range(W):
            for src in range(W):
                off = layouts.striped_key_offset(rank, src)
                for i in range(6):
                    for j in range(6):
                        assert (j + off <= i) == (src + W * j <= rank + W * i)


@pytest.mark.parametrize("W", [1, 2, 3, 4, 8])
def test_striped_ring_equals_causal_attention(W):
    S, d = 6, 8
    N = W * S
    q, k, v = rnd((N, d), 190 + W), rnd((N, d), 200 + W), rnd((N, d), 210 + W)
    shards = [layouts.striped_shard_positions(N, W, r) for r in range(W)]
    full_o, full_l = oracle.attention(q[None, :, None], k[None, :, None], v[None, :, None],
                                      causal=True)
    for r in range(W):
        o, l = recurrences.striped_ring_forward([q[s] for s in shards], [k[s] for s in shards],
                                                [v[s] for s in shards], W, r)
        assert np.allclose(o, full_o[0, shards[r], 0], rtol=0, atol=1e-12)
        assert np.allclose(l, full_l[0, shards[r], 0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("W,rank", [(4, 0), (4, 3), (3, 1)])
def test_contiguous_ring_causal_equals_blocks(W, rank):
    """Contiguous ring: causal attention of device r's block over all key blocks
    equals the merge of the per-step blocks (skip later blocks, mask the own)."""
    S, d = 6, 4
    N = W * S
    q, k, v = rnd((N, d), 120), rnd((N, d), 121), rnd((N, d), 122)
    pos = layouts.contiguous_shard_positions(N, W, rank)
    o = np.zeros((S, d))
    l = np.full(S, -np.inf)
    for step in range(W):
        src = layouts.ring_source(rank, step, W)
        kpos = layouts.contiguous_shard_positions(N, W, src)
        if src > rank:
            continue  # entirely in the future
        bo, bl = oracle.attention(q[None, pos, None], k[None, kpos, None], v[None, kpos, None],
                                  causal=True, q_pos=pos, k_pos=kpos)
        o, l = oracle.merge(o, l, bo[0, :, 0], bl[0, :, 0])
    ref_o, ref_l = textbook(q[None, pos, None], k[None, :, None], v[None, :, None],
                            causal=True, q_pos=pos)
    assert np.allclose(o, ref_o[0, :, 0], rtol=0, atol=1e-12)
    assert np.allclose(l, ref_l[0, :, 0], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# merge


def test_merge_of_split_key_sets_equals_whole():
    N, d = 40, 8
    q, k, v = rnd((1, 7, 1, d), 130), rnd((1, N, 1, d), 131), rnd((1, N, 1, d), 132)
    full_o, full_l = textbook(q, k, v)
    for cuts in ([20], [5, 30], [1, 2, 3, 39], [10, 20, 30]):
        bounds = [0] + cuts + [N]
        o = np.zeros((7, d))
        l = np.full(7, -np.inf)
        for a, b in zip(bounds[:-1], bounds[1:]):
            bo, bl = oracle.attention(q, k[:, a:b], v[:, a:b])
            o, l = oracle.merge(o, l, bo[0, :, 0], bl[0, :, 0])
        assert np.allclose(o, full_o[0, :, 0], rtol=0, atol=1e-12)
        assert np.allclose(l, full_l[0, :, 0], rtol=0, atol=1e-12)


def test_merge_algebra():
    rng = np.random.default_rng(140)
    o = [rng.standard_normal((11, 4)) for _ in range(3)]
    l = [rng.standard_normal(11) * 3 for _ in range(3)]
    ab = oracle.merge(o[0], l[0], o[1], l[1])
    ba = oracle.merge(o[1], l[1], o[0], l[0])
    assert np.allclose(ab[0], ba[0], rtol=0, atol=1e-14) and np.allclose(ab[1], ba[1], atol=1e-14)
    left = oracle.merge(*ab, o[2], l[2])
    bc = oracle.merge(o[1], l[1], o[2], l[2])
    right = oracle.merge(o[0], l[0], *bc)
    assert np.allclose(left[0], right[0], atol=1e-13) and np.allclose(left[1], right[1], atol=1e-13)
    # lse is the log of the summed exponentials
    assert np.allclose(ab[1], np.log(np.exp(l[0]) + np.exp(l[1])), rtol=0, atol=1e-13)


def test_sigmoid_form_equals_logaddexp_form():
    rng = np.random.default_rng(141)
    o_a, o_b = rng.standard_normal((50, 6)), rng.standard_normal((50, 6))
    l_a, l_b = rng.standard_normal(50) * 20, rng.standard_normal(50) * 20
    so, sl = recurrences.sigmoid_merge(o_a, l_a, o_b, l_b)
    mo, ml = oracle.merge(o_a, l_a, o_b, l_b)
    assert np.allclose(so, mo, rtol=0, atol=1e-12) and np.allclose(sl, ml, rtol=0, atol=1e-12)


def test_merge_with_empty_sides():
    o = np.arange(8.0).reshape(2, 4)
    l = np.array([1.5, -2.0])
    empty_o, empty_l = np.zeros((2, 4)), np.full(2, -np.inf)
    for args in ((o, l, empty_o, empty_l), (empty_o, empty_l, o, l)):
        mo, ml = oracle.merge(*args)
        assert np.array_equal(mo, o) and np.array_equal(ml, l)
    mo, ml = oracle.merge(empty_o, empty_l, empty_o, empty_l)
    assert np.all(mo == 0) and np.all(np.isneginf(ml))
    # the page's sigmoid form, taken literally, is NaN here; the reading makes it the identity
    with np.errstate(all="ignore"):
        lit = empty_l - np.log(1 / (1 + np.exp(-(empty_l - l))))
    assert np.all(np.isnan(lit))
    so, sl = recurrences.sigmoid_merge(empty_o, empty_l, o, l)
    assert np.array_equal(so, o) and np.array_equal(sl, l)


# --------------------------------------------------------------------------
# LSE


def test_lse_normalises_the_weights():
    q, k, v = rnd((1, 12, 2, 16), 150), rnd((1, 12, 2, 16), 151), rnd((1, 12, 2, 16), 152)
    _, lse = oracle.attention(q, k, v, causal=True)
    q64, k64 = q.astype(np.float64), k.astype(np.float64)
    for i in range(12):
        for h in range(2):
            s = np.array([q64[0, i, h] @ k64[0, j, h] for j in range(i + 1)]) / 4.0
            assert abs(np.exp(s - lse[0, i, h]).sum() - 1.0) < 1e-13
            assert s.max() <= lse[0, i, h] <= s.max() + math.log(i + 1) + 1e-15


# --------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin


def _pin_battery(lib_path):
    """A fast subset of the pins above, run against a given build of oracle.c.
    Returns the names of the pins that fail."""
    failed = []

    def att(*a, **kw):
        return oracle.attention(*a, lib_path=lib_path, **kw)

    def check(name, fn):
        try:
            if not fn():
                failed.append(name)
        except Exception:  # a crash or a rejected call is a failure too
            failed.append(name)

    q, k, v = rnd((2, 40, 4, 32), 20), rnd((2, 40, 2, 32), 21), rnd((2, 40, 2, 32), 22)

    def textbook_pin():
        out, lse = att(q, k, v, causal=True)
        ro, rl = textbook(q, k, v, causal=True)
        return np.allclose(out, ro, atol=1e-12) and np.allclose(lse, rl, atol=1e-12)

    def large_pin():
        a, b, c = rnd((1, 20, 2, 128), 23, 10.0), rnd((1, 20, 2, 128), 24, 10.0), rnd((1, 20, 2, 128), 25)
        out, lse = att(a, b, c, causal=True)
        ro, rl = textbook(a, b, c, causal=True)
        return np.allclose(out, ro, atol=1e-10) and np.allclose(lse, rl, rtol=1e-13, atol=0)

    def f16_pin():
        a, b, c = (torch.from_numpy(rnd((1, 24, 2, 32), s)).to(torch.float16) for s in (26, 27, 28))
        out, _ = att(a, b, c, causal=True)
        ro, _ = textbook(a.double().numpy(), b.double().numpy(), c.double().numpy(), causal=True)
        return np.allclose(out, ro, atol=1e-12)

    def hand_pin():
        g = golden("hand_d1_n2.json")
        out, lse = att(np.array(g["q"], np.float32).reshape(1, 1, 1, 1),
                       np.array(g["k"], np.float32).reshape(1, 2, 1, 1),
                       np.array(g["v"], np.float32).reshape(1, 2, 1, 1), scale=g["scale"])
        return abs(out[0, 0, 0, 0] - g["out"]) < 1e-13 and abs(lse[0, 0, 0] - g["lse"]) < 1e-13

    def zero_query_pin():
        z = np.zeros((1, 9, 1, 4), np.float32)
        _, lse = att(z, rnd((1, 9, 1, 4), 4), rnd((1, 9, 1, 4), 5), causal=True)
        return np.allclose(lse[0, :, 0], np.log(np.arange(1, 10)), atol=1e-13)

    check("textbook", textbook_pin)
    check("large_scores", large_pin)
    check("f16_storage", f16_pin)
    check("hand_example", hand_pin)
    check("zero_query_causal", zero_query_pin)
    return failed


def test_pin_battery_passes_on_the_oracle():
    assert _pin_battery(None) == []


MUTATIONS = {
    "causal_off_by_one": ("k_pos[j] > q_pos[i]", "k_pos[j] >= q_pos[i]"),
    "dropped_scale": ("s[j] = scale * dot;", "s[j] = dot;"),
    "wrong_gqa_map": ("const int64_t g = hq / group;", "const int64_t g = hq % Hkv;"),
    "lse_without_max": ("*lse_r = M + log(Z);", "*lse_r = log(Z);"),
    "k_used_as_v": ("acc[t] += w * load(v, vbase + t, dtype);",
                    "acc[t] += w * load(k, vbase + t, dtype);"),
    "f16_exponent_off": ("e - 25);", "e - 24);"),
    "unshifted_exp": ("const double w = exp(s[j] - M);", "const double w = exp(s[j]);"),
    "q_head_stride": ("((b * Nq + i) * Hq + hq) * d + t", "((b * Nq + i) * Hq + hq / group) * d + t"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = MUTATIONS[name]
    assert old in src, f"mutation anchor for {name} not found"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = str(tmp_path / "liboracle_mut.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", str(mutated), "-o", lib, "-lm"],
                   check=True)
    assert _pin_battery(lib), f"planted mistake {name} went unnoticed"
