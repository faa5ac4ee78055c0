"""The direct-to-LDS forward kernel (d = 128 and d = 64) vs the fp64 oracle
where the online softmax's running maximum moves (needs a GPU).

The kernel keeps a running row max m and rescales the accumulator by
exp(m_old - m_new) only when a score exceeds m by more than a slack (lazy
rescaling); it takes the exact row max only when a tile's row sums show that
m may have to move.  These cases drive both decisions: scores of large
magnitude, a ramp that moves the max on every key tile, and tiles whose
scores sit just below, at and just above the thresholds.  Each runs through
the whole-schedule call (rattn_fwd) and through ring steps merged by the
log-sum-exp correction, in the step epilogue and as separate merges
(the correction exp(m_old - m_new) of the youngju.dev blockwise attention;
the guijiagi.com page's online-softmax section).

Tolerances as for every 16-bit case: max |dO| <= 2e-2, |dLSE| <= 1e-3.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import layouts
from ring_attention_amd import binding, ring

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 2e-2, 1e-3
LN2 = math.log(2.0)


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(out, lse, ref_o, ref_l, what):
    out = out.detach().float().cpu().numpy().astype(np.float64)
    lse = lse.detach().float().cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref_l)), f"{what}: empty rows differ"
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    fin = ~np.isneginf(ref_l)
    err_o = float(np.max(np.abs(out - ref_o)))
    err_l = float(np.max(np.abs(lse[fin] - ref_l[fin]))) if fin.any() else 0.0
    note(f"{what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
    assert err_o <= TOL_O and err_l <= TOL_LSE, what


def run_all_paths(q, k, v, scale, what, W=2):
    """rattn_fwd (non-causal and causal) and W-device ZigZag ring steps with
    fused and separate merges, each against the oracle."""
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    N = k.shape[1]
    for causal in (False, True):
        out, lse = binding.fwd(qd, kd, vd, causal=causal, scale=scale)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.attention(q, k, v, causal=causal, scale=scale)
        check(out, lse, ref_o, ref_l, f"{what} fwd causal={causal}")
    ks = [ring.shard(kd, W, True, r) for r in range(W)]
    vs = [ring.shard(vd, W, True, r) for r in range(W)]
    for r in range(W):
        qs = ring.shard(q, W, True, r)
        ref_o, ref_l = oracle.attention(qs, k, v, causal=True, scale=scale,
                                        q_pos=layouts.shard_positions(N, W, r, True))
        for fused in (True, False):
            out, lse = ring.ring_forward_steps(qs.to(dev), ks, vs, W, True, r, causal=True,
                                               scale=scale, fused_merge=fused)
            torch.cuda.synchronize()
            check(out, lse, ref_o, ref_l, f"{what} ring steps rank={r} fused={fused}")


HEAD_DIMS = [128, 64, 32]


@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_large_magnitude_scores(gpu, dtype, d):
    """q, k ~ N(0, 10^2): scores of several hundred, softmax close to argmax."""
    g = torch.Generator().manual_seed(61)
    N = 2 * 256 + 88  # three query tiles, ragged last tile; 9 key tiles + 24
    q = (torch.randn(1, N, 4, d, generator=g) * 10).to(dtype)
    k = (torch.randn(1, N, 2, d, generator=g) * 10).to(dtype)
    v = torch.randn(1, N, 2, d, generator=g).to(dtype)
    run_all_paths(q, k, v, None, f"large scores d={d} {dtype}")


@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_max_moves_every_key_tile(gpu, dtype, d):
    """A score ramp: every 64-key tile's scores exceed all earlier ones by
    more than 8 base-2 units (6.4 natural units per tile), so the running
    max moves, and the accumulator is rescaled, on every key tile."""
    g = torch.Generator().manual_seed(62)
    N = 640
    q = torch.zeros(1, N, 2, d)
    q[..., 0] = 1.0
    q[..., 1:] = torch.randn(1, N, 2, d - 1, generator=g) * 0.05
    k = torch.randn(1, N, 1, d, generator=g) * 0.05
    # score of key j for every query: scale * k_j[0] = 0.1 j (+ small noise)
    k[0, :, 0, 0] = 0.1 * torch.arange(N, dtype=torch.float32) * math.sqrt(d)
    v = torch.randn(1, N, 1, d, generator=g)
    run_all_paths(q.to(dtype), k.to(dtype), v.to(dtype), None, f"ramp d={d} {dtype}")


# Raise of each key tile's scores over the first tile's, in base-2 units of
# the scaled score: around 2 a lane's 32 values of p sum to the bound that
# sends the tile to the exact-max path (32 * 2^2 = 128); around 8 a single p
# reaches 2^8, the rescaling threshold; 12 and 20.1 rescale for certain.
JUMPS = [0.0, 1.0, 1.9375, 2.0, 2.0625, 3.0, 7.9375, 8.0, 8.0625, 12.0, 12.0, 20.125, 19.0]


@pytest.mark.parametrize("d", HEAD_DIMS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_thresholds_of_lazy_rescaling(gpu, dtype, d):
    """Every key tile holds 64 equal scores J_t (base-2 units; q = e_0, the
    scale ln2 / 16 and k_j[0] = 16 J_t, all exact in 16 bits), with J_t
    stepping through the values above, below and at the thresholds.  Every
    query is e_0, so all rows see the same scores (causal rows a prefix)."""
    g = torch.Generator().manual_seed(63)
    T = len(JUMPS)
    N = 64 * T
    q = torch.zeros(1, N, 2, d)
    q[..., 0] = 1.0
    k = torch.zeros(1, N, 1, d)
    for t, j in enumerate(JUMPS):
        k[0, 64 * t:64 * (t + 1), 0, 0] = 16.0 * j
    k[..., 1:] = torch.randn(1, N, 1, d - 1, generator=g)  # not seen by q = e_0
    v = torch.randn(1, N, 1, d, generator=g)
    run_all_paths(q.to(dtype), k.to(dtype), v.to(dtype), LN2 / 16, f"thresholds d={d} {dtype}")


@pytest.mark.parametrize("d", HEAD_DIMS)
def test_tile_sums_at_the_slow_path_bound(gpu, d):
    """Scores spread so that some lanes' tile sums land just below and just
    above the exact-max bound while no single p comes near 2^8: per key
    tile, key i has score log2 of a value that makes the 32 keys of a lane
    sum to 127, 128 or 129 times the first tile's p."""
    g = torch.Generator().manual_seed(64)
    base = np.zeros(64)
    tiles = [base]
    for target in (127.0, 128.0, 129.0, 64.0, 200.0):
        # lane halves hold keys 8(r/4) + 4h + r%4 of each 32-key block:
        # give every key the same p = target / 32 (base-2 score log2 of it)
        tiles.append(np.full(64, math.log2(target / 32.0)))
    J = np.concatenate(tiles)
    N = J.size
    q = torch.zeros(1, N, 2, d)
    q[..., 0] = 1.0
    k = torch.zeros(1, N, 1, d)
    k[0, :, 0, 0] = torch.from_numpy(16.0 * J).float()
    k[..., 1:] = torch.randn(1, N, 1, d - 1, generator=g)
    v = torch.randn(1, N, 1, d, generator=g)
    for dtype in (torch.bfloat16, torch.float16):
        run_all_paths(q.to(dtype), k.to(dtype), v.to(dtype), LN2 / 16, f"tile sums d={d} {dtype}")
