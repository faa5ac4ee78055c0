"""The pages' own algorithms, restated in numpy float64 -- TEST INFRASTRUCTURE.

These are not the oracle (the oracle is the definition in ``oracle.c``).  They
exist so that tests can check, against that definition, what the pages claim:
that the blockwise online softmax, the ring simulation and the ZigZag step
rules with the log-sum-exp merge all reach exact attention.  Each one follows
the steps of the algorithm it names in the pages' notation (running row max m,
running sum l, unnormalised accumulator O), written from the description, not
transcribed from a listing.

Single-head arrays: q [Nq, d], k and v [Nk, d], float64.
"""
from __future__ import annotations

import math

import numpy as np


def _exp_shift(x, m):
    """exp(x - m) with exp(-inf - (-inf)) taken as 0 (rows with nothing visible)."""
    with np.errstate(invalid="ignore"):
        r = np.exp(x - m)
    return np.where(np.isneginf(x), 0.0, r)


def _stream_tiles(q, tiles, scale: float):
    """Online softmax of the rows of q over a sequence of key/value tiles.

    State per query row: the running maximum m of the scaled scores and an
    accumulator A = [O | l] over the value columns augmented with a column of
    ones, since the denominator l is the same exponential-weighted sum as O
    with every value replaced by 1.  A tile with scores S (masked entries
    -inf) moves the state to m' = max(m, max_j S_j) and
    A' = exp(m - m') A + exp(S - m') [V | 1]; after the last tile
    O = A[:, :d] / A[:, d] and lse = m' + log A[:, d] (rows that saw no key
    keep O = 0, lse = -inf).  tiles: (K_t, V_t, hidden_t) with hidden_t a
    boolean [rows, keys] mask or None.
    """
    n, dv = q.shape[0], None
    m = np.full(n, -np.inf)
    acc = None
    for kt, vt, hidden in tiles:
        s_t = (q @ kt.T) * scale
        if hidden is not None:
            s_t = np.where(hidden, -np.inf, s_t)
        v_aug = np.concatenate([vt, np.ones((vt.shape[0], 1))], axis=1)
        if acc is None:
            dv = vt.shape[1]
            acc = np.zeros((n, dv + 1))
        m_next = np.maximum(m, s_t.max(axis=1, initial=-np.inf))
        acc = _exp_shift(m, m_next)[:, None] * acc + _exp_shift(s_t, m_next[:, None]) @ v_aug
        m = m_next
    den = acc[:, dv]
    out = np.zeros((n, dv))
    lse = np.full(n, -np.inf)
    seen = den > 0
    out[seen] = acc[seen, :dv] / den[seen, None]
    lse[seen] = m[seen] + np.log(den[seen])
    return out, lse


def tiled_online_softmax(q, k, v, Br: int, Bc: int, scale: float | None = None,
                         causal: bool = False, q_pos=None, k_pos=None):
    """Attention computed tile by tile: query tiles of Br rows, each streaming
    key/value tiles of Bc rows through the online softmax (``_stream_tiles``),
    one division at the end.

    The recurrence is the FlashAttention forward of the yz520gzy chapter
    (ceil(N / B) tiles per side, so ragged tails are kept; the
    FlashAttention-2 variant's single normalisation) with the running-max
    correction of the youngju.dev blockwise attention; causal masking by
    position (a key after the query is hidden).
    Returns (O [Nq, d], lse [Nq]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Nq, d = q.shape
    Nk = k.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qp = np.arange(Nq) if q_pos is None else np.asarray(q_pos)
    kp = np.arange(Nk) if k_pos is None else np.asarray(k_pos)
    out = np.zeros((Nq, v.shape[1]))
    lse = np.full(Nq, -np.inf)
    for i0 in range(0, Nq, Br):
        rows = slice(i0, min(Nq, i0 + Br))
        tiles = [(k[j0:j0 + Bc], v[j0:j0 + Bc],
                  (kp[None, j0:j0 + Bc] > qp[rows, None]) if causal else None)
                 for j0 in range(0, Nk, Bc)]
        out[rows], lse[rows] = _stream_tiles(q[rows], tiles, scale)
    return out, lse


def ring_simulation(q, k, v, n_devices: int, direction: int = -1):
    """The ultralytics page's single-process simulation of a ring of devices.

    Device i keeps query block i; at step s it holds key/value block
    j = (i + direction*s) mod n (direction -1: each device receives from its
    predecessor, as on that page; +1 is the opposite rotation drawn on the
    guijiagi.com page).  As on the ultralytics page, numerator and denominator
    are plain sums of exp(scores) without subtracting a running maximum, and
    the division happens once at the end.  Non-causal.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dim = q.shape[1]
    qb, kb, vb = (np.array_split(x, n_devices) for x in (q, k, v))
    outs = []
    for i in range(n_devices):
        num = np.zeros((qb[i].shape[0], v.shape[1]))
        den = np.zeros((qb[i].shape[0], 1))
        for s in range(n_devices):
            j = (i + direction * s) % n_devices
            p = np.exp(qb[i] @ kb[j].T / math.sqrt(dim))
            num += p @ vb[j]
            den += p.sum(axis=1, keepdims=True)
        outs.append(num / den)
    return np.concatenate(outs)


def sigmoid_merge(out, lse, block_out, block_lse):
    """The log-sum-exp merge in the logistic form of the Twinkle page's
    ``update_out_and_lse``: with a = lse and b = block_lse, the merged output
    is the convex combination sigma(a - b) out + sigma(b - a) block_out
    (sigma the logistic function) and the merged lse is a + softplus(b - a).
    Read literally the page's form is NaN when a side is -inf; the reading
    used here: an empty side (lse = -inf) contributes nothing, so the other
    side is returned unchanged, and two empty sides stay empty (out 0,
    lse -inf).  out: [n, d], lse: [n].
    """
    out = np.array(out, np.float64)
    lse = np.array(lse, np.float64)
    block_out = np.asarray(block_out, np.float64)
    block_lse = np.asarray(block_lse, np.float64)
    a_empty = np.isneginf(lse)
    b_empty = np.isneginf(block_lse)
    both = ~a_empty & ~b_empty
    t = block_lse[both] - lse[both]
    w_b = 1.0 / (1.0 + np.exp(-t))          # sigma(b - a)
    w_a = 1.0 / (1.0 + np.exp(t))           # sigma(a - b)
    out[both] = w_a[:, None] * out[both] + w_b[:, None] * block_out[both]
    softplus = np.maximum(t, 0.0) + np.log1p(np.exp(-np.abs(t)))
    lse[both] = lse[both] + softplus
    take_b = a_empty & ~b_empty
    out[take_b] = block_out[take_b]
    lse[take_b] = block_lse[take_b]
    out[a_empty & b_empty] = 0.0
    return out, lse


def _attend(q, k, v, scale, causal, q_pos=None, k_pos=None):
    """Softmax attention of one block (the local kernel a ring step calls),
    returning the normalised block output and its lse; textbook numpy."""
    S = (q @ k.T) * scale
    if causal:
        S = np.where(k_pos[None, :] > q_pos[:, None], -np.inf, S)
    m = S.max(axis=1)
    fin = np.isfinite(m)
    P = np.zeros_like(S)
    P[fin] = np.exp(S[fin] - m[fin, None])
    l = P.sum(axis=1)
    out = np.zeros((q.shape[0], v.shape[1]))
    out[fin] = (P[fin] @ v) / l[fin, None]
    lse = np.full(q.shape[0], -np.inf)
    lse[fin] = m[fin] + np.log(l[fin])
    return out, lse


def zigzag_ring_forward(q_shards, k_shards, v_shards, W: int, rank: int,
                        scale: float | None = None):
    """One device of the ZigZag ring (Twinkle page, forward-pass section).

    *_shards[r] is device r's [front; back] shard (2c rows each).  Device
    ``rank`` runs W steps; at step s it holds the shard of device (rank - s)
    mod W and applies the step rules (see layouts.zigzag_step_plan); each
    step's normalised output and lse are folded into the running (out, lse)
    with ``sigmoid_merge``, the back-half steps touching only the back rows.
    Returns (out [2c, d], lse [2c]) in the local [front; back] order.
    """
    from .layouts import zigzag_step_plan

    q = np.asarray(q_shards[rank], np.float64)
    two_c, d = q.shape
    c = two_c // 2
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    local = np.arange(two_c)
    out = np.zeros((two_c, np.asarray(v_shards[0]).shape[1]))
    lse = np.full(two_c, -np.inf)
    for step in range(W):
        q_rows, kv_rows, causal, src = zigzag_step_plan(W, rank, step, c)
        k = np.asarray(k_shards[src], np.float64)[kv_rows]
        v = np.asarray(v_shards[src], np.float64)[kv_rows]
        # step 0 is causal on the local [front; back] order; front < back
        # globally, so local row order is a valid stand-in for position.
        bo, bl = _attend(q[q_rows], k, v, scale, causal, local[q_rows], local[kv_rows])
        out[q_rows], lse[q_rows] = sigmoid_merge(out[q_rows], lse[q_rows], bo, bl)
    return out, lse


def online_softmax_over_blocks(q, k_blocks, v_blocks, scale: float | None = None):
    """One pass of the online softmax over key/value blocks in the order
    given (the guijiagi.com page's online-softmax section: a running max and
    sum, a rescaling factor exp(m - m_new), the division at the end), for a
    matrix of query rows; the recurrence is ``_stream_tiles``.
    Returns (O [Nq, d], lse [Nq])."""
    q = np.asarray(q, np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[1])
    tiles = [(np.asarray(kb, np.float64), np.asarray(vb, np.float64), None)
             for kb, vb in zip(k_blocks, v_blocks)]
    return _stream_tiles(q, tiles, scale)


def ring_backward(q, k, v, o, lse, do, W: int, rank: int, scale: float | None = None):
    """The ring backward of one device, simulated: gradients of the device's
    query block and of every key/value block, non-causal.

    What the youngju.dev ring backward relies on, written as whole matrices:
    the probabilities are recomputed from the saved log-sum-exp,
    P = exp(scale Q K^T - lse), and the gradient of sum(dO * O) with respect
    to the scaled scores is G = P * (dO V^T - D) with D = rowsum(dO * O)
    taken from the saved output.  Then dQ = scale G K, dK = scale G^T Q and
    dV = P^T dO.  The ring splits the keys into W blocks: at step s the
    device holds block (rank - s) mod W and adds that block's columns of G
    and P to dQ, and forms that block's dK and dV, which go back to the
    block's owner (here: written into the rows of the block).

    q, o, do: [Nq, d] (this device's query block), lse [Nq]; k, v: [Nk, d]
    (the whole sequence, W equal blocks).  Returns (dQ [Nq, d], dK, dV [Nk, d])
    where dK, dV hold this device's contribution to every block.
    """
    q, k, v, o, do = (np.asarray(x, np.float64) for x in (q, k, v, o, do))
    lse = np.asarray(lse, np.float64)
    Nk, d = k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if Nk % W:
        raise ValueError("Nk must be a multiple of W")
    blk = Nk // W
    P = _exp_shift(scale * (q @ k.T), lse[:, None])
    G = P * (do @ v.T - (do * o).sum(axis=1, keepdims=True))
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for step in range(W):
        cols = slice(((rank - step) % W) * blk, ((rank - step) % W + 1) * blk)
        dQ += scale * (G[:, cols] @ k[cols])
        dK[cols] = scale * (G[:, cols].T @ q)
        dV[cols] = P[:, cols].T @ do
    return dQ, dK, dV


def striped_ring_forward(q_shards, k_shards, v_shards, W: int, rank: int,
                         scale: float | None = None):
    """One device of a causal ring over the Striped layout: at step s device
    ``rank`` holds the shard of device (rank - s) mod W (the ultralytics ring
    order) and attends to it under the striped step rule (layouts.
    striped_key_offset) in local indices; steps are folded with
    ``sigmoid_merge``.  Returns (out [S, d], lse [S])."""
    from .layouts import striped_key_offset

    q = np.asarray(q_shards[rank], np.float64)
    S, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((S, np.asarray(v_shards[0]).shape[1]))
    lse = np.full(S, -np.inf)
    local = np.arange(S)
    for step in range(W):
        src = (rank - step) % W
        k = np.asarray(k_shards[src], np.float64)
        v = np.asarray(v_shards[src], np.float64)
        bo, bl = _attend(q, k, v, scale, True, local,
                         np.arange(k.shape[0]) + striped_key_offset(rank, src))
        out, lse = sigmoid_merge(out, lse, bo, bl)
    return out, lse
