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


def blockwise_attention(q, k, v, Br: int, Bc: int, scale: float | None = None,
                        causal: bool = False, q_pos=None, k_pos=None):
    """Online-softmax attention over query tiles of Br rows and key tiles of Bc
    rows, with the division by l deferred to the end.

    Follows the FlashAttention forward recurrence of the yz520gzy chapter
    (tile counts ceil(N/B), so ragged tails are kept) with the FlashAttention-2
    change described there (keep O unnormalised, divide once), and the
    youngju.dev ``blockwise_attention`` update (m_new = max(m, rowmax S),
    correction exp(m - m_new)).  Causal masking by position: a key later than
    the query gets score -inf (the youngju.dev causal step).
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
        qi = q[i0:i0 + Br]
        m = np.full(qi.shape[0], -np.inf)
        l = np.zeros(qi.shape[0])
        O = np.zeros((qi.shape[0], v.shape[1]))
        for j0 in range(0, Nk, Bc):
            S = (qi @ k[j0:j0 + Bc].T) * scale
            if causal:
                hidden = kp[None, j0:j0 + Bc] > qp[i0:i0 + Br, None]
                S = np.where(hidden, -np.inf, S)
            m_new = np.maximum(m, S.max(axis=1))
            alpha = _exp_shift(m, m_new)
            P = _exp_shift(S, m_new[:, None])
            l = alpha * l + P.sum(axis=1)
            O = alpha[:, None] * O + P @ v[j0:j0 + Bc]
            m = m_new
        seen = l > 0
        out[i0:i0 + Br][seen] = O[seen] / l[seen, None]
        lse[i0:i0 + Br][seen] = m[seen] + np.log(l[seen])
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
    """The Twinkle page's ``update_out_and_lse`` in its sigmoid form:

        out <- out - sigmoid(block_lse - lse) * (out - block_out)
        lse <- lse - logsigmoid(lse - block_lse)

    Taken literally the second line gives NaN when lse = -inf; the reading used
    here: an empty side (lse = -inf) contributes nothing, so the other side is
    returned unchanged, and two empty sides stay empty (out 0, lse -inf).
    out: [n, d], lse: [n].
    """
    out = np.array(out, np.float64)
    lse = np.array(lse, np.float64)
    block_out = np.asarray(block_out, np.float64)
    block_lse = np.asarray(block_lse, np.float64)
    a_empty = np.isneginf(lse)
    b_empty = np.isneginf(block_lse)
    both = ~a_empty & ~b_empty
    diff = block_lse[both] - lse[both]
    sig = 1.0 / (1.0 + np.exp(-diff))
    out[both] = out[both] - sig[:, None] * (out[both] - block_out[both])
    # -logsigmoid(x) = log(1 + exp(-x)) with x = lse - block_lse, written stably
    x = lse[both] - block_lse[both]
    lse[both] = lse[both] + np.where(x > 0, np.log1p(np.exp(-x)), -x + np.log1p(np.exp(x)))
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
    """The guijiagi.com page's online softmax (one pass over key/value blocks,
    running m, l and o rescaled by exp(m - m_new), division at the end),
    for a matrix of query rows and key/value blocks in the order given.
    Returns (O [Nq, d], lse [Nq])."""
    q = np.asarray(q, np.float64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[1])
    m = np.full(q.shape[0], -np.inf)
    l = np.zeros(q.shape[0])
    o = np.zeros((q.shape[0], np.asarray(v_blocks[0]).shape[1]))
    for kb, vb in zip(k_blocks, v_blocks):
        s = (q @ np.asarray(kb, np.float64).T) * scale
        m_new = np.maximum(m, s.max(axis=1))
        alpha = _exp_shift(m, m_new)
        o = o * alpha[:, None]
        l = l * alpha
        p = _exp_shift(s, m_new[:, None])
        o = o + p @ np.asarray(vb, np.float64)
        l = l + p.sum(axis=1)
        m = m_new
    return o / l[:, None], m + np.log(l)


def ring_backward(q, k, v, o, lse, do, W: int, rank: int, scale: float | None = None):
    """The ring backward of one device, simulated: gradients of the device's
    query block and of every key/value block, non-causal.

    Follows the youngju.dev ``ring_attention_backward`` description: the
    device first forms D = rowsum(dO * O) from its saved output; then at each
    of the W steps it holds the key/value block of device (rank - step) mod W,
    recomputes S = scale Q K^T and P = exp(S - lse) from the saved log-sum-exp,
    and forms dV_blk = P^T dO, dP = dO V^T, dS = P (dP - D) scale,
    dQ += dS K, dK_blk = dS^T Q.  The block gradients go back to the block's
    owner, which sums what every device sends it.

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
    S_blk = Nk // W
    D = (do * o).sum(axis=1, keepdims=True)
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    for step in range(W):
        src = (rank - step) % W
        rows = slice(src * S_blk, (src + 1) * S_blk)
        Kb, Vb = k[rows], v[rows]
        P = _exp_shift((q @ Kb.T) * scale, lse[:, None])
        dV[rows] += P.T @ do
        dP = do @ Vb.T
        dS = P * (dP - D) * scale
        dQ += dS @ Kb
        dK[rows] += dS.T @ q
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
