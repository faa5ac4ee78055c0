"""One simulated device of the ring, run step by step on one GPU.

Each step is one call of the step kernel on the key/value shard the device
holds at that step, with a log-sum-exp merge into the running (out, lse) --
the structure of the Twinkle forward pass ("Sequence parallel and Ring
Attention", forward-pass section).  The merge runs in the step kernel's
epilogue (rattn_fwd_step_merge) or as its own launch (rattn_fwd_step, then
rattn_merge).
The fused entry point (rattn_fwd) computes the same thing in one launch.

Ring order: at step s device r holds the shard of device (r - s) mod W
(ultralytics.com "Ring Attention": every device passes its block on to the
next one and receives from the previous one).

ZigZag step rules (Twinkle page, forward pass), for device r with shard
[front; back] of chunks r and 2W-1-r:
  step 0         all local queries x all local keys, causal
  1 <= s <= r    all local queries x the front chunk of the received keys
  s > r          the back half of the queries x all received keys
Contiguous layout with causal masking (youngju.dev "Ring Attention" analysis,
causal step): a block from a later device is skipped, the own block is
masked, earlier blocks are fully visible.
"""
from __future__ import annotations

import torch

from . import binding


def shard_rows(N: int, W: int, zigzag: bool, rank: int):
    """(start_position, length) runs of the rows device ``rank`` holds."""
    if zigzag:
        c = N // (2 * W)
        return [(rank * c, c), ((2 * W - 1 - rank) * c, c)]
    S = N // W
    return [(rank * S, S)]


def shard(x: torch.Tensor, W: int, zigzag: bool, rank: int) -> torch.Tensor:
    """Rows of device ``rank`` of a natural-order [B, N, H, d] tensor, stored
    contiguously in ring layout (front chunk, then back chunk for ZigZag).

    This is data placement done before the timed work: in a real ring each
    device already holds its shard in its own memory."""
    N = x.shape[1]
    parts = [x[:, a:a + n] for a, n in shard_rows(N, W, zigzag, rank)]
    return torch.cat(parts, dim=1).contiguous() if len(parts) > 1 else parts[0].contiguous()


def _direct(kind, fn):
    return fn()


def step_plan(N: int, W: int, zigzag: bool, rank: int, causal: bool):
    """Device ``rank``'s ring steps in order, skipped steps left out:
    (src, query runs, key runs, step causal, first query row of the step)."""
    q_runs = shard_rows(N, W, zigzag, rank)
    plan = []
    for s in range(W):
        src = (rank - s) % W
        k_runs = shard_rows(N, W, zigzag, src)
        row_off = 0  # first query row of the step (rows of the shard are read in place)
        qr, kr, step_causal = q_runs, k_runs, causal
        if zigzag and causal:
            c = N // (2 * W)
            if s == 0:
                pass
            elif s <= rank:
                kr, step_causal = k_runs[:1], False  # the front chunk: key rows [0, c)
            else:
                qr, row_off, step_causal = q_runs[1:], c, False  # back half: rows [c, 2c)
        elif causal:
            if src > rank:
                continue
            step_causal = src == rank
        plan.append((src, qr, kr, step_causal, row_off))
    return plan


def ring_forward_steps(q_shard: torch.Tensor, k_shards, v_shards, W: int, zigzag: bool,
                       rank: int, causal: bool = True, scale: float | None = None,
                       hook=_direct, fused_merge: bool = True):
    """Run device ``rank``'s W ring steps; returns float32 (out, lse).

    q_shard [B, Nq, Hq, d] is the device's query shard; k_shards[src] and
    v_shards[src] are the shards every device would send (see ``shard``).
    fused_merge: steps after the first merge into the running result in the
    step kernel's epilogue (rattn_fwd_step_merge); else each writes a partial
    that rattn_merge folds in.  hook(kind, fn) wraps every library call
    ("step" or "merge") and must return fn(); a benchmark uses it to time
    the launches.
    """
    N = sum(k.shape[1] for k in k_shards)
    out = lse = None
    for src, qr, kr, step_causal, row_off in step_plan(N, W, zigzag, rank, causal):
        kb, vb = k_shards[src], v_shards[src]
        if out is None:
            # the first step writes the running result directly
            out, lse = hook("step", lambda: binding.fwd_step(q_shard, kb, vb, step_causal, qr, kr,
                                                             scale, q_off=row_off))
            continue
        if fused_merge:
            hook("step", lambda: binding.fwd_step_merge(q_shard, kb, vb, step_causal, qr, kr, out,
                                                        lse, row_off=row_off, scale=scale,
                                                        q_off=row_off))
            continue
        bo, bl = hook("step", lambda: binding.fwd_step(q_shard, kb, vb, step_causal, qr, kr, scale,
                                                       q_off=row_off))
        hook("merge", lambda: binding.merge(out, lse, bo, bl, row_off=row_off))
    return out, lse


def ring_backward_steps(q_shard: torch.Tensor, k_shards, v_shards, out_shard: torch.Tensor,
                        lse_shard: torch.Tensor, dout_shard: torch.Tensor, W: int, zigzag: bool,
                        rank: int, causal: bool = True, scale: float | None = None,
                        hook=_direct):
    """Run device ``rank``'s W backward ring steps (youngju.dev "Ring
    Attention" analysis, ring_attention_backward; Twinkle page, backward
    section): D = rowsum(dO * O) once, then at every step the pairs of the
    forward's step rules, adding to dQ of the local queries and to dK, dV of
    the held key/value shard, which in a real ring travel back to the shard's
    owner (here: one float32 accumulator per shard).

    out_shard (q's dtype) and lse_shard are the device's forward results.
    Returns (dq float32 [B, Nq, Hq, d], dk_acc, dv_acc), the last two lists
    indexed by source device, each float32 in that device's shard layout.
    hook(kind, fn) as in ``ring_forward_steps`` ("delta" or "step").
    """
    N = sum(k.shape[1] for k in k_shards)
    delta = hook("delta", lambda: binding.bwd_delta(out_shard, dout_shard))
    dq = torch.zeros(q_shard.shape, dtype=torch.float32, device=q_shard.device)
    dk_acc = [torch.zeros(k.shape, dtype=torch.float32, device=k.device) for k in k_shards]
    dv_acc = [torch.zeros(v.shape, dtype=torch.float32, device=v.device) for v in v_shards]
    q_runs = shard_rows(N, W, zigzag, rank)
    Nq_all = q_shard.shape[1]
    for s in range(W):
        src = (rank - s) % W
        k_runs = shard_rows(N, W, zigzag, src)
        Nk_all = k_shards[src].shape[1]
        q_off, Nq, k_off, Nk = 0, Nq_all, 0, Nk_all
        qr, kr, step_causal = q_runs, k_runs, causal
        if zigzag and causal:
            c = N // (2 * W)
            if s == 0:
                pass
            elif s <= rank:
                Nk, kr, step_causal = c, k_runs[:1], False
            else:
                q_off, Nq, qr, step_causal = c, c, q_runs[1:], False
        elif causal:
            if src > rank:
                continue
            step_causal = src == rank
        hook("step", lambda: binding.bwd_step(
            q_shard, k_shards[src], v_shards[src], dout_shard, lse_shard, delta, dq,
            dk_acc[src], dv_acc[src], step_causal, qr, kr, q_off=q_off, Nq=Nq, k_off=k_off,
            Nk=Nk, scale=scale))
    return dq, dk_acc, dv_acc


# ---- Striped layout ---------------------------------------------------------
# ultralytics.com "Ring Attention": Striped Attention spreads each device's
# tokens evenly over the sequence, so under the causal mask every device and
# every ring step gets about the same work.  Device r keeps positions
# r, r + W, r + 2W, ... (stride W).  Local query i of device r (position
# r + W i) sees local key j of device src (position src + W j) iff
# j + off <= i, off = 0 when src <= r, else 1.  Each step is therefore one
# causal block in local indices, which the step calls express with
# positions: queries at 0 .. S-1, keys at off .. off + S - 1.


def stripe(x: torch.Tensor, W: int, rank: int) -> torch.Tensor:
    """Rows rank, rank + W, ... of a natural-order [B, N, H, d] tensor, stored
    contiguously (the shard device ``rank`` holds under the Striped layout)."""
    return x[:, rank::W].contiguous()


def striped_key_offset(rank: int, src: int) -> int:
    return 0 if src <= rank else 1


def striped_forward_steps(q_shard: torch.Tensor, k_shards, v_shards, W: int, rank: int,
                          causal: bool = True, scale: float | None = None, hook=_direct,
                          fused_merge: bool = True):
    """Device ``rank``'s W ring steps over the Striped layout; returns float32
    (out, lse).  q_shard, k_shards[src], v_shards[src] as ``stripe`` gives
    them; hook and fused_merge as in ``ring_forward_steps``."""
    S = q_shard.shape[1]
    out = lse = None
    for s in range(W):
        src = (rank - s) % W
        kb, vb = k_shards[src], v_shards[src]
        qr = [(0, S)]
        kr = [(striped_key_offset(rank, src) if causal else 0, kb.shape[1])]
        if out is None:
            out, lse = hook("step", lambda: binding.fwd_step(q_shard, kb, vb, causal, qr, kr,
                                                             scale))
        elif fused_merge:
            hook("step", lambda: binding.fwd_step_merge(q_shard, kb, vb, causal, qr, kr, out,
                                                        lse, scale=scale))
        else:
            bo, bl = hook("step", lambda: binding.fwd_step(q_shard, kb, vb, causal, qr, kr,
                                                           scale))
            hook("merge", lambda: binding.merge(out, lse, bo, bl))
    return out, lse


def striped_backward_steps(q_shard: torch.Tensor, k_shards, v_shards, out_shard: torch.Tensor,
                           lse_shard: torch.Tensor, dout_shard: torch.Tensor, W: int, rank: int,
                           causal: bool = True, scale: float | None = None, hook=_direct):
    """Backward of ``striped_forward_steps`` (as ``ring_backward_steps``):
    returns (dq float32, dk_acc, dv_acc) with one float32 accumulator per
    source device's shard."""
    S = q_shard.shape[1]
    delta = hook("delta", lambda: binding.bwd_delta(out_shard, dout_shard))
    dq = torch.zeros(q_shard.shape, dtype=torch.float32, device=q_shard.device)
    dk_acc = [torch.zeros(k.shape, dtype=torch.float32, device=k.device) for k in k_shards]
    dv_acc = [torch.zeros(v.shape, dtype=torch.float32, device=v.device) for v in v_shards]
    for s in range(W):
        src = (rank - s) % W
        kr = [(striped_key_offset(rank, src) if causal else 0, k_shards[src].shape[1])]
        hook("step", lambda: binding.bwd_step(
            q_shard, k_shards[src], v_shards[src], dout_shard, lse_shard, delta, dq,
            dk_acc[src], dv_acc[src], causal, [(0, S)], kr, scale=scale))
    return dq, dk_acc, dv_acc
