"""Global token positions under the ring layouts -- oracle side, TEST INFRASTRUCTURE.

Written from the pages' prose, independently of the HIP path's scheduler:

* Contiguous ring (ultralytics.com glossary "Ring Attention", section on how it
  works; youngju.dev "Ring Attention" analysis, ``ring_attention_forward``):
  the sequence is cut into W equal blocks and device i keeps query block i.
  At step s device i holds the key/value block of device (i - s) mod W,
  because every device sends to its successor and receives from its
  predecessor.
* ZigZag (Twinkle "Sequence parallel and Ring Attention", ZigZag section): the
  sequence is cut into 2W chunks and device r keeps chunk r and chunk
  2W-1-r, stored as [front; back].
* ZigZag step rules (Twinkle page, forward-pass section): step 0 is causal
  attention of the local queries over the local keys; at steps 1..r all local
  queries attend, without mask, to the front half of the received keys; at
  steps after r only the back half of the queries attends, without mask, to
  all received keys.
"""
from __future__ import annotations

import numpy as np


def ring_source(rank: int, step: int, W: int) -> int:
    """Device whose key/value block device ``rank`` holds at ``step``."""
    return (rank - step) % W


def contiguous_shard_positions(N: int, W: int, rank: int) -> np.ndarray:
    """Positions of the rows device ``rank`` keeps under the contiguous split."""
    if N % W:
        raise ValueError("N must be a multiple of W")
    S = N // W
    return np.arange(rank * S, (rank + 1) * S, dtype=np.int64)


def zigzag_shard_positions(N: int, W: int, rank: int) -> np.ndarray:
    """Positions of the rows device ``rank`` keeps under ZigZag: chunk rank, then
    chunk 2W-1-rank."""
    if N % (2 * W):
        raise ValueError("N must be a multiple of 2W")
    c = N // (2 * W)
    front = np.arange(rank * c, (rank + 1) * c, dtype=np.int64)
    back_chunk = 2 * W - 1 - rank
    back = np.arange(back_chunk * c, (back_chunk + 1) * c, dtype=np.int64)
    return np.concatenate([front, back])


def shard_positions(N: int, W: int, rank: int, zigzag: bool) -> np.ndarray:
    return (zigzag_shard_positions if zigzag else contiguous_shard_positions)(N, W, rank)


def zigzag_step_plan(W: int, rank: int, step: int, c: int):
    """Rows used at one ZigZag ring step, as local index arrays.

    Returns (q_rows, kv_rows, causal, src): query rows of the local shard
    [front; back] (each half c rows), key/value rows of the received shard
    (also [front; back]), whether the step masks causally, and the source
    device of the received shard.
    """
    src = ring_source(rank, step, W)
    all_rows = np.arange(2 * c, dtype=np.int64)
    front = np.arange(c, dtype=np.int64)
    back = np.arange(c, 2 * c, dtype=np.int64)
    if step == 0:
        return all_rows, all_rows, True, src
    if step <= rank:
        return all_rows, front, False, src
    return back, all_rows, False, src


def striped_shard_positions(N: int, W: int, rank: int) -> np.ndarray:
    """Striped layout (ultralytics.com glossary "Ring Attention": Striped
    Attention gives each device tokens spread evenly over the sequence):
    device ``rank`` keeps positions rank, rank + W, rank + 2W, ...  (a
    reading: the page gives the idea, not the map; stride W is the even
    spread)."""
    if N % W:
        raise ValueError("N must be a multiple of W")
    return np.arange(rank, N, W, dtype=np.int64)


def striped_key_offset(rank: int, src: int) -> int:
    """Striped causal step rule: local query i of device ``rank`` (position
    rank + W i) sees local key j of device ``src`` (position src + W j) iff
    j + offset <= i, with offset 0 when src <= rank and 1 when src > rank."""
    return 0 if src <= rank else 1
