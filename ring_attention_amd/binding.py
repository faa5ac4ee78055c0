"""ctypes binding of librattn.so -- argument marshalling only.

Every function here checks tensor metadata, allocates outputs with torch on
the inputs' device, and calls the C entry point of the same name on the
current torch stream.  All arithmetic runs in the HIP kernels; there is no
fallback: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librattn.so")

RATTN_OK, RATTN_EINVAL, RATTN_EUNSUPPORTED, RATTN_EHIP = 0, -1, -2, -3
DTYPE_CODES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

# Exported symbols, in the order include/rattn.h declares them.
EXPORTS = ("rattn_fwd", "rattn_fwd_queued", "rattn_fwd_step", "rattn_fwd_step_merge", "rattn_merge",
           "rattn_fwd_varlen", "rattn_fwd_split", "rattn_fwd_split_noalloc",
           "rattn_split_hint", "rattn_bwd_delta",
           "rattn_bwd", "rattn_bwd_varlen", "rattn_bwd_step", "rattn_status_string")


class RattnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load librattn.so and declare signatures.

    With no path: the in-tree build (ring_attention_amd.build), loaded once.
    With a path: that build of the library, which the wrappers below call from
    then on."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(
            f"{p} is missing: build it with `python -m ring_attention_amd.build` "
            "(or __graft_entry__.build()); there is no non-HIP fallback")
    lib = ctypes.CDLL(p)
    i64, i32, vp, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_float
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.rattn_fwd.restype = i32
    lib.rattn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i64, i64, i32, i32, f32,
                              i32, i32, i32, i32, vp]
    lib.rattn_fwd_queued.restype = i32
    lib.rattn_fwd_queued.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i64, i64, i32, i32, f32,
                                     i32, i32, i32, i32, vp, i64, vp]
    lib.rattn_fwd_step.restype = i32
    lib.rattn_fwd_step.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i64, i64, i64, i64, i64,
                                   i64, i32, i32, f32, i32, i64p, i64p, i64p, i64p, vp]
    lib.rattn_fwd_step_merge.restype = i32
    lib.rattn_fwd_step_merge.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i64, i64, i64, i64,
                                         i64, i64, i32, i32, f32, i32, i64p, i64p, i64p, i64p,
                                         i64, i64, vp]
    lib.rattn_merge.restype = i32
    lib.rattn_merge.argtypes = [vp, vp, vp, vp, i32, i32, i64, i64, i64, i32, vp]
    lib.rattn_fwd_varlen.restype = i32
    lib.rattn_fwd_varlen.argtypes = [vp] * 9 + [i32, i64, i64, i64, i32, i32, i32, i32, f32,
                                                i32, vp]
    lib.rattn_fwd_split.restype = i32
    lib.rattn_fwd_split.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i64, i64, i32, i32, f32,
                                    i32, i32, i32, i32, i32, vp, i64, vp]
    lib.rattn_fwd_split_noalloc.restype = i32
    lib.rattn_fwd_split_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i64, i64, i32, i32,
                                            f32, i32, i32, i32, i32, i32, vp]
    lib.rattn_split_hint.restype = i32
    lib.rattn_split_hint.argtypes = [i32, i32, i64, i64, i32, i32, i32, i32, i32, i32]
    lib.rattn_bwd_delta.restype = i32
    lib.rattn_bwd_delta.argtypes = [vp, vp, vp, i64, i32, i32, vp]
    lib.rattn_bwd.restype = i32
    lib.rattn_bwd.argtypes = [vp] * 10 + [i32, i32, i32, i64, i64, i32, i32, f32, i32, i32, i32,
                                          i32, vp]
    lib.rattn_bwd_varlen.restype = i32
    lib.rattn_bwd_varlen.argtypes = [vp] * 14 + [i32, i64, i64, i64, i64, i32, i32, i32, i32,
                                                 f32, i32, vp]
    lib.rattn_bwd_step.restype = i32
    lib.rattn_bwd_step.argtypes = [vp] * 9 + [i32, i32, i32, i64, i64, i64, i64, i64, i64, i32,
                                              i32, f32, i32, i64p, i64p, i64p, i64p, vp]
    lib.rattn_status_string.restype = ctypes.c_char_p
    lib.rattn_status_string.argtypes = [i32]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().rattn_status_string(int(status)).decode()


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(fn: str, rc: int):
    if rc != RATTN_OK:
        raise RattnError(fn, rc)


def _qkv(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D tensor [B, N, H, d]")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in DTYPE_CODES:
        raise ValueError("q, k, v must share one dtype among float32/float16/bfloat16")
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[3] != k.shape[3]:
        raise ValueError("shape mismatch between q and k/v")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")


def _scale(scale):
    return 0.0 if scale is None else float(scale)


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
        n_ring_steps: int = 1, zigzag: bool = False, rank: int = -1,
        scale: float | None = None, out: torch.Tensor | None = None,
        lse: torch.Tensor | None = None):
    """Whole simulated ring schedule in one launch (rattn_fwd).

    q [B, Nq, Hq, d], k/v [B, N, Hkv, d] natural order.  rank=-1: q holds all N
    rows; rank=r: q holds device r's shard.  Returns (out [B,Nq,Hq,d] in q's
    dtype, lse [B,Nq,Hq] float32).
    """
    _qkv(q, k, v)
    B, Nq, Hq, d = q.shape
    N, Hkv = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Nq, Hq), dtype=torch.float32, device=q.device)
    lib = load_library()
    rc = lib.rattn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                       B, Hq, Hkv, Nq, N, d, DTYPE_CODES[q.dtype], _scale(scale),
                       int(bool(causal)), int(n_ring_steps), int(bool(zigzag)), int(rank),
                       _stream(q))
    _check("rattn_fwd", rc)
    return out, lse


QUEUE_WS_BYTES = 64  # RATTN_QUEUE_WS_BYTES


def queue_workspace(device) -> torch.Tensor:
    """A workspace for fwd_queued on `device` (its contents never matter)."""
    return torch.empty(QUEUE_WS_BYTES // 4, dtype=torch.int32, device=device)


def fwd_queued(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
               n_ring_steps: int = 1, zigzag: bool = False, rank: int = -1,
               scale: float | None = None, out: torch.Tensor | None = None,
               lse: torch.Tensor | None = None, queue_ws: torch.Tensor | None = None):
    """fwd() with the query tiles handed out from per-XCD queues
    (rattn_fwd_queued); queue_ws from queue_workspace() is allocated here
    unless given.  Same result as fwd()."""
    _qkv(q, k, v)
    B, Nq, Hq, d = q.shape
    N, Hkv = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Nq, Hq), dtype=torch.float32, device=q.device)
    if queue_ws is None:
        queue_ws = queue_workspace(q.device)
    if queue_ws.device != q.device or not queue_ws.is_contiguous():
        raise ValueError("queue_ws must be a contiguous tensor on q's device")
    lib = load_library()
    rc = lib.rattn_fwd_queued(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr(), B, Hq, Hkv, Nq, N, d, DTYPE_CODES[q.dtype],
                              _scale(scale), int(bool(causal)), int(n_ring_steps),
                              int(bool(zigzag)), int(rank), queue_ws.data_ptr(),
                              queue_ws.numel() * queue_ws.element_size(), _stream(q))
    _check("rattn_fwd_queued", rc)
    return out, lse


def split_hint(q: torch.Tensor, k: torch.Tensor, n_ring_steps: int = 1, zigzag: bool = False,
               rank: int = -1) -> int:
    """rattn_split_hint for these shapes on q's device."""
    B, Nq, Hq, d = q.shape
    n_cu = torch.cuda.get_device_properties(q.device).multi_processor_count
    return int(load_library().rattn_split_hint(B, Hq, Nq, k.shape[1], d, DTYPE_CODES[q.dtype],
                                               int(n_ring_steps), int(bool(zigzag)), int(rank),
                                               n_cu))


def fwd_split(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
              n_ring_steps: int = 1, zigzag: bool = False, rank: int = -1,
              scale: float | None = None, n_splits: int | None = None,
              out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
              ws: torch.Tensor | None = None):
    """rattn_fwd with split-KV (rattn_fwd_split); n_splits=None takes
    rattn_split_hint's count.  The float32 scratch is allocated here unless
    given.  Same result as fwd()."""
    _qkv(q, k, v)
    B, Nq, Hq, d = q.shape
    N, Hkv = k.shape[1], k.shape[2]
    if n_splits is None:
        n_splits = split_hint(q, k, n_ring_steps, zigzag, rank)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Nq, Hq), dtype=torch.float32, device=q.device)
    need = n_splits * B * Nq * Hq * (d + 1) if n_splits > 1 else 0
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.float32, device=q.device)
    lib = load_library()
    rc = lib.rattn_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), B, Hq, Hkv, Nq, N, d, DTYPE_CODES[q.dtype],
                             _scale(scale), int(bool(causal)), int(n_ring_steps),
                             int(bool(zigzag)), int(rank), int(n_splits), ws.data_ptr(),
                             ws.numel(), _stream(q))
    _check("rattn_fwd_split", rc)
    return out, lse


def fwd_split_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                      n_ring_steps: int = 1, zigzag: bool = False, rank: int = -1,
                      scale: float | None = None, n_splits: int | None = None,
                      out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """rattn_fwd_split with the library's fixed scratch for the partials
    (rattn_fwd_split_noalloc: the C call allocates nothing; calls that overlap
    on one GPU race).  n_splits=None takes rattn_split_hint's count."""
    _qkv(q, k, v)
    B, Nq, Hq, d = q.shape
    N, Hkv = k.shape[1], k.shape[2]
    if n_splits is None:
        n_splits = split_hint(q, k, n_ring_steps, zigzag, rank)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Nq, Hq), dtype=torch.float32, device=q.device)
    rc = load_library().rattn_fwd_split_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv,
        Nq, N, d, DTYPE_CODES[q.dtype], _scale(scale), int(bool(causal)), int(n_ring_steps),
        int(bool(zigzag)), int(rank), int(n_splits), _stream(q))
    _check("rattn_fwd_split_noalloc", rc)
    return out, lse


def _segs(pairs):
    """Up to two (start_position, length) pairs as two host int64[2] arrays."""
    pairs = list(pairs) + [(0, 0)] * (2 - len(pairs))
    if len(pairs) != 2:
        raise ValueError("at most two segments")
    starts = (ctypes.c_int64 * 2)(*[int(p[0]) for p in pairs])
    lens = (ctypes.c_int64 * 2)(*[int(p[1]) for p in pairs])
    return starts, lens


def _rows(segs, off, total, what):
    """Rows a step reads: the segment lengths, from row `off` of `total`."""
    n = sum(int(p[1]) for p in segs)
    if off < 0 or off + n > total:
        raise ValueError(f"{what} rows [{off}, {off + n}) exceed the tensor's {total} rows")
    return n


def fwd_step_merge(q: torch.Tensor, k_blk: torch.Tensor, v_blk: torch.Tensor, causal: bool,
                   q_segs, k_segs, out: torch.Tensor, lse: torch.Tensor, row_off: int = 0,
                   scale: float | None = None, q_off: int = 0, k_off: int = 0):
    """One ring step merged into the running float32 (out, lse) at rows
    [row_off, row_off + Nq) (rattn_fwd_step_merge); returns (out, lse).

    The step reads query rows [q_off, q_off + Nq) of q and key/value rows
    [k_off, k_off + Nk) of k_blk, v_blk, Nq and Nk being the segment lengths'
    sums (no copy of a part of a shard)."""
    _qkv(q, k_blk, v_blk)
    B, q_rows, Hq, d = q.shape
    k_rows, Hkv = k_blk.shape[1], k_blk.shape[2]
    Nq = _rows(q_segs, q_off, q_rows, "query")
    Nk = _rows(k_segs, k_off, k_rows, "key")
    for name, t in (("out", out), ("lse", lse)):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous float32 tensor on q's device")
    if out.dim() != 4 or out.shape[0] != B or out.shape[2:] != (Hq, d) or \
            lse.shape != out.shape[:3]:
        raise ValueError("out must be [B, Nq_out, Hq, d] and lse [B, Nq_out, Hq]")
    qs, ql = _segs(q_segs)
    kst, kl = _segs(k_segs)
    rc = load_library().rattn_fwd_step_merge(
        q.data_ptr(), k_blk.data_ptr(), v_blk.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq,
        Hkv, q_rows, int(q_off), Nq, k_rows, int(k_off), Nk, d, DTYPE_CODES[q.dtype],
        _scale(scale), int(bool(causal)), qs, ql, kst, kl, out.shape[1], int(row_off),
        _stream(q))
    _check("rattn_fwd_step_merge", rc)
    return out, lse


def fwd_step(q: torch.Tensor, k_blk: torch.Tensor, v_blk: torch.Tensor, causal: bool,
             q_segs, k_segs, scale: float | None = None,
             out_part: torch.Tensor | None = None, lse_part: torch.Tensor | None = None,
             q_off: int = 0, k_off: int = 0):
    """One ring step (rattn_fwd_step): normalised float32 partial and its lse.

    q_segs / k_segs: up to two (start_position, length) pairs covering, in
    order, the query rows [q_off, q_off + Nq) of q and the key/value rows
    [k_off, k_off + Nk) of k_blk, v_blk (Nq, Nk: the lengths' sums).
    """
    _qkv(q, k_blk, v_blk)
    B, q_rows, Hq, d = q.shape
    k_rows, Hkv = k_blk.shape[1], k_blk.shape[2]
    Nq = _rows(q_segs, q_off, q_rows, "query")
    Nk = _rows(k_segs, k_off, k_rows, "key")
    qs, ql = _segs(q_segs)
    kst, kl = _segs(k_segs)
    if out_part is None:
        out_part = torch.empty((B, Nq, Hq, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, Nq, Hq), dtype=torch.float32, device=q.device)
    lib = load_library()
    rc = lib.rattn_fwd_step(q.data_ptr(), k_blk.data_ptr(), v_blk.data_ptr(),
                            out_part.data_ptr(), lse_part.data_ptr(), B, Hq, Hkv, q_rows,
                            int(q_off), Nq, k_rows, int(k_off), Nk, d,
                            DTYPE_CODES[q.dtype], _scale(scale), int(bool(causal)),
                            qs, ql, kst, kl, _stream(q))
    _check("rattn_fwd_step", rc)
    return out_part, lse_part


def merge(out: torch.Tensor, lse: torch.Tensor, blk_out: torch.Tensor, blk_lse: torch.Tensor,
          row_off: int = 0):
    """In-place log-sum-exp merge (rattn_merge) of a float32 partial into (out, lse)."""
    for name, t in (("out", out), ("lse", lse), ("blk_out", blk_out), ("blk_lse", blk_lse)):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor")
    if out.dim() != 4 or blk_out.dim() != 4:
        raise ValueError("out and blk_out must be [B, N, H, d]")
    B, Nq, H, d = out.shape
    Nb = blk_out.shape[1]
    if blk_out.shape != (B, Nb, H, d) or lse.shape != (B, Nq, H) or blk_lse.shape != (B, Nb, H):
        raise ValueError("merge: shape mismatch")
    lib = load_library()
    rc = lib.rattn_merge(out.data_ptr(), lse.data_ptr(), blk_out.data_ptr(), blk_lse.data_ptr(),
                         B, H, Nq, Nb, int(row_off), d, _stream(out))
    _check("rattn_merge", rc)
    return out, lse


def _like(name, t, ref, dtype=None):
    """t must be a contiguous tensor on ref's device, of dtype (default: ref's)."""
    want = ref.dtype if dtype is None else dtype
    if not isinstance(t, torch.Tensor) or t.dtype != want or not t.is_contiguous() or \
            t.device != ref.device:
        raise ValueError(f"{name} must be a contiguous {want} tensor on {ref.device}")


def bwd_delta(out: torch.Tensor, dout: torch.Tensor, delta: torch.Tensor | None = None):
    """D = rowsum(dout * out) over the last dim (rattn_bwd_delta), float32."""
    _like("dout", dout, out)
    if out.dtype not in DTYPE_CODES or dout.shape != out.shape or not out.is_cuda:
        raise ValueError("out and dout must be matching GPU tensors")
    d = out.shape[-1]
    rows = out.numel() // d if d else 0
    if delta is None:
        delta = torch.empty(out.shape[:-1], dtype=torch.float32, device=out.device)
    _like("delta", delta, out, torch.float32)
    if delta.numel() != rows:
        raise ValueError("delta must hold one value per row")
    rc = load_library().rattn_bwd_delta(out.data_ptr(), dout.data_ptr(), delta.data_ptr(), rows,
                                        d, DTYPE_CODES[out.dtype], _stream(out))
    _check("rattn_bwd_delta", rc)
    return delta


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
        lse: torch.Tensor, dout: torch.Tensor, causal: bool = False, n_ring_steps: int = 1,
        zigzag: bool = False, rank: int = -1, scale: float | None = None,
        dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
        dv: torch.Tensor | None = None, delta_ws: torch.Tensor | None = None):
    """Backward of ``fwd`` (rattn_bwd): returns (dq, dk, dv) in q's dtype.

    out, lse: the forward's results; dout: the gradient of the loss with
    respect to out.  Layout arguments as ``fwd``."""
    _qkv(q, k, v)
    B, Nq, Hq, d = q.shape
    N, Hkv = k.shape[1], k.shape[2]
    _like("out", out, q)
    _like("dout", dout, q)
    _like("lse", lse, q, torch.float32)
    if out.shape != q.shape or dout.shape != q.shape or lse.shape != (B, Nq, Hq):
        raise ValueError("out, dout must be [B, Nq, Hq, d] and lse [B, Nq, Hq]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if delta_ws is None:
        delta_ws = torch.empty((B, Nq, Hq), dtype=torch.float32, device=q.device)
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _like(name, t, ref)
        if t.shape != ref.shape:
            raise ValueError(f"{name} must have the shape of its input")
    _like("delta_ws", delta_ws, q, torch.float32)
    if delta_ws.numel() < B * Nq * Hq:
        raise ValueError("delta_ws must hold B*Nq*Hq floats")
    rc = load_library().rattn_bwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
        dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta_ws.data_ptr(),
        B, Hq, Hkv, Nq, N, d, DTYPE_CODES[q.dtype], _scale(scale), int(bool(causal)),
        int(n_ring_steps), int(bool(zigzag)), int(rank), _stream(q))
    _check("rattn_bwd", rc)
    return dq, dk, dv


def bwd_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor,
             lse: torch.Tensor, delta: torch.Tensor, dq_acc: torch.Tensor,
             dk_acc: torch.Tensor, dv_acc: torch.Tensor, causal: bool, q_segs, k_segs,
             q_off: int = 0, Nq: int | None = None, k_off: int = 0, Nk: int | None = None,
             scale: float | None = None):
    """One backward ring step (rattn_bwd_step): adds the contributions of the
    pairs between query rows [q_off, q_off+Nq) of q and key rows
    [k_off, k_off+Nk) of k/v to the float32 accumulators dq_acc (q's shape),
    dk_acc and dv_acc (k's shape).  q_segs / k_segs: up to two
    (start_position, length) pairs covering those rows in order."""
    _qkv(q, k, v)
    B, q_rows, Hq, d = q.shape
    k_rows, Hkv = k.shape[1], k.shape[2]
    Nq = q_rows - q_off if Nq is None else Nq
    Nk = k_rows - k_off if Nk is None else Nk
    _like("dout", dout, q)
    for name, t in (("lse", lse), ("delta", delta)):
        _like(name, t, q, torch.float32)
        if t.shape != (B, q_rows, Hq):
            raise ValueError(f"{name} must be [B, Nq, Hq]")
    for name, t, ref in (("dq_acc", dq_acc, q), ("dk_acc", dk_acc, k), ("dv_acc", dv_acc, v)):
        _like(name, t, ref, torch.float32)
        if t.shape != ref.shape:
            raise ValueError(f"{name} must have the shape of its input")
    qs, ql = _segs(q_segs)
    kst, kl = _segs(k_segs)
    rc = load_library().rattn_bwd_step(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), lse.data_ptr(),
        delta.data_ptr(), dq_acc.data_ptr(), dk_acc.data_ptr(), dv_acc.data_ptr(), B, Hq, Hkv,
        q_rows, int(q_off), int(Nq), k_rows, int(k_off), int(Nk), d, DTYPE_CODES[q.dtype],
        _scale(scale), int(bool(causal)), qs, ql, kst, kl, _stream(q))
    _check("rattn_bwd_step", rc)
    return dq_acc, dk_acc, dv_acc


def varlen_from_cu_seqlens(cu_seqlens):
    """(starts, lengths) of a packed batch given its prefix sums cu_seqlens
    (n_seq + 1 non-decreasing integers starting at 0)."""
    cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
    if not cu or cu[0] != 0 or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0 and not decrease")
    return cu[:-1], [b - a for a, b in zip(cu, cu[1:])]


def _varlen_ranges(q, k, q_start, q_len, k_start, k_len):
    """Checked host ranges and their int32 device copies."""
    Nq, Nk = q.shape[0], k.shape[0]
    ranges = [list(map(int, x)) for x in (q_start, q_len, k_start, k_len)]
    n_seq = len(ranges[0])
    if any(len(x) != n_seq for x in ranges):
        raise ValueError("q_start, q_len, k_start, k_len must have one entry per sequence")
    for (qs, ql, ks, kl) in zip(*ranges):
        if qs < 0 or ql < 0 or qs + ql > Nq or ks < 0 or kl < 0 or ks + kl > Nk:
            raise ValueError("a sequence range lies outside q or k")
    dev = [torch.tensor(x if x else [0], dtype=torch.int32, device=q.device) for x in ranges]
    return ranges, n_seq, dev


def bwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
               lse: torch.Tensor, dout: torch.Tensor, q_start, q_len, k_start, k_len,
               causal: bool = False, scale: float | None = None):
    """Backward of ``fwd_varlen`` (rattn_bwd_varlen): returns (dq, dk, dv) in
    q's dtype, zero on rows outside every sequence."""
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        if not isinstance(t, torch.Tensor) or t.dim() != 3 or not t.is_cuda or \
                not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 3-D GPU tensor [N, H, d]")
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype) or \
            q.dtype not in DTYPE_CODES or k.shape != v.shape or out.shape != q.shape or \
            dout.shape != q.shape or q.shape[2] != k.shape[2]:
        raise ValueError("q, out, dout [Nq, Hq, d] and k, v [Nk, Hkv, d] of one dtype")
    Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[0], k.shape[1]
    _like("lse", lse, q, torch.float32)
    if lse.shape != (Nq, Hq):
        raise ValueError("lse must be [Nq, Hq]")
    ranges, n_seq, dev = _varlen_ranges(q, k, q_start, q_len, k_start, k_len)
    dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    ws = torch.empty((Nq, Hq), dtype=torch.float32, device=q.device)
    rc = load_library().rattn_bwd_varlen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
        dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
        *[t.data_ptr() for t in dev], n_seq, max(ranges[1], default=0),
        max(ranges[3], default=0), Nq, Nk, Hq, Hkv, d, DTYPE_CODES[q.dtype], _scale(scale),
        int(bool(causal)), _stream(q))
    _check("rattn_bwd_varlen", rc)
    return dq, dk, dv


def fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_start, q_len, k_start,
               k_len, causal: bool = False, scale: float | None = None,
               out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Variable-length batch (rattn_fwd_varlen): sequence i attends from query
    rows [q_start[i], +q_len[i]) of q [Nq, Hq, d] to key/value rows
    [k_start[i], +k_len[i]) of k, v [Nk, Hkv, d].  The ranges are host lists
    (checked here) copied to the device as int32.  Returns (out [Nq, Hq, d],
    lse [Nq, Hq]); rows outside every sequence keep what out/lse held
    (zeros / -inf when allocated here)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 3 or not t.is_cuda or \
                not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 3-D GPU tensor [N, H, d]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in DTYPE_CODES or \
            k.shape != v.shape or q.shape[2] != k.shape[2]:
        raise ValueError("q, k, v must share dtype and head dim; k, v one shape")
    Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[0], k.shape[1]
    ranges, n_seq, dev = _varlen_ranges(q, k, q_start, q_len, k_start, k_len)
    if out is None:
        out = torch.zeros_like(q)
    if lse is None:
        lse = torch.full((Nq, Hq), float("-inf"), dtype=torch.float32, device=q.device)
    _like("out", out, q)
    _like("lse", lse, q, torch.float32)
    if out.shape != q.shape or lse.shape != (Nq, Hq):
        raise ValueError("out must be [Nq, Hq, d] and lse [Nq, Hq]")
    max_len_q = max(ranges[1]) if n_seq else 0
    rc = load_library().rattn_fwd_varlen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
        *[t.data_ptr() for t in dev], n_seq, max_len_q, Nq, Nk, Hq, Hkv, d,
        DTYPE_CODES[q.dtype], _scale(scale), int(bool(causal)), _stream(q))
    _check("rattn_fwd_varlen", rc)
    return out, lse

