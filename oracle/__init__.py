"""fp64 CPU oracle for exact (ring) attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP path (``ring_attention_amd``)
never imports it, and it imports nothing from the HIP path.

Contents
  oracle.c        the definition softmax(scale*QK^T)V in double (C + OpenMP),
                  and its gradients dQ, dK, dV (backward pass)
  __init__.py     ctypes wrapper: ``attention``, ``merge``, ``attention_bwd``
                  (with ``bwd_stats``, ``bwd_dq``, ``bwd_dkv`` for sampled
                  rows), ``build``
  layouts.py      global positions of query/key rows under the ring layouts
                  (contiguous blocks, ZigZag chunk pairs) and the per-step plan
                  of the ZigZag ring
  recurrences.py  the pages' own algorithms restated in numpy fp64 (blockwise
                  online softmax, the 4-device ring simulation, the ZigZag
                  step rules with the sigmoid merge); used only to pin the
                  oracle against what the pages claim
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, F16, BF16 = 0, 1, 2

_lib = None


def build(verbose: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile oracle.c into oracle/liboracle.so (gcc, -O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-std=c11", "-Wall", "-Wextra", "-shared",
           "-fPIC", src, "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _load(path: str | None = None):
    """Load liboracle.so (building it if absent or stale); ``path`` loads a
    separately compiled copy instead (tests use this to plant mistakes)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    if path is None and (not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))):
        build()
    lib = ctypes.CDLL(path or _LIB_PATH)
    i64p = ctypes.POINTER(ctypes.c_int64)
    f64p = ctypes.POINTER(ctypes.c_double)
    lib.oracle_attention_rows.restype = ctypes.c_int
    lib.oracle_attention_rows.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int, i64p, i64p, ctypes.c_int, ctypes.c_double, ctypes.c_int64,
        i64p, f64p, f64p, ctypes.c_int]
    lib.oracle_merge_rows.restype = ctypes.c_int
    lib.oracle_merge_rows.argtypes = [f64p, f64p, f64p, f64p, ctypes.c_int64,
                                      ctypes.c_int, f64p, f64p]
    bwd_head = [ctypes.c_void_p] * 4 + [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int, i64p, i64p, ctypes.c_int, ctypes.c_double]
    lib.oracle_bwd_stats.restype = ctypes.c_int
    lib.oracle_bwd_stats.argtypes = bwd_head + [ctypes.c_int64, i64p, f64p, f64p, ctypes.c_int]
    lib.oracle_bwd_dq.restype = ctypes.c_int
    lib.oracle_bwd_dq.argtypes = bwd_head + [f64p, f64p, ctypes.c_int64, i64p, f64p,
                                             ctypes.c_int]
    lib.oracle_bwd_dkv.restype = ctypes.c_int
    lib.oracle_bwd_dkv.argtypes = bwd_head + [f64p, f64p, ctypes.c_int64, i64p, f64p, f64p,
                                              ctypes.c_int]
    lib.oracle_f16_to_double.restype = ctypes.c_double
    lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    if path is None:
        _lib = lib
    return lib


def default_threads() -> int:
    """Threads the oracle uses: OMP_NUM_THREADS if set, else all cores, at most 16."""
    env = os.environ.get("OMP_NUM_THREADS")
    n = int(env) if env and env.isdigit() else (os.cpu_count() or 1)
    return max(1, min(n, 16))


def _as_storage(x):
    """Return (contiguous numpy array holding the storage bits, dtype code).

    Accepts numpy float32/float16 arrays or CPU torch tensors of float32,
    float16 or bfloat16.  bf16 and fp16 are passed as their raw 16-bit
    patterns; the C side decodes them exactly.
    """
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            if x.dtype == torch.float16:
                return x.view(torch.int16).numpy().view(np.uint16), F16
            if x.dtype == torch.float32:
                return x.numpy(), F32
            raise TypeError(f"oracle: unsupported torch dtype {x.dtype}")
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.float16:
        return x.view(np.uint16), F16
    raise TypeError(f"oracle: unsupported numpy dtype {x.dtype}")


def _i64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def attention(q, k, v, causal: bool = False, scale: float | None = None,
              q_pos=None, k_pos=None, rows=None, n_threads: int | None = None,
              lib_path: str | None = None):
    """softmax(scale * Q K^T) V and its log-sum-exp, in float64.

    q: [B, Nq, Hq, d]; k, v: [B, Nk, Hkv, d] (same storage dtype).
    q_pos / k_pos: global positions of the rows (default: 0..Nq-1, 0..Nk-1);
    with ``causal`` a key is visible iff k_pos <= q_pos.
    rows: optional (n, 3) int array of (b, i, hq) triples; then the result is
    (out [n, d], lse [n]).  Without rows: (out [B, Nq, Hq, d], lse [B, Nq, Hq]).
    scale: default 1/sqrt(d).
    lib_path: use a separately compiled copy of oracle.c (tests only).
    """
    lib = _load(lib_path)
    qs, dt = _as_storage(q)
    ks, dtk = _as_storage(k)
    vs, dtv = _as_storage(v)
    if not (dt == dtk == dtv):
        raise TypeError("oracle: q, k, v must share one dtype")
    if qs.ndim != 4 or ks.ndim != 4 or vs.ndim != 4:
        raise ValueError("oracle: q, k, v must be [B, N, H, d]")
    B, Nq, Hq, d = qs.shape
    Bk, Nk, Hkv, dk = ks.shape
    if vs.shape != ks.shape or Bk != B or dk != d:
        raise ValueError("oracle: shape mismatch")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    qp = _i64(np.arange(Nq) if q_pos is None else q_pos)
    kp = _i64(np.arange(Nk) if k_pos is None else k_pos)
    if qp.shape != (Nq,) or kp.shape != (Nk,):
        raise ValueError("oracle: position arrays must have one entry per row")
    if rows is None:
        n = B * Nq * Hq
        rows_arr = None
    else:
        rows_arr = _i64(rows).reshape(-1, 3)
        n = rows_arr.shape[0]
    out = np.empty((n, d), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = lib.oracle_attention_rows(
        qs.ctypes.data, ks.ctypes.data, vs.ctypes.data, dt, B, Hq, Hkv, Nq, Nk, d,
        _ptr(qp, ctypes.c_int64), _ptr(kp, ctypes.c_int64), int(bool(causal)),
        float(scale), n,
        None if rows_arr is None else _ptr(rows_arr, ctypes.c_int64),
        _ptr(out, ctypes.c_double), _ptr(lse, ctypes.c_double),
        n_threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_attention_rows rejected its arguments")
    if rows is None:
        return out.reshape(B, Nq, Hq, d), lse.reshape(B, Nq, Hq)
    return out, lse


def merge(o_a, l_a, o_b, l_b, lib_path: str | None = None):
    """Combine two partial results over disjoint key sets (float64).

    o_*: [..., d], l_*: [...] with matching leading shapes.  Returns (o, lse).
    """
    lib = _load(lib_path)
    o_a = np.ascontiguousarray(o_a, dtype=np.float64)
    o_b = np.ascontiguousarray(o_b, dtype=np.float64)
    l_a = np.ascontiguousarray(l_a, dtype=np.float64)
    l_b = np.ascontiguousarray(l_b, dtype=np.float64)
    if o_a.shape != o_b.shape or l_a.shape != l_b.shape or o_a.shape[:-1] != l_a.shape:
        raise ValueError("oracle.merge: shape mismatch")
    d = o_a.shape[-1]
    n = int(np.prod(l_a.shape)) if l_a.ndim else 1
    o = np.empty_like(o_a)
    lse = np.empty_like(l_a)
    f = ctypes.c_double
    rc = lib.oracle_merge_rows(_ptr(o_a, f), _ptr(l_a, f), _ptr(o_b, f), _ptr(l_b, f),
                               n, d, _ptr(o, f), _ptr(lse, f))
    if rc != 0:
        raise ValueError("oracle_merge_rows rejected its arguments")
    return o, lse


class _BwdArgs:
    """Storage views, shapes and positions shared by the backward wrappers."""

    def __init__(self, q, k, v, dout, causal, scale, q_pos, k_pos):
        self.qs, dt = _as_storage(q)
        self.ks, dtk = _as_storage(k)
        self.vs, dtv = _as_storage(v)
        self.ds, dtd = _as_storage(dout)
        if not (dt == dtk == dtv == dtd):
            raise TypeError("oracle: q, k, v, dout must share one dtype")
        if self.qs.ndim != 4 or self.ks.shape != self.vs.shape or self.ds.shape != self.qs.shape:
            raise ValueError("oracle: q, dout [B, Nq, Hq, d]; k, v [B, Nk, Hkv, d]")
        self.dtype = dt
        self.B, self.Nq, self.Hq, self.d = self.qs.shape
        _, self.Nk, self.Hkv, _ = self.ks.shape
        if self.ks.shape[0] != self.B or self.ks.shape[3] != self.d:
            raise ValueError("oracle: shape mismatch")
        self.scale = 1.0 / np.sqrt(self.d) if scale is None else float(scale)
        self.qp = _i64(np.arange(self.Nq) if q_pos is None else q_pos)
        self.kp = _i64(np.arange(self.Nk) if k_pos is None else k_pos)
        if self.qp.shape != (self.Nq,) or self.kp.shape != (self.Nk,):
            raise ValueError("oracle: position arrays must have one entry per row")
        self.causal = int(bool(causal))

    def head(self):
        return (self.qs.ctypes.data, self.ks.ctypes.data, self.vs.ctypes.data,
                self.ds.ctypes.data, self.dtype, self.B, self.Hq, self.Hkv, self.Nq, self.Nk,
                self.d, _ptr(self.qp, ctypes.c_int64), _ptr(self.kp, ctypes.c_int64),
                self.causal, self.scale)


def _rows(rows, n_all):
    if rows is None:
        return None, n_all
    r = _i64(rows).reshape(-1, 3)
    return r, r.shape[0]


def bwd_stats(q, k, v, dout, causal=False, scale=None, q_pos=None, k_pos=None, rows=None,
              n_threads=None, lib_path=None):
    """Per query row: LSE and D = dO . O (float64).  rows: optional (n, 3)
    (b, i, hq) triples; returns (lse, delta) of shape [n] or [B, Nq, Hq]."""
    lib = _load(lib_path)
    a = _BwdArgs(q, k, v, dout, causal, scale, q_pos, k_pos)
    r, n = _rows(rows, a.B * a.Nq * a.Hq)
    lse = np.empty(n, np.float64)
    delta = np.empty(n, np.float64)
    f = ctypes.c_double
    rc = lib.oracle_bwd_stats(*a.head(), n, None if r is None else _ptr(r, ctypes.c_int64),
                              _ptr(lse, f), _ptr(delta, f), n_threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_bwd_stats rejected its arguments")
    if rows is None:
        return lse.reshape(a.B, a.Nq, a.Hq), delta.reshape(a.B, a.Nq, a.Hq)
    return lse, delta


def bwd_dq(q, k, v, dout, lse_all, delta_all, causal=False, scale=None, q_pos=None,
           k_pos=None, rows=None, n_threads=None, lib_path=None):
    """dQ rows (float64).  lse_all, delta_all: [B, Nq, Hq] from ``bwd_stats``
    (only the requested rows' entries are read).  Returns [n, d] for (b, i, hq)
    rows, else [B, Nq, Hq, d]."""
    lib = _load(lib_path)
    a = _BwdArgs(q, k, v, dout, causal, scale, q_pos, k_pos)
    la = np.ascontiguousarray(lse_all, np.float64)
    da = np.ascontiguousarray(delta_all, np.float64)
    if la.shape != (a.B, a.Nq, a.Hq) or da.shape != la.shape:
        raise ValueError("oracle.bwd_dq: lse_all / delta_all must be [B, Nq, Hq]")
    r, n = _rows(rows, a.B * a.Nq * a.Hq)
    dq = np.empty((n, a.d), np.float64)
    f = ctypes.c_double
    rc = lib.oracle_bwd_dq(*a.head(), _ptr(la, f), _ptr(da, f), n,
                           None if r is None else _ptr(r, ctypes.c_int64), _ptr(dq, f),
                           n_threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_bwd_dq rejected its arguments")
    return dq if rows is not None else dq.reshape(a.B, a.Nq, a.Hq, a.d)


def bwd_dkv(q, k, v, dout, lse_all, delta_all, causal=False, scale=None, q_pos=None,
            k_pos=None, rows=None, n_threads=None, lib_path=None):
    """dK and dV rows (float64), summed over the query heads of each key/value
    head's group.  rows: optional (n, 3) (b, j, g) triples.  Returns (dk, dv)
    of shape [n, d] or [B, Nk, Hkv, d]."""
    lib = _load(lib_path)
    a = _BwdArgs(q, k, v, dout, causal, scale, q_pos, k_pos)
    la = np.ascontiguousarray(lse_all, np.float64)
    da = np.ascontiguousarray(delta_all, np.float64)
    if la.shape != (a.B, a.Nq, a.Hq) or da.shape != la.shape:
        raise ValueError("oracle.bwd_dkv: lse_all / delta_all must be [B, Nq, Hq]")
    r, n = _rows(rows, a.B * a.Nk * a.Hkv)
    dk = np.empty((n, a.d), np.float64)
    dv = np.empty((n, a.d), np.float64)
    f = ctypes.c_double
    rc = lib.oracle_bwd_dkv(*a.head(), _ptr(la, f), _ptr(da, f), n,
                            None if r is None else _ptr(r, ctypes.c_int64), _ptr(dk, f),
                            _ptr(dv, f), n_threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_bwd_dkv rejected its arguments")
    if rows is None:
        shp = (a.B, a.Nk, a.Hkv, a.d)
        return dk.reshape(shp), dv.reshape(shp)
    return dk, dv


def attention_bwd(q, k, v, dout, causal=False, scale=None, q_pos=None, k_pos=None,
                  n_threads=None, lib_path=None):
    """Gradients of sum(dout * attention(q, k, v)) with respect to q, k, v, in
    float64: returns (dq [B,Nq,Hq,d], dk, dv [B,Nk,Hkv,d], lse, delta [B,Nq,Hq])."""
    kw = dict(causal=causal, scale=scale, q_pos=q_pos, k_pos=k_pos, n_threads=n_threads,
              lib_path=lib_path)
    lse, delta = bwd_stats(q, k, v, dout, **kw)
    dq = bwd_dq(q, k, v, dout, lse, delta, **kw)
    dk, dv = bwd_dkv(q, k, v, dout, lse, delta, **kw)
    return dq, dk, dv, lse, delta


def decode_f16(bits: int) -> float:
    """The oracle's own fp16 decoder (exposed so tests can pin it)."""
    return _load().oracle_f16_to_double(bits)


def decode_bf16(bits: int) -> float:
    """The oracle's own bf16 decoder (exposed so tests can pin it)."""
    return _load().oracle_bf16_to_double(bits)
