"""fp64 CPU oracle for exact (ring) attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP path (``ring_attention_amd``)
never imports it, and it imports nothing from the HIP path.

Contents
  oracle.c        the definition softmax(scale*QK^T)V in double (C + OpenMP)
  __init__.py     ctypes wrapper: ``attention``, ``merge``, ``build``
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


def decode_f16(bits: int) -> float:
    """The oracle's own fp16 decoder (exposed so tests can pin it)."""
    return _load().oracle_f16_to_double(bits)


def decode_bf16(bits: int) -> float:
    """The oracle's own bf16 decoder (exposed so tests can pin it)."""
    return _load().oracle_bf16_to_double(bits)
