"""The C ABI without a GPU: exports and host-side argument checks.

Every call here is rejected (or has no work) before anything is enqueued, so
these tests never launch a kernel.  Fake device pointers are plain aligned
integers that are never dereferenced.  The two checks that make a valid call
(and expect RATTN_EHIP from its failed launch) skip where a GPU is visible.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from ring_attention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rattn.h")

OK, EINVAL, EUNSUP, EHIP = 0, -1, -2, -3
P = [0x10000 * (i + 1) for i in range(8)]  # 16-byte aligned, never dereferenced


def declared():
    text = open(HEADER).read()
    return set(re.findall(r"RATTN_API\s+[\w\s\*]*?\b(rattn_\w+)\s*\(", text))


def test_header_declares_the_binding_exports():
    assert declared() == set(binding.EXPORTS)


def test_library_exports_exactly_the_header(rattn_lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.split()[1:2] == ["T"]}
    assert syms == declared()
    for name in declared():
        assert hasattr(rattn_lib, name)


def test_status_strings(rattn_lib):
    for code in (OK, EINVAL, EUNSUP, EHIP, 12345):
        s = binding.status_string(code)
        assert isinstance(s, str) and s
    assert binding.status_string(12345) == "unknown status"


def fwd(lib, q=P[0], k=P[1], v=P[2], out=P[3], lse=P[4], B=1, Hq=2, Hkv=2, Nq=64, N=64, d=64,
        dtype=2, scale=0.0, causal=1, W=1, zigzag=0, rank=-1):
    return lib.rattn_fwd(q, k, v, out, lse, B, Hq, Hkv, Nq, N, d, dtype, scale, causal, W,
                         zigzag, rank, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), EINVAL), (dict(lse=0), EINVAL), (dict(B=0), EINVAL), (dict(Hq=3, Hkv=2), EINVAL),
    (dict(Hkv=0), EINVAL), (dict(d=48), EUNSUP), (dict(d=256), EUNSUP), (dict(dtype=3), EINVAL),
    (dict(causal=2), EINVAL), (dict(zigzag=2), EINVAL), (dict(W=0), EINVAL), (dict(W=33), EUNSUP),
    (dict(W=3, N=64, Nq=64), EINVAL), (dict(W=4, zigzag=1, N=68, Nq=68), EINVAL),
    (dict(W=4, rank=4), EINVAL), (dict(W=4, rank=-2), EINVAL),
    (dict(W=4, rank=-1, Nq=16), EINVAL), (dict(W=4, rank=1, Nq=64), EINVAL),
    (dict(q=P[0] + 2), EINVAL), (dict(out=P[3] + 8), EINVAL), (dict(lse=P[4] + 2), EINVAL),
    (dict(N=-4, Nq=-4), EINVAL), (dict(B=1 << 30, Hq=1 << 30, Hkv=1 << 30, N=1 << 20,
                                       Nq=1 << 20, d=128), EUNSUP),
    # a sequence of 2^31 rows (the kernels count a run's rows in 32 bits)
    (dict(B=1, Hq=1, Hkv=1, N=1 << 31, Nq=1 << 31), EUNSUP),
])
def test_fwd_rejects(rattn_lib, kw, status):
    assert fwd(rattn_lib, **kw) == status


def test_fwd_empty_is_ok_without_launch(rattn_lib):
    assert fwd(rattn_lib, N=0, Nq=0) == OK
    assert fwd(rattn_lib, N=0, Nq=0, W=4, zigzag=1) == OK
    # empty tensors may come with null pointers
    assert fwd(rattn_lib, q=0, k=0, v=0, out=0, lse=0, N=0, Nq=0) == OK
    assert fwd(rattn_lib, k=0, N=64, Nq=64) == EINVAL


QUEUE_WS = 64  # RATTN_QUEUE_WS_BYTES


def fwd_queued(lib, ws=P[5], ws_bytes=QUEUE_WS, **kw):
    a = dict(q=P[0], k=P[1], v=P[2], out=P[3], lse=P[4], B=1, Hq=2, Hkv=2, Nq=64, N=64, d=64,
             dtype=2, scale=0.0, causal=1, W=1, zigzag=0, rank=-1)
    a.update(kw)
    return lib.rattn_fwd_queued(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"],
                                a["Hkv"], a["Nq"], a["N"], a["d"], a["dtype"], a["scale"],
                                a["causal"], a["W"], a["zigzag"], a["rank"], ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(ws=0), EINVAL), (dict(ws_bytes=QUEUE_WS - 4), EINVAL), (dict(ws=P[5] + 2), EINVAL),
    (dict(q=0), EINVAL), (dict(Hq=3), EINVAL), (dict(d=48), EUNSUP), (dict(W=3), EINVAL),
    (dict(B=1, Hq=1, Hkv=1, N=1 << 31, Nq=1 << 31), EUNSUP),
])
def test_fwd_queued_rejects(rattn_lib, kw, status):
    """The queued forward checks what rattn_fwd checks, and its workspace."""
    assert fwd_queued(rattn_lib, **kw) == status


def test_fwd_queued_empty_is_ok_without_launch(rattn_lib):
    assert fwd_queued(rattn_lib, N=0, Nq=0) == OK
    # the tensor checks come first: an empty call needs no workspace either
    assert fwd_queued(rattn_lib, N=0, Nq=0, ws=0) == OK


def fwd_split(lib, n_splits=4, ws=P[5], ws_floats=None, **kw):
    a = dict(q=P[0], k=P[1], v=P[2], out=P[3], lse=P[4], B=1, Hq=2, Hkv=2, Nq=64, N=64, d=64,
             dtype=2, scale=0.0, causal=1, W=1, zigzag=0, rank=-1)
    a.update(kw)
    need = n_splits * a["B"] * a["Nq"] * a["Hq"] * (a["d"] + 1)
    return lib.rattn_fwd_split(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"],
                               a["Hkv"], a["Nq"], a["N"], a["d"], a["dtype"], a["scale"],
                               a["causal"], a["W"], a["zigzag"], a["rank"], n_splits, ws,
                               need if ws_floats is None else ws_floats, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_splits=0), EINVAL), (dict(n_splits=65), EUNSUP), (dict(ws=0), EINVAL),
    (dict(ws_floats=100), EINVAL), (dict(ws=P[5] + 4), EINVAL), (dict(q=0), EINVAL),
    (dict(d=48), EUNSUP), (dict(W=3), EINVAL),
])
def test_fwd_split_rejects(rattn_lib, kw, status):
    assert fwd_split(rattn_lib, **kw) == status


def test_fwd_split_empty_is_ok_without_launch(rattn_lib):
    assert fwd_split(rattn_lib, N=0, Nq=0) == OK
    assert fwd_split(rattn_lib, N=0, Nq=0, ws=0) == OK


def split_noalloc(lib, n_splits=4, **kw):
    a = dict(q=P[0], k=P[1], v=P[2], out=P[3], lse=P[4], B=1, Hq=2, Hkv=2, Nq=64, N=64, d=64,
             dtype=2, scale=0.0, causal=1, W=1, zigzag=0, rank=-1)
    a.update(kw)
    return lib.rattn_fwd_split_noalloc(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"],
                                       a["Hq"], a["Hkv"], a["Nq"], a["N"], a["d"], a["dtype"],
                                       a["scale"], a["causal"], a["W"], a["zigzag"], a["rank"],
                                       n_splits, None)


ESCRATCH = -4
SCRATCH_FLOATS = 8 << 20  # RATTN_NOALLOC_SCRATCH_FLOATS


@pytest.mark.parametrize("kw,status", [
    (dict(n_splits=0), EINVAL), (dict(n_splits=65), EUNSUP), (dict(q=0), EINVAL),
    (dict(Hq=3), EINVAL), (dict(d=48), EUNSUP), (dict(out=P[3] + 4), EINVAL),
    # partials beyond the fixed scratch: 64 * 1 * 65536 * 2 * 129 floats > 8M
    (dict(n_splits=64, Nq=65536, N=65536), ESCRATCH),
    (dict(n_splits=2, B=1, Hq=32, Hkv=8, Nq=1024, N=1024, d=128), ESCRATCH),
])
def test_fwd_split_noalloc_rejects(rattn_lib, kw, status):
    """Argument checks, and calls whose partials exceed the library's fixed
    scratch, are refused on the host before any device work."""
    assert split_noalloc(rattn_lib, **kw) == status


def test_fwd_split_noalloc_scratch_bound(rattn_lib):
    def need(n, B, Nq, Hq, d):
        return n * B * Nq * Hq * (d + 1)
    assert need(2, 1, 1024, 32, 128) > SCRATCH_FLOATS          # the last case above
    assert need(8, 1, 4096, 1, 128) <= SCRATCH_FLOATS          # one 4096-row head, 8 splits
    assert b"scratch" in rattn_lib.rattn_status_string(ESCRATCH)


def test_fwd_split_noalloc_empty_needs_no_scratch(rattn_lib):
    assert split_noalloc(rattn_lib, N=0, Nq=0) == OK


def test_fwd_split_noalloc_single_split_needs_no_scratch_without_gpu(rattn_lib):
    """A single split is rattn_fwd: no scratch check at any size.  The call is
    valid, so it launches: with the fake pointers of this file it may only run
    where launches must fail."""
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: a valid call would launch on fake pointers")
    assert split_noalloc(rattn_lib, n_splits=1, Nq=65536, N=65536) == EHIP


def test_split_hint(rattn_lib):
    h = rattn_lib.rattn_split_hint
    # (B, Hq, Nq, N, d, dtype, W, zigzag, rank, n_cu)
    assert h(1, 1, 4096, 4096, 128, 2, 1, 0, -1, 256) == 8   # 16 tiles of 256 rows -> 128 items
    assert h(1, 8, 16384, 131072, 128, 2, 8, 1, 2, 256) == 1   # 512 query tiles already
    assert h(1, 1, 256, 256, 128, 2, 1, 0, -1, 256) == 1       # 4 key tiles: no split
    assert h(1, 1, 1024, 1024, 128, 2, 1, 0, -1, 256) == 2     # 16 key tiles: at most 2
    assert h(1, 1, 64, 1 << 20, 64, 1, 1, 0, -1, 256) == 64    # capped at 64
    assert h(1, 1, 4096, 4096, 48, 2, 1, 0, -1, 256) == 1      # unsupported d
    assert h(0, 1, 4096, 4096, 128, 2, 1, 0, -1, 256) == 1


def seg(a, b):
    return (ctypes.c_int64 * 2)(a, b)


def step(lib, Nq=32, Nk=32, qs=(0, 0), ql=(32, 0), ks=(0, 0), kl=(32, 0), d=128, dtype=1,
         causal=1, q=P[0], out=P[3], nulls=False, q_rows=None, q_off=0, k_rows=None, k_off=0):
    arrs = [None] * 4 if nulls else [seg(*qs), seg(*ql), seg(*ks), seg(*kl)]
    q_rows = Nq if q_rows is None else q_rows
    k_rows = Nk if k_rows is None else k_rows
    return lib.rattn_fwd_step(q, P[1], P[2], out, P[4], 1, 4, 2, q_rows, q_off, Nq, k_rows,
                              k_off, Nk, d, dtype, 0.0, causal, *arrs, None)


@pytest.mark.parametrize("kw,status", [
    (dict(nulls=True), EINVAL), (dict(q=0), EINVAL), (dict(ql=(30, 0)), EINVAL),
    (dict(kl=(16, 8)), EINVAL), (dict(ql=(40, -8)), EINVAL), (dict(d=12), EUNSUP),
    (dict(dtype=-1), EINVAL), (dict(causal=-1), EINVAL), (dict(out=P[3] + 4), EINVAL),
    # row ranges outside the query / key row spaces
    (dict(q_off=1), EINVAL), (dict(q_off=-1, q_rows=64), EINVAL), (dict(q_rows=31), EINVAL),
    (dict(k_off=40, k_rows=64), EINVAL), (dict(k_off=-1, k_rows=64), EINVAL),
])
def test_fwd_step_rejects(rattn_lib, kw, status):
    assert step(rattn_lib, **kw) == status


def step_merge(lib, Nq=32, Nq_out=64, off=0, q=P[0], out=P[3], q_rows=None, q_off=0):
    q_rows = Nq if q_rows is None else q_rows
    return lib.rattn_fwd_step_merge(q, P[1], P[2], out, P[4], 1, 4, 2, q_rows, q_off, Nq, 32, 0,
                                    32, 128, 1, 0.0, 1, seg(0, 0), seg(Nq, 0), seg(0, 0),
                                    seg(32, 0), Nq_out, off, None)


@pytest.mark.parametrize("kw,status", [
    (dict(off=40), EINVAL), (dict(off=-1), EINVAL), (dict(Nq_out=16), EINVAL),
    (dict(Nq_out=-1), EINVAL), (dict(q=0), EINVAL), (dict(out=P[3] + 4), EINVAL),
    (dict(q_off=8, q_rows=32), EINVAL),
])
def test_fwd_step_merge_rejects(rattn_lib, kw, status):
    assert step_merge(rattn_lib, **kw) == status


def test_fwd_step_empty_is_ok_without_launch(rattn_lib):
    assert step(rattn_lib, Nq=0, ql=(0, 0)) == OK
    assert step(rattn_lib, Nq=0, ql=(0, 0), q=0, out=0) == OK


def merge(lib, out=P[0], lse=P[1], bo=P[2], bl=P[3], B=1, H=2, Nq=8, Nb=4, off=0, d=64):
    return lib.rattn_merge(out, lse, bo, bl, B, H, Nq, Nb, off, d, None)


@pytest.mark.parametrize("kw,status", [
    (dict(out=0), EINVAL), (dict(bl=0), EINVAL), (dict(B=0), EINVAL), (dict(Nb=-1), EINVAL),
    (dict(off=5), EINVAL), (dict(off=-1), EINVAL), (dict(Nb=9), EINVAL), (dict(d=8), EUNSUP),
    (dict(out=P[0] + 4), EINVAL), (dict(lse=P[1] + 1), EINVAL),
])
def test_merge_rejects(rattn_lib, kw, status):
    assert merge(rattn_lib, **kw) == status


def test_merge_empty_is_ok_without_launch(rattn_lib):
    assert merge(rattn_lib, Nb=0) == OK
    assert merge(rattn_lib, Nb=0, bo=0, bl=0) == OK


def test_launch_error_maps_to_status_without_gpu(rattn_lib):
    """With no GPU present, a valid call reports RATTN_EHIP instead of crashing."""
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: this check only runs where launches must fail")
    assert merge(rattn_lib) == EHIP
    assert fwd(rattn_lib) == EHIP


def test_binding_checks_tensors_before_calling():
    q = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError):
        binding.fwd(q, q, q)  # CPU tensors are refused before any library call
    with pytest.raises(ValueError):
        binding.merge(q, torch.zeros(1, 4, 1), q, torch.zeros(1, 4, 1))


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        binding.load_library(str(tmp_path / "librattn.so"))


# ---- backward entry points --------------------------------------------------

def bwd(lib, q=P[0], k=P[1], v=P[2], out=P[3], lse=P[4], dout=P[5], dq=P[6], dk=P[7],
        dv=P[7] + 0x100000, ws=P[7] + 0x200000, B=1, Hq=2, Hkv=2, Nq=64, N=64, d=64, dtype=2,
        scale=0.0, causal=1, W=1, zigzag=0, rank=-1):
    return lib.rattn_bwd(q, k, v, out, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, Nq, N, d, dtype,
                         scale, causal, W, zigzag, rank, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), EINVAL), (dict(dout=0), EINVAL), (dict(dq=0), EINVAL), (dict(dk=0), EINVAL),
    (dict(ws=0), EINVAL), (dict(lse=0), EINVAL), (dict(B=0), EINVAL),
    (dict(Hq=3, Hkv=2), EINVAL), (dict(d=48), EUNSUP), (dict(dtype=3), EINVAL),
    (dict(causal=2), EINVAL), (dict(W=0), EINVAL), (dict(W=33), EUNSUP),
    (dict(W=3), EINVAL), (dict(W=4, zigzag=1, N=68, Nq=68), EINVAL), (dict(W=4, rank=4), EINVAL),
    (dict(W=4, rank=1, Nq=64), EINVAL), (dict(dout=P[5] + 8), EINVAL),
    (dict(dv=P[7] + 0x100008), EINVAL), (dict(ws=P[7] + 0x200002), EINVAL),
])
def test_bwd_rejects(rattn_lib, kw, status):
    assert bwd(rattn_lib, **kw) == status


def test_bwd_empty_is_ok_without_launch(rattn_lib):
    assert bwd(rattn_lib, N=0, Nq=0) == OK
    assert bwd(rattn_lib, q=0, k=0, v=0, out=0, lse=0, dout=0, dq=0, dk=0, dv=0, ws=0, N=0,
               Nq=0) == OK


def bwd_step(lib, q=P[0], k=P[1], v=P[2], dout=P[3], lse=P[4], delta=P[5], dq=P[6], dk=P[7],
             dv=P[7] + 0x100000, B=1, Hq=2, Hkv=1, q_rows=64, q_off=0, Nq=64, k_rows=64,
             k_off=0, Nk=64, d=64, dtype=2, scale=0.0, causal=1, qs=(0, 32), ql=(32, 32),
             ks=(0, 32), kl=(32, 32)):
    arr = lambda t: (ctypes.c_int64 * 2)(*t)  # noqa: E731
    return lib.rattn_bwd_step(q, k, v, dout, lse, delta, dq, dk, dv, B, Hq, Hkv, q_rows, q_off,
                              Nq, k_rows, k_off, Nk, d, dtype, scale, causal, arr(qs), arr(ql),
                              arr(ks), arr(kl), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), EINVAL), (dict(delta=0), EINVAL), (dict(dk=0), EINVAL),
    (dict(Hq=3, Hkv=2), EINVAL),
    (dict(d=8), EUNSUP), (dict(q_off=8), EINVAL), (dict(k_off=-1), EINVAL),
    (dict(Nq=65), EINVAL), (dict(ql=(32, 31)), EINVAL), (dict(kl=(-1, 65)), EINVAL),
    (dict(q_rows=128, q_off=96, Nq=64, ql=(64, 0)), EINVAL),
    (dict(dq=P[6] + 4), EINVAL), (dict(causal=3), EINVAL),
])
def test_bwd_step_rejects(rattn_lib, kw, status):
    assert bwd_step(rattn_lib, **kw) == status


def test_bwd_step_without_pairs_is_ok(rattn_lib):
    assert bwd_step(rattn_lib, Nk=0, kl=(0, 0)) == OK
    assert bwd_step(rattn_lib, q_rows=128, q_off=128, Nq=0, ql=(0, 0), qs=(0, 0)) == OK


@pytest.mark.parametrize("args,status", [
    ((P[0], P[1], P[2], -1, 64, 2), EINVAL), ((0, P[1], P[2], 8, 64, 2), EINVAL),
    ((P[0], P[1], P[2], 8, 24, 2), EUNSUP), ((P[0], P[1], P[2], 8, 64, 5), EINVAL),
    ((P[0] + 8, P[1], P[2], 8, 64, 2), EINVAL), ((0, 0, 0, 0, 64, 2), OK),
])
def test_bwd_delta_rejects(rattn_lib, args, status):
    assert rattn_lib.rattn_bwd_delta(*args, None) == status


def fwd_varlen(lib, q=P[0], k=P[1], v=P[2], out=P[3], lse=P[4], qs=P[5], ql=P[5] + 256,
               ks=P[5] + 512, kl=P[5] + 768, n_seq=3, max_len_q=64, Nq=128, Nk=128, Hq=2,
               Hkv=1, d=64, dtype=2, scale=0.0, causal=1):
    return lib.rattn_fwd_varlen(q, k, v, out, lse, qs, ql, ks, kl, n_seq, max_len_q, Nq, Nk, Hq,
                                Hkv, d, dtype, scale, causal, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), EINVAL), (dict(qs=0), EINVAL), (dict(kl=0), EINVAL), (dict(Hq=3, Hkv=2), EINVAL),
    (dict(n_seq=-1), EINVAL), (dict(max_len_q=-5), EINVAL), (dict(d=48), EUNSUP),
    (dict(dtype=7), EINVAL), (dict(causal=5), EINVAL), (dict(out=P[3] + 4), EINVAL),
    (dict(ql=P[5] + 258), EINVAL), (dict(Nq=-1), EINVAL),
])
def test_fwd_varlen_rejects(rattn_lib, kw, status):
    assert fwd_varlen(rattn_lib, **kw) == status


def test_fwd_varlen_without_work_is_ok(rattn_lib):
    assert fwd_varlen(rattn_lib, n_seq=0) == OK
    assert fwd_varlen(rattn_lib, max_len_q=0) == OK
    assert fwd_varlen(rattn_lib, q=0, out=0, lse=0, Nq=0) == OK


def test_varlen_from_cu_seqlens():
    assert binding.varlen_from_cu_seqlens([0, 3, 3, 10]) == ([0, 3, 3], [3, 0, 7])
    with pytest.raises(ValueError):
        binding.varlen_from_cu_seqlens([1, 3])
    with pytest.raises(ValueError):
        binding.varlen_from_cu_seqlens([0, 5, 4])


def bwd_varlen(lib, q=P[0], k=P[1], v=P[2], out=P[3], lse=P[4], dout=P[5], dq=P[6], dk=P[7],
               dv=P[7] + 0x100000, ws=P[7] + 0x200000, qs=P[5] + 256, ql=P[5] + 512,
               ks=P[5] + 768, kl=P[5] + 1024, n_seq=3, max_q=64, max_k=64, Nq=128, Nk=128,
               Hq=2, Hkv=1, d=64, dtype=2, scale=0.0, causal=1):
    return lib.rattn_bwd_varlen(q, k, v, out, lse, dout, dq, dk, dv, ws, qs, ql, ks, kl, n_seq,
                                max_q, max_k, Nq, Nk, Hq, Hkv, d, dtype, scale, causal, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), EINVAL), (dict(dq=0), EINVAL), (dict(ws=0), EINVAL), (dict(kl=0), EINVAL),
    (dict(Hq=3, Hkv=2), EINVAL), (dict(n_seq=-2), EINVAL), (dict(max_k=-1), EINVAL),
    (dict(d=100), EUNSUP), (dict(dtype=9), EINVAL), (dict(causal=4), EINVAL),
    (dict(dk=P[7] + 2), EINVAL), (dict(qs=P[5] + 258), EINVAL),
    (dict(max_q=1 << 40), EUNSUP),
])
def test_bwd_varlen_rejects(rattn_lib, kw, status):
    assert bwd_varlen(rattn_lib, **kw) == status


def test_bwd_varlen_without_work_is_ok(rattn_lib):
    assert bwd_varlen(rattn_lib, n_seq=0) == OK
    assert bwd_varlen(rattn_lib, Nq=0, Nk=0) == OK
