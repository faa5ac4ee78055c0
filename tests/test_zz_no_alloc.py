"""rattn_fwd_split_noalloc (split-KV forward with the library's fixed scratch)
against rattn_fwd_split (caller workspace), through the C ABI (needs a GPU).

Both run the same kernels; only where the split partials live differs, so
the outputs must agree bit for bit.  Two calls in a row on the same GPU, the
second smaller and on another kernel (d = 64, causal, ZigZag), so the
second reuses the scratch that still holds the first call's partials.
"""
import sys

import pytest
import torch

from ring_attention_amd import binding, workloads

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def call_noalloc(lib, q, k, v, causal, W, zigzag, rank, n_splits):
    B, Nq, Hq, d = q.shape
    N, Hkv = k.shape[1], k.shape[2]
    out = torch.empty_like(q)
    lse = torch.empty((B, Nq, Hq), dtype=torch.float32, device=q.device)
    rc = lib.rattn_fwd_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), B, Hq, Hkv, Nq, N, d,
                                     binding.DTYPE_CODES[q.dtype], 0.0, int(causal), W,
                                     int(zigzag), rank, n_splits,
                                     torch.cuda.current_stream().cuda_stream)
    assert rc == 0, binding.status_string(rc)
    return out, lse


CASES = [
    # (name, B, N, Hq, Hkv, d, dtype, causal, W, zigzag, n_splits)
    ("one head 4096, d=128 bf16, 8 splits", 1, 4096, 1, 1, 128, torch.bfloat16, False, 1, False,
     8),
    ("2 heads 1024 GQA, d=64 f16, causal ZigZag W=2, 4 splits", 1, 1024, 2, 1, 64,
     torch.float16, True, 2, True, 4),
]


def test_noalloc_split_equals_workspace_split(gpu):
    lib = binding.load_library()
    for i, (name, B, N, Hq, Hkv, d, dtype, causal, W, zz, ns) in enumerate(CASES):
        note(f"case no-alloc split: {name}")
        q, k, v = workloads.make_qkv(B, N, N, Hq, Hkv, d, dtype, seed=90 + i, device=gpu)
        need = ns * B * N * Hq * (d + 1)
        assert need <= 8 << 20
        out_a, lse_a = call_noalloc(lib, q, k, v, causal, W, zz, -1, ns)
        out_b, lse_b = binding.fwd_split(q, k, v, causal=causal, n_ring_steps=W, zigzag=zz,
                                         rank=-1, n_splits=ns)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), name
        assert torch.equal(lse_a, lse_b), name
        # and the same result as the unsplit call, to the 16-bit bar
        out_c, lse_c = binding.fwd(q, k, v, causal=causal, n_ring_steps=W, zigzag=zz, rank=-1)
        torch.cuda.synchronize()
        assert (out_a.float() - out_c.float()).abs().max().item() <= 2e-2
        fin = torch.isfinite(lse_c)
        assert torch.equal(torch.isfinite(lse_a), fin)
        assert (lse_a[fin] - lse_c[fin]).abs().max().item() <= 1e-3
