"""bsr_run_decode_scratch (decode on the library's static scratch, no caller workspace) against
bsr_run_decode on the same plan and inputs: two calls in a row, the second on a smaller batch, each
bitwise equal to the workspace entry point (same kernels, same plan) and within the bf16 tolerance
of the fp64 oracle.  A plan that needs more than the scratch is rejected on the host.
"""
import ctypes as C
import math
import os

import numpy as np
import pytest

import workloads as I
from block_sparse_paged_bsr_amd import _lib
from tests.gpu_helpers import compare, log, make_plan, oracle


def _have_gpu():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libbsr_attn.so not built")
def test_scratch_capacity_rejected_on_the_host():
    """A plan whose workspace exceeds the 32 MiB scratch returns BSR_CAPACITY before any GPU
    call (runs without a GPU)."""
    lens = np.full(2048, 8192)
    ip, ix, la = I.page_table_from_lengths(lens, 16, np.arange(int((lens // 16).sum())))
    from block_sparse_paged_bsr_amd import api

    p = api.Plan(ip, ix, la, num_pages=len(ix), num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                 num_workers=4096)
    assert p.workspace_bytes() > 32 << 20
    rc = _lib.lib().bsr_run_decode_scratch(p.handle, None, None, None, None, None, 1, 0.1, None)
    assert rc == _lib.BSR_CAPACITY
    assert "32" in _lib.lib().bsr_last_error().decode() or "33554432" in _lib.lib().bsr_last_error().decode()


@pytest.mark.gpu
def test_scratch_decode_matches_workspace_decode():
    import torch
    from block_sparse_paged_bsr_amd import api

    if not _have_gpu():
        pytest.skip("no GPU")
    api.version()
    cases = [
        ("batch-64 decode", I.batched_decode_bf16(seed=0), 256),
        ("smaller batch", I.make_paged_batch(7, [300, 17, 1000, 0, 64], None, page_size=16, num_qo_heads=32,
                                             num_kv_heads=8, head_dim=128), 16),
    ]
    sm = 1.0 / math.sqrt(128)
    for name, b, C_ in cases:
        log(f"[decode scratch] {name}: batch {b.batch}, tokens {int(b.kv_lens.sum())}, workers {C_}")
        p = make_plan(b, num_workers=C_)
        assert p.workspace_bytes() <= 32 << 20
        q, k, v = b.torch_values("cuda")
        ws = api.alloc_workspace(p)
        p.upload(ws)
        o_ref, l_ref = api.run_decode(p, ws, q, k, v, sm_scale=sm)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((q.shape[0], 32), float("nan"), dtype=torch.float32, device="cuda")
        api.run_decode_scratch(p, q, k, v, o, lse, sm_scale=sm)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), name
        ro, rl = oracle(b)
        compare(o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, "bf16", f"decode scratch, {name}")
