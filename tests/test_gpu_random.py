"""Randomised GPU parity: seeded random shapes across every path the library dispatches to
(decode and tiled kernels, fp32 and bf16, every page-size class, GQA group sizes 1-8, tile
sizes, worker counts, causal, sliding window and soft cap), each case against the oracle.
The seed of a case is printed before it runs."""
import math

import numpy as np
import pytest

import workloads as I
from tests.gpu_helpers import compare, log, make_plan, oracle, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_paged_bsr_amd import api

    api.version()  # loads the library or raises


def _case(seed):
    rng = np.random.default_rng(7000 + seed)
    B = int(rng.integers(1, 7))
    kv = rng.integers(0, 1500, size=B)
    decode = bool(rng.random() < 0.4)
    if decode:
        qo = None
    else:
        qo = np.minimum(rng.integers(1, 400, size=B), np.maximum(kv, 1))
        kv = np.maximum(kv, qo)  # queries are the last positions of their request
    f32 = bool(rng.random() < 0.2)
    d = int(rng.choice([16, 64, 128])) if f32 else int(rng.choice([64, 128]))
    Hk = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    P = int(rng.choice([1, 4, 8, 12, 16, 32]))
    causal = (not decode) and bool(rng.random() < 0.7)
    window = int(rng.choice([-1, -1, 0, 17, 300]))
    cap = float(rng.choice([0.0, 0.0, 2.0, 7.5]))
    C = int(rng.integers(1, 300))
    tq = int(rng.choice([0, 0, 16, 32, 64, 128]))
    return dict(kv=kv.tolist(), qo=None if qo is None else qo.tolist(), f32=f32, d=d, Hk=Hk, g=g, P=P,
                causal=causal, window=window, cap=cap, C=C, tq=tq)


@pytest.mark.parametrize("seed", range(24))
def test_random_case(seed):
    c = _case(seed)
    log(f"[random {seed}] {c}")
    b = I.make_paged_batch(8000 + seed, c["kv"], c["qo"], page_size=c["P"], num_qo_heads=c["Hk"] * c["g"],
                           num_kv_heads=c["Hk"], head_dim=c["d"], dtype="f32" if c["f32"] else "bf16",
                           causal=c["causal"], num_pages=sum((x + c["P"] - 1) // c["P"] for x in c["kv"]) + 3)
    p = make_plan(b, num_workers=c["C"], tile_q=c["tq"], window_left=c["window"], soft_cap=c["cap"])
    o, l, _ = run_gpu(b, p)
    ro, rl = oracle(b, window_left=c["window"], soft_cap=c["cap"])
    compare(o, l, ro, rl, "f32" if c["f32"] else "bf16", f"random {seed}")
