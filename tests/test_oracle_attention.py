"""Pins of the oracle's attention against closed forms, a library routine and invariants."""
import math

import numpy as np
import pytest
import torch

import workloads as I
from oracle import attention as A
from tests.conftest import load_golden


def test_online_softmax_example():
    """Tiled online softmax of the notes page equals the closed-form softmax mean."""
    g = load_golden("online_softmax_example.json")
    s = np.array(g["scores"])
    v = np.array(g["values"])[:, None]
    # the oracle materialises the row; closed form (1 + 3e + 5e^2) / (1 + e + e^2)
    o, l = A.attention_one_head(np.array([[1.0]]), s[:, None], v, 1.0)
    e = math.e
    closed = (1 + 3 * e + 5 * e * e) / (1 + e + e * e)
    assert abs(o[0, 0] - closed) < 1e-14
    assert abs(l[0] - math.log(1 + e + e * e)) < 1e-14
    # the page's tiling: first tile [0, 2) has max 1 and sum exp(-1) + 1
    (a0, a1), (b0, b1) = g["tiles"]
    oa, la = A.attention_one_head(np.array([[1.0]]), s[a0:a1, None], v[a0:a1], 1.0)
    assert abs(la[0] - (1.0 + math.log(math.exp(-1) + 1))) < 1e-14
    ob, lb = A.attention_one_head(np.array([[1.0]]), s[b0:b1, None], v[b0:b1], 1.0)
    om, lm = A.merge_state(oa, la, ob, lb)
    assert abs(om[0, 0] - closed) < 1e-14 and abs(lm[0] - l[0]) < 1e-14


def test_single_key_closed_form():
    rng = np.random.default_rng(0)
    q, k, v = rng.standard_normal((3, 8)), rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    o, l = A.attention_one_head(q, k, v, 0.3)
    assert np.allclose(o, np.repeat(v, 3, 0), atol=1e-15)
    assert np.allclose(l, 0.3 * (q @ k.T)[:, 0], atol=1e-14)


def test_equal_scores_closed_form():
    rng = np.random.default_rng(1)
    n, d = 9, 4
    k = np.tile(rng.standard_normal((1, d)), (n, 1))
    v = rng.standard_normal((n, d))
    q = rng.standard_normal((2, d))
    o, l = A.attention_one_head(q, k, v, 0.7)
    assert np.allclose(o, np.tile(v.mean(0), (2, 1)), atol=1e-14)
    s = 0.7 * (q @ k[0])
    assert np.allclose(l, s + math.log(n), atol=1e-13)


def test_empty_rows():
    q = np.ones((2, 4))
    k = np.ones((3, 4))
    v = np.ones((3, 4))
    allowed = np.array([[False] * 3, [True, False, False]])
    o, l = A.attention_one_head(q, k, v, 1.0, allowed)
    assert np.all(o[0] == 0) and l[0] == -np.inf
    assert np.allclose(o[1], 1.0) and abs(l[1] - 4.0) < 1e-15
    o, l = A.attention_one_head(q, np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(l))


def _sdpa(q, k, v, scale, causal):
    """torch's fp64 scaled_dot_product_attention on the CPU, [H, L, d] layout."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), is_causal=causal, scale=scale
    ).numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", [0, 1])
def test_matches_library_sdpa_contiguous(seed, causal):
    """Contiguous, non-GQA, l_qo = l_kv: equals torch SDPA (top-left = bottom-right here)."""
    rng = np.random.default_rng(seed)
    H, L, d = 3, 23, 16
    q, k, v = (rng.standard_normal((L, H, d)) for _ in range(3))
    b = _contiguous_batch([L], q, k, v, H, H, qo=[L])
    o, _ = A.batch_attention(
        q, b["k"], b["v"], b["kv_indptr"], b["kv_indices"], b["last"], 1, H, H,
        1 / math.sqrt(d), qo_indptr=b["qo_indptr"], causal=causal,
    )
    ref = _sdpa(q.transpose(1, 0, 2), k.transpose(1, 0, 2), v.transpose(1, 0, 2), 1 / math.sqrt(d), causal)
    assert np.allclose(o.transpose(1, 0, 2), ref, atol=1e-12, rtol=0)


def _contiguous_batch(lens, q, k, v, Hq, Hk, qo=None):
    """Page size 1, rows in order: K/V given as [total_kv, Hk, d]."""
    lens = np.asarray(lens)
    kv_indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    out = {
        "k": k.reshape(-1, 1, Hk, k.shape[-1]),
        "v": v.reshape(-1, 1, Hk, v.shape[-1]),
        "kv_indptr": kv_indptr,
        "kv_indices": np.arange(kv_indptr[-1], dtype=np.int32),
        "last": np.where(lens > 0, 1, 0).astype(np.int32),
        "qo_indptr": None if qo is None else np.concatenate([[0], np.cumsum(qo)]).astype(np.int32),
    }
    return out


def test_bottom_right_causal_is_key_prefix():
    """Row q of a causal request sees exactly its first l_kv - l_qo + q + 1 keys."""
    rng = np.random.default_rng(3)
    Lq, Lk, d, H = 5, 12, 8, 2
    q = rng.standard_normal((Lq, H, d))
    k = rng.standard_normal((Lk, H, d))
    v = rng.standard_normal((Lk, H, d))
    b = _contiguous_batch([Lk], q, k, v, H, H, qo=[Lq])
    o, l = A.batch_attention(q, b["k"], b["v"], b["kv_indptr"], b["kv_indices"], b["last"], 1,
                             H, H, 0.25, qo_indptr=b["qo_indptr"], causal=True)
    for r in range(Lq):
        n = Lk - Lq + r + 1
        ref = _sdpa(q[r : r + 1].transpose(1, 0, 2), k[:n].transpose(1, 0, 2), v[:n].transpose(1, 0, 2), 0.25, False)
        assert np.allclose(o[r], ref[:, 0], atol=1e-12, rtol=0)


def test_causal_decode_equals_noncausal():
    b = I.make_paged_batch(4, [7, 30, 1], None, page_size=4, num_qo_heads=4, num_kv_heads=2,
                           head_dim=8, dtype="f32")
    args = (b.q_f32, b.k_f32, b.v_f32, b.kv_indptr, b.kv_indices, b.last_page_len, 4, 4, 2, 0.35)
    o1, l1 = A.batch_attention(*args, causal=True)
    o2, l2 = A.batch_attention(*args, causal=False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_gqa_equals_repeated_kv_heads():
    rng = np.random.default_rng(7)
    g, Hk, d = 4, 2, 8
    b = I.make_paged_batch(7, [9, 17], [3, 2], page_size=4, num_qo_heads=g * Hk, num_kv_heads=Hk,
                           head_dim=d, dtype="f32", causal=True)
    o, l = A.batch_attention(b.q_f32, b.k_f32, b.v_f32, b.kv_indptr, b.kv_indices, b.last_page_len,
                             4, g * Hk, Hk, 0.3, qo_indptr=b.qo_indptr, causal=True)
    krep = np.repeat(b.k_f32, g, axis=2)
    vrep = np.repeat(b.v_f32, g, axis=2)
    o2, l2 = A.batch_attention(b.q_f32, krep, vrep, b.kv_indptr, b.kv_indices, b.last_page_len,
                               4, g * Hk, g * Hk, 0.3, qo_indptr=b.qo_indptr, causal=True)
    assert np.allclose(o, o2, atol=1e-14, rtol=0) and np.allclose(l, l2, atol=1e-14, rtol=0)
    # and a wrong head mapping (h % H_kv instead of h // g) would differ
    assert not np.allclose(o[:, 1], o[:, g])


@pytest.mark.parametrize("seed", [0, 1])
def test_paged_equals_contiguous_and_permutation_invariance(seed):
    rng = np.random.default_rng(seed)
    lens = [13, 1, 32, 6]
    P, Hq, Hk, d = 4, 4, 2, 8
    b = I.make_paged_batch(seed, lens, None, page_size=P, num_qo_heads=Hq, num_kv_heads=Hk,
                           head_dim=d, dtype="f32", num_pages=40)
    o, l = A.batch_attention(b.q_f32, b.k_f32, b.v_f32, b.kv_indptr, b.kv_indices, b.last_page_len,
                             P, Hq, Hk, 0.3)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), "NaN-poisoned slots must not be read"
    # contiguous copy of the same tokens
    kc = np.concatenate([b.k_f32.reshape(-1, Hk, d)[A.physical_rows(b.kv_indptr, b.kv_indices, b.last_page_len, P, i)] for i in range(4)])
    vc = np.concatenate([b.v_f32.reshape(-1, Hk, d)[A.physical_rows(b.kv_indptr, b.kv_indices, b.last_page_len, P, i)] for i in range(4)])
    c = _contiguous_batch(lens, b.q_f32, kc, vc, Hq, Hk)
    o2, l2 = A.batch_attention(b.q_f32, c["k"], c["v"], c["kv_indptr"], c["kv_indices"], c["last"], 1, Hq, Hk, 0.3)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)
    # relabel the physical pages with a random permutation
    perm = rng.permutation(40)
    k2 = np.empty_like(b.k_f32)
    v2 = np.empty_like(b.v_f32)
    k2[perm] = b.k_f32
    v2[perm] = b.v_f32
    o3, l3 = A.batch_attention(b.q_f32, k2, v2, b.kv_indptr, perm[b.kv_indices], b.last_page_len,
                               P, Hq, Hk, 0.3)
    assert np.array_equal(o, o3) and np.array_equal(l, l3)


def test_scale_and_transpose_are_not_interchangeable():
    """A transposed or unscaled product would change the result of a non-symmetric case."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal((3, 4))
    k = rng.standard_normal((5, 4))
    v = rng.standard_normal((5, 4))
    o, l = A.attention_one_head(q, k, v, 0.5)
    # brute force with scalar loops for one row
    r = 1
    s = [0.5 * sum(q[r, c] * k[j, c] for c in range(4)) for j in range(5)]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    Z = sum(w)
    ov = [sum(w[j] * v[j, c] for j in range(5)) / Z for c in range(4)]
    assert np.allclose(o[r], ov, atol=1e-14) and abs(l[r] - (m + math.log(Z))) < 1e-14


def test_composable_equals_union():
    """Prefix level (+) suffix level equals single-level attention over prefix ++ suffix."""
    b = I.shared_prefix_decode(seed=0, groups=2, per_group=4, prefix_len=32, suffix_lo=3,
                               suffix_hi=20, page_size=4, num_qo_heads=8, num_kv_heads=2,
                               head_dim=16, dtype="f32")
    o, l, _, _ = A.composable_attention(
        b.q_f32, b.k_f32, b.v_f32,
        (b.l1_qo_indptr, b.l1_kv_indptr, b.l1_kv_indices, b.l1_last_page_len),
        (b.l2_kv_indptr, b.l2_kv_indices, b.l2_last_page_len),
        4, 8, 2, 0.25,
    )
    of, lf = A.batch_attention(b.q_f32, b.k_f32, b.v_f32, b.full_kv_indptr, b.full_kv_indices,
                               b.full_last_page_len, 4, 8, 2, 0.25)
    assert np.allclose(o, of, atol=1e-13, rtol=0) and np.allclose(l, lf, atol=1e-13, rtol=0)


def test_cascade_three_levels_equals_union():
    """Level 0 (one prompt for all) (+) level 1 (group prefixes) (+) private suffixes equals
    single-level attention over the concatenated pages of each request (the union check)."""
    b = I.cascade_decode(seed=1, requests=8, groups=(1, 4), prefix_lens=(12, 8), suffix_lo=0,
                         suffix_hi=9, page_size=4, num_qo_heads=8, num_kv_heads=2, head_dim=16,
                         dtype="f32")
    o, l, states = A.cascade_attention(b.q_f32, b.k_f32, b.v_f32, b.levels, b.suffix, 4, 8, 2, 0.25)
    assert len(states) == 3
    of, lf = A.batch_attention(b.q_f32, b.k_f32, b.v_f32, *b.full, 4, 8, 2, 0.25)
    assert np.allclose(o, of, atol=1e-13, rtol=0) and np.allclose(l, lf, atol=1e-13, rtol=0)
    # an empty suffix leaves the prefix levels' state unchanged (the merge's identity)
    empty = np.nonzero(b.suffix_lens == 0)[0]
    for r in empty:
        assert np.all(np.isneginf(states[2][1][r]))


@pytest.mark.parametrize("br,bc", [(4, 8), (16, 16), (1, 4)])
def test_bsr_block_rows_equal_dense_attention_under_the_block_mask(br, bc):
    """The BSR view of a block-sparse mask (block row = B_r queries, its column blocks = pages
    of B_c keys) gives the attention of the dense sequence under the expanded mask ("FlashInfer:
    Engineering ..." §III.1, §IV; block-sparse matrix of B_r x B_c blocks)."""
    bs = I.block_sparse_attention(5, 64, br, bc, 0.35, num_qo_heads=4, num_kv_heads=2, head_dim=16, dtype="f32")
    b = bs.dense
    o, l = A.batch_attention(b.q_f32, b.k_f32, b.v_f32, b.kv_indptr, b.kv_indices, b.last_page_len, bc, 4, 2,
                             0.25, qo_indptr=b.qo_indptr)
    dense_mask = np.kron(bs.block_mask, np.ones((br, bc), dtype=bool))
    npg = b.k_f32.shape[0]
    od, ld = A.batch_attention(b.q_f32, b.k_f32, b.v_f32, [0, npg], np.arange(npg), [bc], bc, 4, 2, 0.25,
                               qo_indptr=[0, 64], custom_mask=[dense_mask])
    assert np.array_equal(np.isneginf(l), np.isneginf(ld))
    fin = np.isfinite(l)
    assert np.allclose(o, od, atol=1e-12) and np.allclose(l[fin], ld[fin], atol=1e-12)
