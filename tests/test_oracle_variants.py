"""Oracle pins for the attention variants: sliding window and logits soft cap.

Sliding window ("FlashInfer 原理" §⑧): key k visible to query q iff
k + l_qo + window_left >= l_kv + q.  Soft cap (review §5, eq. 8): every score s is
replaced by c * tanh(s / c), c > 0, before masking.  Each pin below is a closed form or a
loop written from those sentences, independent of the oracle's matrix code.
"""
import math

import numpy as np

import workloads as I
from oracle import attention as A
from oracle import plan as PL


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_soft_cap_one_key_closed_form():
    q, k, v = _rand(0, 1, 8), _rand(1, 1, 8), _rand(2, 1, 5)
    s = 0.3 * float(q[0] @ k[0])
    o, l = A.attention_one_head(q, k, v, 0.3, soft_cap=0.7)
    assert np.allclose(o[0], v[0], atol=1e-15) and abs(l[0] - 0.7 * math.tanh(s / 0.7)) < 1e-15


def test_soft_cap_saturation_gives_equal_weights():
    # scores far above the cap all map to ~c: the weights become equal, O = mean(V),
    # LSE = c + ln(n)
    q = np.ones((1, 4))
    k = np.array([[50.0, 0, 0, 0], [60.0, 0, 0, 0], [70.0, 0, 0, 0]])
    v = _rand(3, 3, 6)
    o, l = A.attention_one_head(q, k, v, 1.0, soft_cap=1.0)
    assert np.allclose(o[0], v.mean(axis=0), atol=1e-12)
    assert abs(l[0] - (1.0 + math.log(3))) < 1e-12


def test_soft_cap_brute_force_loop():
    q, k, v = _rand(4, 3, 6), _rand(5, 7, 6), _rand(6, 7, 4)
    sm, cap = 0.4, 1.3
    o, l = A.attention_one_head(q, k, v, sm, soft_cap=cap)
    for r in range(3):
        t = [cap * math.tanh(sm * sum(q[r, c] * k[j, c] for c in range(6)) / cap) for j in range(7)]
        m = max(t)
        w = [math.exp(x - m) for x in t]
        Z = sum(w)
        ref = [sum(w[j] * v[j, c] for j in range(7)) / Z for c in range(4)]
        assert np.allclose(o[r], ref, atol=1e-14) and abs(l[r] - (m + math.log(Z))) < 1e-14


def test_soft_cap_large_cap_is_identity():
    q, k, v = _rand(7, 4, 8), _rand(8, 9, 8), _rand(9, 9, 8)
    o0, l0 = A.attention_one_head(q, k, v, 0.35)
    o1, l1 = A.attention_one_head(q, k, v, 0.35, soft_cap=1e7)
    assert np.allclose(o0, o1, atol=1e-9) and np.allclose(l0, l1, atol=1e-9)


def _batch(seed, kv, qo, P=4, Hq=4, Hk=2, d=8):
    return I.make_paged_batch(seed, kv, qo, page_size=P, num_qo_heads=Hq, num_kv_heads=Hk, head_dim=d,
                              dtype="f32", poison=False)


def test_window_predicate_by_hand():
    """Masks written out by hand from the meaning of the window: with 3 queries over 6 keys, query
    q's aligned position is q + 3 (bottom-right), and a window of w keys to the left shows keys
    q + 3 - w onwards; causal adds the upper bound q + 3."""
    # w = 1: query 0 (aligned to key 3) sees keys 2.., query 1 keys 3.., query 2 keys 4..
    w1 = [[0, 0, 1, 1, 1, 1],
          [0, 0, 0, 1, 1, 1],
          [0, 0, 0, 0, 1, 1]]
    assert A.window_allowed(3, 6, 1).astype(int).tolist() == w1
    # w = 0: from the aligned key on
    w0 = [[0, 0, 0, 1, 1, 1],
          [0, 0, 0, 0, 1, 1],
          [0, 0, 0, 0, 0, 1]]
    assert A.window_allowed(3, 6, 0).astype(int).tolist() == w0
    # w = 4: query 0 would start at key -1, i.e. sees every key; query 2 starts at key 1
    w4 = [[1, 1, 1, 1, 1, 1],
          [1, 1, 1, 1, 1, 1],
          [0, 1, 1, 1, 1, 1]]
    assert A.window_allowed(3, 6, 4).astype(int).tolist() == w4
    # more queries than keys (4 over 2): query q is aligned to key q - 2, so a window of w = 1
    # starts at key q - 3 <= 0 and shows both keys to every query; with causal and w = 0 each
    # query sees only its aligned key, which exists for queries 2 and 3 alone
    assert A.window_allowed(4, 2, 1).astype(int).tolist() == [[1, 1], [1, 1], [1, 1], [1, 1]]
    both = A.window_allowed(4, 2, 0) & A.causal_allowed(4, 2)
    assert both.astype(int).tolist() == [[0, 0], [0, 0], [1, 0], [0, 1]]
    # combined with causal through the attention itself: each row of 3 queries over 6 keys with
    # w = 1 sees exactly its aligned key and the one before it
    b = I.make_paged_batch(5, [6], [3], page_size=2, num_qo_heads=1, num_kv_heads=1, head_dim=4, dtype="f32",
                           poison=False)
    o, l = A.batch_attention(b.q_f32, b.k_f32, b.v_f32, b.kv_indptr, b.kv_indices, b.last_page_len, 2, 1, 1, 0.7,
                             qo_indptr=b.qo_indptr, causal=True, window_left=1)
    rows = A.physical_rows(b.kv_indptr, b.kv_indices, b.last_page_len, 2, 0)
    kf, vf = b.k_f32.reshape(-1, 1, 4)[rows, 0], b.v_f32.reshape(-1, 1, 4)[rows, 0]
    for r, keys in enumerate(([2, 3], [3, 4], [4, 5])):
        o_ref, l_ref = A.attention_one_head(b.q_f32[r:r + 1, 0], kf[keys], vf[keys], 0.7)
        assert np.allclose(o[r, 0], o_ref[0], atol=1e-14) and abs(l[r, 0] - l_ref[0]) < 1e-14


def test_window_wider_than_context_is_no_window():
    b = _batch(1, [9, 14, 3], [5, 14, 2])
    args = (b.q_f32, b.k_f32, b.v_f32, b.kv_indptr, b.kv_indices, b.last_page_len, 4, 4, 2, 0.5)
    o0, l0 = A.batch_attention(*args, qo_indptr=b.qo_indptr, causal=True)
    o1, l1 = A.batch_attention(*args, qo_indptr=b.qo_indptr, causal=True, window_left=100)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_window_zero_causal_sees_only_the_diagonal():
    b = _batch(2, [7, 4], [7, 4])
    o, l = A.batch_attention(b.q_f32, b.k_f32, b.v_f32, b.kv_indptr, b.kv_indices, b.last_page_len, 4,
                             4, 2, 0.5, qo_indptr=b.qo_indptr, causal=True, window_left=0)
    kf = b.k_f32.reshape(-1, 2, 8)
    vf = b.v_f32.reshape(-1, 2, 8)
    for i in range(2):
        rows = A.physical_rows(b.kv_indptr, b.kv_indices, b.last_page_len, 4, i)
        for pos in range(len(rows)):
            r = b.qo_indptr[i] + pos
            for h in range(4):
                kv = rows[pos]
                assert np.allclose(o[r, h], vf[kv, h // 2], atol=1e-15)
                s = 0.5 * float(b.q_f32[r, h].astype(np.float64) @ kf[kv, h // 2].astype(np.float64))
                assert abs(l[r, h] - s) < 1e-12


def test_window_decode_equals_attention_over_last_keys():
    # one query: window w keeps the last w + 1 keys, the same as a request whose page
    # list holds only those keys (paging is exact, so compare against a sliced view)
    b = _batch(3, [13, 22, 5], None)
    w = 6
    o, l = A.batch_attention(b.q_f32, b.k_f32, b.v_f32, b.kv_indptr, b.kv_indices, b.last_page_len, 4,
                             4, 2, 0.5, window_left=w)
    kf = b.k_f32.reshape(-1, 2, 8)
    vf = b.v_f32.reshape(-1, 2, 8)
    for i in range(3):
        rows = A.physical_rows(b.kv_indptr, b.kv_indices, b.last_page_len, 4, i)[-(w + 1):]
        for h in range(4):
            oo, ll = A.attention_one_head(b.q_f32[i:i + 1, h], kf[rows, h // 2], vf[rows, h // 2], 0.5)
            assert np.allclose(o[i, h], oo[0], atol=1e-14) and abs(l[i, h] - ll[0]) < 1e-14


def test_window_plan_covers_exactly_the_windowed_ranges():
    kv, qo = [300, 17, 64, 129, 0, 40], [300, 17, 64, 129, 3, 1]
    for w in (0, 5, 31, 64, 1000):
        for causal in (False, True):
            p = PL.make_plan(kv, qo, 8, 2, 5, causal=causal, window_left=w)
            g = 4
            for t in p.tiles:
                first = t.row_start // g
                lo = min(t.vis, max(0, kv[t.req] - qo[t.req] + first - w))
                assert t.lo == lo
                covered = []
                for m in t.items:
                    it = p.items[m]
                    assert it.kv_len <= p.chunk_limit
                    covered.extend(range(it.kv_start, it.kv_start + it.kv_len))
                assert covered == list(range(lo, t.vis))
                # every key some row of the tile may see lies in [lo, vis)
                last = (t.row_end - 1) // g
                for pos in (first, last):
                    row_lo = kv[t.req] - qo[t.req] + pos - w
                    assert row_lo >= lo or lo == 0
            assert p.total_work == sum(t.vis - t.lo for t in p.tiles)


def test_no_window_plan_unchanged():
    # window_left = -1 is the plain plan: the pinned worked example still holds
    p = PL.make_plan([1000, 100, 100, 50], None, 1, 1, 4, alpha=0, beta=1, window_left=-1)
    assert p.chunk_limit == 313


# ---------------------------------------------------------------------------
# Custom masks (LogitsMask with an arbitrary per-request boolean matrix)
# ---------------------------------------------------------------------------


def test_custom_mask_unpacking_worked_example():
    # two requests: 2 x 3 and 1 x 2; bits written out by hand, little-endian within a byte
    # request 0: rows [1 0 1], [0 1 1] -> bits 0..5 = 1,0,1,0,1,1; request 1: [1, 1] -> bits 6, 7
    bits = np.array([0b11110101], dtype=np.uint8)
    m = A.unpack_custom_mask(bits, [2, 1], [3, 2])
    assert m[0].tolist() == [[True, False, True], [False, True, True]]
    assert m[1].tolist() == [[True, True]]


def test_custom_mask_unpacking_matches_numpy_packbits():
    rng = np.random.default_rng(11)
    qo, kv = [3, 1, 5], [7, 12, 4]
    mats = [rng.random((a, b)) < 0.5 for a, b in zip(qo, kv)]
    bits = np.packbits(np.concatenate([m.reshape(-1) for m in mats]), bitorder="little")
    for a, b in zip(A.unpack_custom_mask(bits, qo, kv), mats):
        assert np.array_equal(a, b)


def test_all_true_custom_mask_is_no_mask_and_causal_mask_is_causal():
    b = I.make_paged_batch(21, [40, 9], [6, 9], page_size=4, num_qo_heads=4, num_kv_heads=2, head_dim=16,
                           dtype="f32", causal=True)
    args = (b.q_f32, b.k_f32, b.v_f32, b.kv_indptr, b.kv_indices, b.last_page_len, 4, 4, 2, 0.25)
    ones = [np.ones((q, k), dtype=bool) for q, k in zip([6, 9], [40, 9])]
    o1, l1 = A.batch_attention(*args, qo_indptr=b.qo_indptr, causal=True, custom_mask=ones)
    o2, l2 = A.batch_attention(*args, qo_indptr=b.qo_indptr, causal=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    cm = [A.causal_allowed(q, k) for q, k in zip([6, 9], [40, 9])]
    o3, l3 = A.batch_attention(*args, qo_indptr=b.qo_indptr, causal=False, custom_mask=cm)
    assert np.array_equal(o3, o2) and np.array_equal(l3, l2)


def test_custom_mask_row_with_no_key_is_empty_and_single_key_row_is_v():
    b = I.make_paged_batch(22, [10], [3], page_size=4, num_qo_heads=2, num_kv_heads=1, head_dim=8, dtype="f32")
    m = np.zeros((3, 10), dtype=bool)
    m[1, 4] = True
    m[2, [2, 7]] = True
    o, l = A.batch_attention(b.q_f32, b.k_f32, b.v_f32, b.kv_indptr, b.kv_indices, b.last_page_len, 4, 2, 1,
                             0.5, qo_indptr=b.qo_indptr, custom_mask=[m])
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
    rows = A.physical_rows(b.kv_indptr, b.kv_indices, b.last_page_len, 4, 0)
    vflat = b.v_f32.reshape(-1, 1, 8)
    kflat = b.k_f32.reshape(-1, 1, 8)
    for h in range(2):
        assert np.allclose(o[1, h], vflat[rows[4], 0])
        s = 0.5 * kflat[rows[[2, 7]], 0].astype(np.float64) @ b.q_f32[2, h].astype(np.float64)
        w = np.exp(s - s.max())
        assert np.allclose(o[2, h], (w / w.sum()) @ vflat[rows[[2, 7]], 0])
        assert math.isclose(l[2, h], s.max() + math.log(w.sum()), rel_tol=1e-12)
