"""Pins of the oracle's attention state and merge against the pages and algebra."""
import math

import numpy as np
import pytest

from oracle import attention as A
from tests.conftest import load_golden


def _close(x, pair):
    value, tol = pair
    assert abs(x - value) <= tol, (x, value, tol)


def test_worked_example_states_and_merge():
    g = load_golden("merge_worked_example.json")
    q = np.array([g["q"]])
    K = np.array(g["keys"])
    V = np.array(g["values"])[:, None]
    a0, a1 = g["chunk_a"]
    b0, b1 = g["chunk_b"]
    oa, la = A.attention_one_head(q, K[a0:a1], V[a0:a1], g["sm_scale"])
    ob, lb = A.attention_one_head(q, K[b0:b1], V[b0:b1], g["sm_scale"])
    e = g["expected"]
    _close(oa[0, 0], e["O_A"])
    _close(la[0], e["LSE_A"])
    _close(ob[0, 0], e["O_B"])
    _close(lb[0], e["LSE_B"])
    _close(math.exp(la[0]), e["exp_LSE_A"])
    _close(math.exp(lb[0]), e["exp_LSE_B"])
    om, lm = A.merge_state(oa, la, ob, lb)
    _close(om[0, 0], e["O_merged"])
    # the naive average of the two partial outputs is the wrong answer
    _close((oa[0, 0] + ob[0, 0]) / 2, e["naive_average_is_wrong"])
    assert abs(om[0, 0] - (oa[0, 0] + ob[0, 0]) / 2) > 7.0
    # and the merge equals single-shot attention over all four keys
    of, lf = A.attention_one_head(q, K, V, g["sm_scale"])
    assert abs(of[0, 0] - om[0, 0]) < 1e-12 and abs(lf[0] - lm[0]) < 1e-12


def test_scalar_example():
    g = load_golden("merge_scalar_example.json")
    o, l = A.merge_state(
        np.array([[g["O_A"]]]), np.array([math.log(g["Z_A"])]),
        np.array([[g["O_B"]]]), np.array([math.log(g["Z_B"])]),
    )
    assert abs(o[0, 0] - g["expected_merged_O"]) < 1e-14
    assert abs(l[0] - math.log(g["Z_A"] + g["Z_B"])) < 1e-14
    assert abs(o[0, 0] - g["wrong_average"]) > 0.5


def _rand_state(rng, n, d, empty_frac=0.0):
    o = rng.standard_normal((n, d))
    l = rng.standard_normal(n) * 3
    if empty_frac:
        mask = rng.random(n) < empty_frac
        o[mask] = 0.0
        l[mask] = -np.inf
    return o, l


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_commutative_associative_identity(seed):
    rng = np.random.default_rng(seed)
    a, b, c = (_rand_state(rng, 40, 7, 0.2) for _ in range(3))
    ab = A.merge_state(*a, *b)
    ba = A.merge_state(*b, *a)
    assert np.allclose(ab[0], ba[0], atol=1e-14, rtol=0) and np.allclose(ab[1], ba[1], atol=1e-14, rtol=0, equal_nan=False)
    left = A.merge_state(*A.merge_state(*a, *b), *c)
    right = A.merge_state(*a, *A.merge_state(*b, *c))
    assert np.allclose(left[0], right[0], atol=1e-13, rtol=0)
    assert np.array_equal(np.isinf(left[1]), np.isinf(right[1]))
    fin = np.isfinite(left[1])
    assert np.allclose(left[1][fin], right[1][fin], atol=1e-13, rtol=0)
    e = A.empty_state((40, 7))
    ae = A.merge_state(*a, *e)
    assert np.array_equal(ae[0], a[0]) and np.array_equal(ae[1], a[1])
    ee = A.merge_state(*e, *e)
    assert np.all(ee[0] == 0) and np.all(np.isneginf(ee[1]))


def test_merge_is_not_sensitive_to_large_lse():
    # eq. 6 subtracts the shared maximum; exp(800) would overflow without it
    o, l = A.merge_state(np.array([[1.0]]), np.array([800.0]), np.array([[3.0]]), np.array([800.0]))
    assert o[0, 0] == 2.0 and abs(l[0] - (800.0 + math.log(2.0))) < 1e-12


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_split_equals_union(seed):
    """Folding the states of any disjoint partition of the keys gives attention over the union."""
    rng = np.random.default_rng(seed)
    Lq, Lk, d = 5, 37, 8
    q = rng.standard_normal((Lq, d))
    k = rng.standard_normal((Lk, d))
    v = rng.standard_normal((Lk, d))
    scale = 1 / math.sqrt(d)
    perm = rng.permutation(Lk)
    cuts = np.sort(rng.choice(np.arange(1, Lk), size=4, replace=False))
    parts = np.split(perm, cuts)
    states = [A.attention_one_head(q, k[p], v[p], scale) for p in parts]
    o, l = A.fold_states(states)
    of, lf = A.attention_one_head(q, k, v, scale)
    assert np.allclose(o, of, atol=1e-13, rtol=0) and np.allclose(l, lf, atol=1e-13, rtol=0)


def test_overlap_double_counts():
    """Keys must not overlap: merging a chunk with itself does not reproduce it (review §3.3)."""
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal((1, 4)), rng.standard_normal((6, 4)), rng.standard_normal((6, 4))
    s = A.attention_one_head(q, k, v, 0.5)
    o, l = A.merge_state(*s, *s)
    assert np.allclose(o, s[0]) and abs(l[0] - (s[1][0] + math.log(2))) < 1e-12
