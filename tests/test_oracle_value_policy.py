"""Pins of the oracle's A^2-weighted value policy (CPU only): the weights in
closed form and their bounds, the selection against brute force, the choice
of uniform widths for equal weights (convexity of the distortion in the bit
width), the expected surrogate by Monte Carlo over rotation seeds, the
log-sum-exp merge of two tiers against attention over their union, order
invariance, and the pages' claim that the policy beats uniform values at 2
bits when attention is concentrated ([P3] section 5)."""
import itertools
import math

import numpy as np

from oracle import attention as oat
from oracle import metrics as ome
from oracle import quantizer as oqz
from oracle import value_policy as vp


def test_weights_equal_keys_and_bounds():
    """Equal keys: every p_j = 1/T, so A_j = 1/T^2 exactly.  Any keys:
    sum_j A_j <= 1 (p^2 <= p) and >= 1/T (Cauchy-Schwarz: sum p^2 >= 1/T)."""
    rng = np.random.default_rng(0)
    T, d = 37, 16
    K = np.tile(rng.standard_normal(d), (T, 1))
    A = vp.a2_weights(rng.standard_normal((5, d)), K)
    assert np.allclose(A, 1.0 / T ** 2, rtol=1e-12, atol=0)
    K = rng.standard_normal((T, d)) * 3
    A = vp.a2_weights(rng.standard_normal((6, d)), K)
    assert 1.0 / T - 1e-15 <= A.sum() <= 1.0 + 1e-15


def test_weights_dominant_key():
    """One key aligned with every probe at a score margin of m over the rest
    gets p = 1 / (1 + (T-1) e^-m): A of it -> 1, the others -> 0."""
    T, d = 20, 8
    K = np.zeros((T, d))
    K[7, 0] = 40.0 * math.sqrt(d)           # score 40 q_0 for q_0 = 1
    Qp = np.zeros((3, d))
    Qp[:, 0] = 1.0
    A = vp.a2_weights(Qp, K)
    p7 = 1.0 / (1.0 + (T - 1) * math.exp(-40.0))
    assert abs(A[7] - p7 ** 2) < 1e-15
    assert np.all(A[np.arange(T) != 7] < 1e-30)


def test_selection_against_brute_force():
    """The R largest w with ties to the lower index: the chosen set has the
    largest sum of all R-subsets, and of those the lexicographically
    smallest index set."""
    rng = np.random.default_rng(1)
    for trial in range(30):
        T = 7
        w = rng.integers(0, 4, T).astype(float)      # many ties
        R = int(rng.integers(0, T + 1))
        m = vp.select(w, R)
        assert m.sum() == R
        best = max(sum(w[list(c)]) for c in itertools.combinations(range(T), R))
        winners = [c for c in itertools.combinations(range(T), R) if sum(w[list(c)]) == best]
        assert tuple(np.flatnonzero(m)) == min(winners)
        perm = vp.permutation(m)
        assert sorted(perm) == list(range(T))
        assert list(perm[:R]) == sorted(np.flatnonzero(m)) and list(perm[R:]) == sorted(np.flatnonzero(~m))


def test_distortion_convex_in_bits_so_equal_weights_stay_uniform():
    """D_b of the TQ-MSE quantiser is strictly convex in b (each extra bit
    saves less than the one before), so with equal weights every two-tier
    split at the same mean is worse than uniform and the policy keeps
    uniform widths."""
    d = 128
    D = [vp.value_distortion(d, b) for b in (1, 2, 3, 4)]
    assert all(D[i] > D[i + 1] for i in range(3))
    assert all(D[i - 1] + D[i + 1] > 2 * D[i] for i in (1, 2))
    # Known values: 1 bit is 1 - 2/pi in the large-d limit (0.3634); d=128 is close.
    assert abs(D[0] - (1 - 2 / math.pi)) < 0.003
    A = np.full((2, 300), 1.0 / 300 ** 2)
    res = vp.plan(A, np.ones((2, 300)), d, 2)
    assert (res["b_lo"], res["b_hi"]) == (2, 2) and res["R"] == 0
    assert np.array_equal(res["perm"], np.tile(np.arange(300), (2, 1)))


def test_concentrated_weights_take_the_skewed_tiers():
    """A handful of tokens holding the A^2 mass: the (1, 4) split with a
    third high wins, and the heavy tokens are in the high tier."""
    d, T = 64, 90
    A = np.full((1, T), 1e-8)
    heavy = [3, 40, 77]
    A[0, heavy] = 0.3
    res = vp.plan(A, np.ones((1, T)), d, 2)
    assert (res["b_lo"], res["b_hi"], res["R"]) == (1, 4, 30)
    assert set(heavy) <= set(res["perm"][0, :30])
    # The chosen candidate has the smallest surrogate, computed independently.
    for (b_lo, b_hi, num, den), s in zip(res["candidates"], res["surrogate"]):
        R = (T * num) // den
        heavy_first = sorted(range(T), key=lambda j: (-A[0, j], j))[:R]
        Dh, Dl = vp.value_distortion(d, b_hi), vp.value_distortion(d, b_lo)
        want = sum(A[0, j] * (Dh if j in heavy_first else Dl) for j in range(T))
        assert abs(s - want) <= 1e-12 * want
    assert res["surrogate"][2] < res["surrogate"][1] < res["surrogate"][0]


def test_expected_surrogate_by_monte_carlo():
    """Over random rotation seeds the measured sum_j A_j ||v_hat_j - v_j||^2
    averages to sum_j A_j ||v_j||^2 D_{b_j} (the seeded sign flip plus
    Hadamard spreads each direction close to uniformly)."""
    rng = np.random.default_rng(3)
    T, d = 40, 64
    V = rng.standard_normal((T, d))
    A = rng.random(T) ** 3
    high = vp.select(A, T // 3)
    vals = [vp.surrogate_of(A, V, vp.tiered_values(V, high, 1, 4, seed)) for seed in range(60)]
    want = vp.expected_surrogate(A, V, high, 1, 4)
    assert abs(np.mean(vals) - want) < 0.03 * want + 3 * np.std(vals) / math.sqrt(len(vals))


def test_merge_of_two_tiers_is_attention_over_the_union():
    rng = np.random.default_rng(4)
    T, d, R = 50, 32, 17
    K, V, Q = rng.standard_normal((T, d)) * 2, rng.standard_normal((T, d)), rng.standard_normal((3, d))
    o, _, _, lse = oat.attend(Q, K, V)
    oa, _, _, la = oat.attend(Q, K[:R], V[:R])
    ob, _, _, lb = oat.attend(Q, K[R:], V[R:])
    om, lm = vp.merge(oa, la, ob, lb)
    assert np.allclose(om, o, rtol=1e-12, atol=1e-13) and np.allclose(lm, lse, rtol=0, atol=1e-12)
    # Order of the (key, value) pairs does not matter.
    perm = rng.permutation(T)
    o2, _, _, l2 = oat.attend(Q, K[perm], V[perm])
    assert np.allclose(o2, o, atol=1e-13) and np.allclose(l2, lse, atol=1e-12)


def test_policy_beats_uniform_values_when_attention_is_concentrated():
    """[P3] section 5: the A^2-weighted value policy improves on uniform
    values at 2 bits.  Keys N(0, 1), queries N(0, 1.5^2 I), so the scores
    q.k/sqrt(d) have a spread of 1.5 (concentrated attention), probes = the queries of the
    step (a query-aware write); 2-bit budget.  Both the A^2 measure and the
    output error fall."""
    rng = np.random.default_rng(5)
    T, d, G = 600, 64, 8
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    Q = rng.standard_normal((G, d)) * 1.5
    A = vp.a2_weights(Q, K)
    res = vp.plan(A[None], np.sum(V * V, axis=1)[None], d, 2)
    assert res["b_lo"] < res["b_hi"]
    high = np.zeros(T, dtype=bool)
    high[res["perm"][0, :res["R"]]] = True
    Vp = vp.tiered_values(V, high, res["b_lo"], res["b_hi"], seed=9)
    st = oqz.QState(d, oqz.MSE, 2, 9)
    Vu = oqz.dequantize(oqz.quantize(V, st), st)
    o, p, _, _ = oat.attend(Q, K, V)
    op, _, _, _ = oat.attend(Q, K, Vp)
    ou, _, _, _ = oat.attend(Q, K, Vu)
    a2p = ome.a2_value_distortion(p, V, Vp).mean()
    a2u = ome.a2_value_distortion(p, V, Vu).mean()
    ep, eu = np.sum((op - o) ** 2), np.sum((ou - o) ** 2)
    print("A2 policy %.4g uniform %.4g; output err policy %.4g uniform %.4g" % (a2p, a2u, ep, eu))
    assert a2p < 0.8 * a2u
    assert ep < eu
