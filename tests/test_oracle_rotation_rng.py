"""Pins of the oracle's rotation and random state (CPU only)."""
import os

import numpy as np
import pytest
from scipy import stats

from oracle import rng, rotation

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("d", [16, 32, 128, 1024])
def test_hadamard_is_hadamard(d):
    H = rotation.hadamard(d)
    assert np.array_equal(H @ H.T, d * np.eye(d, dtype=np.int64))


@pytest.mark.parametrize("d", [2, 4, 8, 64])
def test_hadamard_matches_sylvester_recursion(d):
    # Independent construction: H_2n = [[H, H], [H, -H]].
    H = np.array([[1]])
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    assert np.array_equal(rotation.hadamard(d), H)


@pytest.mark.parametrize("d", [128, 1024])
def test_rotation_orthogonal_and_norm_preserving(d):
    P = rotation.rotation_matrix(7, d)
    assert np.max(np.abs(P.T @ P - np.eye(d))) < 1e-12
    x = np.random.default_rng(0).standard_normal((5, d))
    assert np.allclose(np.linalg.norm(x @ P.T, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_splitmix64_reference_outputs():
    vals = [int(l.strip(), 16) for l in open(os.path.join(GOLDEN, "splitmix64.txt"))
            if l.strip() and not l.startswith("#")]
    assert [int(v) for v in rng.splitmix64_stream(0, 3)] == vals
    assert [rng.mix64((i + 1) * rng.GOLDEN_GAMMA) for i in range(3)] == vals


def test_sign_vector_balanced_and_seeded():
    D = rng.sign_vector(0, 4096)
    assert set(np.unique(D)) == {-1.0, 1.0}
    # Binomial(4096, 1/2): 5 sigma = 160.
    assert abs(np.sum(D)) < 160
    assert np.array_equal(D, rng.sign_vector(0, 4096))
    assert not np.array_equal(D, rng.sign_vector(1, 4096))
    # A prefix property: the vector for d is the first d entries of the stream.
    assert np.array_equal(rng.sign_vector(0, 128), D[:128])


def test_gaussian_sketch_is_standard_normal():
    S = rng.gaussian_sketch(3, 128)
    assert S.shape == (128, 128)
    assert np.all(S == S.astype(np.float16))
    z = S.ravel()
    assert stats.kstest(z, "norm").pvalue > 1e-3
    assert abs(z.mean()) < 5 / 128 and abs(z.var() - 1) < 5 * np.sqrt(2 / z.size)
    # Rows are uncorrelated: S S^T / d ~ I.
    G = S @ S.T / 128
    assert np.max(np.abs(np.diag(G) - 1)) < 0.6
    assert np.max(np.abs(G - np.diag(np.diag(G)))) < 0.5
