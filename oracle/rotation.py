"""Randomised normalised Walsh-Hadamard rotation, as a dense matrix.   [oracle]

[P1] section "Esquemas de Cuantización" (KQV, QKQV) and [P2] section
"Configuração Experimental": a Walsh-Hadamard transform with random signs is
applied to K and V before scalar quantisation, spreading energy and outliers.

Reading: Pi = H D / sqrt(d), H the Sylvester Hadamard matrix in natural order,
H_ij = (-1)^popcount(i & j), D = diag(sign vector), D applied first.
Pi is orthogonal, so Pi^T undoes it.
"""
import numpy as np

from .rng import sign_vector


def hadamard(d):
    """Sylvester Hadamard matrix from the popcount formula (integers)."""
    i = np.arange(d)
    bits = np.bitwise_and(i[:, None], i[None, :])
    pc = np.zeros_like(bits)
    while np.any(bits):
        pc += bits & 1
        bits >>= 1
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def rotation_matrix(seed, d):
    """Pi = H diag(D) / sqrt(d), float64 d x d."""
    H = hadamard(d).astype(np.float64)
    D = sign_vector(seed, d)
    return H * D[None, :] / np.sqrt(d)
