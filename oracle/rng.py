"""Seeded random state of the quantiser: sign vector D and Gaussian sketch S.   [oracle]

[P2] section "Configuração Experimental": the rotation is a random
Walsh-Hadamard transform and the optional residual stage is a 1-bit
Johnson-Lindenstrauss (QJL) sketch.  [P1] section "Contribuciones Clave" 1:
the QJL estimator is unbiased with variance (pi/2)||r||^2/d, which fixes S
as a dense standard-Gaussian matrix with m = d rows.

The pages fix only the distributions.  Both sides of the parity check draw
them from one counter-based generator, SplitMix64 (Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014), written here
from its published definition in Python integers:

  out(i) = mix64(base + (i+1) * 0x9E3779B97F4A7C15  mod 2^64),
  mix64(z): z ^= z>>30; z *= 0xBF58476D1CE4E5B9; z ^= z>>27;
            z *= 0x94D049BB133111EB; z ^= z>>31   (all mod 2^64)

with base = seed XOR tag.  Tags (hex digits of pi after the point):
  sign stream  0x243F6A8885A308D3,   Gaussian stream  0x13198A2E03707344.

Sign vector: D_i = +1 if bit 63 of out_sign(i) is 0, else -1, i < d.
Gaussian sketch: S (m x d, m = d, row-major) from Box-Muller pairs in
double: pair p uses o1 = out_gauss(2p), o2 = out_gauss(2p+1),
u1 = ((o1>>11)+1) 2^-53 in (0,1], u2 = (o2>>11) 2^-53 in [0,1),
R = sqrt(-2 ln u1), S_flat[2p] = R cos(2 pi u2), S_flat[2p+1] = R sin(2 pi u2);
S is defined as the float16 rounding (round to nearest even, straight from
the double) of these values: an N(0,1) draw perturbed by at most 2^-11
relative, exactly representable in fp16 and fp32 alike.
"""
import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15
TAG_SIGN = 0x243F6A8885A308D3
TAG_GAUSS = 0x13198A2E03707344
TWO_PI = 6.283185307179586


def mix64(z):
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def splitmix64_stream(base, count):
    """First `count` outputs of the SplitMix64 stream started at `base`
    (numpy uint64 arithmetic wraps modulo 2^64, as the definition needs)."""
    i = np.arange(1, count + 1, dtype=np.uint64)
    z = np.uint64(base & MASK64) + i * np.uint64(GOLDEN_GAMMA)
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def sign_vector(seed, d):
    """D in {+1,-1}^d as float64."""
    o = splitmix64_stream((seed ^ TAG_SIGN) & MASK64, d)
    top = (o >> np.uint64(63)).astype(np.int64)
    return np.where(top == 0, 1.0, -1.0)


def gaussian_draws(seed, d, m=None):
    """The Box-Muller doubles behind S, before the float16 rounding, [m, d]."""
    m = d if m is None else m
    n = m * d
    npairs = (n + 1) // 2
    o = splitmix64_stream((seed ^ TAG_GAUSS) & MASK64, 2 * npairs)
    o1 = o[0::2] >> np.uint64(11)
    o2 = o[1::2] >> np.uint64(11)
    u1 = (o1.astype(np.float64) + 1.0) * 2.0 ** -53
    u2 = o2.astype(np.float64) * 2.0 ** -53
    r = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(2 * npairs)
    z[0::2] = r * np.cos(TWO_PI * u2)
    z[1::2] = r * np.sin(TWO_PI * u2)
    return z[:n].reshape(m, d)


def gaussian_sketch(seed, d, m=None):
    """S in R^{m x d}: the float16 values, returned as float64."""
    return gaussian_draws(seed, d, m).astype(np.float16).astype(np.float64)
