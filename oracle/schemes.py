"""Scheme presets: per-tensor (mode, bits) at a budget of n bits per coordinate.   [oracle]

  KV (Plain-KV) : K PLAIN(n),  V PLAIN(n)   [P1] "Esquemas" 1; [P2] "Contribuições" 1
  TQ-KV         : K MSE(n),    V MSE(n)     [P2] "Contribuições" 1
  KQV           : K MSE(n),    V PROD(n)    [P1] "Esquemas" 2
  QKQV          : K PROD(n),   V PROD(n)    [P1] "Esquemas" 3
  TQ-QKV        : K PROD(n),   V MSE(n)     [P2] "Contribuições" 1 (QJL on the key path)
  HEADQ         : K HEADQ(base MSE 2 + side code), V MSE(n)   [P3] section 3
  SQU-KV        : K SPECTRAL(n), V SPECTRAL(n)   [P2] "Recomendações Práticas" 2 (see spectral.py)
PROD(n) spends n-1 bits on the Lloyd-Max index and 1 bit per coordinate on
the QJL sketch (m = d), so every preset keeps n bits per coordinate
(HEADQ aside, whose key budget is 2 bits plus the side code).
"""
from .quantizer import PLAIN, MSE, PROD, HEADQ

SPECTRAL = "spectral"

TABLE = {
    "kv": (PLAIN, PLAIN),
    "tq-kv": (MSE, MSE),
    "kqv": (MSE, PROD),
    "qkqv": (PROD, PROD),
    "tq-qkv": (PROD, MSE),
    "headq": (HEADQ, MSE),
    "squ-kv": (SPECTRAL, SPECTRAL),
}


def modes(scheme, n):
    """((k_mode, k_bits), (v_mode, v_bits)); bits = the tensor's total budget."""
    km, vm = TABLE[scheme]
    kb = 2 if km == HEADQ else n
    return (km, kb), (vm, n)
