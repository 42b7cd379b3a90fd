"""Read side by its plain definition: dense dequantised keys and values,
then textbook softmax attention in float64.   [oracle]

[P3] section 2.1: a query q scores key j as s_j = q^T k_j / sqrt(d), and
softmax is invariant to adding one constant to all scores.  [P3] section
2.2: values are read by the attention-weighted sum o = sum_j p_j v_j.
[P3] section 3: the HeadQ score adds q^T U_h z_hat / sqrt(d) (folded into the
dense effective key by headq.quantize).

Grouped queries: query head g reads KV head floor(g / (Hq / Hkv)).
"""
import numpy as np


def logsumexp(s, axis=-1):
    m = np.max(s, axis=axis, keepdims=True)
    return (m + np.log(np.sum(np.exp(s - m), axis=axis, keepdims=True))).squeeze(axis)


def attend(Q, K, V):
    """Q [G, d], K [T, d], V [T, d] -> out [G, d], probabilities [G, T],
    scores [G, T], lse [G]."""
    Q = np.asarray(Q, dtype=np.float64)
    d = Q.shape[1]
    s = Q @ np.asarray(K, dtype=np.float64).T / np.sqrt(d)
    lse = logsumexp(s, axis=1)
    p = np.exp(s - lse[:, None])
    o = p @ np.asarray(V, dtype=np.float64)
    return o, p, s, lse


def attend_batched(Q, K, V):
    """Q [B, Hq, d], K/V [B, Hkv, T, d] -> out [B, Hq, d], lse [B, Hq]."""
    B, Hq, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    for b in range(B):
        for h in range(Hkv):
            o, _, _, l = attend(Q[b, h * G:(h + 1) * G], K[b, h], V[b, h])
            out[b, h * G:(h + 1) * G] = o
            lse[b, h * G:(h + 1) * G] = l
    return out, lse
