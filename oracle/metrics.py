"""Quality measures.   [oracle]

[P1] section "Métricas de Evaluación": KL divergence between the reference
and the quantised softmax distributions, and top-5 routing recall.
[P1] section "Significado y Afirmaciones" 1: mean KL is optimistic; the
worst case is reported too.  [P2] section "Configuração Experimental":
relMSE_K, relMSE_V and the direction error through cosine similarity.

Readings: KL(p_ref || p_quant) in nats; mean and max over all queries.
Top-5 ties go to the lower token index.  relMSE pooled over the tensor:
sum ||x - x_hat||^2 / sum ||x||^2.  Direction error: mean over vectors of
1 - cos(x, x_hat), vectors with a zero norm on either side left out.

Score-space and site measures:
[P3] section 2.1 (Eq. 6): KL between the reference and the perturbed
attention is locally a Fisher-weighted variance of the score errors.  Read
as the second-order term of KL(p || p_hat): 1/2 Var_{j~p}(ds_j), with
ds = s_hat - s in the natural units of s = q^T k / sqrt(d).
[P3] section 4 "Cadeia de Evidências": score-space error predicts KL better
than raw key MSE, by Spearman rank correlation.  Spearman = Pearson
correlation of the ranks, ties given their average rank.
[P1] section "Métricas de Evaluación": the 6D error framework splits the
error into scale (SNR) and direction (phi) at three sites (keys, values,
attention output).  The pages give no formulas; read as the pooled
SNR = 10 log10(sum ||x||^2 / sum ||x - x_hat||^2) in dB and phi = the mean
angle arccos(cos(x, x_hat)) in radians over vectors with non-zero norms.
[P3] section 2.2: value distortion weighted by A^2, sum_j p_j^2 ||dv_j||^2
per query.
"""
import numpy as np

from .attention import logsumexp


def kl_from_scores(s_ref, s_q):
    """KL(softmax(s_ref) || softmax(s_q)) per row, from logits."""
    s_ref = np.asarray(s_ref, dtype=np.float64)
    s_q = np.asarray(s_q, dtype=np.float64)
    lr = logsumexp(s_ref, axis=-1)
    lq = logsumexp(s_q, axis=-1)
    p = np.exp(s_ref - lr[..., None])
    return np.sum(p * (s_ref - s_q), axis=-1) - lr + lq


def topk_indices(s, k=5):
    """Indices of the k largest entries per row, ties to the lower index."""
    s = np.asarray(s, dtype=np.float64)
    order = np.lexsort((np.broadcast_to(np.arange(s.shape[-1]), s.shape), -s), axis=-1)
    return order[..., :k]


def topk_recall(s_ref, s_q, k=5):
    a = topk_indices(s_ref, k)
    b = topk_indices(s_q, k)
    hits = np.array([len(set(x) & set(y)) for x, y in zip(a.reshape(-1, k), b.reshape(-1, k))])
    return hits / k


def rel_mse(X, Xhat):
    X = np.asarray(X, dtype=np.float64)
    Xhat = np.asarray(Xhat, dtype=np.float64)
    return float(np.sum((X - Xhat) ** 2) / np.sum(X * X))


def direction_error(X, Xhat):
    X = np.asarray(X, dtype=np.float64).reshape(-1, X.shape[-1])
    Xhat = np.asarray(Xhat, dtype=np.float64).reshape(-1, X.shape[-1])
    nx = np.linalg.norm(X, axis=1)
    nh = np.linalg.norm(Xhat, axis=1)
    ok = (nx > 0) & (nh > 0)
    cos = np.sum(X[ok] * Xhat[ok], axis=1) / (nx[ok] * nh[ok])
    return float(np.mean(1.0 - cos))


def fisher_score_error(s_ref, s_q):
    """1/2 Var_{j~p}(s_q - s_ref) per row, p = softmax(s_ref) ([P3] Eq. 6)."""
    s_ref = np.asarray(s_ref, dtype=np.float64)
    ds = np.asarray(s_q, dtype=np.float64) - s_ref
    p = np.exp(s_ref - logsumexp(s_ref, axis=-1)[..., None])
    m = np.sum(p * ds, axis=-1)
    return 0.5 * np.sum(p * (ds - m[..., None]) ** 2, axis=-1)


def average_ranks(a):
    """Ranks 1..n of a (1-D), tied values sharing the mean of their ranks."""
    a = np.asarray(a, dtype=np.float64)
    order = np.argsort(a, kind="stable")
    r = np.empty(len(a))
    i = 0
    while i < len(a):
        j = i
        while j + 1 < len(a) and a[order[j + 1]] == a[order[i]]:
            j += 1
        r[order[i:j + 1]] = 0.5 * (i + j) + 1.0
        i = j + 1
    return r


def spearman(a, b):
    """Spearman rank correlation of two equal-length 1-D samples (NaN when a
    sample is constant)."""
    ra = average_ranks(a)
    rb = average_ranks(b)
    ra -= ra.mean()
    rb -= rb.mean()
    den = np.sqrt(np.sum(ra * ra) * np.sum(rb * rb))
    return float(np.sum(ra * rb) / den) if den > 0 else float("nan")


def snr_db(X, Xhat):
    """Pooled signal-to-noise ratio of x_hat as an estimate of x, in dB."""
    X = np.asarray(X, dtype=np.float64)
    Xhat = np.asarray(Xhat, dtype=np.float64)
    return float(10.0 * np.log10(np.sum(X * X) / np.sum((X - Xhat) ** 2)))


def direction_angle(X, Xhat):
    """Mean angle (radians) between x and x_hat over vectors with non-zero
    norms on both sides."""
    X = np.asarray(X, dtype=np.float64).reshape(-1, X.shape[-1])
    Xhat = np.asarray(Xhat, dtype=np.float64).reshape(-1, X.shape[-1])
    nx = np.linalg.norm(X, axis=1)
    nh = np.linalg.norm(Xhat, axis=1)
    ok = (nx > 0) & (nh > 0)
    cos = np.clip(np.sum(X[ok] * Xhat[ok], axis=1) / (nx[ok] * nh[ok]), -1.0, 1.0)
    return float(np.mean(np.arccos(cos)))


def a2_value_distortion(P, V, Vhat):
    """sum_j p_j^2 ||v_hat_j - v_j||^2 per query: P [G, T] attention
    probabilities, V, Vhat [T, d]."""
    dv2 = np.sum((np.asarray(Vhat, dtype=np.float64) - np.asarray(V, dtype=np.float64)) ** 2, axis=1)
    return np.asarray(P, dtype=np.float64) ** 2 @ dv2
