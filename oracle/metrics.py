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
