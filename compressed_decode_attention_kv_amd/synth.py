"""Seeded synthetic inputs shaped like the pages' regimes.

This module only draws inputs.  It holds none of the quantiser's or the
attention's arithmetic, so both the library tests and the oracle tests can
feed it to either side.

Regimes (the pages name them; the exact laws below are readings):
  isotropic     -- i.i.d. Gaussian keys and values.
  heavy_tailed  -- i.i.d. Student-t (nu = 3) scaled to unit variance, plus a
                   1 % fraction of token vectors carrying one +-20 outlier
                   coordinate.
  low_rank      -- K = Z diag(sqrt(lambda)) W^T + 0.01 E, lambda_i = 0.7^i,
                   W an orthonormal d x 16 basis; queries half inside span(W)
                   (norm matched), half isotropic.
  structured    -- K and V each a per-head mean plus a rank-16 part with
                   lambda_i = 0.7^i on an orthonormal basis of its own, plus
                   0.01 E; mean entries N(0, 1/d); queries half inside the key
                   span (norm matched), half isotropic; separate calibration
                   draws of K and V from the same law.
  rope          -- post-RoPE-like keys: N(0,1) pairs rotated by position *
                   theta_i, theta_i = 10000^(-2i/d); queries whose pair i has
                   variance proportional to 0.7^i (E||q||^2 = d), rotated by
                   their position; calibration queries at uniform positions.

Small inputs are drawn on the host with numpy (PCG64); full-size inputs are
drawn on the device with torch's seeded generator.  Either way every tensor
is a deterministic function of its seed.
"""
import math

import numpy as np

# Workload definitions: name -> sizes.  "G" = query heads per KV head.
WORKLOADS = {
    "isotropic_small": dict(B=1, H=1, G=16, T=4096, d=128, dtype="f32"),
    "isotropic_decode": dict(B=16, H=32, G=1, T=32768, d=128, dtype="f16"),
    "heavy_tailed": dict(B=4, H=8, G=0, T=131072, d=128, dtype="f32"),
    "low_rank": dict(B=1, H=4, G=64, T=65536, d=1024, dtype="f32"),
    "rope_gqa": dict(B=8, H=8, G=4, T=131072, d=128, dtype="f16"),
    "structured_decode": dict(B=16, H=32, G=1, T=32768, d=128, dtype="f16"),
}


def isotropic_small(seed=0, T=4096, d=128, nq=16):
    """K, V [1,1,T,d] and Q [1,nq,d], all N(0,1) float32; one default_rng(seed)
    drawn in the order K, V, Q."""
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((T, d)).astype(np.float32)
    V = rng.standard_normal((T, d)).astype(np.float32)
    Q = rng.standard_normal((nq, d)).astype(np.float32)
    return K[None, None], V[None, None], Q[None]


def _np_rng(seed, *key):
    return np.random.default_rng(np.random.SeedSequence([seed, *key]))


def isotropic(B, H, G, T, d, seed=1, kv_std=None, dtype=np.float16):
    """K, V [B,H,T,d] ~ N(0, kv_std^2) (default 1/sqrt(d)); Q [B,H*G,d] ~ N(0,1)."""
    s = 1.0 / math.sqrt(d) if kv_std is None else kv_std
    K = (_np_rng(seed, 0).standard_normal((B, H, T, d)) * s).astype(dtype)
    V = (_np_rng(seed, 1).standard_normal((B, H, T, d)) * s).astype(dtype)
    Q = _np_rng(seed, 2).standard_normal((B, H * G, d)).astype(dtype)
    return K, V, Q


def _student_t3(rng, shape):
    z = rng.standard_normal(shape)
    chi2 = np.sum(rng.standard_normal((3,) + tuple(shape)) ** 2, axis=0)
    return z / np.sqrt(chi2 / 3.0) / math.sqrt(3.0)


def _outliers(rng, X, frac=0.01, mag=20.0):
    B, H, T, d = X.shape
    hit = rng.random((B, H, T)) < frac
    coord = rng.integers(0, d, size=(B, H, T))
    sign = np.where(rng.random((B, H, T)) < 0.5, -1.0, 1.0)
    b, h, t = np.nonzero(hit)
    X[b, h, t, coord[b, h, t]] = sign[b, h, t] * mag
    return X


def heavy_tailed(B, H, T, d, seed=3, dtype=np.float32):
    """K, V [B,H,T,d]: Student-t(3)/sqrt(3) with 1 % outlier tokens (one
    coordinate set to +-20); K and V drawn independently."""
    out = []
    for tid in range(2):
        rng = _np_rng(seed, tid)
        X = _student_t3(rng, (B, H, T, d))
        out.append(_outliers(rng, X).astype(dtype))
    return out[0], out[1]


def low_rank(H, T, d, nq, seed=4, rank=16, decay=0.7, noise=0.01, dtype=np.float32):
    """K [1,H,T,d] low-rank + noise, V [1,H,T,d] N(0,1), Q [1,H*nq,d] with the
    first half of each head's queries inside span(W) and the rest isotropic."""
    rng = _np_rng(seed, 0)
    lam = decay ** np.arange(rank)
    K = np.empty((1, H, T, d))
    Q = np.empty((1, H * nq, d))
    for h in range(H):
        W, _ = np.linalg.qr(rng.standard_normal((d, rank)))
        Z = rng.standard_normal((T, rank))
        K[0, h] = (Z * np.sqrt(lam)) @ W.T + noise * rng.standard_normal((T, d))
        ni = nq // 2
        g = rng.standard_normal((ni, rank)) * math.sqrt(d / rank)
        Q[0, h * nq:h * nq + ni] = g @ W.T
        Q[0, h * nq + ni:(h + 1) * nq] = rng.standard_normal((nq - ni, d))
    V = _np_rng(seed, 1).standard_normal((1, H, T, d))
    return K.astype(dtype), V.astype(dtype), Q.astype(dtype)


def _structured_law(rng, H, d, rank, decay):
    lam = decay ** np.arange(rank)
    laws = []
    for _ in range(H):
        W, _ = np.linalg.qr(rng.standard_normal((d, rank)))
        laws.append((rng.standard_normal(d) / math.sqrt(d), W))
    return lam, laws


def _structured_draw(rng, lam, law, n, noise):
    mu, W = law
    d, rank = W.shape
    return mu + (rng.standard_normal((n, rank)) * np.sqrt(lam)) @ W.T + noise * rng.standard_normal((n, d))


def structured(B, H, G, T, d, seed=6, rank=16, decay=0.7, noise=0.01, n_calib=4096, dtype=np.float32):
    """K, V [B,H,T,d] (structured regime), Q [B,H*G,d], and the calibration
    draws CK, CV [H, n_calib, d] (float32)."""
    rng = _np_rng(seed, 0)
    lam, klaws = _structured_law(rng, H, d, rank, decay)
    _, vlaws = _structured_law(rng, H, d, rank, decay)
    K = np.empty((B, H, T, d))
    V = np.empty((B, H, T, d))
    Q = np.empty((B, H * G, d))
    drng = _np_rng(seed, 1)
    for b in range(B):
        for h in range(H):
            K[b, h] = _structured_draw(drng, lam, klaws[h], T, noise)
            V[b, h] = _structured_draw(drng, lam, vlaws[h], T, noise)
            ni = G // 2
            g = drng.standard_normal((ni, rank)) * math.sqrt(d / rank)
            Q[b, h * G:h * G + ni] = g @ klaws[h][1].T
            Q[b, h * G + ni:(h + 1) * G] = drng.standard_normal((G - ni, d))
    crng = _np_rng(seed, 2)
    CK = np.stack([_structured_draw(crng, lam, klaws[h], n_calib, noise) for h in range(H)])
    CV = np.stack([_structured_draw(crng, lam, vlaws[h], n_calib, noise) for h in range(H)])
    return K.astype(dtype), V.astype(dtype), Q.astype(dtype), CK.astype(np.float32), CV.astype(np.float32)


def _rope(X, pos, d):
    """Rotate pairs (2i, 2i+1) of X [..., d] by pos * 10000^(-2i/d)."""
    i = np.arange(d // 2)
    theta = 10000.0 ** (-2.0 * i / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = X[..., 0::2], X[..., 1::2]
    out = np.empty_like(X)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def rope_gqa(B, Hkv, G, T, d, seed=5, n_calib=4096, decay=0.7, dtype=np.float16):
    """Keys [B,Hkv,T,d] = RoPE(N(0,1), position t); values N(0,1);
    queries [B,Hkv*G,d] with pair variance ~ decay^i (E||q||^2 = d), rotated
    to position T; calibration queries [Hkv, n_calib, d] from the same law at
    uniform positions in [0, T)."""
    rng = _np_rng(seed, 0)
    lam = decay ** np.arange(d // 2)
    lam = lam * (d / (2.0 * lam.sum()))          # sum over pairs of 2 lam_i = d
    pair_std = np.repeat(np.sqrt(lam), 2)
    K = _rope(rng.standard_normal((B, Hkv, T, d)), np.arange(T)[None, None, :], d)
    V = _np_rng(seed, 1).standard_normal((B, Hkv, T, d))
    Q = _rope(_np_rng(seed, 2).standard_normal((B, Hkv * G, d)) * pair_std, T, d)
    crng = _np_rng(seed, 3)
    pos = crng.integers(0, T, size=(Hkv, n_calib))
    C = _rope(crng.standard_normal((Hkv, n_calib, d)) * pair_std, pos, d)
    return K.astype(dtype), V.astype(dtype), Q.astype(dtype), C.astype(np.float32)


def device_isotropic(B, H, G, T, d, seed=1, device="cuda"):
    """Full-size isotropic decode workload drawn on the device:
    K, V [B,H,T,d] ~ N(0, 1/d) float16, Q [B,H*G,d] ~ N(0,1) float16."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    s = 1.0 / math.sqrt(d)
    K = (torch.randn((B, H, T, d), generator=g, device=device, dtype=torch.float32) * s).half()
    V = (torch.randn((B, H, T, d), generator=g, device=device, dtype=torch.float32) * s).half()
    Q = torch.randn((B, H * G, d), generator=g, device=device, dtype=torch.float32).half()
    return K, V, Q


def device_heavy_tailed(B, H, T, d, seed=3, frac=0.01, mag=20.0, device="cuda"):
    """Full-size heavy-tailed regime drawn on the device: K, V [B,H,T,d]
    float32, Student-t(3)/sqrt(3) per coordinate (normal over the root of a
    chi-square with 3 degrees of freedom / 3), with a `frac` fraction of token
    vectors carrying one +-`mag` outlier coordinate; K and V independent."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for _ in range(2):
        X = torch.empty((B, H, T, d), device=device, dtype=torch.float32)
        for b in range(B):  # one batch row at a time bounds the temporaries
            z = torch.randn((H, T, d), generator=g, device=device)
            chi2 = torch.zeros_like(z)
            for _ in range(3):
                e = torch.randn((H, T, d), generator=g, device=device)
                chi2.addcmul_(e, e)
            X[b] = z / torch.sqrt(chi2 / 3.0) / math.sqrt(3.0)
        hit = torch.rand((B, H, T), generator=g, device=device) < frac
        coord = torch.randint(0, d, (B, H, T), generator=g, device=device)
        sign = torch.where(torch.rand((B, H, T), generator=g, device=device) < 0.5, -1.0, 1.0)
        rows = torch.nonzero(hit.reshape(-1)).squeeze(1)
        flat = X.view(-1, d)
        flat[rows, coord.reshape(-1)[rows]] = sign.reshape(-1)[rows] * mag
        out.append(X)
    return out[0], out[1]


def device_rope_gqa(B, Hkv, G, T, d, seed=5, n_calib=4096, decay=0.7, device="cuda"):
    """Full-size post-RoPE GQA regime, the law of rope_gqa drawn on the device:
    keys [B,Hkv,T,d] float16 = RoPE(N(0,1), position t), values N(0,1)
    float16, queries [B,Hkv*G,d] float16 with pair variance ~ decay^i rotated
    to position T; calibration queries [Hkv, n_calib, d] float32 drawn on the
    host (numpy) from the same law at uniform positions in [0, T)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    i = torch.arange(d // 2, device=device, dtype=torch.float64)
    theta = 10000.0 ** (-2.0 * i / d)
    lam_np = decay ** np.arange(d // 2)
    lam_np = lam_np * (d / (2.0 * lam_np.sum()))
    pair_std = torch.from_numpy(np.repeat(np.sqrt(lam_np), 2)).float().to(device)

    def rope(X, pos):
        ang = pos.to(torch.float64)[..., None] * theta
        c, s = torch.cos(ang).float(), torch.sin(ang).float()
        x0, x1 = X[..., 0::2], X[..., 1::2]
        r = torch.empty_like(X)
        r[..., 0::2] = x0 * c - x1 * s
        r[..., 1::2] = x0 * s + x1 * c
        return r

    pos = torch.arange(T, device=device)
    K = torch.empty((B, Hkv, T, d), dtype=torch.float16, device=device)
    for b in range(B):
        K[b] = rope(torch.randn((Hkv, T, d), generator=g, device=device), pos).half()
    V = torch.empty((B, Hkv, T, d), dtype=torch.float16, device=device)
    for b in range(B):
        V[b] = torch.randn((Hkv, T, d), generator=g, device=device).half()
    Qr = torch.randn((B, Hkv * G, d), generator=g, device=device) * pair_std
    Q = rope(Qr, torch.full((B, Hkv * G), T, device=device)).half()
    crng = _np_rng(seed, 3)
    cpos = crng.integers(0, T, size=(Hkv, n_calib))
    C = _rope(crng.standard_normal((Hkv, n_calib, d)) * np.repeat(np.sqrt(lam_np), 2), cpos, d)
    return K, V, Q, C.astype(np.float32)


def device_structured(B, H, G, T, d, seed=6, rank=16, decay=0.7, noise=0.01, n_calib=4096, device="cuda"):
    """Full-size structured regime drawn on the device: K, V [B,H,T,d]
    float16, Q [B,H*G,d] float16, and the calibration draws CK, CV
    [H, n_calib, d] (host float32); the law of `structured`."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    f32 = torch.float32
    sl = torch.sqrt(torch.tensor([decay ** i for i in range(rank)], dtype=f32, device=device))

    def law():
        W = torch.linalg.qr(torch.randn((H, d, rank), generator=g, device=device, dtype=f32))[0]
        mu = torch.randn((H, 1, d), generator=g, device=device, dtype=f32) / math.sqrt(d)
        return mu, W.transpose(1, 2).contiguous()          # [H, rank, d]

    def draw(mu, Wt, n):
        Z = torch.randn((H, n, rank), generator=g, device=device, dtype=f32) * sl
        return mu + torch.matmul(Z, Wt) + noise * torch.randn((H, n, d), generator=g, device=device, dtype=f32)

    (mk, Wk), (mv, Wv) = law(), law()
    K = torch.empty((B, H, T, d), dtype=torch.float16, device=device)
    V = torch.empty((B, H, T, d), dtype=torch.float16, device=device)
    for b in range(B):
        K[b] = draw(mk, Wk, T).half()
        V[b] = draw(mv, Wv, T).half()
    # Half the queries in the key span (norm matched): the first G/2 of each
    # head, or with one query per head those of the even heads.
    Q = torch.randn((B, H, G, d), generator=g, device=device, dtype=f32)
    c = torch.randn((B, H, G, rank), generator=g, device=device, dtype=f32) * math.sqrt(d / rank)
    inspan = torch.matmul(c, Wk.unsqueeze(0))
    sel = torch.zeros((H, G), dtype=torch.bool, device=device)
    if G >= 2:
        sel[:, :G // 2] = True
    else:
        sel[0::2, 0] = True
    Q = torch.where(sel[None, :, :, None], inspan, Q).reshape(B, H * G, d).half()
    CK = draw(mk, Wk, n_calib).cpu().numpy().astype(np.float32)
    CV = draw(mv, Wv, n_calib).cpu().numpy().astype(np.float32)
    return K, V, Q, CK, CV
