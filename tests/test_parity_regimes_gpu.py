"""GPU parity on the pages' other regimes, each with its own input law
(inputs: compressed_decode_attention_kv_amd/synth.py):

  * heavy-tailed K/V (Student-t, nu = 3, 1 % outlier tokens), fp32, the
    schemes Plain-KV, TQ-KV, TQ-QKV at n = 2 and 3, with relMSE_K/V and the
    cosine direction error the regime reports;
  * low-rank keys at d = 1024 (rank 16, eigenvalues 0.7^i, 0.01 noise) with
    queries half inside the key subspace, KQV and QKQV at n = 4, with KL and
    top-5 recall;
  * the full-size heavy-tailed cache (B=4, 8 heads, T=131072; every scheme
    and budget), the full-size low-rank cache (H=4, T=65536, d=1024, 64
    queries per head; KQV and QKQV) and the full-size HeadQ cache under GQA
    (B=8, 8 KV heads x 4 query heads, T=131072, fp16, rank-16 basis fitted
    from 4096 calibration queries), with a sampled (batch, head) slice
    checked element by element against the oracle.
Same bar as the other parity tests: codes, sign bits and side codes
bit-exact outside the decision band; outputs within 1e-3 relative L2;
metrics against the oracle's."""
import numpy as np
import pytest

from compressed_decode_attention_kv_amd import synth
from oracle import headq as ohq
from oracle import metrics as ome
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from compressed_decode_attention_kv_amd import tq as lib
    return lib


def _pooled(X):
    """The input vectors of every (b, h) in the order run_case visits them."""
    B, H = X.shape[:2]
    return np.concatenate([X[b, h] for b in range(B) for h in range(H)])


@pytest.mark.parametrize("scheme", ["kv", "tq-kv", "tq-qkv"])
@pytest.mark.parametrize("n", [2, 3])
def test_heavy_tailed_schemes(tq, scheme, n):
    """B=1, 2 heads, T=3000 (ragged), fp32; two queries per head exercise the
    read side as well."""
    from tests import gpu_util
    K, V = synth.heavy_tailed(1, 2, 3000, 128, seed=30 + n)
    Q = np.random.default_rng(31 + n).standard_normal((1, 4, 128)).astype(np.float32) * 0.5
    worst, n_band, kp, vp, (Kd, Vd, Qd), heads = gpu_util.run_case(tq, K, V, Q, scheme, n, seed=7,
                                                                    label="heavy %s n=%d" % (scheme, n))
    print("heavy", scheme, n, "worst rel L2 %.3g band %d" % (worst, n_band))
    m = tq.metrics(None, Kd, Vd, kp, vp)
    Kr = _pooled(Kd.double().cpu().numpy())
    Vr = _pooled(Vd.double().cpu().numpy())
    Kh = np.concatenate([k for k, _ in heads])
    Vh = np.concatenate([v for _, v in heads])
    for key, ref, hat in (("k", Kr, Kh), ("v", Vr, Vh)):
        rel = ome.rel_mse(ref, hat)
        assert abs(m["relmse_" + key] - rel) <= 1e-5 * rel, (key, m["relmse_" + key], rel)
        assert abs(m["dir_err_" + key] - ome.direction_error(ref, hat)) <= 1e-5, key
    assert np.isnan(m["kl_mean"])


@pytest.mark.parametrize("scheme", ["kqv", "qkqv"])
def test_low_rank_d1024(tq, scheme):
    """H=2, T=2500, d=1024, 8 queries per head (half in the key subspace),
    fp32, n=4: codes, outputs, KL and top-5 recall."""
    from tests import gpu_util
    K, V, Q = synth.low_rank(2, 2500, 1024, 8, seed=40)
    worst, n_band, kp, vp, (Kd, Vd, Qd), heads = gpu_util.run_case(tq, K, V, Q, scheme, 4, seed=11,
                                                                    label="lowrank %s" % scheme)
    print("low-rank", scheme, "worst rel L2 %.3g band %d" % (worst, n_band))
    m = tq.metrics(Qd, Kd, Vd, kp, vp)
    Kn, Qn = Kd.double().cpu().numpy(), Qd.double().cpu().numpy()
    kls, recs, amb = [], [], 0
    for h, (Khat, _) in enumerate(heads):
        kl, rec, s, sh = pu.kl_and_recall(Qn[0, 8 * h:8 * h + 8], Kn[0, h], Khat)
        kls.append(kl)
        recs.append(rec)
        amb += int(pu.top5_ambiguous(s).sum() + pu.top5_ambiguous(sh).sum())
    kls, recs = np.concatenate(kls), np.concatenate(recs)
    assert abs(m["kl_mean"] - kls.mean()) <= pu.KL_ATOL and abs(m["kl_max"] - kls.max()) <= pu.KL_ATOL
    assert abs(m["top5_recall"] - recs.mean()) <= amb / (5.0 * len(recs)) + 1e-12


@pytest.fixture(scope="module")
def heavy_full(tq):
    """The heavy-tailed cache at full size, drawn once on the device."""
    B, H, T, d = 4, 8, 131072, 128
    K, V = synth.device_heavy_tailed(B, H, T, d, seed=33)
    return K, V


@pytest.mark.parametrize("scheme,n", [("tq-qkv", 3), ("tq-qkv", 2), ("kv", 2), ("kv", 3), ("tq-kv", 2),
                                      ("tq-kv", 3)])
def test_heavy_tailed_full_size_sampled(tq, heavy_full, scheme, n):
    """B=4, 8 heads, T=131072, d=128, fp32, every scheme and budget of the
    regime: full quantisation on the GPU, finiteness of every norm, and one
    sampled (batch, head) slice against the oracle (codes, sign bits, norms;
    relMSE and direction error of that slice)."""
    B, H, T, d = 4, 8, 131072, 128
    K, V = heavy_full
    kp = tq.quantize(K, tq.KEYS, scheme, n, 21)
    vp = tq.quantize(V, tq.VALUES, scheme, n, 21)
    torch.cuda.synchronize()
    kpl, vpl = kp.planes(), vp.planes()
    assert np.isfinite(kpl["norms"]).all() and np.isfinite(vpl["norms"]).all()
    if "gamma" in kpl:
        assert np.isfinite(kpl["gamma"]).all()
    b, h = (2, 5) if n == 3 else (3, 1)
    sl = slice((b * H + h) * T, (b * H + h + 1) * T)
    Kn = K[b, h].double().cpu().numpy()
    Vn = V[b, h].double().cpu().numpy()
    _, Khat, _, nb1, nd1 = pu.oracle_match(Kn, {k: v[sl] for k, v in kpl.items()}, pu.MODE_NAMES[kp.c.mode],
                                           kp.c.bits, 21, label="heavy full %s %d K" % (scheme, n))
    _, Vhat, _, nb2, nd2 = pu.oracle_match(Vn, {k: v[sl] for k, v in vpl.items()}, pu.MODE_NAMES[vp.c.mode],
                                           vp.c.bits, 21, label="heavy full %s %d V" % (scheme, n))
    assert nb1 + nb2 <= max(1, pu.MAX_BAND_FRACTION * (nd1 + nd2))
    m = tq.metrics(None, K[b:b + 1, h:h + 1], V[b:b + 1, h:h + 1], kp.head_view(b, h), vp.head_view(b, h))
    for key, ref, hat in (("k", Kn, Khat), ("v", Vn, Vhat)):
        rel = ome.rel_mse(ref, hat)
        assert abs(m["relmse_" + key] - rel) <= 1e-5 * rel, (key, m["relmse_" + key], rel)
        assert abs(m["dir_err_" + key] - ome.direction_error(ref, hat)) <= 1e-5, key


@pytest.mark.parametrize("scheme", ["kqv", "qkqv"])
def test_low_rank_full_size_sampled(tq, scheme):
    """The low-rank workload at its own size: H=4, T=65536, d=1024, fp32,
    64 queries per head (half inside the key subspace), n=4, in the launch
    configuration the benchmark times.  Full quantisation and decode on the
    GPU; every output finite; one sampled head with its 64 queries against the
    oracle (codes and signs, norms, gamma, outputs, LSE, KL and top-5)."""
    H, T, d, G = 4, 65536, 1024, 64
    K, V, Q = synth.low_rank(H, T, d, G, seed=40)
    Kd, Vd, Qd = (torch.from_numpy(x).cuda() for x in (K, V, Q))
    kp = tq.quantize(Kd, tq.KEYS, scheme, 4, 3)
    vp = tq.quantize(Vd, tq.VALUES, scheme, 4, 3)
    out, lse = tq.decode_attention(Qd, kp, vp)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item() and torch.isfinite(lse).all().item()
    h = 2 if scheme == "kqv" else 1
    sl = slice(h * T, (h + 1) * T)
    Kn, Vn = K[0, h].astype(np.float64), V[0, h].astype(np.float64)
    qn = Q[0, G * h:G * h + G].astype(np.float64)
    kpl, vpl = kp.planes(), vp.planes()
    _, Khat, _, nb1, nd1 = pu.oracle_match(Kn, {k: v[sl] for k, v in kpl.items()}, pu.MODE_NAMES[kp.c.mode],
                                           kp.c.bits, 3, label="low-rank full K")
    _, Vhat, _, nb2, nd2 = pu.oracle_match(Vn, {k: v[sl] for k, v in vpl.items()}, pu.MODE_NAMES[vp.c.mode],
                                           vp.c.bits, 3, label="low-rank full V")
    assert nb1 + nb2 <= max(1, pu.MAX_BAND_FRACTION * (nd1 + nd2))
    o_ref, lse_ref, _ = pu.oracle_decode(qn, Khat, Vhat)
    err = pu.rel_l2(out[0, G * h:G * h + G].cpu().numpy(), o_ref)
    print("low-rank full %s: worst rel L2 %.3g, in-band %d" % (scheme, err.max(), nb1 + nb2))
    assert err.max() <= pu.OUT_RTOL, err
    assert np.allclose(lse[0, G * h:G * h + G].cpu().numpy(), lse_ref, atol=2e-4, rtol=1e-5)
    m = tq.metrics(Qd[:, G * h:G * h + G].contiguous(), Kd[:, h:h + 1], None, kp.head_view(0, h), None)
    kl, rec, s, sh = pu.kl_and_recall(qn, Kn, Khat)
    assert abs(m["kl_mean"] - kl.mean()) <= pu.KL_ATOL and abs(m["kl_max"] - kl.max()) <= pu.KL_ATOL
    amb = int(pu.top5_ambiguous(s).sum() + pu.top5_ambiguous(sh).sum())
    assert abs(m["top5_recall"] - rec.mean()) <= amb / (5.0 * len(rec)) + 1e-12


def test_headq_gqa_full_size_sampled(tq):
    """B=8, 8 KV heads x 4 query heads, T=131072, d=128, fp16 post-RoPE keys;
    HeadQ keys (2-bit base + rank-16 4-bit side code, basis fitted from 4096
    calibration queries per head) and TQ-4 values.  Full quantisation and
    decode on the GPU; every output finite; one sampled (batch, KV head) with
    its 4 queries against the oracle (codes, side codes, outputs, LSE, KL)."""
    B, Hkv, G, T, d, r = 8, 8, 4, 131072, 128, 16
    K, V, Q, C = synth.device_rope_gqa(B, Hkv, G, T, d, seed=55)
    U = np.stack([ohq.fit_basis(C[h].astype(np.float64), r)[0] for h in range(Hkv)])
    basis = torch.from_numpy(np.ascontiguousarray(U, dtype=np.float32)).cuda()
    kp = tq.quantize(K, tq.KEYS, "headq", 4, 13, basis=basis)
    vp = tq.quantize(V, tq.VALUES, "headq", 4, 13)
    out, lse = tq.decode_attention(Q, kp, vp)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item() and torch.isfinite(lse).all().item()
    b, h = 5, 3
    sl = slice((b * Hkv + h) * T, (b * Hkv + h + 1) * T)
    Kn = K[b, h].double().cpu().numpy()
    Vn = V[b, h].double().cpu().numpy()
    qn = Q[b, G * h:G * h + G].double().cpu().numpy()
    kpl, vpl = kp.planes(), vp.planes()
    _, Khat, _, nb1, nd1 = pu.oracle_match(Kn, {k: v[sl] for k, v in kpl.items()}, pu.MODE_NAMES[kp.c.mode],
                                           kp.c.bits, 13, U=U[h], label="headq full K")
    _, Vhat, _, nb2, nd2 = pu.oracle_match(Vn, {k: v[sl] for k, v in vpl.items()}, pu.MODE_NAMES[vp.c.mode],
                                           vp.c.bits, 13, label="headq full V")
    assert nb1 + nb2 <= max(1, pu.MAX_BAND_FRACTION * (nd1 + nd2))
    o_ref, lse_ref, _ = pu.oracle_decode(qn, Khat, Vhat)
    err = pu.rel_l2(out[b, G * h:G * h + G].cpu().numpy(), o_ref)
    assert err.max() <= pu.OUT_RTOL, err
    assert np.allclose(lse[b, G * h:G * h + G].cpu().numpy(), lse_ref, atol=2e-4, rtol=1e-5)
    m = tq.metrics(Q[b:b + 1, G * h:G * h + G], K[b:b + 1, h:h + 1], None, kp.head_view(b, h), None)
    kl, _, _, _ = pu.kl_and_recall(qn, Kn, Khat)
    assert abs(m["kl_mean"] - kl.mean()) <= pu.KL_ATOL and abs(m["kl_max"] - kl.max()) <= pu.KL_ATOL


@pytest.mark.parametrize("scheme,d,H,T,dtype", [("kqv", 512, 1, 40000, torch.float32),
                                                ("qkqv", 256, 5, 16001, torch.float32),
                                                ("qkqv", 1024, 3, 1000, torch.float16)])
def test_sketch_tiles(tq, scheme, d, H, T, dtype):
    """B=1, n=4: at d >= 256 the QJL sketch S r runs on the matrix cores over
    tiles of 32768 / d tokens of one head (the residuals staged in LDS as
    fp16 hi + lo).  Many tiles per head with a ragged last tile (T = 40000
    at d=512: 625 tiles of 64; T = 16001 at d=256: the last tile holds one
    token), several heads, fp32 and fp16 inputs.  Codes, signs, norms, gamma
    and outputs against the oracle."""
    from tests import gpu_util
    K, V, Q = synth.isotropic(1, H, 2, T, d, seed=77, kv_std=1.0, dtype=np.float32)
    worst, n_band, *_ = gpu_util.run_case(tq, K, V, Q, scheme, 4, seed=19, dtype=dtype,
                                          label="sketch %s d=%d" % (scheme, d))
    print("sketch tiles", scheme, d, "worst rel L2 %.3g band %d" % (worst, n_band))
