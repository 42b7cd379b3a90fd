"""GPU parity of tq_metrics' score-space and site measures, through the C ABI,
against the float64 oracle on the same packed planes:

  * Fisher score error 1/2 Var_p(s_hat - s) per query ([P3] Eq. 6), mean and
    max over queries;
  * Spearman rank correlation, across the queries, of KL with the Fisher
    error and with the raw key MSE of the query's head ([P3] section 4);
  * SNR (dB) and mean angle at the key cache, the value cache and the
    attention output (the 6D error framework of [P1]);
  * the A^2-weighted value distortion ([P3] section 2.2).

The oracle's dense dequantised K_hat / V_hat come from the same planes
(tests.parity_util.oracle_match, which also checks the planes themselves);
its output-site estimate is the GPU decode output, whose own parity with
the oracle is covered by the decode tests.  Tolerances: relative 1e-4 for the
Fisher and A^2 measures and the angles (fp32 scores and errors against
float64), 1e-3 dB for SNRs; Spearman exactly, after checking that the
oracle's per-query values are far enough apart (relative gap > 1e-3) that
rounding cannot swap two ranks.
"""
import numpy as np
import pytest

from oracle import attention as oat
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


def _separated(x, rel=1e-3):
    """Distinct values (up to exact ties) lie more than rel apart."""
    u = np.unique(np.asarray(x))
    return len(u) < 2 or np.all(np.diff(u) > rel * np.maximum(np.abs(u[1:]), 1e-30))


@pytest.mark.parametrize("scheme,d,G,dtype", [
    ("kqv", 128, 2, torch.float32),
    ("qkqv", 128, 1, torch.float16),
    ("tq-qkv", 64, 2, torch.float32),
    ("headq", 128, 2, torch.float32),
])
def test_score_space_and_site_measures(tq, scheme, d, G, dtype):
    B, H, T, seed = 2, 2, 700, 4
    rng = np.random.default_rng(17)
    K = (rng.standard_normal((B, H, T, d)) / np.sqrt(d) * rng.uniform(0.5, 2.0, (B, H, 1, 1))).astype(np.float32)
    V = (rng.standard_normal((B, H, T, d)) / np.sqrt(d)).astype(np.float32)
    Q = rng.standard_normal((B, H * G, d)).astype(np.float32) * 1.5
    Kd, Vd, Qd = (torch.from_numpy(x).to(dtype).cuda() for x in (K, V, Q))
    K, V, Q = (x.double().cpu().numpy() for x in (Kd, Vd, Qd))   # the values the GPU sees
    U = None
    basis = None
    if scheme == "headq":
        U = np.stack([np.linalg.qr(rng.standard_normal((d, 16)))[0] for _ in range(H)])
        basis = torch.from_numpy(np.ascontiguousarray(U, dtype=np.float32)).cuda()
        U = basis.double().cpu().numpy()
    kp = tq.quantize(Kd, tq.KEYS, scheme, 4, seed, basis=basis)
    vp = tq.quantize(Vd, tq.VALUES, scheme, 4, seed)
    m = tq.metrics(Qd, Kd, Vd, kp, vp)
    o_hat, _ = tq.decode_attention(Qd, kp, vp)
    torch.cuda.synchronize()
    o_hat = o_hat.double().cpu().numpy()

    kpl, vpl = kp.planes(), vp.planes()
    kl, fisher, a2, kmse = [], [], [], []
    Kh_all, Vh_all, o_ref_all = [], [], []
    for b in range(B):
        for h in range(H):
            sl = slice((b * H + h) * T, (b * H + h + 1) * T)
            _, Kh, _, _, _ = pu.oracle_match(K[b, h], {k: v[sl] for k, v in kpl.items()}, pu.MODE_NAMES[kp.c.mode],
                                             kp.c.bits, seed, U=U[h] if U is not None else None, label="metrics K")
            _, Vh, _, _, _ = pu.oracle_match(V[b, h], {k: v[sl] for k, v in vpl.items()}, pu.MODE_NAMES[vp.c.mode],
                                             vp.c.bits, seed, label="metrics V")
            Kh_all.append(Kh)
            Vh_all.append(Vh)
            q = Q[b, h * G:(h + 1) * G]
            o_ref, p_ref, s_ref, _ = oat.attend(q, K[b, h], V[b, h])
            s_hat = q @ Kh.T / np.sqrt(d)
            kl.append(ome.kl_from_scores(s_ref, s_hat))
            fisher.append(ome.fisher_score_error(s_ref, s_hat))
            a2.append(ome.a2_value_distortion(p_ref, V[b, h], Vh))
            kmse.append(np.full(G, np.mean(np.sum((K[b, h] - Kh) ** 2, axis=1))))
            o_ref_all.append(o_ref)
    kl, fisher, a2, kmse = (np.concatenate(x) for x in (kl, fisher, a2, kmse))
    o_ref_all = np.concatenate(o_ref_all)
    Kflat = K.reshape(-1, d)
    Vflat = V.reshape(-1, d)
    Khf, Vhf = np.concatenate(Kh_all), np.concatenate(Vh_all)
    # Query order of the oracle lists is (b, h, g) = (b, query head), as on the GPU.
    o_hat = o_hat.reshape(-1, d)

    def close(name, ref, rtol=1e-4, atol=0.0):
        got = m[name]
        assert abs(got - ref) <= atol + rtol * abs(ref), "%s %s: gpu %.9g oracle %.9g" % (scheme, name, got, ref)

    assert m["n_queries"] == len(kl)
    close("kl_mean", kl.mean(), rtol=0, atol=pu.KL_ATOL)
    close("fisher_mean", fisher.mean())
    close("fisher_max", fisher.max())
    close("a2_value_mean", a2.mean())
    close("snr_k_db", ome.snr_db(Kflat, Khf), rtol=0, atol=1e-3)
    close("snr_v_db", ome.snr_db(Vflat, Vhf), rtol=0, atol=1e-3)
    close("phi_k", ome.direction_angle(Kflat, Khf))
    close("phi_v", ome.direction_angle(Vflat, Vhf))
    close("snr_out_db", ome.snr_db(o_ref_all, o_hat), rtol=0, atol=1e-3)
    close("phi_out", ome.direction_angle(o_ref_all, o_hat))
    assert _separated(fisher) and _separated(kl) and _separated(kmse), "oracle values too close to rank robustly"
    close("spearman_fisher_kl", ome.spearman(fisher, kl), rtol=0, atol=1e-12)
    close("spearman_keymse_kl", ome.spearman(kmse, kl), rtol=0, atol=1e-12)
    print(scheme, "fisher/KL rho %.3f, key-MSE/KL rho %.3f, SNR k/v/out %.2f/%.2f/%.2f dB"
          % (m["spearman_fisher_kl"], m["spearman_keymse_kl"], m["snr_k_db"], m["snr_v_db"], m["snr_out_db"]))


def test_measures_missing_inputs_are_nan(tq):
    """Without queries the score-space measures are NaN; without the raw
    values the value-side and output-site measures are NaN."""
    rng = np.random.default_rng(2)
    K = torch.from_numpy((rng.standard_normal((1, 2, 300, 128)) / np.sqrt(128)).astype(np.float32)).cuda()
    Q = torch.from_numpy(rng.standard_normal((1, 2, 128)).astype(np.float32)).cuda()
    kp = tq.quantize(K, tq.KEYS, "kqv", 4, 0)
    vp = tq.quantize(K, tq.VALUES, "kqv", 4, 0)
    m = tq.metrics(None, K, None, kp, None)
    assert np.isfinite(m["snr_k_db"]) and np.isfinite(m["phi_k"])
    for f in ("fisher_mean", "spearman_fisher_kl", "snr_v_db", "snr_out_db", "a2_value_mean"):
        assert np.isnan(m[f]), f
    m = tq.metrics(Q, K, None, kp, vp)
    assert np.isfinite(m["fisher_mean"]) and np.isnan(m["a2_value_mean"]) and np.isnan(m["snr_out_db"])
