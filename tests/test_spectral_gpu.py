"""GPU parity of SpectralQuant with uniform allocation (SQU-KV) through the C
ABI against the float64 oracle (oracle/spectral.py) on the structured
regime: codes exact outside the 1e-6 decision band (the distance of z_i to
its nearest boundary s_i t_k), norms to float32 rounding, attention outputs
within 1e-3 relative L2 per query, log-sum-exp (which carries the mean's
offset q . mu / sqrt(d)) within 2e-4, reconstruction measures within 1e-5
relative.  The per-head state (basis, mean, spreads) is fitted by the
oracle on a separate calibration draw and rounded to float32; both sides
read those float32 values."""
import numpy as np
import pytest

from compressed_decode_attention_kv_amd import synth
from oracle import metrics as ome
from oracle import spectral as osq
from tests import gpu_util
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from compressed_decode_attention_kv_amd import tq as lib
    return lib


def _case(B, H, G, T, d, seed):
    K, V, Q, CK, CV = synth.structured(B, H, G, T, d, seed=seed, n_calib=2048)
    return K, V, Q, gpu_util.spectral_states(CK, CV)


@pytest.mark.parametrize("d,n,dt", [
    (128, 2, "f16"), (128, 3, "f32"), (128, 4, "f16"), (128, 1, "f32"),
    (64, 2, "f32"), (64, 3, "f16"), (32, 2, "f16"), (32, 4, "f32"),
])
def test_squ_kv_quantize_and_decode(tq, d, n, dt):
    """B=2, H=2, 2 queries per KV head, T=777 (a ragged tail in every tile
    size: 8192/d tokens per quantiser tile), fp16 or fp32 inputs.  d=128 at
    3-4 bits decodes on the table-driven kernel, the rest on the generic one."""
    K, V, Q, spec = _case(2, 2, 2, 777, d, seed=40 + d + n)
    dtype = torch.float16 if dt == "f16" else torch.float32
    worst, n_band, kp, vp, _ = gpu_util.run_case(tq, K, V, Q, "squ-kv", n, seed=0, dtype=dtype,
                                                 spectral=spec, label="squ-kv d=%d n=%d" % (d, n))[:5]
    assert (kp.c.mode, kp.c.bits, vp.c.mode, vp.c.bits) == (4, n, 4, n)
    print("squ-kv d=%d n=%d %s worst rel L2 %.3g in-band %d" % (d, n, dt, worst, n_band))


def test_squ_kv_metrics(tq):
    """tq_metrics on a SPECTRAL cache: relMSE and direction error of both
    tensors, KL and top-5 against the oracle's dense reconstruction."""
    K, V, Q, spec = _case(1, 2, 4, 1500, 128, seed=51)
    worst, n_band, kp, vp, (Kd, Vd, Qd), heads = gpu_util.run_case(tq, K, V, Q, "squ-kv", 3, spectral=spec,
                                                                   label="metrics")
    m = tq.metrics(Qd, Kd, Vd, kp, vp)
    Kf = Kd.double().cpu().numpy()[0]
    Vf = Vd.double().cpu().numpy()[0]
    Qf = Qd.double().cpu().numpy()[0]
    Khat = np.concatenate([kh for kh, _ in heads])
    Vhat = np.concatenate([vh for _, vh in heads])
    Kall, Vall = Kf.reshape(-1, 128), Vf.reshape(-1, 128)
    for got, want in ((m["relmse_k"], ome.rel_mse(Kall, Khat)), (m["relmse_v"], ome.rel_mse(Vall, Vhat))):
        assert abs(got - want) <= 1e-5 * want, (got, want)
    assert abs(m["dir_err_k"] - ome.direction_error(Kall, Khat)) <= 1e-5
    assert abs(m["dir_err_v"] - ome.direction_error(Vall, Vhat)) <= 1e-5
    kls, recs, amb = [], [], 0
    for h in range(2):
        kl, rec, s, sh = pu.kl_and_recall(Qf[h * 4:(h + 1) * 4], Kf[h], heads[h][0])
        kls.append(kl)
        recs.append(rec)
        amb += pu.top5_ambiguous(sh).sum() + pu.top5_ambiguous(s).sum()
    kl = np.concatenate(kls)
    assert abs(m["kl_mean"] - kl.mean()) <= pu.KL_ATOL
    assert abs(m["kl_max"] - kl.max()) <= pu.KL_ATOL
    assert abs(m["top5_recall"] - np.concatenate(recs).mean()) <= amb / (5.0 * len(kl)) + 1e-12


@pytest.mark.parametrize("n,dt", [(3, "f16"), (4, "f32"), (1, "f16")])
def test_squ_kv_many_tiles(tq, n, dt):
    """d = 128 over many 64-token tiles and several blocks per head (T=2500,
    a ragged last tile), the matrix-core projection with certified
    decisions against the oracle."""
    K, V, Q, spec = _case(1, 2, 2, 2500, 128, seed=60 + n)
    dtype = torch.float16 if dt == "f16" else torch.float32
    gpu_util.run_case(tq, K, V, Q, "squ-kv", n, seed=0, dtype=dtype, spectral=spec, label="tiles n=%d" % n)


def test_squ_kv_degenerate_calibration(tq):
    """A calibration without noise: 112 of 128 spreads are (numerically)
    zero, so most decisions cannot be certified and every tile takes the
    exact path for all its decisions; keys with and without a component
    outside the calibrated span."""
    rng = np.random.default_rng(70)
    d, T, r = 128, 700, 16
    W, _ = np.linalg.qr(rng.standard_normal((d, r)))
    lam = 0.7 ** np.arange(r)
    C = (rng.standard_normal((2048, r)) * np.sqrt(lam)) @ W.T
    X = (rng.standard_normal((1, 1, T, r)) * np.sqrt(lam)) @ W.T
    X[0, 0, T // 2:] += 0.05 * rng.standard_normal((T - T // 2, d))   # half the tokens leave the span
    V0, mu, sc = (a.astype(np.float32) for a in osq.fit(C.astype(np.float64)))
    spec = {"K": (V0[None], mu[None], sc[None]), "V": (V0[None], mu[None], sc[None])}
    Q = rng.standard_normal((1, 2, d))
    gpu_util.run_case(tq, X, X, Q, "squ-kv", 3, spectral=spec, label="degenerate")


@pytest.mark.parametrize("d", [64, 128])
def test_squ_kv_append_matches_full_quantize(tq, d):
    """Appending a SPECTRAL cache in pieces at per-sequence positions writes
    the same bytes as quantising it whole."""
    K, V, Q, spec = _case(2, 2, 1, 400, d, seed=52)
    Kd = gpu_util.dev(K)
    sd = tuple(gpu_util.dev(a) for a in spec["K"])
    full = tq.quantize(Kd, tq.KEYS, "squ-kv", 3, spectral=sd)
    cache = tq.quantize(Kd[:, :, :100].contiguous(), tq.KEYS, "squ-kv", 3, spectral=sd, T_cap=400)
    for t0, t1 in ((100, 101), (101, 333), (333, 400)):
        pos = torch.full((2,), t0, dtype=torch.int32, device="cuda")
        tq.quantize_append(Kd[:, :, t0:t1].contiguous(), tq.KEYS, "squ-kv", 3, pos, cache)
    torch.cuda.synchronize()
    a, b = full.planes(), cache.planes()
    assert np.array_equal(a["codes"], b["codes"])
    assert np.array_equal(a["norms"], b["norms"])


def test_squ_kv_static_decode_and_lengths(tq):
    """The allocation-free decode and per-sequence lengths on a SPECTRAL
    cache agree with the allocating decode, and a zero length gives out = 0,
    lse = -inf (the mean's offset does not leak into empty sequences)."""
    K, V, Q, spec = _case(2, 2, 2, 600, 128, seed=53)
    sd = {k: tuple(gpu_util.dev(a) for a in v) for k, v in spec.items()}
    Kd, Vd, Qd = gpu_util.dev(K), gpu_util.dev(V), gpu_util.dev(Q)
    kp = tq.quantize(Kd, tq.KEYS, "squ-kv", 4, spectral=sd["K"])
    vp = tq.quantize(Vd, tq.VALUES, "squ-kv", 4, spectral=sd["V"])
    lens = torch.tensor([0, 600], dtype=torch.int32, device="cuda")
    o1, l1 = tq.decode_attention(Qd, kp, vp, lens=lens)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    tq.decode_attention_static(Qd, kp, vp, o2, l2, lens=lens)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.all(o1[0] == 0) and torch.all(torch.isneginf(l1[0]))
    o3, l3 = tq.decode_attention(Qd, kp, vp)
    assert torch.allclose(o3[1], o1[1], rtol=0, atol=0) and torch.equal(l3[1], l1[1])


@pytest.mark.parametrize("kmode,kbits,vmode,vbits", [(4, 3, 2, 2), (1, 3, 4, 2), (2, 2, 4, 4)])
def test_spectral_mixed_with_rotated_modes(tq, kmode, kbits, vmode, vbits):
    """Per-tensor overrides that pair a SPECTRAL tensor with a rotated one
    (MSE or QJL): the decode combines the two domains."""
    K, V, Q, spec = _case(1, 2, 2, 500, 128, seed=54)
    worst, n_band, kp, vp, _ = gpu_util.run_case(tq, K, V, Q, "kqv", 4, seed=7, spectral=spec,
                                                 modes=((kmode, kbits), (vmode, vbits)), label="mixed")[:5]
    assert (kp.c.mode, vp.c.mode) == (kmode, vmode)


def test_structured_data_quality_ordering(tq):
    """[P2] "Resultados e Recomendações": on structured data at 2 bits the
    SQU-KV keys reconstruct better than TQ-KV's, through the library."""
    K, V, Q, spec = _case(1, 2, 4, 2048, 128, seed=55)
    Kd, Vd, Qd = gpu_util.dev(K), gpu_util.dev(V), gpu_util.dev(Q)
    sd = {k: tuple(gpu_util.dev(a) for a in v) for k, v in spec.items()}
    sk = tq.quantize(Kd, tq.KEYS, "squ-kv", 2, spectral=sd["K"])
    sv = tq.quantize(Vd, tq.VALUES, "squ-kv", 2, spectral=sd["V"])
    tk = tq.quantize(Kd, tq.KEYS, "tq-kv", 2)
    tv = tq.quantize(Vd, tq.VALUES, "tq-kv", 2)
    ms = tq.metrics(Qd, Kd, Vd, sk, sv)
    mt = tq.metrics(Qd, Kd, Vd, tk, tv)
    print("relMSE K: squ-kv %.4g tq-kv %.4g; KL: %.4g vs %.4g" % (ms["relmse_k"], mt["relmse_k"],
                                                                   ms["kl_mean"], mt["kl_mean"]))
    assert ms["relmse_k"] < mt["relmse_k"]
    assert ms["relmse_v"] < mt["relmse_v"]
