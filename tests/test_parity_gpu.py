"""GPU parity: the HIP path through the C ABI against the float64 oracle on
the same seeded inputs.  Bar: codes and sign bits bit-exact outside the 1e-6
decision band (in-band mismatches counted, < 1e-5 of all); attention outputs
within 1e-3 relative L2 per query; KL within 1e-5 absolute."""
import math

import numpy as np
import pytest

from compressed_decode_attention_kv_amd import synth
from oracle import quantizer as oqz
from oracle import metrics as ome
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


_dev = gpu_util.dev


def _run_case(*args, **kw):
    return gpu_util.run_case(*args, **kw)[:5]


def test_config1_kqv_full(tq):
    """Single head, d=128, T=4096, fp32 N(0,1), 16 queries, KQV at n=4."""
    K, V, Q = synth.isotropic_small(seed=0)
    worst, n_band, kp, vp, (Kd, Vd, Qd) = _run_case(tq, K, V, Q, "kqv", 4, seed=0, label="cfg1")
    print("config1 worst rel L2 %.3g, in-band mismatches %d" % (worst, n_band))
    # Metrics vs the oracle.
    m = tq.metrics(Qd, Kd, Vd, kp, vp)
    Kf, Vf, Qf = K[0, 0].astype(np.float64), V[0, 0].astype(np.float64), Q[0].astype(np.float64)
    _, Khat, _, _, _ = pu.oracle_match(Kf, kp.planes(), oqz.MSE, 4, 0)
    _, Vhat, _, _, _ = pu.oracle_match(Vf, vp.planes(), oqz.PROD, 3, 0)
    kl, rec, s, sh = pu.kl_and_recall(Qf, Kf, Khat)
    assert abs(m["kl_mean"] - kl.mean()) <= pu.KL_ATOL
    assert abs(m["kl_max"] - kl.max()) <= pu.KL_ATOL
    amb = pu.top5_ambiguous(sh).sum() + pu.top5_ambiguous(s).sum()
    assert abs(m["top5_recall"] - rec.mean()) <= amb / (5.0 * len(rec)) + 1e-12
    assert abs(m["relmse_k"] - ome.rel_mse(Kf, Khat)) <= 1e-5 * ome.rel_mse(Kf, Khat)
    assert abs(m["relmse_v"] - ome.rel_mse(Vf, Vhat)) <= 1e-5 * ome.rel_mse(Vf, Vhat)
    assert abs(m["dir_err_k"] - ome.direction_error(Kf, Khat)) <= 1e-5
    assert abs(m["dir_err_v"] - ome.direction_error(Vf, Vhat)) <= 1e-5
    assert m["n_queries"] == 16


@pytest.mark.parametrize("scheme", ["kv", "tq-kv", "kqv", "qkqv", "tq-qkv"])
@pytest.mark.parametrize("n", [2, 3, 4])
def test_schemes_ragged_gqa(tq, scheme, n):
    """Every preset and budget; T=1000 (ragged tail), B=2, H=2, 3 queries per
    KV head, fp16 inputs."""
    K, V, Q = synth.isotropic(2, 2, 3, 1000, 128, seed=10 + n, kv_std=1.0, dtype=np.float32)
    worst, n_band, *_ = _run_case(tq, K, V, Q, scheme, n, seed=n, dtype=torch.float16, label=scheme)
    print(scheme, n, "worst rel L2 %.3g band %d" % (worst, n_band))


@pytest.mark.parametrize("d,kmode,kbits,vmode,vbits", [
    (128, 1, 3, 2, 2),    # K MSE(3), V PROD(2 + 1): 3 bits per coordinate on both sides
    (128, 0, 4, 2, 1),    # K PLAIN(4), V PROD(1 + 1)
    (256, 2, 2, 0, 3),    # K PROD(2 + 1), V PLAIN(3)
    (64, 1, 4, 1, 2),     # K MSE(4), V MSE(2)
])
def test_per_tensor_override(tq, d, kmode, kbits, vmode, vbits):
    """Per-tensor (mode, index bits) chosen outside the presets through the
    ABI's override, fp16 inputs, ragged T, 2 queries per KV head."""
    K, V, Q = synth.isotropic(1, 2, 2, 900, d, seed=20 + d, kv_std=1.0, dtype=np.float32)
    worst, n_band, kp, vp, _ = _run_case(tq, K, V, Q, "kqv", 4, seed=3, dtype=torch.float16,
                                         modes=((kmode, kbits), (vmode, vbits)), label="override")
    assert (kp.c.mode, kp.c.bits, vp.c.mode, vp.c.bits) == (kmode, kbits, vmode, vbits)
    print("override", d, kmode, kbits, vmode, vbits, "worst rel L2 %.3g band %d" % (worst, n_band))


@pytest.mark.parametrize("d", [32, 64, 256, 512, 1024])
@pytest.mark.parametrize("scheme", ["kqv", "qkqv", "kv"])
def test_head_dims(tq, d, scheme):
    T = 700 if d < 1024 else 300
    K, V, Q = synth.isotropic(1, 2, 2, T, d, seed=d, kv_std=1.0, dtype=np.float32)
    _run_case(tq, K, V, Q, scheme, 4, seed=5, label="%s d=%d" % (scheme, d))


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_single_token_and_zero_vectors(tq, dtype):
    K, V, Q = synth.isotropic(1, 1, 4, 1, 128, seed=1, kv_std=1.0, dtype=np.float32)
    _run_case(tq, K, V, Q, "kqv", 4, label="T=1", dtype=dtype)
    K, V, Q = synth.isotropic(1, 2, 2, 300, 128, seed=2, kv_std=1.0, dtype=np.float32)
    K[0, 0, ::7] = 0.0
    V[0, 1, ::5] = 0.0
    _, _, kp, vp, _ = _run_case(tq, K, V, Q, "qkqv", 4, label="zeros", dtype=dtype)
    pl = kp.planes()
    z = np.arange(0, 300, 7)
    assert np.all(pl["codes"][z] == 0) and np.all(pl["gamma"][z] == 0)   # code fields hold the signs too


@pytest.mark.parametrize("scheme", ["kqv", "kv", "qkqv"])
def test_value_norms_across_orders_of_magnitude(tq, scheme):
    """Value vectors scaled by 10^u, u uniform in [-6, 6], with zero vectors
    among them, and keys scaled up so that the softmax weights spread too.
    The table-driven decode adds two tokens' values with fp16 weights kept in
    range by a running exponent frame; the outputs must still match the
    oracle's exact sums (T odd, so the last pair of a slot is a single token)."""
    K, V, Q = synth.isotropic(1, 2, 2, 701, 128, seed=11, kv_std=1.0, dtype=np.float32)
    rng = np.random.default_rng(12)
    V = (V * 10.0 ** rng.uniform(-6.0, 6.0, size=V.shape[:3] + (1,))).astype(np.float32)
    V[0, 0, ::9] = 0.0
    K = (K * 3.0).astype(np.float32)
    _run_case(tq, K, V, Q, scheme, 4, label="value norms " + scheme)


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_strided_input_and_large_values(tq, dtype):
    base = np.random.default_rng(3).standard_normal((1, 2, 400, 256)).astype(np.float32) * 300.0
    Kd = torch.from_numpy(base).to(dtype).cuda()[..., :128]       # row stride 256
    Vd = torch.from_numpy(base[..., 128:].copy()).to(dtype).cuda()
    Q = np.random.default_rng(4).standard_normal((1, 2, 128)).astype(np.float32) * 0.01
    kp = tq.quantize(Kd, tq.KEYS, "kqv", 4, 9)
    vp = tq.quantize(Vd, tq.VALUES, "kqv", 4, 9)
    out, _ = tq.decode_attention(torch.from_numpy(Q).cuda(), kp, vp)
    out = out.cpu().numpy()
    Kn = Kd.double().cpu().numpy()
    Vn = Vd.double().cpu().numpy()
    for h in range(2):
        sl = slice(h * 400, (h + 1) * 400)
        _, Khat, _, _, _ = pu.oracle_match(Kn[0, h], {k: v[sl] for k, v in kp.planes().items()}, oqz.MSE, 4, 9)
        _, Vhat, _, _, _ = pu.oracle_match(Vn[0, h], {k: v[sl] for k, v in vp.planes().items()}, oqz.PROD, 3, 9)
        o_ref, _, _ = pu.oracle_decode(Q[0, h:h + 1].astype(np.float64), Khat, Vhat)
        assert pu.rel_l2(out[0, h:h + 1], o_ref).max() <= pu.OUT_RTOL


def test_headq_gqa(tq):
    """HeadQ keys (2-bit base + rank-16 4-bit side code) with TQ-4 values,
    post-RoPE-like keys, 4 query heads per KV head."""
    d, r = 128, 16
    K, V, Q, C = synth.rope_gqa(1, 2, 4, 1500, d, seed=5, n_calib=4096, dtype=np.float32)
    from oracle import headq as ohq
    U = np.stack([ohq.fit_basis(C[h].astype(np.float64), r)[0] for h in range(2)])
    worst, n_band, kp, vp, (Kd, Vd, Qd) = _run_case(tq, K, V, Q, "headq", 4, seed=3, U=U, label="headq")
    m = tq.metrics(Qd, Kd, None, kp, None)
    kls = []
    for h in range(2):
        Kf = Kd[0, h].double().cpu().numpy()
        sl = slice(h * 1500, (h + 1) * 1500)
        _, Khat, _, _, _ = pu.oracle_match(Kf, {k: v[sl] for k, v in kp.planes().items()}, oqz.HEADQ, 2, 3, U=U[h])
        kl, _, _, _ = pu.kl_and_recall(Qd[0, 4 * h:4 * h + 4].double().cpu().numpy(), Kf, Khat)
        kls.append(kl)
    kls = np.concatenate(kls)
    assert abs(m["kl_mean"] - kls.mean()) <= pu.KL_ATOL and abs(m["kl_max"] - kls.max()) <= pu.KL_ATOL


@pytest.mark.parametrize("d,kmode,kbits,vmode,vbits", [
    (128, 1, 2, 1, 2),    # TQ-KV at n = 2
    (128, 1, 2, 1, 1),
    (128, 1, 4, 1, 1),
    (128, 2, 2, 1, 2),    # K PROD(2 + 1), V MSE(2)
    (128, 1, 2, 2, 2),    # K MSE(2), V PROD(2 + 1)
    (256, 1, 2, 1, 2),
    (512, 1, 3, 1, 1),
    (1024, 1, 2, 1, 2),
    (128, 0, 2, 0, 2),    # Plain-KV at n = 2
])
def test_table_decode_low_bits(tq, d, kmode, kbits, vmode, vbits):
    """The table-driven decode at 2-bit keys (fp32 centroid quads per byte)
    and 1- and 2-bit values (fp16 centroid octets and quads per byte), every
    head dim it serves; B=1, H=2, 3 queries per KV head, ragged T, fp16."""
    K, V, Q = synth.isotropic(1, 2, 3, 1100, d, seed=30 + d + kbits + vbits, kv_std=1.0, dtype=np.float32)
    worst, n_band, kp, vp, _ = _run_case(tq, K, V, Q, "kqv", 4, seed=6, dtype=torch.float16,
                                         modes=((kmode, kbits), (vmode, vbits)), label="lowbits")
    assert (kp.c.mode, kp.c.bits, vp.c.mode, vp.c.bits) == (kmode, kbits, vmode, vbits)
    print("low bits d=%d K(%d,%d) V(%d,%d) worst %.3g" % (d, kmode, kbits, vmode, vbits, worst))


@pytest.mark.parametrize("G,kbits,vbits,T", [
    (2, 4, 4, 700), (4, 3, 4, 1000), (16, 2, 2, 333), (17, 4, 3, 900), (64, 4, 4, 257), (5, 2, 3, 1),
    (4, 4, 1, 513), (16, 3, 1, 70),
])
def test_grouped_query_decode(tq, G, kbits, vbits, T):
    """The grouped-query matrix-core decode (G >= 2 query heads per KV head at
    d = 128, unsketched tensors): one block of 16 queries per pass, ragged
    query blocks (G = 17: 16 + 1), T not a multiple of the 16-token step,
    T = 1, 1-bit values (four tokens' bits per table entry); fp16 inputs, B=2,
    H=2."""
    K, V, Q = synth.isotropic(2, 2, G, T, 128, seed=80 + G + T, kv_std=1.0, dtype=np.float32)
    _run_case(tq, K, V, Q, "kqv", 4, seed=2, dtype=torch.float16, modes=((1, kbits), (1, vbits)),
              label="gqa G=%d" % G)


@pytest.mark.parametrize("d,G,scheme", [
    (128, 4, "kqv"), (128, 3, "qkqv"), (256, 2, "tq-kv"), (256, 16, "qkqv"), (512, 5, "kqv"),
    (1024, 2, "qkqv"), (1024, 17, "kqv"), (1024, 8, "tq-kv"),
])
def test_grouped_query_decode_wide_and_sketched(tq, d, G, scheme):
    """The grouped-query decode over wider heads (d / 128 waves per unit adding
    partial scores through LDS) and over sketched keys and values (QJL sign
    products on the matrix cores), n = 4, fp16, ragged T."""
    K, V, Q = synth.isotropic(1, 2, G, 530, d, seed=100 + d + G, kv_std=1.0, dtype=np.float32)
    _run_case(tq, K, V, Q, scheme, 4, seed=4, dtype=torch.float16, label="gqa %s d=%d G=%d" % (scheme, d, G))


@pytest.mark.parametrize("d,G,kbits,vbits", [(256, 4, 2, 1), (512, 3, 3, 2), (1024, 5, 4, 1)])
def test_grouped_query_decode_wide_narrow_values(tq, d, G, kbits, vbits):
    """The grouped-query decode over wider heads with 1- and 2-bit values
    (quad table entries, the 1-bit ones from a bit transpose of four tokens)
    and 2- to 4-bit keys, fp16, ragged T."""
    K, V, Q = synth.isotropic(1, 2, G, 301, d, seed=120 + d + G, kv_std=1.0, dtype=np.float32)
    _run_case(tq, K, V, Q, "kqv", 4, seed=5, dtype=torch.float16, modes=((1, kbits), (1, vbits)),
              label="gqa d=%d G=%d K%d V%d" % (d, G, kbits, vbits))


def test_grouped_query_decode_lengths_and_static(tq):
    """Per-sequence lengths (0, ragged, full) and the allocation-free decode
    through the grouped-query path agree with the oracle on each prefix."""
    from oracle import attention as oat
    B, H, G, T, d = 3, 2, 4, 600, 128
    K, V, Q = synth.isotropic(B, H, G, T, d, seed=91, kv_std=1.0, dtype=np.float32)
    Kd, Vd, Qd = _dev(K, torch.float16), _dev(V, torch.float16), _dev(Q, torch.float16)
    kp = tq.quantize(Kd, tq.KEYS, "tq-kv", 4, 3)
    vp = tq.quantize(Vd, tq.VALUES, "tq-kv", 3, 3)
    lens = torch.tensor([0, 301, 600], dtype=torch.int32, device="cuda")
    out, lse = tq.decode_attention(Qd, kp, vp, lens=lens)
    o2 = torch.empty_like(out)
    l2 = torch.empty_like(lse)
    tq.decode_attention_static(Qd, kp, vp, o2, l2, lens=lens)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    Kh, Vh, Qh = Kd.double().cpu().numpy(), Vd.double().cpu().numpy(), Qd.double().cpu().numpy()
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    for b, n in ((1, 301), (2, 600)):
        for h in range(H):
            sl = slice((b * H + h) * T, (b * H + h) * T + n)
            _, Khat, _, _, _ = pu.oracle_match(Kh[b, h, :n], {k: v[sl] for k, v in kp.planes().items()}, oqz.MSE, 4, 3)
            _, Vhat, _, _, _ = pu.oracle_match(Vh[b, h, :n], {k: v[sl] for k, v in vp.planes().items()}, oqz.MSE, 3, 3)
            o_ref, _, _, l_ref = oat.attend(Qh[b, h * G:(h + 1) * G], Khat, Vhat)
            assert np.all(pu.rel_l2(out[b, h * G:(h + 1) * G], o_ref) <= pu.OUT_RTOL)
            assert np.allclose(lse[b, h * G:(h + 1) * G], l_ref, atol=2e-4)


@pytest.mark.parametrize("vbits", [1, 2, 3])
def test_headq_keys_low_bit_values(tq, vbits):
    """HeadQ keys over 1-, 2- and 3-bit values (the value tiers of the A^2
    policy), 4 query heads per KV head."""
    d, r = 128, 16
    K, V, Q, C = synth.rope_gqa(1, 2, 4, 900, d, seed=7, n_calib=2048, dtype=np.float32)
    from oracle import headq as ohq
    U = np.stack([ohq.fit_basis(C[h].astype(np.float64), r)[0] for h in range(2)])
    worst, n_band, kp, vp, _ = _run_case(tq, K, V, Q, "headq", 4, seed=4, U=U, modes=((3, 2), (1, vbits)),
                                         label="headq v%d" % vbits)
    assert (kp.c.mode, vp.c.bits) == (3, vbits)


@pytest.mark.parametrize("scheme", ["kqv", "kv", "qkqv"])
def test_isotropic_decode_full_size_sampled(tq, scheme):
    """The benchmark workload at full size (B=16, 32 heads, T=32768, d=128,
    fp16, one query per head), in the launch configuration the benchmark
    times; sampled (batch, head) slices are checked against the oracle
    element by element, every output for finiteness, and the metrics call on
    the same slices against the oracle's KL and top-5."""
    B, H, T, d = 16, 32, 32768, 128
    K, V, Q = synth.device_isotropic(B, H, 1, T, d, seed=1)
    kp = tq.quantize(K, tq.KEYS, scheme, 4, 0)
    vp = tq.quantize(V, tq.VALUES, scheme, 4, 0)
    out, lse = tq.decode_attention(Q, kp, vp)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item() and torch.isfinite(lse).all().item()
    kmode, vmode = pu.MODE_NAMES[kp.c.mode], pu.MODE_NAMES[vp.c.mode]
    kpl, vpl = kp.planes(), vp.planes()
    for (b, h) in [(0, 0), (7, 13), (15, 31)]:
        sl = slice((b * H + h) * T, (b * H + h + 1) * T)
        Kn = K[b, h].double().cpu().numpy()
        Vn = V[b, h].double().cpu().numpy()
        qn = Q[b, h:h + 1].double().cpu().numpy()
        _, Khat, _, _, _ = pu.oracle_match(Kn, {k: v[sl] for k, v in kpl.items()}, kmode, kp.c.bits, 0, label="K")
        _, Vhat, _, _, _ = pu.oracle_match(Vn, {k: v[sl] for k, v in vpl.items()}, vmode, vp.c.bits, 0, label="V")
        o_ref, lse_ref, _ = pu.oracle_decode(qn, Khat, Vhat)
        err = pu.rel_l2(out[b, h:h + 1].cpu().numpy(), o_ref)
        assert err.max() <= pu.OUT_RTOL, (scheme, b, h, err)
        assert abs(lse[b, h].item() - lse_ref[0]) <= 1e-4
        m = tq.metrics(Q[b:b + 1, h:h + 1], K[b:b + 1, h:h + 1], None, kp.head_view(b, h), None)
        kl, rec, s, sh = pu.kl_and_recall(qn, Kn, Khat)
        assert abs(m["kl_mean"] - kl[0]) <= pu.KL_ATOL
        amb = int(pu.top5_ambiguous(s).sum() + pu.top5_ambiguous(sh).sum())
        assert abs(m["top5_recall"] - rec[0]) <= amb / 5.0 + 1e-12


@pytest.mark.parametrize("scheme", ["kqv", "qkqv", "headq"])
def test_capacity_larger_than_length(tq, scheme):
    """T_cap > T: the planes of each head are padded to the capacity; the
    decode must read only the first T tokens of each head."""
    B, H, G, T, d, cap = 2, 2, 2, 777, 128, 1000
    if scheme == "headq":
        K, V, Q, C = synth.rope_gqa(B, H, G, T, d, seed=8, n_calib=2048, dtype=np.float32)
        from oracle import headq as ohq
        U = np.stack([ohq.fit_basis(C[h].astype(np.float64), 16)[0] for h in range(H)])
        basis = gpu_util.dev(U.astype(np.float32))
    else:
        K, V, Q = synth.isotropic(B, H, G, T, d, seed=9, kv_std=1.0, dtype=np.float32)
        U, basis = None, None
    Kd, Vd, Qd = gpu_util.dev(K, torch.float16), gpu_util.dev(V, torch.float16), gpu_util.dev(Q, torch.float16)
    kp = tq.quantize(Kd, tq.KEYS, scheme, 4, 6, basis=basis, T_cap=cap)
    vp = tq.quantize(Vd, tq.VALUES, scheme, 4, 6, T_cap=cap)
    out, lse = tq.decode_attention(Qd, kp, vp)
    torch.cuda.synchronize()
    kpl, vpl = kp.planes(), vp.planes()
    kmode, vmode = pu.MODE_NAMES[kp.c.mode], pu.MODE_NAMES[vp.c.mode]
    for b in range(B):
        for h in range(H):
            sl = slice((b * H + h) * cap, (b * H + h) * cap + T)
            Kn, Vn = Kd[b, h].double().cpu().numpy(), Vd[b, h].double().cpu().numpy()
            _, Khat, _, _, _ = pu.oracle_match(Kn, {k: v[sl] for k, v in kpl.items()}, kmode, kp.c.bits, 6,
                                               U=U[h] if U is not None else None, label="cap K")
            _, Vhat, _, _, _ = pu.oracle_match(Vn, {k: v[sl] for k, v in vpl.items()}, vmode, vp.c.bits, 6,
                                               label="cap V")
            qn = Qd[b, G * h:G * h + G].double().cpu().numpy()
            o_ref, lse_ref, _ = pu.oracle_decode(qn, Khat, Vhat)
            assert pu.rel_l2(out[b, G * h:G * h + G].cpu().numpy(), o_ref).max() <= pu.OUT_RTOL
            assert np.allclose(lse[b, G * h:G * h + G].cpu().numpy(), lse_ref, atol=2e-4, rtol=1e-5)


def test_fp32_input_path_matches_fp16_path(tq):
    """fp32 inputs at d=128 take the matrix-core quantiser through an fp16
    hi + lo split of x * 2^14 / ||x||.  On fp16-representable data the fp32
    and fp16 paths see the same values: codes agree except next to a
    decision boundary (fraction < 1e-5), norms and gamma to 2e-6 relative.
    4 x 8 x 4096 vectors (16.8M coordinates): an inconsistent split (hi and
    lo rounded from different values next to an fp16 rounding tie) shows up
    here in hundreds of rows."""
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    X16 = (torch.randn((4, 8, 4096, 128), generator=g, device="cuda") / np.sqrt(128)).half()
    X32 = X16.float()
    for scheme, which in (("tq-kv", tq.KEYS), ("kqv", tq.VALUES), ("kv", tq.KEYS)):
        a, b = tq.quantize(X16, which, scheme, 4, 2), tq.quantize(X32, which, scheme, 4, 2)
        torch.cuda.synchronize()
        pa, pb = a.planes(), b.planes()
        fw = a.c.bits + (1 if a.c.mode == tq.MODE_PROD else 0)   # PROD fields carry the sign bit
        ia = oqz.unpack_bits(pa["codes"], fw, 128)
        ib = oqz.unpack_bits(pb["codes"], fw, 128)
        diff = ia != ib
        assert diff.mean() < pu.MAX_BAND_FRACTION, (scheme, diff.sum())
        na, nb = pa["norms"].astype(np.float64), pb["norms"].astype(np.float64)
        assert np.all(np.abs(na - nb) <= 1e-6 * na), scheme
        if "gamma" in pa:
            same = ~diff.any(axis=1)
            ga, gb = pa["gamma"][same].astype(np.float64), pb["gamma"][same].astype(np.float64)
            assert np.all(np.abs(ga - gb) <= 2e-6 * ga + 1e-12), (scheme, np.max(np.abs(ga - gb) / ga))
