"""C-ABI contract tests that need no GPU: the library loads, exports every
symbol include/tq.h declares, its host-only functions agree with the oracle,
and every validation error is returned before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import codebook as ocb
from oracle import headq as ohq
from oracle import rng as orng
from oracle import spectral as osq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "tq.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|tq_status|int32_t)\s+(tq_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol(tqlib):
    names = _declared()
    assert len(names) >= 14
    lib = ctypes.CDLL(tqlib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(tqlib.EXPORTS) == names
    assert tqlib.lib().tq_abi_version() == 7


@pytest.mark.parametrize("d,bits", [(32, 1), (128, 2), (128, 3), (128, 4), (1024, 2), (1024, 4)])
def test_codebook_matches_oracle(tqlib, d, bits):
    c, t = tqlib.codebook_build(d, bits)
    oc, ot = ocb.lloyd_max(d, bits)
    # Both are Lloyd fixed points computed independently (continued-fraction
    # incomplete beta here, scipy's betainc in the oracle); they agree far
    # inside the 1e-6 decision band.
    assert np.max(np.abs(c - oc)) < 2e-12
    assert np.max(np.abs(t - ot)) < 2e-12
    # The fp32 boundaries the kernels compare against are identical.
    assert np.array_equal(t.astype(np.float32), ot.astype(np.float32))


@pytest.mark.parametrize("seed,d", [(0, 32), (0, 128), (12345, 128), (2**63 + 7, 256), (3, 1024)])
def test_rotation_state_matches_oracle(tqlib, seed, d):
    s, S = tqlib.rotation_state(seed, d)
    assert np.array_equal(s.astype(np.float64), orng.sign_vector(seed, d))
    assert np.array_equal(S.astype(np.float64), orng.gaussian_sketch(seed, d))


def test_scheme_modes_table(tqlib):
    K, V = tqlib.KEYS, tqlib.VALUES
    P, M, Q, H = tqlib.MODE_PLAIN, tqlib.MODE_MSE, tqlib.MODE_PROD, tqlib.MODE_HEADQ
    assert tqlib.scheme_modes("kv", 4, K) == (P, 4) and tqlib.scheme_modes("kv", 4, V) == (P, 4)
    assert tqlib.scheme_modes("tq-kv", 3, K) == (M, 3)
    assert tqlib.scheme_modes("kqv", 4, K) == (M, 4) and tqlib.scheme_modes("kqv", 4, V) == (Q, 3)
    assert tqlib.scheme_modes("qkqv", 4, K) == (Q, 3) and tqlib.scheme_modes("qkqv", 2, V) == (Q, 1)
    assert tqlib.scheme_modes("tq-qkv", 3, K) == (Q, 2) and tqlib.scheme_modes("tq-qkv", 3, V) == (M, 3)
    assert tqlib.scheme_modes("headq", 4, K) == (H, 2) and tqlib.scheme_modes("headq", 4, V) == (M, 4)
    S = tqlib.MODE_SPECTRAL
    assert tqlib.scheme_modes("squ-kv", 2, K) == (S, 2) and tqlib.scheme_modes("squ-kv", 3, V) == (S, 3)


def test_layouts(tqlib):
    # PROD: 3-bit index + sign in 4-bit fields, no separate sign plane.
    lay = tqlib.packed_layout(128, tqlib.MODE_PROD, 3)
    assert (lay.code_bytes, lay.qjl_bytes, lay.has_gamma) == (64, 0, 1)
    lay = tqlib.packed_layout(128, tqlib.MODE_PROD, 2)
    assert (lay.code_bytes, lay.qjl_bytes, lay.has_gamma) == (48, 0, 1)
    lay = tqlib.packed_layout(128, tqlib.MODE_MSE, 4)
    assert (lay.code_bytes, lay.qjl_bytes, lay.has_gamma, lay.side_bytes) == (64, 0, 0, 0)
    lay = tqlib.packed_layout(128, tqlib.MODE_HEADQ, 2, 16, 4)
    assert (lay.code_bytes, lay.side_bytes, lay.has_side_scale) == (32, 8, 1)
    lay = tqlib.packed_layout(1024, tqlib.MODE_PROD, 3)
    assert (lay.code_bytes, lay.qjl_bytes) == (512, 0)
    lay = tqlib.packed_layout(128, tqlib.MODE_SPECTRAL, 3)
    assert (lay.code_bytes, lay.qjl_bytes, lay.has_gamma, lay.side_bytes) == (48, 0, 0, 0)
    lay = tqlib.packed_layout(32, tqlib.MODE_SPECTRAL, 1)
    assert lay.code_bytes == 4
    # The head's basis is held on chip: d <= 128.
    with pytest.raises(tqlib.TQError):
        tqlib.packed_layout(256, tqlib.MODE_SPECTRAL, 2)


@pytest.mark.parametrize("bad", [
    dict(d=48), dict(d=2048), dict(d=16), dict(n_bits=0), dict(n_bits=5),
    dict(scheme="kqv", which=1, n_bits=1), dict(scheme=99), dict(which=7),
    dict(dtype=9), dict(T=0), dict(B=0), dict(align=8), dict(stride_t=10),
    dict(no_codes=True), dict(scheme="kqv", which=1, no_gamma=True),
    dict(scheme="headq", which=0, no_hq=True), dict(scheme="tq-kv", which=0, give_hq=True),
    dict(scheme="headq", which=0, hq_rank=12), dict(scheme="headq", which=0, hq_bits=1),
    dict(T_cap=3),
    # per-tensor overrides (mode, index bits)
    dict(ovr=(1, 0)), dict(ovr=(1, 5)), dict(ovr=(2, 4)), dict(ovr=(2, 0)), dict(ovr=(7, 2)),
    dict(ovr=(3, 2), which=1, give_hq=True), dict(ovr=(3, 3), give_hq=True), dict(ovr=(3, 2), no_hq=True),
    dict(ovr=(2, 2), no_gamma=True),
    # SPECTRAL: state missing, misaligned, too wide, with a HeadQ basis, bad bits
    dict(scheme="squ-kv"), dict(scheme="squ-kv", spec_align=2), dict(scheme="squ-kv", basis_align=4), dict(scheme="squ-kv", d=256, give_spec=True),
    dict(scheme="squ-kv", give_spec=True, give_hq=True), dict(ovr=(4, 5), give_spec=True),
    dict(ovr=(4, 0), give_spec=True), dict(ovr=(4, 2), which=1),
])
def test_quantize_rejects_before_any_gpu_call(tqlib, bad):
    """Fake (never dereferenced) but aligned pointers: every case must be
    rejected by host validation, so no HIP call is made."""
    fake = 1 << 20
    d = bad.get("d", 128)
    desc = tqlib.TensorDesc(fake + bad.get("align", 0), bad.get("dtype", tqlib.F16), bad.get("B", 1), 2,
                            bad.get("T", 8), d, 2 * 8 * d, 8 * d, bad.get("stride_t", d))
    out = tqlib.Packed()
    out.T_cap = bad.get("T_cap", 0)
    out.codes = None if bad.get("no_codes") else fake
    out.norms = fake
    out.qjl = None
    out.gamma = None if bad.get("no_gamma") else fake
    out.side = fake
    out.side_scale = fake
    if bad.get("give_spec") or "spec_align" in bad or "basis_align" in bad:
        out.basis = fake + bad.get("basis_align", 0)
        out.mean = fake + bad.get("spec_align", 0)
        out.scale = fake
    hq = None
    scheme = bad.get("scheme", "tq-kv")
    if (scheme == "headq" and not bad.get("no_hq")) or bad.get("give_hq"):
        hq = tqlib.HeadQ(fake, bad.get("hq_rank", 16), bad.get("hq_bits", 4))
    sid = tqlib.SCHEMES.get(scheme, scheme)
    ovr = tqlib.ModeOverride(*bad["ovr"]) if "ovr" in bad else None
    st = tqlib.lib().tq_quantize(ctypes.byref(desc), bad.get("which", 0), sid, bad.get("n_bits", 4), 0,
                                 ctypes.byref(ovr) if ovr else None, ctypes.byref(hq) if hq else None,
                                 ctypes.byref(out), None)
    assert st in (tqlib.EINVAL, tqlib.EUNSUPPORTED), st
    assert tqlib.lib().tq_last_error().decode()


def _packed(tqlib, mode, bits, B=1, H=2, T=8, d=128, fake=1 << 20):
    p = tqlib.Packed(B, H, T, T, d, mode, bits, 0, 0, 0, fake, fake, fake, fake, fake, fake, fake)
    return p


def test_decode_rejects_mismatches(tqlib):
    lib = tqlib.lib()
    fake = 1 << 20
    k = _packed(tqlib, tqlib.MODE_MSE, 4)
    v = _packed(tqlib, tqlib.MODE_PROD, 3, T=9)
    n = ctypes.c_size_t()
    assert lib.tq_decode_workspace_size(ctypes.byref(k), ctypes.byref(v), 2, ctypes.byref(n)) == tqlib.EMISMATCH
    v = _packed(tqlib, tqlib.MODE_PROD, 3)
    assert lib.tq_decode_workspace_size(ctypes.byref(k), ctypes.byref(v), 3, ctypes.byref(n)) == tqlib.EMISMATCH
    assert lib.tq_decode_workspace_size(ctypes.byref(k), ctypes.byref(v), 4, ctypes.byref(n)) == tqlib.OK
    assert n.value > 0 and n.value % 256 == 0
    q = tqlib.TensorDesc(fake, tqlib.F16, 1, 4, 1, 64, 4 * 64, 64, 64)   # wrong d
    out = fake
    assert lib.tq_decode_attention(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), out, None, fake,
                                   n.value, None) == tqlib.EMISMATCH
    q = tqlib.TensorDesc(fake, tqlib.F16, 1, 4, 1, 128, 4 * 128, 128, 128)
    assert lib.tq_decode_attention(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), out, None, fake,
                                   n.value - 256, None) == tqlib.ENOMEM
    assert lib.tq_decode_attention(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), out, None, fake + 16,
                                   n.value, None) == tqlib.EINVAL
    # K and V with different capacities: the kernels address both with one head stride.
    vcap = _packed(tqlib, tqlib.MODE_PROD, 3)
    vcap.T_cap = 16
    assert lib.tq_decode_workspace_size(ctypes.byref(k), ctypes.byref(vcap), 4, ctypes.byref(n)) == tqlib.EMISMATCH
    assert lib.tq_decode_attention(ctypes.byref(q), ctypes.byref(k), ctypes.byref(vcap), out, None, fake,
                                   1 << 30, None) == tqlib.EMISMATCH
    hv = _packed(tqlib, tqlib.MODE_HEADQ, 2)
    assert lib.tq_decode_workspace_size(ctypes.byref(k), ctypes.byref(hv), 4, ctypes.byref(n)) != tqlib.OK
    # A hand-made PROD header with 4 index bits has no kernel: rejected before launch.
    k4 = _packed(tqlib, tqlib.MODE_PROD, 4)
    assert lib.tq_decode_workspace_size(ctypes.byref(k4), ctypes.byref(v), 4, ctypes.byref(n)) == tqlib.OK
    assert lib.tq_decode_attention(ctypes.byref(q), ctypes.byref(k4), ctypes.byref(v), out, None, fake,
                                   1 << 30, None) == tqlib.EUNSUPPORTED


def test_decode_rejects_spectral_without_state(tqlib):
    """A SPECTRAL header without its basis, mean or spreads is refused on the
    host, by the workspace query and the decode."""
    lib = tqlib.lib()
    fake = 1 << 20
    k = _packed(tqlib, tqlib.MODE_SPECTRAL, 3)
    v = _packed(tqlib, tqlib.MODE_SPECTRAL, 3)
    n = ctypes.c_size_t()
    for missing in ("basis", "mean", "scale"):
        k.basis, k.mean, k.scale = fake, fake, fake
        setattr(k, missing, None)
        assert lib.tq_decode_workspace_size(ctypes.byref(k), ctypes.byref(v), 2, ctypes.byref(n)) == tqlib.EINVAL
    k.basis, k.mean, k.scale = fake, fake, fake
    v.basis, v.mean, v.scale = fake, fake, fake
    assert lib.tq_decode_workspace_size(ctypes.byref(k), ctypes.byref(v), 2, ctypes.byref(n)) == tqlib.OK
    # The workspace grows by the per-query score offsets of SPECTRAL keys.
    m = _packed(tqlib, tqlib.MODE_MSE, 3)
    n2 = ctypes.c_size_t()
    assert lib.tq_decode_workspace_size(ctypes.byref(m), ctypes.byref(v), 2, ctypes.byref(n2)) == tqlib.OK
    assert n.value >= n2.value


def test_spectral_fit_matches_oracle(tqlib):
    """tq_spectral_fit (Jacobi in double on the host) against the oracle's
    fit (LAPACK eigh): the same mean, spreads, eigenvectors with the same
    sign convention (well separated spectrum), orthonormal columns."""
    rng = np.random.default_rng(11)
    d = 64
    W, _ = np.linalg.qr(rng.standard_normal((d, d)))
    lam = 0.8 ** np.arange(d)
    X = ((rng.standard_normal((5000, d)) * np.sqrt(lam)) @ W.T + 0.3).astype(np.float32)
    V, mu, s = tqlib.spectral_fit(X)
    Vo, muo, so = osq.fit(X.astype(np.float64))
    assert np.max(np.abs(V.T.astype(np.float64) @ V - np.eye(d))) < 1e-5
    assert np.max(np.abs(mu - muo)) < 1e-6
    assert np.max(np.abs(s - so)) < 1e-6
    assert abs(float(np.sum(s.astype(np.float64) ** 2)) - 1.0) < 1e-5
    assert np.max(np.abs(V - Vo)) < 1e-3
    with pytest.raises(tqlib.TQError):
        tqlib.spectral_fit(np.zeros((10, 256), dtype=np.float32))


def test_binding_refuses_bad_spectral_state(tqlib):
    torch = pytest.importorskip("torch")
    x = torch.zeros((1, 2, 8, 64), dtype=torch.float32)
    good = (torch.zeros((2, 64, 64)), torch.zeros((2, 64)), torch.zeros((2, 64)))
    for bad in (None, good[:2], (good[0].transpose(1, 2), good[1], good[2]),
                (good[0], good[1].double(), good[2]), (good[0], good[1], torch.zeros((2, 32)))):
        with pytest.raises(ValueError):
            tqlib.quantize(x, tqlib.KEYS, "squ-kv", 2, spectral=bad)


def test_headq_fit_matches_oracle_projector(tqlib):
    rng = np.random.default_rng(0)
    d, r = 128, 16
    scales = 0.8 ** np.arange(d)
    X = (rng.standard_normal((3000, d)) * scales + 0.5).astype(np.float32)
    U = tqlib.headq_fit(X, r)
    Uo, _ = ohq.fit_basis(X.astype(np.float64), r)
    assert np.max(np.abs(U.T @ U - np.eye(r))) < 1e-5
    assert np.max(np.abs(U @ U.T - Uo @ Uo.T)) < 1e-4
    # Same sign convention, so the columns agree too (eigenvalues well separated).
    assert np.max(np.abs(U - Uo)) < 1e-3


@pytest.mark.parametrize("case", ["strided", "shape", "dtype", "missing"])
def test_binding_refuses_bad_headq_basis(tqlib, case):
    """The ABI reads the HeadQ basis as dense [H][d][rank] fp32 at its pointer:
    the binding refuses a strided view (e.g. numpy eigenvectors, column-major)
    or a wrong shape or dtype before calling the library."""
    torch = pytest.importorskip("torch")
    x = torch.zeros((1, 2, 8, 128), dtype=torch.float32)
    bases = {
        "strided": torch.zeros((2, 16, 128), dtype=torch.float32).transpose(1, 2),  # [2, 128, 16] view
        "shape": torch.zeros((2, 64, 16), dtype=torch.float32),
        "dtype": torch.zeros((2, 128, 16), dtype=torch.float64),
        "missing": None,
    }
    if case == "strided":
        assert not bases[case].is_contiguous()
    with pytest.raises(ValueError):
        tqlib.quantize(x, tqlib.KEYS, "headq", 4, 0, basis=bases[case])


def test_append_and_lengths_reject_before_any_gpu_call(tqlib):
    """tq_quantize_append checks the new tokens against the cache header
    (mode, bits, seed, B, H, d, capacity) and tq_decode_attention_lens its
    length vector, on the host; fake pointers, invalid cases only."""
    lib = tqlib.lib()
    fake = 1 << 20
    cache = _packed(tqlib, tqlib.MODE_MSE, 4, B=1, H=2, T=8)
    cache.seed = 5

    def desc(H=2, T=1):
        return tqlib.TensorDesc(fake, tqlib.F16, 1, H, T, 128, H * T * 128, T * 128, 128)

    kqv, qkqv = tqlib.SCHEMES["kqv"], tqlib.SCHEMES["qkqv"]
    cases = [
        (desc(), kqv, 4, 6, fake, tqlib.EMISMATCH),       # seed differs
        (desc(), kqv, 3, 5, fake, tqlib.EMISMATCH),       # index bits differ
        (desc(), qkqv, 4, 5, fake, tqlib.EMISMATCH),      # mode differs (PROD keys)
        (desc(H=3), kqv, 4, 5, fake, tqlib.EMISMATCH),    # heads differ
        (desc(), kqv, 4, 5, None, tqlib.EINVAL),          # no positions
        (desc(), kqv, 4, 5, fake + 2, tqlib.EINVAL),      # misaligned positions
        (desc(T=9), kqv, 4, 5, fake, tqlib.EINVAL),       # more new tokens than the capacity
    ]
    for d, scheme, n, seed, pos, want in cases:
        st = lib.tq_quantize_append(ctypes.byref(d), tqlib.KEYS, scheme, n, seed, None, None, pos, ctypes.byref(cache),
                                    None)
        assert st == want, (scheme, n, seed, pos, st)
        assert lib.tq_last_error().decode()
    hq = tqlib.HeadQ(fake, 16, 4)
    assert lib.tq_quantize_append(ctypes.byref(desc()), tqlib.KEYS, kqv, 4, 5, None, ctypes.byref(hq), fake,
                                  ctypes.byref(cache), None) == tqlib.EINVAL
    # An override must name the cache's own mode and bits.
    for mode, bits, want in ((tqlib.MODE_MSE, 3, tqlib.EMISMATCH), (tqlib.MODE_PROD, 3, tqlib.EMISMATCH),
                             (tqlib.MODE_MSE, 9, tqlib.EINVAL)):
        ovr = tqlib.ModeOverride(mode, bits)
        assert lib.tq_quantize_append(ctypes.byref(desc()), tqlib.KEYS, kqv, 4, 5, ctypes.byref(ovr), None, fake,
                                      ctypes.byref(cache), None) == want
    v = _packed(tqlib, tqlib.MODE_PROD, 3, B=1, H=2, T=8)
    q = tqlib.TensorDesc(fake, tqlib.F16, 1, 2, 1, 128, 2 * 128, 128, 128)
    for lens in (None, fake + 2):
        assert lib.tq_decode_attention_lens(ctypes.byref(q), ctypes.byref(cache), ctypes.byref(v), lens, fake, None,
                                            fake, 1 << 30, None) == tqlib.EINVAL


def test_value_policy_rejects_before_any_gpu_call(tqlib):
    """Host validation of the value-policy entry points (fake pointers)."""
    lib = tqlib.lib()
    fake = 1 << 20
    n = ctypes.c_size_t()

    def desc(B=1, H=2, T=8, d=64, dtype=None):
        return tqlib.TensorDesc(fake, tqlib.F16 if dtype is None else dtype, B, H, T, d, H * T * d, T * d, d)
    k = desc()
    assert lib.tq_a2_workspace_size(ctypes.byref(desc(H=3)), ctypes.byref(k), ctypes.byref(n)) == tqlib.EMISMATCH
    assert lib.tq_a2_workspace_size(ctypes.byref(desc(B=2, H=4)), ctypes.byref(k), ctypes.byref(n)) == tqlib.EMISMATCH
    # 2 query heads per KV head x 200 probes x d=64 > 16384
    assert lib.tq_a2_workspace_size(ctypes.byref(desc(H=4, T=200)), ctypes.byref(k), ctypes.byref(n)) == tqlib.EUNSUPPORTED
    assert lib.tq_a2_workspace_size(ctypes.byref(desc(H=4, T=3)), ctypes.byref(k), ctypes.byref(n)) == tqlib.OK
    assert lib.tq_a2_weights(ctypes.byref(desc(H=4, T=3)), ctypes.byref(k), fake, fake, n.value - 1, None) == tqlib.ENOMEM
    assert lib.tq_a2_weights(ctypes.byref(desc(H=4, T=3)), ctypes.byref(k), None, fake, n.value, None) == tqlib.EINVAL
    v = desc()
    assert lib.tq_value_policy_workspace_size(ctypes.byref(v), ctypes.byref(n)) == tqlib.OK
    plan = tqlib.ValuePlan()
    for budget in (0, 5):
        assert lib.tq_value_policy(fake, ctypes.byref(v), budget, fake, ctypes.byref(plan), fake, n.value,
                                   None) == tqlib.EINVAL
    assert lib.tq_value_policy(fake, ctypes.byref(v), 2, fake, None, fake, n.value, None) == tqlib.EINVAL
    assert lib.tq_value_policy(fake, ctypes.byref(v), 2, fake, ctypes.byref(plan), fake, n.value - 256,
                               None) == tqlib.ENOMEM
    out = desc(T=4)
    assert lib.tq_gather_tokens(ctypes.byref(v), fake, 5, ctypes.byref(out), None) == tqlib.EINVAL
    assert lib.tq_gather_tokens(ctypes.byref(v), fake, -1, ctypes.byref(out), None) == tqlib.EINVAL
    assert lib.tq_gather_tokens(ctypes.byref(v), fake, 0, ctypes.byref(desc(T=4, d=32)), None) == tqlib.EMISMATCH
    assert lib.tq_gather_tokens(ctypes.byref(v), fake, 0, ctypes.byref(desc(T=4, dtype=tqlib.F32)), None) == tqlib.EMISMATCH
    assert lib.tq_attention_merge(fake, fake, None, fake, 4, 64, fake, None, None) == tqlib.EINVAL
    assert lib.tq_attention_merge(fake, fake, fake, fake, 0, 64, fake, None, None) == tqlib.EINVAL



def test_stream_rw_rejects_before_any_gpu_call(tqlib):
    """Host validation of the write-side traffic diagnostic (fake pointers)."""
    lib = tqlib.lib()
    fake = 1 << 20

    def call(src=fake, rows=1024, ib=256, dst=fake, ob=64, planes=fake, np_=2):
        return lib.tq_stream_rw(src, rows, ib, dst, ob, planes, np_, None)
    assert call(src=None) == tqlib.EINVAL
    assert call(dst=None) == tqlib.EINVAL
    assert call(planes=None) == tqlib.EINVAL
    assert call(src=fake + 8) == tqlib.EINVAL
    assert call(planes=fake + 2) == tqlib.EINVAL
    for ib, ob in ((0, 64), (96, 64), (8192, 64), (256, 0), (256, 80), (256, 8192)):
        assert call(ib=ib, ob=ob) == tqlib.EINVAL, (ib, ob)
    for np_ in (-1, 5):
        assert call(np_=np_) == tqlib.EINVAL
    for rows in (0, -3, (1 << 35) + 1):
        assert call(rows=rows) == tqlib.EINVAL
