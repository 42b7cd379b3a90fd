"""GPU tests of the generation-loop entry points, through the C ABI:
tq_quantize_append (new tokens written at per-sequence slots of an existing
packed cache) and tq_decode_attention_lens (each sequence attends over its own
length).

  * Appended planes equal those of quantising the whole sequence at once,
    slot by slot, at ragged per-sequence positions: bit-exact, since every
    token is quantised on its own by the same sequence of operations whatever
    its slot in a tile.  Matrix-core path (fp16 and fp32, d=128), the
    matrix-core sketch at d=256 (fp32 PROD keys), HeadQ.  Slots past T_cap are
    skipped and the neighbouring head's slots keep their bytes.  The appended
    sketched slots are also checked against the oracle (codes and signs exact
    outside the decision band).
  * Decode over ragged lengths (full, partial, one token, zero) against the
    float64 oracle on each sequence's own prefix; a length-0 sequence gives
    out = 0 and lse = -inf.  Table-driven (d=128) and generic (d=64) kernels.
  * A serving loop: a ragged prefix, then steps of "append one token per
    sequence, decode over the grown lengths", each step against the oracle.
"""
import numpy as np
import pytest

from tests import parity_util as pu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from compressed_decode_attention_kv_amd import tq as lib
    return lib


def _basis(H, d, r, seed):
    rng = np.random.default_rng(seed)
    U = np.stack([np.linalg.qr(rng.standard_normal((d, r)))[0] for _ in range(H)])
    return np.ascontiguousarray(U, dtype=np.float32)


def _cmp_slots(a, b, slots, label, sign_tol=0, field_bits=0):
    """Planes a, b (dicts of [n, bytes] arrays) equal on the given slots;
    with sign_tol, the code plane of a sketched tensor may differ in at most
    sign_tol bits, each of them the sign bit (top bit) of a field_bits-bit
    field."""
    for name in a:
        x, y = a[name][slots], b[name][slots]
        if name == "codes" and sign_tol:
            diff = np.unpackbits(np.bitwise_xor(x, y), axis=-1, bitorder="little")
            pos = np.nonzero(diff)[-1]
            assert len(pos) <= sign_tol, "%s: %d bits differ" % (label, len(pos))
            assert np.all(pos % field_bits == field_bits - 1), "%s: a code bit differs" % label
        else:
            assert np.array_equal(x, y), "%s: plane %s differs" % (label, name)


@pytest.mark.parametrize("scheme,dtype,d", [
    ("kqv", torch.float16, 128),    # matrix-core quantiser, MSE keys, PROD values
    ("qkqv", torch.float16, 128),
    ("kqv", torch.float32, 128),    # matrix-core quantiser on the fp32 hi + lo split
    ("tq-qkv", torch.float32, 256), # PROD keys through the matrix-core sketch kernel
    ("qkqv", torch.float16, 64),    # generic quantiser with the in-kernel sketch
    ("headq", torch.float16, 128),  # HeadQ side code (generic quantiser)
])
def test_append_matches_whole_sequence(tq, scheme, dtype, d):
    B, H, T0, Tmax, Tn = 3, 2, 64, 320, 37
    rng = np.random.default_rng(5)
    X = torch.from_numpy((rng.standard_normal((B, H, Tmax, d)) / np.sqrt(d)).astype(np.float32)).to(dtype).cuda()
    basis = torch.from_numpy(_basis(H, d, 16, 6)).cuda() if scheme == "headq" else None
    for which in (tq.KEYS, tq.VALUES):
        whole = tq.quantize(X, which, scheme, 4, 9, basis=basis)
        cache = tq.quantize(X[:, :, :T0].contiguous(), which, scheme, 4, 9, basis=basis, T_cap=Tmax)
        # Ragged positions; sequence 2 runs past T_cap (the last 37 - 5 tokens are skipped).
        pos = [T0, 101, Tmax - 5]
        xn = torch.stack([X[b, :, min(p, Tmax - Tn):min(p, Tmax - Tn) + Tn] for b, p in enumerate(pos)]).contiguous()
        # Sequence 2's new tokens are X[2, :, Tmax-Tn : Tmax]; only the first 5 land (slots Tmax-5 .. Tmax-1),
        # so compare those slots with tokens Tmax-Tn .. Tmax-Tn+4 of the whole-sequence cache below.
        tq.quantize_append(xn, which, scheme, 4, torch.tensor(pos, dtype=torch.int32, device="cuda"), cache, seed=9)
        torch.cuda.synchronize()
        a, c = whole.planes(), cache.planes()
        sign_tol = 0
        fb = cache.c.bits + 1
        label = "%s %s d=%d which=%d" % (scheme, dtype, d, which)
        for b in range(B):
            for h in range(H):
                base = (b * H + h) * Tmax
                _cmp_slots(a, c, slice(base, base + T0), label + " prefix b=%d h=%d" % (b, h), sign_tol, fb)
                if b < 2:
                    sl = slice(base + pos[b], base + pos[b] + Tn)
                    _cmp_slots(a, c, sl, label + " appended b=%d h=%d" % (b, h), sign_tol, fb)
                else:
                    src = Tmax - Tn
                    for k in range(5):
                        got = {n: v[base + Tmax - 5 + k:base + Tmax - 4 + k] for n, v in c.items()}
                        ref = {n: v[base + src + k:base + src + k + 1] for n, v in a.items()}
                        _cmp_slots(ref, got, slice(0, 1), label + " clipped b=%d h=%d k=%d" % (b, h, k), sign_tol, fb)
                if cache.c.mode == tq.MODE_PROD and b < 2:
                    # The appended slots against the oracle on their source tokens.
                    sl = slice(base + pos[b], base + pos[b] + Tn)
                    src = xn[b, h].double().cpu().numpy()
                    pu.oracle_match(src, {n: v[sl] for n, v in c.items()}, pu.MODE_NAMES[cache.c.mode],
                                    cache.c.bits, 9, label=label + " appended vs oracle")


def test_append_rejects_mismatched_cache(tq):
    X = torch.zeros((1, 2, 8, 128), dtype=torch.float16, device="cuda")
    cache = tq.quantize(X, tq.KEYS, "kqv", 4, 3, T_cap=16)
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    for kw in (dict(scheme="kqv", n=3, seed=3), dict(scheme="qkqv", n=4, seed=3), dict(scheme="kqv", n=4, seed=4)):
        with pytest.raises(tq.TQError) as e:
            tq.quantize_append(X[:, :, :1].contiguous(), tq.KEYS, kw["scheme"], kw["n"], pos, cache, seed=kw["seed"])
        assert e.value.status == tq.EMISMATCH
    with pytest.raises(tq.TQError) as e:
        tq.quantize_append(torch.zeros((1, 3, 1, 128), dtype=torch.float16, device="cuda"), tq.KEYS, "kqv", 4, pos,
                           cache, seed=3)
    assert e.value.status == tq.EMISMATCH
    with pytest.raises(ValueError):
        tq.quantize_append(X[:, :, :1].contiguous(), tq.KEYS, "kqv", 4, pos.to(torch.int64), cache, seed=3)


@pytest.mark.parametrize("scheme,d", [("kqv", 128), ("qkqv", 128), ("tq-qkv", 64)])
def test_decode_lengths_against_oracle(tq, scheme, d):
    """B=4, 2 KV heads x 2 query heads, T=1500 (several splits, ragged),
    lengths (1500, 777, 1, 0)."""
    from tests import gpu_util
    B, H, G, T = 4, 2, 2, 1500
    rng = np.random.default_rng(11)
    K = (rng.standard_normal((B, H, T, d)) / np.sqrt(d)).astype(np.float32)
    V = (rng.standard_normal((B, H, T, d)) / np.sqrt(d)).astype(np.float32)
    Q = rng.standard_normal((B, H * G, d)).astype(np.float32)
    Kd, Vd, Qd = gpu_util.dev(K), gpu_util.dev(V), gpu_util.dev(Q)
    kp = tq.quantize(Kd, tq.KEYS, scheme, 4, 2)
    vp = tq.quantize(Vd, tq.VALUES, scheme, 4, 2)
    lens = [T, 777, 1, 0]
    out, lse = tq.decode_attention(Qd, kp, vp, lens=torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    kpl, vpl = kp.planes(), vp.planes()
    for b in range(B):
        for h in range(H):
            qs = slice(h * G, (h + 1) * G)
            if lens[b] == 0:
                assert np.all(out[b, qs] == 0) and np.all(np.isneginf(lse[b, qs])), "empty sequence"
                continue
            sl = slice((b * H + h) * T, (b * H + h) * T + lens[b])
            _, Khat, _, _, _ = pu.oracle_match(K[b, h, :lens[b]].astype(np.float64), {k: v[sl] for k, v in kpl.items()},
                                               pu.MODE_NAMES[kp.c.mode], kp.c.bits, 2, label="lens K")
            _, Vhat, _, _, _ = pu.oracle_match(V[b, h, :lens[b]].astype(np.float64), {k: v[sl] for k, v in vpl.items()},
                                               pu.MODE_NAMES[vp.c.mode], vp.c.bits, 2, label="lens V")
            o_ref, lse_ref, _ = pu.oracle_decode(Q[b, qs].astype(np.float64), Khat, Vhat)
            err = pu.rel_l2(out[b, qs], o_ref)
            assert np.all(err <= pu.OUT_RTOL), "%s b=%d h=%d len=%d: rel L2 %.3g" % (scheme, b, h, lens[b], err.max())
            assert np.allclose(lse[b, qs], lse_ref, atol=2e-4, rtol=1e-5)


def test_append_decode_loop(tq):
    """KQV n=4, fp16, d=128, B=2, 2 KV heads x 2 query heads, prefixes of 150
    and 97 tokens in a cache of capacity 200; three steps of append-one-token
    + decode over the grown lengths, each against the oracle."""
    B, H, G, d, Tcap = 2, 2, 2, 128, 200
    rng = np.random.default_rng(21)
    X = {w: torch.from_numpy((rng.standard_normal((B, H, Tcap, d)) / np.sqrt(d)).astype(np.float32)).half().cuda()
         for w in ("k", "v")}
    lens = [150, 97]
    kp = tq.quantize(X["k"][:, :, :150].contiguous(), tq.KEYS, "kqv", 4, 1, T_cap=Tcap)
    vp = tq.quantize(X["v"][:, :, :150].contiguous(), tq.VALUES, "kqv", 4, 1, T_cap=Tcap)
    for step in range(3):
        pos = torch.tensor(lens, dtype=torch.int32, device="cuda")
        for w, p, which in (("k", kp, tq.KEYS), ("v", vp, tq.VALUES)):
            xn = torch.stack([X[w][b, :, lens[b]:lens[b] + 1] for b in range(B)]).contiguous()
            tq.quantize_append(xn, which, "kqv", 4, pos, p, seed=1)
        lens = [n + 1 for n in lens]
        kp.c.T = vp.c.T = max(lens)
        Q = torch.from_numpy(rng.standard_normal((B, H * G, d)).astype(np.float32)).half().cuda()
        out, lse = tq.decode_attention(Q, kp, vp, lens=torch.tensor(lens, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        out, lse = out.cpu().numpy(), lse.cpu().numpy()
        kpl, vpl = kp.planes(), vp.planes()
        Qn = Q.double().cpu().numpy()
        for b in range(B):
            for h in range(H):
                sl = slice((b * H + h) * Tcap, (b * H + h) * Tcap + lens[b])
                Kn = X["k"][b, h, :lens[b]].double().cpu().numpy()
                Vn = X["v"][b, h, :lens[b]].double().cpu().numpy()
                _, Khat, _, _, _ = pu.oracle_match(Kn, {k: v[sl] for k, v in kpl.items()}, pu.MODE_NAMES[kp.c.mode],
                                                   kp.c.bits, 1, label="loop K")
                _, Vhat, _, _, _ = pu.oracle_match(Vn, {k: v[sl] for k, v in vpl.items()}, pu.MODE_NAMES[vp.c.mode],
                                                   vp.c.bits, 1, label="loop V")
                qs = slice(h * G, (h + 1) * G)
                o_ref, lse_ref, _ = pu.oracle_decode(Qn[b, qs], Khat, Vhat)
                err = pu.rel_l2(out[b, qs], o_ref)
                assert np.all(err <= pu.OUT_RTOL), "step %d b=%d h=%d: rel L2 %.3g" % (step, b, h, err.max())
                assert np.allclose(lse[b, qs], lse_ref, atol=2e-4, rtol=1e-5)
