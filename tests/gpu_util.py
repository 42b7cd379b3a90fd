"""Shared pieces of the GPU parity tests: run a case through the C ABI and
compare it with the float64 oracle head by head."""
import numpy as np
import torch

from oracle import spectral as osq
from tests import parity_util as pu

MODE_SPECTRAL = 4


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def spectral_states(CK, CV):
    """Per-head SpectralQuant state (basis, mean, spreads) of the keys and
    values, fitted by the oracle on the calibration draws CK, CV [H, N, d]
    and rounded to float32 (the values both sides then read)."""
    out = {}
    for name, C in (("K", CK), ("V", CV)):
        fits = [osq.fit(C[h].astype(np.float64)) for h in range(C.shape[0])]
        out[name] = tuple(np.stack([f[i] for f in fits]).astype(np.float32) for i in range(3))
    return out


def run_case(tq, K, V, Q, scheme, n, seed=0, U=None, dtype=None, label="", modes=None, spectral=None):
    """K, V [B, H, T, d], Q [B, H*G, d] (numpy).  Quantise and decode on the
    GPU, run the oracle per (b, h), compare everything.  Returns the worst
    output error, the in-band mismatch count, the packed tensors, the device
    inputs and the oracle's dense (K_hat, V_hat) per (b, h).  modes:
    ((k_mode, k_bits), (v_mode, v_bits)) per-tensor overrides of the preset.
    spectral: {"K": (basis [H,d,d], mean [H,d], scale [H,d]), "V": ...}
    float32 numpy, for SPECTRAL tensors."""
    B, H, T, d = K.shape
    Hq = Q.shape[1]
    G = Hq // H
    dtype = torch.float32 if dtype is None else dtype
    Kd, Vd, Qd = dev(K, dtype), dev(V, dtype), dev(Q, dtype)
    # The oracle sees exactly the values the GPU sees.
    Kh_in = Kd.double().cpu().numpy()
    Vh_in = Vd.double().cpu().numpy()
    Qh_in = Qd.double().cpu().numpy()
    basis = dev(U.astype(np.float32)) if U is not None else None
    (km, kb), (vm, vb) = modes if modes is not None else ((None, None), (None, None))
    spec = {k: tuple(dev(a) for a in v) for k, v in spectral.items()} if spectral else {}
    kp = tq.quantize(Kd, tq.KEYS, scheme, n, seed, basis=basis, mode=km, bits=kb, spectral=spec.get("K"))
    vp = tq.quantize(Vd, tq.VALUES, scheme, n, seed, mode=vm, bits=vb, spectral=spec.get("V"))
    out, lse = tq.decode_attention(Qd, kp, vp)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    kplanes, vplanes = kp.planes(), vp.planes()
    kmode, vmode = pu.MODE_NAMES.get(kp.c.mode), pu.MODE_NAMES.get(vp.c.mode)

    def match(X, planes, pk, mode, name, h, Uh=None):
        if pk.c.mode == MODE_SPECTRAL:
            Vb, mu, sc = spectral[name]
            st = osq.SQState(Vb[h], mu[h], sc[h], pk.c.bits)
            return pu.spectral_match(X, planes, st, label=label + " " + name)
        return pu.oracle_match(X, planes, mode, pk.c.bits, seed, U=Uh, label=label + " " + name)

    n_band, n_dec = 0, 0
    worst = 0.0
    heads = []
    for b in range(B):
        for h in range(H):
            sl = slice((b * H + h) * T, (b * H + h + 1) * T)
            Uh = U[h] if U is not None else None
            _, Khat, _, nb1, nd1 = match(Kh_in[b, h], {k: v[sl] for k, v in kplanes.items()}, kp, kmode, "K", h, Uh)
            _, Vhat, _, nb2, nd2 = match(Vh_in[b, h], {k: v[sl] for k, v in vplanes.items()}, vp, vmode, "V", h)
            heads.append((Khat, Vhat))
            n_band += nb1 + nb2
            n_dec += nd1 + nd2
            qs = Qh_in[b, h * G:(h + 1) * G]
            o_ref, lse_ref, _ = pu.oracle_decode(qs, Khat, Vhat)
            err = pu.rel_l2(out[b, h * G:(h + 1) * G], o_ref)
            worst = max(worst, float(err.max()))
            assert np.all(err <= pu.OUT_RTOL), "%s: output rel L2 %.3g at b=%d h=%d" % (label, err.max(), b, h)
            assert np.allclose(lse[b, h * G:(h + 1) * G], lse_ref, atol=2e-4, rtol=1e-5), label + " lse"
    assert n_band <= max(1, pu.MAX_BAND_FRACTION * n_dec), "%s: %d in-band mismatches of %d" % (label, n_band, n_dec)
    return worst, n_band, kp, vp, (Kd, Vd, Qd), heads
