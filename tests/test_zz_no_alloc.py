"""tq_decode_attention_static: the decode with the library's static device
workspace (no allocation), through the C ABI, against tq_decode_attention
with a workspace of its own on the same packed caches.  Same kernels, same
plan: outputs and log-sum-exps must be identical.  Two calls in a row, the
second on a smaller cache, so the second reads a workspace the first left
behind; plus per-sequence lengths, a head dim whose kernel writes one
partial per wave, and the host-side refusals."""
import ctypes

import numpy as np
import pytest

from compressed_decode_attention_kv_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def tq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from compressed_decode_attention_kv_amd import tq as lib
    return lib


def _case(tq, B, H, G, T, d, scheme, seed, lens=None):
    K, V, Q = synth.isotropic(B, H, G, T, d, seed=seed, kv_std=1.0, dtype=np.float32)
    Kd, Vd, Qd = (torch.from_numpy(x).half().cuda() for x in (K, V, Q))
    kp = tq.quantize(Kd, tq.KEYS, scheme, 4, seed)
    vp = tq.quantize(Vd, tq.VALUES, scheme, 4, seed)
    ln = torch.tensor(lens, dtype=torch.int32, device="cuda") if lens is not None else None
    ref_out, ref_lse = tq.decode_attention(Qd, kp, vp, lens=ln)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    tq.decode_attention_static(Qd, kp, vp, out, lse, lens=ln)
    torch.cuda.synchronize()
    print("static decode %s d=%d B=%d H=%d G=%d T=%d: max |diff| %.3g" % (
        scheme, d, B, H, G, T, (out - ref_out).abs().max().item()), flush=True)
    assert torch.equal(out, ref_out), (scheme, d, T)
    assert torch.equal(lse, ref_lse), (scheme, d, T)
    assert torch.isfinite(out).all().item()


def test_static_workspace_two_calls_second_smaller(tq):
    _case(tq, 2, 4, 2, 3000, 128, "kqv", 1)
    _case(tq, 1, 2, 1, 500, 128, "kqv", 2)


def test_static_workspace_lengths_and_other_kernels(tq):
    _case(tq, 3, 2, 2, 1500, 128, "qkqv", 3, lens=[1500, 700, 0])
    _case(tq, 1, 2, 4, 600, 1024, "kqv", 4)       # one partial per wave
    _case(tq, 1, 2, 2, 700, 64, "tq-qkv", 5)       # generic decode kernel
    _case(tq, 1, 1, 1, 40, 128, "kv", 6)


def test_static_workspace_refusals(tq):
    lib = tq.lib()
    # A sketched cache whose sketch (seed, d) was never made resident: refused
    # on the host.  The planes are real (zeroed) and sized, so nothing would be
    # out of bounds in any case.
    B, H, T, d = 1, 1, 64, 256
    k = tq.PackedTensor(B, H, T, d, tq.MODE_MSE, 4)
    v = tq.PackedTensor(B, H, T, d, tq.MODE_PROD, 3)
    for p, mode, bits in ((k, tq.MODE_MSE, 4), (v, tq.MODE_PROD, 3)):
        for t in (p.codes, p.norms, p.gamma):
            if t is not None:
                t.zero_()
        p.c.B, p.c.H, p.c.T, p.c.d, p.c.mode, p.c.bits, p.c.seed = B, H, T, d, mode, bits, 987654321
    q = torch.zeros((B, H, d), dtype=torch.float16, device="cuda")
    out = torch.zeros((B, H, d), dtype=torch.float32, device="cuda")
    with pytest.raises(tq.TQError) as e:
        tq.decode_attention_static(q, k, v, out)
    assert e.value.status == tq.EINVAL and "not resident" in str(e.value)
    # A decode whose workspace exceeds the static array: refused before any launch.
    fake = 1 << 20
    kb = tq.Packed(64, 32, 64, 64, 1024, tq.MODE_MSE, 4, 0, 0, 0, fake, fake, fake, fake, fake, fake, fake)
    vb = tq.Packed(64, 32, 64, 64, 1024, tq.MODE_PROD, 3, 0, 0, 0, fake, fake, fake, fake, fake, fake, fake)
    qd = tq.TensorDesc(fake, tq.F16, 64, 32, 1, 1024, 32 * 1024, 1024, 1024)
    st = lib.tq_decode_attention_static(ctypes.byref(qd), ctypes.byref(kb), ctypes.byref(vb), None, fake, None, None)
    assert st == tq.ENOMEM, st
    assert "static" in lib.tq_last_error().decode()
