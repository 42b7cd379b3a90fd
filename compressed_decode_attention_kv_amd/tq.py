"""ctypes binding of libtq.so, the C-ABI library declared in include/tq.h.

Argument marshalling only: every step of the quantiser and of the decode
runs in the library's HIP kernels.  PyTorch supplies device memory and the
current stream.  Importing this module loads libtq.so and raises if it is
missing -- there is no CPU fallback.
"""
import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libtq.so is not built (%s); run `python -m compressed_decode_attention_kv_amd.build`" % LIB_PATH)
_lib = ctypes.CDLL(LIB_PATH)

# ---- enums (include/tq.h) -------------------------------------------------------
OK, EINVAL, EUNSUPPORTED, EMISMATCH, ENOMEM, EDEVICE = range(6)
F32, F16 = 0, 1
KEYS, VALUES = 0, 1
MODE_PLAIN, MODE_MSE, MODE_PROD, MODE_HEADQ, MODE_SPECTRAL = range(5)
SCHEMES = {"kv": 0, "tq-kv": 1, "kqv": 2, "qkqv": 3, "tq-qkv": 4, "headq": 5, "squ-kv": 6}

EXPORTS = ["tq_abi_version", "tq_status_str", "tq_last_error", "tq_codebook_build", "tq_scheme_modes",
           "tq_packed_layout", "tq_rotation_state", "tq_quantize", "tq_quantize_append",
           "tq_decode_workspace_size", "tq_decode_attention", "tq_decode_attention_lens",
           "tq_decode_attention_static",
           "tq_metrics_workspace_size", "tq_metrics", "tq_spectral_fit", "tq_headq_fit",
           "tq_a2_workspace_size", "tq_a2_weights", "tq_value_policy_workspace_size", "tq_value_policy",
           "tq_gather_tokens", "tq_attention_merge",
           "tq_stream_read", "tq_stream_rw", "tq_release_cache"]


class ModeOverride(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("bits", ctypes.c_int32)]


class TensorDesc(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("B", ctypes.c_int32),
                ("H", ctypes.c_int32), ("T", ctypes.c_int32), ("d", ctypes.c_int32),
                ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64), ("stride_t", ctypes.c_int64)]


class Layout(ctypes.Structure):
    _fields_ = [("code_bytes", ctypes.c_int32), ("qjl_bytes", ctypes.c_int32), ("side_bytes", ctypes.c_int32),
                ("has_gamma", ctypes.c_int32), ("has_side_scale", ctypes.c_int32)]


class HeadQ(ctypes.Structure):
    _fields_ = [("basis", ctypes.c_void_p), ("rank", ctypes.c_int32), ("side_bits", ctypes.c_int32)]


class Packed(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32), ("T_cap", ctypes.c_int32),
                ("d", ctypes.c_int32), ("mode", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("side_rank", ctypes.c_int32), ("side_bits", ctypes.c_int32), ("seed", ctypes.c_uint64),
                ("codes", ctypes.c_void_p), ("norms", ctypes.c_void_p), ("qjl", ctypes.c_void_p),
                ("gamma", ctypes.c_void_p), ("side", ctypes.c_void_p), ("side_scale", ctypes.c_void_p),
                ("basis", ctypes.c_void_p), ("mean", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class MetricsOut(ctypes.Structure):
    _fields_ = [("kl_mean", ctypes.c_double), ("kl_max", ctypes.c_double), ("top5_recall", ctypes.c_double),
                ("relmse_k", ctypes.c_double), ("relmse_v", ctypes.c_double), ("dir_err_k", ctypes.c_double),
                ("dir_err_v", ctypes.c_double), ("n_queries", ctypes.c_int64),
                ("fisher_mean", ctypes.c_double), ("fisher_max", ctypes.c_double),
                ("spearman_fisher_kl", ctypes.c_double), ("spearman_keymse_kl", ctypes.c_double),
                ("snr_k_db", ctypes.c_double), ("snr_v_db", ctypes.c_double), ("snr_out_db", ctypes.c_double),
                ("phi_k", ctypes.c_double), ("phi_v", ctypes.c_double), ("phi_out", ctypes.c_double),
                ("a2_value_mean", ctypes.c_double)]


class ValuePlan(ctypes.Structure):
    _fields_ = [("b_lo", ctypes.c_int32), ("b_hi", ctypes.c_int32), ("n_high", ctypes.c_int32),
                ("n_candidates", ctypes.c_int32), ("cand_lo", ctypes.c_int32 * 3), ("cand_hi", ctypes.c_int32 * 3),
                ("cand_high", ctypes.c_int32 * 3), ("surrogate", ctypes.c_double * 3)]


_P = ctypes.POINTER
_sigs = {
    "tq_abi_version": ([], ctypes.c_int32),
    "tq_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "tq_last_error": ([], ctypes.c_char_p),
    "tq_codebook_build": ([ctypes.c_int32, ctypes.c_int32, _P(ctypes.c_double), _P(ctypes.c_double)], ctypes.c_int),
    "tq_scheme_modes": ([ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P(ctypes.c_int32), _P(ctypes.c_int32)], ctypes.c_int),
    "tq_packed_layout": ([ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P(Layout)], ctypes.c_int),
    "tq_rotation_state": ([ctypes.c_uint64, ctypes.c_int32, _P(ctypes.c_float), _P(ctypes.c_float)], ctypes.c_int),
    "tq_quantize": ([_P(TensorDesc), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint64,
                     _P(ModeOverride), _P(HeadQ), _P(Packed), ctypes.c_void_p], ctypes.c_int),
    "tq_quantize_append": ([_P(TensorDesc), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint64,
                            _P(ModeOverride), _P(HeadQ), ctypes.c_void_p, _P(Packed), ctypes.c_void_p], ctypes.c_int),
    "tq_decode_workspace_size": ([_P(Packed), _P(Packed), ctypes.c_int32, _P(ctypes.c_size_t)], ctypes.c_int),
    "tq_decode_attention": ([_P(TensorDesc), _P(Packed), _P(Packed), ctypes.c_void_p, ctypes.c_void_p,
                             ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "tq_decode_attention_lens": ([_P(TensorDesc), _P(Packed), _P(Packed), ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "tq_decode_attention_static": ([_P(TensorDesc), _P(Packed), _P(Packed), ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
    "tq_metrics_workspace_size": ([_P(TensorDesc), _P(Packed), _P(Packed), _P(ctypes.c_size_t)], ctypes.c_int),
    "tq_metrics": ([_P(TensorDesc), _P(TensorDesc), _P(TensorDesc), _P(Packed), _P(Packed), _P(MetricsOut),
                    ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "tq_headq_fit": ([_P(ctypes.c_float), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P(ctypes.c_float)], ctypes.c_int),
    "tq_spectral_fit": ([_P(ctypes.c_float), ctypes.c_int32, ctypes.c_int32, _P(ctypes.c_float), _P(ctypes.c_float),
                         _P(ctypes.c_float)], ctypes.c_int),
    "tq_a2_workspace_size": ([_P(TensorDesc), _P(TensorDesc), _P(ctypes.c_size_t)], ctypes.c_int),
    "tq_a2_weights": ([_P(TensorDesc), _P(TensorDesc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                       ctypes.c_void_p], ctypes.c_int),
    "tq_value_policy_workspace_size": ([_P(TensorDesc), _P(ctypes.c_size_t)], ctypes.c_int),
    "tq_value_policy": ([ctypes.c_void_p, _P(TensorDesc), ctypes.c_int32, ctypes.c_void_p, _P(ValuePlan),
                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "tq_gather_tokens": ([_P(TensorDesc), ctypes.c_void_p, ctypes.c_int32, _P(TensorDesc), ctypes.c_void_p],
                         ctypes.c_int),
    "tq_attention_merge": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                            ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
    "tq_stream_read": ([ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
    "tq_stream_rw": ([ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                      ctypes.c_int32, ctypes.c_void_p], ctypes.c_int),
    "tq_release_cache": ([], ctypes.c_int),
}
for _name, (_args, _res) in _sigs.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res


class TQError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (_lib.tq_status_str(status).decode(), msg))
        self.status = status


def _check(status):
    if status != OK:
        raise TQError(status, _lib.tq_last_error().decode())


def lib():
    return _lib


# ---- host-only calls ---------------------------------------------------------------
def codebook_build(d, bits):
    c = np.zeros(1 << bits, dtype=np.float64)
    t = np.zeros((1 << bits) - 1, dtype=np.float64)
    _check(_lib.tq_codebook_build(d, bits, c.ctypes.data_as(_P(ctypes.c_double)), t.ctypes.data_as(_P(ctypes.c_double))))
    return c, t


def scheme_modes(scheme, n_bits, which):
    m, b = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.tq_scheme_modes(SCHEMES.get(scheme, scheme), n_bits, which, ctypes.byref(m), ctypes.byref(b)))
    return m.value, b.value


def packed_layout(d, mode, bits, side_rank=0, side_bits=0):
    lay = Layout()
    _check(_lib.tq_packed_layout(d, mode, bits, side_rank, side_bits, ctypes.byref(lay)))
    return lay


def rotation_state(seed, d):
    s = np.zeros(d, dtype=np.float32)
    S = np.zeros((d, d), dtype=np.float32)
    _check(_lib.tq_rotation_state(seed, d, s.ctypes.data_as(_P(ctypes.c_float)), S.ctypes.data_as(_P(ctypes.c_float))))
    return s, S


def spectral_fit(calib):
    """(basis [d, d] with the eigenvectors as columns, mean [d], scale [d]),
    float32, of one head's calibration vectors calib [N, d]."""
    calib = np.ascontiguousarray(calib, dtype=np.float32)
    N, d = calib.shape
    V = np.zeros((d, d), dtype=np.float32)
    mu = np.zeros(d, dtype=np.float32)
    sc = np.zeros(d, dtype=np.float32)
    f = _P(ctypes.c_float)
    _check(_lib.tq_spectral_fit(calib.ctypes.data_as(f), N, d, V.ctypes.data_as(f), mu.ctypes.data_as(f),
                                sc.ctypes.data_as(f)))
    return V, mu, sc


def headq_fit(calib, rank):
    calib = np.ascontiguousarray(calib, dtype=np.float32)
    N, d = calib.shape
    U = np.zeros((d, rank), dtype=np.float32)
    _check(_lib.tq_headq_fit(calib.ctypes.data_as(_P(ctypes.c_float)), N, d, rank, U.ctypes.data_as(_P(ctypes.c_float))))
    return U


# ---- device calls ------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def tensor_desc(t):
    """Descriptor of a device tensor shaped [B, H, T, d] (or [B, Hq, d] for
    queries) whose last dimension is contiguous."""
    torch = _torch()
    if t.dim() == 3:
        t = t.unsqueeze(2)
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected [B, H, T, d] with a contiguous last dimension")
    if t.dtype == torch.float16:
        dt = F16
    elif t.dtype == torch.float32:
        dt = F32
    else:
        raise ValueError("dtype must be float16 or float32")
    B, H, T, d = t.shape
    return TensorDesc(t.data_ptr(), dt, B, H, T, d, t.stride(0), t.stride(1), t.stride(2)), t


class PackedTensor:
    """Device planes of one packed tensor (K or V) plus its C descriptor.
    The planes are torch tensors owned by this object."""

    def __init__(self, B, H, T_cap, d, mode, bits, side_rank=0, side_bits=0, device="cuda"):
        torch = _torch()
        lay = packed_layout(d, mode, bits, side_rank, side_bits)
        n = B * H * T_cap
        self.layout = lay

        def plane(nbytes):
            # 16-byte aligned (torch allocations are 256-byte aligned).
            return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)

        self.codes = plane(n * lay.code_bytes)
        self.norms = plane(n * 4)
        self.qjl = None   # PROD keeps its sign bits in the code fields (qjl_bytes is 0)
        self.gamma = plane(n * 4) if lay.has_gamma else None
        self.side = plane(n * lay.side_bytes) if lay.side_bytes else None
        self.side_scale = plane(n * 4) if lay.has_side_scale else None
        self.basis = None
        self.spectral = None
        self.c = Packed()
        self.c.T_cap = T_cap
        self.c.codes = self.codes.data_ptr()
        self.c.norms = self.norms.data_ptr()
        self.c.qjl = None
        self.c.gamma = self.gamma.data_ptr() if self.gamma is not None else None
        self.c.side = self.side.data_ptr() if self.side is not None else None
        self.c.side_scale = self.side_scale.data_ptr() if self.side_scale is not None else None

    def head_view(self, b, h):
        """A descriptor of the single (b, h) slice of this cache (B = H = 1),
        pointing into the same planes."""
        v = PackedTensor.__new__(PackedTensor)
        v.layout = self.layout
        v.basis = self.basis
        v.spectral = self.spectral
        v.c = Packed()
        ctypes.pointer(v.c)[0] = self.c
        v.c.B, v.c.H = 1, 1
        off = (b * self.c.H + h) * self.c.T_cap
        lay = self.layout
        v.c.codes = self.c.codes + off * lay.code_bytes
        v.c.norms = self.c.norms + off * 4
        if self.c.gamma:
            v.c.gamma = self.c.gamma + off * 4
        if self.c.side:
            v.c.side = self.c.side + off * lay.side_bytes
            v.c.side_scale = self.c.side_scale + off * 4
        if self.c.basis and self.c.mode == MODE_SPECTRAL:
            d = self.c.d
            v.c.basis = self.c.basis + h * d * d * 4
            v.c.mean = self.c.mean + h * d * 4
            v.c.scale = self.c.scale + h * d * 4
        elif self.c.basis:
            d, r = self.c.d, self.c.side_rank
            v.c.basis = self.c.basis + h * d * r * 4
        v._parent = self
        return v

    @property
    def n(self):
        return self.c.B * self.c.H * self.c.T_cap

    def planes(self):
        """Host copies (numpy) of the planes, shaped per vector."""
        n = self.n
        out = {"codes": self.codes[: n * self.layout.code_bytes].cpu().numpy().reshape(n, -1),
               "norms": self.norms[: n * 4].cpu().numpy().view(np.float32).copy()}
        if self.gamma is not None:
            out["gamma"] = self.gamma[: n * 4].cpu().numpy().view(np.float32).copy()
        if self.side is not None:
            out["side"] = self.side[: n * self.layout.side_bytes].cpu().numpy().reshape(n, -1)
            out["side_scale"] = self.side_scale[: n * 4].cpu().numpy().view(np.float32).copy()
        return out


def _check_basis(basis, x, H, d):
    """The ABI reads the HeadQ basis as a dense float32 [H][d][rank] array at
    basis.data_ptr(): refuse anything else (a strided view would be read in
    the wrong order)."""
    torch = _torch()
    if basis is None:
        raise ValueError("HeadQ keys need a basis [H, d, rank]")
    if basis.dtype != torch.float32 or basis.dim() != 3 or tuple(basis.shape[:2]) != (H, d):
        raise ValueError("HeadQ basis must be float32 [H=%d, d=%d, rank], got %s %s"
                         % (H, d, basis.dtype, tuple(basis.shape)))
    if not basis.is_contiguous():
        raise ValueError("HeadQ basis must be contiguous (dense [H][d][rank]); pass basis.contiguous()")
    if basis.device != x.device:
        raise ValueError("HeadQ basis must be on the input's device (%s, got %s)" % (x.device, basis.device))


def _check_spectral(spectral, x, H, d):
    """The ABI reads the SPECTRAL state as dense float32 arrays on the input's
    device: basis [H][d][d] (V[h][k][i], eigenvector i in column i), mean and
    scale [H][d]."""
    torch = _torch()
    if spectral is None or len(spectral) != 3:
        raise ValueError("SPECTRAL needs spectral=(basis [H, d, d], mean [H, d], scale [H, d])")
    for t, shape, name in zip(spectral, [(H, d, d), (H, d), (H, d)], ["basis", "mean", "scale"]):
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError("SPECTRAL %s must be contiguous float32 %s, got %s %s"
                             % (name, shape, t.dtype, tuple(t.shape)))
        if t.device != x.device:
            raise ValueError("SPECTRAL %s must be on the input's device (%s, got %s)" % (name, x.device, t.device))


def _override(mode, bits):
    """The per-tensor (mode, index bits) override, or None for the preset."""
    if mode is None and bits is None:
        return None
    if mode is None or bits is None:
        raise ValueError("a per-tensor override needs both mode and bits")
    return ModeOverride(mode, bits)


def quantize(x, which, scheme, n_bits, seed=0, basis=None, rank=16, side_bits=4, T_cap=None, mode=None, bits=None,
             spectral=None):
    """Quantise x [B, H, T, d] (device, fp16/fp32) into a new PackedTensor.
    The tensor's (mode, index bits) come from (scheme, n_bits, which), or
    from `mode` and `bits` when both are given (per-tensor override).
    HEADQ takes `basis` [H, d, rank]; SPECTRAL takes `spectral` = (basis
    [H, d, d], mean [H, d], scale [H, d]), device float32."""
    desc, x4 = tensor_desc(x)
    ovr = _override(mode, bits)
    if ovr is None:
        mode, bits = scheme_modes(scheme, n_bits, which)
    hq = None
    if mode == MODE_HEADQ:
        _check_basis(basis, x, desc.H, desc.d)
        rank = basis.shape[-1]
        hq = HeadQ(basis.data_ptr(), rank, side_bits)
    pt = PackedTensor(desc.B, desc.H, T_cap or desc.T, desc.d, mode, bits,
                      rank if hq else 0, side_bits if hq else 0, device=x.device)
    pt.basis = basis
    if mode == MODE_SPECTRAL:
        _check_spectral(spectral, x, desc.H, desc.d)
        pt.spectral = tuple(spectral)
        pt.c.basis, pt.c.mean, pt.c.scale = (t.data_ptr() for t in spectral)
    _check(_lib.tq_quantize(ctypes.byref(desc), which, SCHEMES.get(scheme, scheme), n_bits, seed,
                            ctypes.byref(ovr) if ovr else None, ctypes.byref(hq) if hq else None,
                            ctypes.byref(pt.c), _stream()))
    pt._keep = x4
    return pt


def _check_index_vector(v, B, like, what):
    """Positions and lengths are read by the kernels as dense int32 [B] on the
    device: refuse anything else."""
    torch = _torch()
    if v is None or v.dtype != torch.int32 or v.dim() != 1 or v.shape[0] != B or not v.is_contiguous():
        raise ValueError("%s must be a contiguous int32 tensor of shape [%d]" % (what, B))
    if v.device != like.device:
        raise ValueError("%s must be on %s (got %s)" % (what, like.device, v.device))


def quantize_append(x, which, scheme, n_bits, pos, cache, seed=0, mode=None, bits=None):
    """Quantise the new tokens x [B, H, Tn, d] and write token t of sequence b
    at slot pos[b] + t of the PackedTensor `cache` (same scheme or override,
    bits and seed as it was written with).  cache.c.T is left as is."""
    desc, x4 = tensor_desc(x)
    ovr = _override(mode, bits)
    _check_index_vector(pos, desc.B, x, "pos")
    hq = None
    if cache.c.mode == MODE_HEADQ:
        hq = HeadQ(cache.c.basis, cache.c.side_rank, cache.c.side_bits)
    _check(_lib.tq_quantize_append(ctypes.byref(desc), which, SCHEMES.get(scheme, scheme), n_bits, seed,
                                   ctypes.byref(ovr) if ovr else None, ctypes.byref(hq) if hq else None,
                                   pos.data_ptr(), ctypes.byref(cache.c), _stream()))
    cache._keep_append = (x4, pos)


def decode_workspace_size(kp, vp, Hq):
    n = ctypes.c_size_t()
    _check(_lib.tq_decode_workspace_size(ctypes.byref(kp.c), ctypes.byref(vp.c), Hq, ctypes.byref(n)))
    return n.value


def decode_attention(q, kp, vp, out=None, lse=None, ws=None, lens=None):
    """out [B, Hq, d] fp32 = softmax attention of q [B, Hq, d] over the packed
    cache; with lens (device int32 [B]) sequence b attends over its first
    lens[b] tokens.  Returns (out, lse)."""
    torch = _torch()
    desc, q4 = tensor_desc(q)
    B, Hq, d = desc.B, desc.H, desc.d
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = decode_workspace_size(kp, vp, Hq)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if lens is None:
        _check(_lib.tq_decode_attention(ctypes.byref(desc), ctypes.byref(kp.c), ctypes.byref(vp.c), out.data_ptr(),
                                        lse.data_ptr(), ws.data_ptr(), ws.numel(), _stream()))
    else:
        _check_index_vector(lens, B, q, "lens")
        _check(_lib.tq_decode_attention_lens(ctypes.byref(desc), ctypes.byref(kp.c), ctypes.byref(vp.c),
                                             lens.data_ptr(), out.data_ptr(), lse.data_ptr(), ws.data_ptr(),
                                             ws.numel(), _stream()))
    return out, lse


def decode_attention_static(q, kp, vp, out, lse=None, lens=None):
    """decode_attention into the caller's out [B, Hq, d] fp32 (and lse
    [B, Hq]) with the library's static workspace: allocates nothing."""
    desc, q4 = tensor_desc(q)
    if lens is not None:
        _check_index_vector(lens, desc.B, q, "lens")
    _check(_lib.tq_decode_attention_static(ctypes.byref(desc), ctypes.byref(kp.c), ctypes.byref(vp.c),
                                           lens.data_ptr() if lens is not None else None, out.data_ptr(),
                                           lse.data_ptr() if lse is not None else None, _stream()))
    return out, lse


def metrics(q=None, k_ref=None, v_ref=None, kp=None, vp=None):
    """Quality measures (synchronous).  Returns a dict."""
    torch = _torch()
    dq = tensor_desc(q)[0] if q is not None else None
    dk = tensor_desc(k_ref)[0] if k_ref is not None else None
    dv = tensor_desc(v_ref)[0] if v_ref is not None else None
    n = ctypes.c_size_t()
    _check(_lib.tq_metrics_workspace_size(ctypes.byref(dq) if dq else None, ctypes.byref(kp.c) if kp else None,
                                          ctypes.byref(vp.c) if vp else None, ctypes.byref(n)))
    dev = (q if q is not None else (k_ref if k_ref is not None else v_ref)).device
    ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device=dev)
    res = MetricsOut()
    _check(_lib.tq_metrics(ctypes.byref(dq) if dq else None, ctypes.byref(dk) if dk else None,
                           ctypes.byref(dv) if dv else None, ctypes.byref(kp.c) if kp else None,
                           ctypes.byref(vp.c) if vp else None, ctypes.byref(res), ws.data_ptr(), ws.numel(),
                           _stream()))
    return {f: getattr(res, f) for f, _ in MetricsOut._fields_}


def stream_read(buf, sink):
    """Stream-read the device tensor `buf` (non-temporal 128-bit loads)."""
    _check(_lib.tq_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), _stream()))


def stream_rw(src, rows, in_row_bytes, dst, out_row_bytes, planes=None, nplanes=0):
    """The write side's traffic with no arithmetic: per row, read in_row_bytes
    of the device tensor `src`, write out_row_bytes of `dst` and one float to
    each of `nplanes` planes of `planes` ([nplanes][rows] float32)."""
    _check(_lib.tq_stream_rw(src.data_ptr(), rows, in_row_bytes, dst.data_ptr(), out_row_bytes,
                             planes.data_ptr() if planes is not None else None, nplanes, _stream()))


def release_cache():
    _check(_lib.tq_release_cache())


# ---- A^2-weighted value policy ------------------------------------------------------
def a2_weights(q_probe, k):
    """A [B, H, T] fp32: per token, the mean over the probe queries of its KV
    head of the squared attention probability.  q_probe [B, Hq, Np, d], k
    [B, H, T, d] (device)."""
    torch = _torch()
    dq, q4 = tensor_desc(q_probe)
    dk, k4 = tensor_desc(k)
    n = ctypes.c_size_t()
    _check(_lib.tq_a2_workspace_size(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(n)))
    ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device=k.device)
    w = torch.empty((dk.B, dk.H, dk.T), dtype=torch.float32, device=k.device)
    _check(_lib.tq_a2_weights(ctypes.byref(dq), ctypes.byref(dk), w.data_ptr(), ws.data_ptr(), ws.numel(), _stream()))
    return w


def value_policy(weights, v, budget_bits):
    """(perm [B, H, T] int32, plan dict) of the two-tier value policy."""
    torch = _torch()
    dv, v4 = tensor_desc(v)
    if weights.dtype != torch.float32 or tuple(weights.shape) != (dv.B, dv.H, dv.T) or not weights.is_contiguous():
        raise ValueError("weights must be contiguous float32 [B, H, T]")
    n = ctypes.c_size_t()
    _check(_lib.tq_value_policy_workspace_size(ctypes.byref(dv), ctypes.byref(n)))
    ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device=v.device)
    perm = torch.empty((dv.B, dv.H, dv.T), dtype=torch.int32, device=v.device)
    plan = ValuePlan()
    _check(_lib.tq_value_policy(weights.data_ptr(), ctypes.byref(dv), budget_bits, perm.data_ptr(),
                                ctypes.byref(plan), ws.data_ptr(), ws.numel(), _stream()))
    k = plan.n_candidates
    return perm, {"b_lo": plan.b_lo, "b_hi": plan.b_hi, "n_high": plan.n_high,
                  "candidates": [(plan.cand_lo[i], plan.cand_hi[i], plan.cand_high[i]) for i in range(k)],
                  "surrogate": [plan.surrogate[i] for i in range(k)]}


def gather_tokens(x, perm, t0, tn):
    """x[b, h, perm[b, h, t0 + t]] for t < tn, as a new [B, H, tn, d] tensor."""
    torch = _torch()
    dx, x4 = tensor_desc(x)
    if perm.dtype != torch.int32 or tuple(perm.shape) != (dx.B, dx.H, dx.T) or not perm.is_contiguous():
        raise ValueError("perm must be contiguous int32 [B, H, T]")
    out = torch.empty((dx.B, dx.H, tn, dx.d), dtype=x.dtype, device=x.device)
    do, _ = tensor_desc(out)
    _check(_lib.tq_gather_tokens(ctypes.byref(dx), perm.data_ptr(), t0, ctypes.byref(do), _stream()))
    return out


def attention_merge(out_a, lse_a, out_b, lse_b):
    """Attention over the union of two disjoint token sets."""
    torch = _torch()
    for t in (out_a, lse_a, out_b, lse_b):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("merge operands must be contiguous float32")
    d = out_a.shape[-1]
    n = out_a.numel() // d
    out = torch.empty_like(out_a)
    lse = torch.empty_like(lse_a)
    _check(_lib.tq_attention_merge(out_a.data_ptr(), lse_a.data_ptr(), out_b.data_ptr(), lse_b.data_ptr(), n, d,
                                   out.data_ptr(), lse.data_ptr(), _stream()))
    return out, lse


class TwoTierCache:
    """A packed cache under the A^2-weighted value policy: the tokens of each
    (batch, head) permuted (high tier first), keys quantised with their own
    scheme over both tiers, values at the plan's two widths (TQ-MSE)."""

    def __init__(self, q_probe, K, V, key_scheme, budget_bits, seed=0, key_bits=None, basis=None, side_bits=4):
        self.weights = a2_weights(q_probe, K)
        self.perm, self.plan = value_policy(self.weights, V, budget_bits)
        T = K.shape[2]
        R = self.plan["n_high"]
        kb = budget_bits if key_bits is None else key_bits
        self.tiers = []
        for t0, tn, vbits in ((0, R, self.plan["b_hi"]), (R, T - R, self.plan["b_lo"])):
            if tn == 0:
                continue
            Kt = gather_tokens(K, self.perm, t0, tn)
            Vt = gather_tokens(V, self.perm, t0, tn)
            kp = quantize(Kt, KEYS, key_scheme, kb, seed, basis=basis, side_bits=side_bits)
            vp = quantize(Vt, VALUES, key_scheme, kb, seed, mode=MODE_MSE, bits=vbits)
            self.tiers.append((kp, vp))

    def decode(self, q):
        outs = [decode_attention(q, kp, vp) for kp, vp in self.tiers]
        if len(outs) == 1:
            return outs[0]
        return attention_merge(outs[0][0], outs[0][1], outs[1][0], outs[1][1])
