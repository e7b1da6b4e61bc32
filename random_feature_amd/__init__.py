"""random_feature_amd — FAVOR+ random-feature attention on MI355X (gfx950).

A thin ctypes binding over the C ABI of `libfavor.so` (declared in
include/favor.h). Every step of the computation runs in the library's HIP
kernels; this module only checks tensors, passes device pointers, sizes and
the current HIP stream, and allocates outputs/workspace with torch.

The library must be built first (`python random_feature_amd/build.py`, or
`__graft_entry__.build()`); importing this package without it raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfavor.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libfavor.so not found at {LIB_PATH}: build it with `python random_feature_amd/build.py` "
        "(there is no fallback implementation)")

_lib = ctypes.CDLL(LIB_PATH)

F32, BF16 = 0, 1
PRF, RELU, TRIG = 0, 1, 2
OMEGA_MODES = {"ortho_chi": 0, "iid": 1, "ortho_sqrtd": 2, "hyperbolic": 3, "trig_pairs": 4}
KINDS = {"prf": PRF, "relu": RELU, "trig": TRIG}
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "hip error"}

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

_lib.favor_make_omega.argtypes = [ctypes.c_uint64, _i, _i, _i, _i, _vp, _vp]
_lib.favor_make_omega_host.argtypes = [ctypes.c_uint64, _i, _i, _i, _i, _vp]
_lib.favor_features.argtypes = [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp]
_lib.favor_bidir.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _vp, _sz, _vp]
_lib.favor_bidir_noalloc.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _vp]
_lib.favor_bidir_cross.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp, _vp, _sz,
                                   _vp]
_lib.favor_causal.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp, _vp,
                              _sz, _vp]
_lib.favor_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp]
_lib.favor_decode_gated.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp]
_lib.favor_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i]
_lib.favor_omega_prepared_size.argtypes = [_i, _i, _i, _i, _i]
_lib.favor_omega_prepared_size.restype = _sz
_lib.favor_omega_prepare.argtypes = [_vp, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]
_lib.favor_bidir_prepared.argtypes = _lib.favor_bidir.argtypes
_lib.favor_causal_prepared.argtypes = _lib.favor_causal.argtypes
_lib.favor_bidir_backward.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _vp,
                                      _vp, _vp, _sz, _vp]
_lib.favor_backward_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i, _i]
_lib.favor_backward_workspace_size.restype = _sz
_lib.favor_causal_backward.argtypes = _lib.favor_bidir_backward.argtypes
_lib.favor_causal_backward_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i, _i]
_lib.favor_causal_backward_workspace_size.restype = _sz
_lib.favor_workspace_size.restype = _sz
_lib.favor_timing_enable.argtypes = [_i]
_lib.favor_timing_enable.restype = _i
_lib.favor_timing_read.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float), _i]
_lib.favor_timing_read.restype = _i
_lib.favor_status_string.argtypes = [_i]
_lib.favor_status_string.restype = ctypes.c_char_p
for _fn in ("favor_make_omega", "favor_make_omega_host", "favor_features", "favor_bidir", "favor_bidir_noalloc",
            "favor_bidir_cross",
            "favor_bidir_backward", "favor_causal", "favor_causal_backward", "favor_decode", "favor_decode_gated",
            "favor_omega_prepare", "favor_bidir_prepared", "favor_causal_prepared"):
    getattr(_lib, _fn).restype = _i

EXPORTED = ["favor_make_omega", "favor_make_omega_host", "favor_features", "favor_bidir", "favor_bidir_noalloc",
            "favor_bidir_cross",
            "favor_bidir_backward", "favor_backward_workspace_size", "favor_causal", "favor_causal_backward",
            "favor_causal_backward_workspace_size",
            "favor_decode", "favor_decode_gated", "favor_workspace_size", "favor_timing_enable", "favor_timing_read",
            "favor_status_string", "favor_omega_prepared_size", "favor_omega_prepare", "favor_bidir_prepared",
            "favor_causal_prepared"]


class FavorError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {_lib.favor_status_string(status).decode()} (status {status})")


def _check(fn: str, st: int):
    if st != 0:
        raise FavorError(fn, st)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, ndim: int, shape=None, dtype=None):
    """Rank, then (when given) exact shape and dtype, then contiguity of one argument. The C ABI sees only
    pointers and the sizes taken from q, so these checks are what keeps every kernel read and write inside the
    caller's buffers. Device residence is checked after every argument's structure (_resident)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _resident(**named):
    """Every named tensor (None: absent) is a device tensor, all on one device."""
    devs = set()
    for name, t in named.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        devs.add(t.device)
    if len(devs) > 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(map(str, devs))}")


def _check_seq(q, k, v, omega, cross: bool = False, resident: bool = True):
    """q [B,H,Lq,d], k [B,H,Lk,d], v [B,H,Lk,dv] of one dtype (fp32 or bf16), Lq = Lk unless cross;
    omega fp32 [H,m,d]. Returns (B, H, Lq, Lk, d, dv, m)."""
    _need(q, "q", 4)
    _dtype_code(q)
    B, H, Lq, d = q.shape
    _need(k, "k", 4, dtype=q.dtype)
    Lk = k.shape[2]
    if not cross and Lk != Lq:
        raise ValueError(f"k must have the length of q ({Lq}), got {Lk}")
    _need(k, "k", 4, shape=(B, H, Lk, d), dtype=q.dtype)
    _need(v, "v", 4, dtype=q.dtype)
    dv = v.shape[-1]
    _need(v, "v", 4, shape=(B, H, Lk, dv), dtype=q.dtype)
    _need(omega, "omega", 3, dtype=torch.float32)
    m = omega.shape[1]
    _need(omega, "omega", 3, shape=(H, m, d), dtype=torch.float32)
    if resident:
        _resident(q=q, k=k, v=v, omega=omega)
    return B, H, Lq, Lk, d, dv, m


def _check_ws(ws, device, need: int):
    if not isinstance(ws, torch.Tensor) or not ws.is_contiguous() or not ws.is_cuda or ws.device != device:
        raise ValueError("ws must be a contiguous device tensor on the inputs' device")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"ws holds {ws.numel() * ws.element_size()} bytes, {need} needed")
    return ws.numel() * ws.element_size()


def _check_out(out, name, shape, dtype, device):
    _need(out, name, len(shape), shape=shape, dtype=dtype)
    _resident(**{name: out})
    if out.device != device:
        raise ValueError(f"{name} must be on {device}")


def _kind(kind) -> int:
    return KINDS[kind] if isinstance(kind, str) else int(kind)


def make_omega_host(seed: int, H: int, m: int, d: int, mode: str = "ortho_chi"):
    """Omega [H,m,d] fp32 in host memory (numpy), computed by the library's host code."""
    import numpy as np
    out = np.empty((H, m, d), dtype=np.float32)
    _check("favor_make_omega_host",
           _lib.favor_make_omega_host(ctypes.c_uint64(seed & (2 ** 64 - 1)), H, m, d, OMEGA_MODES[mode],
                                      out.ctypes.data_as(ctypes.c_void_p)))
    return out


def make_omega(seed: int, H: int, m: int, d: int, mode: str = "ortho_chi", device="cuda") -> torch.Tensor:
    """Omega [H,m,d] fp32 on the device (built on the host, copied on the current stream)."""
    out = torch.empty((H, m, d), dtype=torch.float32, device=device)
    _check("favor_make_omega",
           _lib.favor_make_omega(ctypes.c_uint64(seed & (2 ** 64 - 1)), H, m, d, OMEGA_MODES[mode], _ptr(out),
                                 ctypes.c_void_p(_stream(out.device))))
    return out


def workspace_size(causal: bool, B, H, L, d, dv, m, dtype: torch.dtype) -> int:
    code = F32 if dtype == torch.float32 else BF16
    return int(_lib.favor_workspace_size(1 if causal else 0, B, H, L, d, dv, m, code))


def workspace(causal: bool, q: torch.Tensor, v: torch.Tensor, omega: torch.Tensor) -> torch.Tensor:
    """Device scratch for bidir()/causal() (k's length for cross attention), reusable across calls of that shape."""
    B, H, L, d = q.shape
    n = workspace_size(causal, B, H, L, d, v.shape[-1], omega.shape[1], q.dtype)
    # 0: arguments the library rejects; the entry point itself then reports which status applies
    return torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)


def backward_workspace(q: torch.Tensor, v: torch.Tensor, omega: torch.Tensor) -> torch.Tensor:
    """Device scratch for bidir_backward() at q's shape (reusable across calls of that shape)."""
    B, H, L, d = q.shape
    n = int(_lib.favor_backward_workspace_size(B, H, L, d, v.shape[-1], omega.shape[1], _dtype_code(q)))
    if n == 0:
        raise FavorError("favor_backward_workspace_size", 1)
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def causal_backward_workspace(q: torch.Tensor, v: torch.Tensor, omega: torch.Tensor) -> torch.Tensor:
    """Device scratch for causal_backward() at q's shape (reusable across calls of that shape)."""
    B, H, L, d = q.shape
    n = int(_lib.favor_causal_backward_workspace_size(B, H, L, d, v.shape[-1], omega.shape[1], _dtype_code(q)))
    if n == 0:
        raise FavorError("favor_causal_backward_workspace_size", 1)
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def features(x: torch.Tensor, omega: torch.Tensor, kind="prf", eps: float = 0.0):
    """phi [B,H,L,m] and logscale [B,H,L] with phi_true = phi * exp(logscale)."""
    _need(x, "x", 4)
    _dtype_code(x)
    B, H, L, d = x.shape
    _need(omega, "omega", 3, dtype=torch.float32)
    m = omega.shape[1]
    _need(omega, "omega", 3, shape=(H, m, d), dtype=torch.float32)
    _resident(x=x, omega=omega)
    phi = torch.empty((B, H, L, m), dtype=torch.float32, device=x.device)
    ls = torch.empty((B, H, L), dtype=torch.float32, device=x.device)
    _check("favor_features",
           _lib.favor_features(_ptr(x), _ptr(omega), B, H, L, d, m, _dtype_code(x), _kind(kind), float(eps),
                               _ptr(phi), _ptr(ls), ctypes.c_void_p(_stream(x.device))))
    return phi, ls


class PreparedOmega:
    """Omega' fragments written by favor_omega_prepare for one omega [H,m,d] and (dv, dtype, kind): pass as
    `prep=` to bidir() or causal() with that omega, value width, input dtype and kind (checked here: the library
    itself cannot tell). Valid until omega changes."""

    def __init__(self, buf, H, d, dv, m, dtype, kind):
        self.buf, self.key = buf, (H, d, dv, m, dtype, _kind(kind))

    def check(self, H, d, dv, m, dtype, kind):
        if self.key != (H, d, dv, m, dtype, _kind(kind)):
            raise ValueError(f"prepared omega is for (H, d, dv, m, dtype, kind) = {self.key}, "
                             f"not {(H, d, dv, m, dtype, _kind(kind))}")


def prepare_omega(omega, dv: int, dtype=torch.bfloat16, kind="prf") -> PreparedOmega:
    """favor_omega_prepare: omega [H,m,d] fp32 on the device into the kernels' fragments for value width dv and
    inputs of `dtype`, on the current stream."""
    _need(omega, "omega", 3, dtype=torch.float32)
    _resident(omega=omega)
    H, m, d = omega.shape
    code = {torch.float32: 0, torch.bfloat16: 1}.get(dtype)
    if code is None:
        raise ValueError(f"dtype {dtype}: float32 or bfloat16")
    n = int(_lib.favor_omega_prepared_size(H, d, dv, m, code))
    if n == 0:
        raise FavorError("favor_omega_prepared_size", 2)
    buf = torch.empty(n, dtype=torch.uint8, device=omega.device)
    _check("favor_omega_prepare",
           _lib.favor_omega_prepare(_ptr(omega), H, d, dv, m, code, _kind(kind), _ptr(buf), n,
                                    ctypes.c_void_p(_stream(omega.device))))
    return PreparedOmega(buf, H, d, dv, m, dtype, kind)


def bidir(q, k, v, omega, kind="prf", eps: float = 0.0, out_f32: bool = False, ws=None, out=None, prep=None):
    """Bidirectional FAVOR+ (Performer equation 4). Returns out [B,H,L,dv]. prep: a PreparedOmega of this omega
    (favor_bidir_prepared: no per-call conversion of omega)."""
    _check_seq(q, k, v, omega)
    return bidir_cross(q, k, v, omega, kind=kind, eps=eps, renormalize=True, out_f32=out_f32, ws=ws, out=out,
                       _fn="favor_bidir", _prep=prep)


NOALLOC_MAX_BYTES = 64 << 20  # FAVOR_BIDIR_NOALLOC_MAX_BYTES


def bidir_noalloc(q, k, v, omega, kind="prf", eps: float = 0.0, out_f32: bool = False, out=None):
    """bidir() through favor_bidir_noalloc: the library's own workspace array on the device (no allocation in
    the library; `out` is allocated here unless given). Calls overlapping on one device race."""
    B, H, L, _, d, dv, m = _check_seq(q, k, v, omega)
    odt = torch.float32 if out_f32 else q.dtype
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=odt, device=q.device)
    _check_out(out, "out", (B, H, L, dv), odt, q.device)
    _check("favor_bidir_noalloc",
           _lib.favor_bidir_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(omega), B, H, L, d, dv, m, _dtype_code(q),
                                    _kind(kind), float(eps), 1 if out_f32 else 0, _ptr(out),
                                    ctypes.c_void_p(_stream(q.device))))
    return out


def bidir_cross(q, k, v, omega, kind="prf", eps: float = 0.0, renormalize: bool = True, out_f32: bool = False,
                ws=None, out=None, _fn="favor_bidir_cross", _prep=None):
    """Bidirectional FAVOR+ between q [B,H,Lq,d] and k [B,H,Lk,d], v [B,H,Lk,dv]; without renormalisation the
    output is phi(q).S in canonical feature scale. Returns out [B,H,Lq,dv]."""
    B, H, Lq, Lk, d, dv, m = _check_seq(q, k, v, omega, cross=True)
    need = workspace_size(False, B, H, Lk, d, dv, m, q.dtype)
    if ws is None:
        ws = workspace(False, k, v, omega)
    ws_bytes = _check_ws(ws, q.device, need)
    odt = torch.float32 if out_f32 else q.dtype
    if out is None:
        out = torch.empty((B, H, Lq, dv), dtype=odt, device=q.device)
    _check_out(out, "out", (B, H, Lq, dv), odt, q.device)
    st = ctypes.c_void_p(_stream(q.device))
    if _prep is not None:
        _prep.check(H, d, dv, m, q.dtype, kind)
        _fn = "favor_bidir_prepared"
        r = _lib.favor_bidir_prepared(_ptr(q), _ptr(k), _ptr(v), _ptr(_prep.buf), B, H, Lq, d, dv, m,
                                      _dtype_code(q), _kind(kind), float(eps), 1 if out_f32 else 0, _ptr(out),
                                      _ptr(ws), ws_bytes, st)
    elif _fn == "favor_bidir":
        r = _lib.favor_bidir(_ptr(q), _ptr(k), _ptr(v), _ptr(omega), B, H, Lq, d, dv, m, _dtype_code(q),
                             _kind(kind), float(eps), 1 if out_f32 else 0, _ptr(out), _ptr(ws), ws_bytes, st)
    else:
        r = _lib.favor_bidir_cross(_ptr(q), _ptr(k), _ptr(v), _ptr(omega), B, H, Lq, Lk, d, dv, m, _dtype_code(q),
                                   _kind(kind), float(eps), 1 if renormalize else 0, 1 if out_f32 else 0,
                                   _ptr(out), _ptr(ws), ws_bytes, st)
    _check(_fn, r)
    return out


def bidir_backward(q, k, v, omega, dout, kind="prf", eps: float = 0.0, grad_f32: bool = False, ws=None, out=None):
    """Gradients (dq, dk, dv) of bidir()'s output for the upstream gradient `dout` (the forward sums are
    recomputed; kind "prf" or "relu" with the forward's eps). `out`: optional preallocated (dq, dk, dv)."""
    return _backward("favor_bidir_backward", backward_workspace, q, k, v, omega, dout, kind, eps, grad_f32, ws, out)


def _backward(fn, wsfn, q, k, v, omega, dout, kind, eps, grad_f32, ws, out):
    B, H, L, _, d, dv, m = _check_seq(q, k, v, omega, resident=False)
    _need(dout, "dout", 4, shape=(B, H, L, dv), dtype=q.dtype)
    _resident(q=q, k=k, v=v, omega=omega, dout=dout)
    if ws is None:
        ws = wsfn(q, v, omega)
    sz = (_lib.favor_backward_workspace_size if fn == "favor_bidir_backward"
          else _lib.favor_causal_backward_workspace_size)
    ws_bytes = _check_ws(ws, q.device, int(sz(B, H, L, d, dv, m, _dtype_code(q))))
    gdt = torch.float32 if grad_f32 else q.dtype
    if out is None:
        dq = torch.empty((B, H, L, d), dtype=gdt, device=q.device)
        dk = torch.empty((B, H, L, d), dtype=gdt, device=q.device)
        dvv = torch.empty((B, H, L, dv), dtype=gdt, device=q.device)
    else:
        dq, dk, dvv = out
        for t, n, last in ((dq, "dq", d), (dk, "dk", d), (dvv, "dv", dv)):
            _check_out(t, n, (B, H, L, last), gdt, q.device)
    _check(fn, getattr(_lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(omega), _ptr(dout), B, H, L, d, dv, m,
                                 _dtype_code(q), _kind(kind), float(eps), 1 if grad_f32 else 0, _ptr(dq), _ptr(dk),
                                 _ptr(dvv),
                                 _ptr(ws), ws_bytes, ctypes.c_void_p(_stream(q.device))))
    return dq, dk, dvv


def causal_backward(q, k, v, omega, dout, kind="prf", eps: float = 0.0, grad_f32: bool = False, ws=None, out=None):
    """Gradients (dq, dk, dv) of causal()'s output for the upstream gradient `dout` (the forward is
    recomputed). `out`: optional preallocated (dq, dk, dv)."""
    return _backward("favor_causal_backward", causal_backward_workspace, q, k, v, omega, dout, kind, eps, grad_f32,
                     ws, out)


def causal(q, k, v, omega, kind="prf", eps: float = 0.0, out_f32: bool = False, return_state: bool = False,
           ws=None, out=None, prep=None):
    """Causal FAVOR+ (Performer appendix B.1). Returns out, or (out, S_final, z_final) in canonical scale.
    prep: a PreparedOmega of this omega (favor_causal_prepared)."""
    B, H, L, _, d, dv, m = _check_seq(q, k, v, omega)
    need = workspace_size(True, B, H, L, d, dv, m, q.dtype)
    if ws is None:
        ws = workspace(True, q, v, omega)
    ws_bytes = _check_ws(ws, q.device, need)
    odt = torch.float32 if out_f32 else q.dtype
    if out is None:
        out = torch.empty((B, H, L, dv), dtype=odt, device=q.device)
    _check_out(out, "out", (B, H, L, dv), odt, q.device)
    S = z = None
    if return_state:
        S = torch.empty((B, H, m, dv), dtype=torch.float32, device=q.device)
        z = torch.empty((B, H, m), dtype=torch.float32, device=q.device)
    fn, om = "favor_causal", omega
    if prep is not None:
        prep.check(H, d, dv, m, q.dtype, kind)
        fn, om = "favor_causal_prepared", prep.buf
    _check(fn, getattr(_lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(om), B, H, L, d, dv, m, _dtype_code(q), _kind(kind),
                                 float(eps), 1 if out_f32 else 0, _ptr(out), _ptr(S), _ptr(z), _ptr(ws), ws_bytes,
                                 ctypes.c_void_p(_stream(q.device))))
    return (out, S, z) if return_state else out


def _check_decode(q, k, v, omega, S, z, out):
    """q, k [N,H,d] and v [N,H,dv] of one dtype; omega fp32 [H,m,d]; S fp32 [N,H,m,dv]; z fp32 [N,H,m];
    out fp32 [N,H,dv] if given. Returns (N, H, d, dv, m)."""
    _need(q, "q", 3)
    _dtype_code(q)
    N, H, d = q.shape
    _need(k, "k", 3, shape=(N, H, d), dtype=q.dtype)
    _need(v, "v", 3, dtype=q.dtype)
    dv = v.shape[-1]
    _need(v, "v", 3, shape=(N, H, dv), dtype=q.dtype)
    _need(omega, "omega", 3, dtype=torch.float32)
    m = omega.shape[1]
    _need(omega, "omega", 3, shape=(H, m, d), dtype=torch.float32)
    _need(S, "S", 4, shape=(N, H, m, dv), dtype=torch.float32)
    _need(z, "z", 3, shape=(N, H, m), dtype=torch.float32)
    if out is not None:
        _need(out, "out", 3, shape=(N, H, dv), dtype=torch.float32)
    return N, H, d, dv, m


def decode(q, k, v, omega, S, z, kind="prf", eps: float = 0.0, out=None):
    """One decode step: q,k [N,H,d], v [N,H,dv]; S [N,H,m,dv], z [N,H,m] updated in place. Returns out [N,H,dv]."""
    N, H, d, dv, m = _check_decode(q, k, v, omega, S, z, out)
    _resident(q=q, k=k, v=v, omega=omega, S=S, z=z, out=out)
    if out is None:
        out = torch.empty((N, H, dv), dtype=torch.float32, device=q.device)
    _check("favor_decode",
           _lib.favor_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(omega), _ptr(S), _ptr(z), N, H, d, dv, m,
                             _dtype_code(q), _kind(kind), float(eps), _ptr(out), ctypes.c_void_p(_stream(q.device))))
    return out


def decode_gated(q, k, v, omega, S, z, gate, in_weight=None, kind="prf", eps: float = 0.0, out=None):
    """One gated decode step: S = g S + w phi(k) v^T, z = g z + w phi(k) with gate g and optional input weight w
    (fp32 [N,H], device); otherwise as decode(). Returns out [N,H,dv]."""
    N, H, d, dv, m = _check_decode(q, k, v, omega, S, z, out)
    _need(gate, "gate", 2, shape=(N, H), dtype=torch.float32)
    if in_weight is not None:
        _need(in_weight, "in_weight", 2, shape=(N, H), dtype=torch.float32)
    _resident(q=q, k=k, v=v, omega=omega, S=S, z=z, out=out, gate=gate, in_weight=in_weight)
    if out is None:
        out = torch.empty((N, H, dv), dtype=torch.float32, device=q.device)
    _check("favor_decode_gated",
           _lib.favor_decode_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(omega), _ptr(S), _ptr(z), _ptr(gate),
                                   _ptr(in_weight) if in_weight is not None else None, N, H, d, dv, m,
                                   _dtype_code(q), _kind(kind), float(eps), _ptr(out),
                                   ctypes.c_void_p(_stream(q.device))))
    return out


def timing_enable(on: bool = True) -> None:
    """Start (or stop) recording per-launch kernel durations with HIP events; clears earlier records."""
    _check("favor_timing_enable", _lib.favor_timing_enable(1 if on else 0))


def timing_read():
    """[(kernel name, ms), ...] for every launch recorded since timing_enable(True), in launch order."""
    n = _lib.favor_timing_read(None, None, 0)
    names = (ctypes.c_char_p * max(n, 1))()
    ms = (ctypes.c_float * max(n, 1))()
    n = _lib.favor_timing_read(names, ms, n)
    return [(names[i].decode(), float(ms[i])) for i in range(n)]


def raw_call(name: str, *args) -> int:
    """Call a C entry point with raw ctypes arguments and return its status (for error-path tests)."""
    return int(getattr(_lib, name)(*args))
