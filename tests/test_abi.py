"""Host-side checks of libfavor that need no GPU.

* The library loads and exports every entry point declared in include/favor.h.
* Argument checks return their documented status before anything is launched
  (the pointers passed here are never dereferenced: each call fails its checks).
* The host Omega generator reproduces the oracle's Omega bit for bit (two
  independent implementations of one recipe; Performer section 2.4, appendix B.2).
"""
import ctypes
import os
import re

import numpy as np
import torch
import pytest

import oracle
import random_feature_amd as rf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "favor.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced by the checks under test
MISALIGNED = ctypes.c_void_p(0x10008)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:favor_status|size_t|int|const char\*)\s+(favor_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) == 21
    lib = ctypes.CDLL(rf.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(rf.EXPORTED) == names


def test_status_strings():
    for code in range(5):
        assert rf._lib.favor_status_string(code)
    assert rf._lib.favor_status_string(99) == b"unknown status"


def _bidir(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, om=FAKE, B=1, H=1, L=64, d=64, dv=64, m=256, dt=1, kind=0, eps=0.0, of=0,
             out=FAKE, ws=FAKE, wsb=1 << 30, st=None)
    a.update(kw)
    return rf.raw_call("favor_bidir", a["q"], a["k"], a["v"], a["om"], a["B"], a["H"], a["L"], a["d"], a["dv"],
                       a["m"], a["dt"], a["kind"], ctypes.c_float(a["eps"]), a["of"], a["out"], a["ws"],
                       ctypes.c_size_t(a["wsb"]), a["st"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID),
    (dict(out=None), INVALID),
    (dict(ws=None), INVALID),
    (dict(v=MISALIGNED), INVALID),
    (dict(L=0), INVALID),
    (dict(B=-1), INVALID),
    (dict(dt=7), INVALID),
    (dict(kind=5), INVALID),
    (dict(eps=-1.0), INVALID),
    (dict(eps=float("nan")), INVALID),
    (dict(d=48), UNSUPPORTED),
    (dict(m=200), UNSUPPORTED),
    (dict(dv=24), UNSUPPORTED),
    (dict(wsb=16), WORKSPACE),
])
def test_bidir_argument_checks(kw, status):
    assert _bidir(**kw) == status


def test_causal_argument_checks():
    def call(S=None, z=None, wsb=1 << 30, d=64, kind=0):
        return rf.raw_call("favor_causal", FAKE, FAKE, FAKE, FAKE, 1, 1, 64, d, d, 256, 1, kind, ctypes.c_float(0.0),
                           0, FAKE, S, z, FAKE, ctypes.c_size_t(wsb), None)
    assert call(S=FAKE, z=None) == INVALID          # both or neither
    assert call(wsb=8) == WORKSPACE
    assert call(d=48) == UNSUPPORTED
    assert call(kind=2, wsb=8) == WORKSPACE    # trigonometric features: accepted up to the workspace check
    assert call(kind=2, S=FAKE, z=FAKE) == UNSUPPORTED  # but no canonical final state for them


def test_trig_argument_checks():
    def cross(renorm=1, m=256):
        return rf.raw_call("favor_bidir_cross", FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, 64, 64, m, 1, 2,
                           ctypes.c_float(0.0), renorm, 0, FAKE, FAKE, ctypes.c_size_t(8), None)
    assert cross() == WORKSPACE                 # accepted up to the workspace check
    assert cross(renorm=0) == UNSUPPORTED       # no canonical scale for the trigonometric map
    assert rf.raw_call("favor_make_omega_host", ctypes.c_uint64(0), 1, 33, 16, 4, FAKE) == INVALID


def test_decode_argument_checks():
    def call(N=4, H=2, d=64, dv=64, m=256, q=FAKE, S=FAKE):
        return rf.raw_call("favor_decode", q, FAKE, FAKE, FAKE, S, FAKE, N, H, d, dv, m, 1, 0, ctypes.c_float(0.0),
                           FAKE, None)
    assert call(q=None) == INVALID
    assert call(S=MISALIGNED) == INVALID
    assert call(N=0) == INVALID
    assert call(d=128) == UNSUPPORTED
    assert call(dv=40) == UNSUPPORTED   # value widths: multiples of 16 up to 256
    assert call(dv=272) == UNSUPPORTED
    assert call(m=100) == UNSUPPORTED


def test_decode_gated_argument_checks():
    def call(gate=FAKE, inw=None, q=FAKE, d=64):
        return rf.raw_call("favor_decode_gated", q, FAKE, FAKE, FAKE, FAKE, FAKE, gate, inw, 4, 2, d, 64, 256, 1, 0,
                           ctypes.c_float(0.0), FAKE, None)
    assert call(gate=None) == INVALID
    assert call(gate=ctypes.c_void_p(0x10002)) == INVALID
    assert call(inw=ctypes.c_void_p(0x10001)) == INVALID
    assert call(q=None) == INVALID
    assert call(d=128) == UNSUPPORTED


@pytest.mark.parametrize("fn,wsfn", [("favor_bidir_backward", "favor_backward_workspace_size"),
                                     ("favor_causal_backward", "favor_causal_backward_workspace_size")])
def test_backward_argument_checks(fn, wsfn):
    def call(kind=0, d=64, dv=64, m=256, wsb=1 << 30, q=FAKE, eps=0.0):
        return rf.raw_call(fn, q, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, d, dv, m, 1, kind, ctypes.c_float(eps), 0, FAKE,
                           FAKE, FAKE, FAKE, ctypes.c_size_t(wsb), None)
    assert call(q=None) == INVALID
    assert call(kind=1, eps=-1.0) == INVALID
    assert call(kind=2) == UNSUPPORTED          # the trigonometric features have no backward kernels
    assert call(d=16, dv=16, m=256) == UNSUPPORTED
    assert call(wsb=8) == WORKSPACE
    assert getattr(rf._lib, wsfn)(1, 1, 64, 64, 64, 256, 1) > 0
    assert getattr(rf._lib, wsfn)(0, 1, 64, 64, 64, 256, 1) == 0


def test_features_and_omega_argument_checks():
    st = rf.raw_call("favor_features", FAKE, FAKE, 1, 1, 8, 48, 64, 1, 0, ctypes.c_float(0.0), FAKE, FAKE, None)
    assert st == UNSUPPORTED
    assert rf.raw_call("favor_make_omega", ctypes.c_uint64(0), 1, 16, 16, 0, None, None) == INVALID
    # the hyperbolic mode pairs every row with its negative: m must be even
    assert rf.raw_call("favor_make_omega_host", ctypes.c_uint64(0), 1, 33, 16, 3, FAKE) == INVALID
    assert rf.raw_call("favor_make_omega", ctypes.c_uint64(0), 1, 33, 16, 3, FAKE, None) == INVALID
    assert rf.raw_call("favor_make_omega", ctypes.c_uint64(0), 1, 16, 16, 9, FAKE, None) == INVALID
    assert rf.raw_call("favor_make_omega_host", ctypes.c_uint64(0), 0, 16, 16, 0, FAKE) == INVALID


def test_workspace_size_query():
    assert rf.workspace_size(False, 8, 12, 4096, 64, 64, 256, __import__("torch").bfloat16) > 0
    assert rf.workspace_size(True, 4, 8, 8192, 64, 64, 256, __import__("torch").bfloat16) > 0
    assert rf._lib.favor_workspace_size(0, 1, 1, 16, 48, 48, 64, 1) == 0      # unsupported -> 0
    assert rf._lib.favor_workspace_size(0, 0, 1, 16, 64, 64, 64, 1) == 0      # invalid -> 0


@pytest.mark.parametrize("seed,H,m,d,mode", [
    (0, 1, 32, 16, "ortho_chi"),
    (1, 8, 128, 16, "ortho_chi"),
    (2, 3, 256, 64, "ortho_chi"),
    (3, 2, 40, 16, "ortho_chi"),
    (4, 2, 96, 32, "ortho_sqrtd"),
    (6, 3, 128, 64, "hyperbolic"),
    (7, 2, 64, 16, "trig_pairs"),
    (5, 2, 48, 16, "iid"),
    (2 ** 64 - 1, 1, 64, 64, "ortho_chi"),
    (12345678901234, 1, 20, 7, "ortho_chi"),
])
def test_host_omega_bit_exact_against_oracle(seed, H, m, d, mode):
    lib_om = rf.make_omega_host(seed, H, m, d, mode)
    ref = oracle.make_omega(seed, H, m, d, mode)
    assert lib_om.dtype == np.float32 and lib_om.shape == (H, m, d)
    assert np.array_equal(lib_om.view(np.uint32), ref.view(np.uint32))


def test_host_omega_head_rows_independent_of_H():
    a = rf.make_omega_host(9, 2, 64, 16)
    b = rf.make_omega_host(9, 5, 64, 16)
    assert np.array_equal(a, b[:2])


def test_prepared_omega_checks():
    """favor_omega_prepare and the prepared calls check their arguments before any launch: the prepared size is
    the workspace's fragment area; a short buffer is FAVOR_ERR_WORKSPACE; the prepared calls check `prep` as
    favor_bidir and favor_causal check omega."""
    n = rf._lib.favor_omega_prepared_size(12, 64, 64, 256, 1)
    assert n == 12 * 16 * 2 * 512 * 2  # H * (m/16) * (d/32) * 512 fragments' 2-byte elements
    assert rf._lib.favor_omega_prepared_size(12, 48, 64, 256, 1) == 0   # d outside the built set
    assert rf._lib.favor_omega_prepared_size(0, 64, 64, 256, 1) == 0

    def prep_call(om=FAKE, prep=FAKE, nbytes=n, kind=0, d=64, m=256):
        return rf.raw_call("favor_omega_prepare", om, 12, d, 64, m, 1, kind, prep, ctypes.c_size_t(nbytes), None)
    assert prep_call(om=None) == INVALID
    assert prep_call(prep=MISALIGNED) == INVALID
    assert prep_call(nbytes=n - 1) == WORKSPACE
    assert prep_call(d=48) == UNSUPPORTED
    assert prep_call(kind=2, m=160) == UNSUPPORTED  # trigonometric features: exact shapes only

    def call(fn, prep=FAKE, ws=FAKE, wsb=1 << 30):
        extra = (FAKE, FAKE) if fn == "favor_causal_prepared" else ()
        return rf.raw_call(fn, FAKE, FAKE, FAKE, prep, 1, 12, 64, 64, 64, 256, 1, 0, ctypes.c_float(0.0), 0, FAKE,
                           *extra, ws, ctypes.c_size_t(wsb), None)
    for fn in ("favor_bidir_prepared", "favor_causal_prepared"):
        assert call(fn, prep=None) == INVALID
        assert call(fn, prep=MISALIGNED) == INVALID
        assert call(fn, wsb=8) == WORKSPACE


def test_bidir_noalloc_checks_before_any_device_call():
    """favor_bidir_noalloc takes favor_bidir's checks, and refuses a workspace beyond its array
    (FAVOR_BIDIR_NOALLOC_MAX_BYTES) before it touches the device."""
    def call(**kw):
        a = dict(q=FAKE, out=FAKE, B=1, H=1, L=64, d=64, dv=64, m=256, dt=1)
        a.update(kw)
        return rf.raw_call("favor_bidir_noalloc", a["q"], FAKE, FAKE, FAKE, a["B"], a["H"], a["L"], a["d"], a["dv"],
                           a["m"], a["dt"], 0, ctypes.c_float(0.0), 0, a["out"], None)
    assert call(q=None) == INVALID
    assert call(out=MISALIGNED) == INVALID
    assert call(d=48) == UNSUPPORTED
    big = dict(B=64, H=16, L=4096)
    assert rf.workspace_size(False, 64, 16, 4096, 64, 64, 256, torch.bfloat16) > rf.NOALLOC_MAX_BYTES
    assert call(**big) == WORKSPACE
    # the headline workload's workspace fits
    assert rf.workspace_size(False, 8, 12, 4096, 64, 64, 256, torch.bfloat16) <= rf.NOALLOC_MAX_BYTES


@pytest.mark.parametrize("d,dv,m,dt,status", [
    (128, 256, 512, 1, OK), (64, 208, 240, 1, OK), (16, 48, 16, 1, OK), (32, 80, 96, 0, OK), (64, 256, 256, 0, OK),
    (128, 64, 64, 0, UNSUPPORTED),   # fp32: d <= 64 and m <= 256 outside the exact shapes
    (64, 64, 512, 0, UNSUPPORTED),
    (16, 16, 16, 0, OK),             # an exact shape
    (64, 64, 528, 1, UNSUPPORTED), (64, 272, 64, 1, UNSUPPORTED), (48, 64, 64, 1, UNSUPPORTED),
    (64, 40, 64, 1, UNSUPPORTED), (64, 64, 72, 1, UNSUPPORTED),
])
def test_shape_set(d, dv, m, dt, status):
    """The sequence entry points take d in {16, 32, 64, 128}, dv and m multiples of 16 up to 256 and 512 (fp32: d <= 64
    and m <= 256 outside the exact shapes): a supported shape has a workspace size and passes every check (it fails
    only on the workspace size given here); others return FAVOR_ERR_UNSUPPORTED."""
    n = rf._lib.favor_workspace_size(0, 2, 3, 100, d, dv, m, dt)
    assert (n > 0) == (status == OK)
    got = _bidir(d=d, dv=dv, m=m, dt=dt, wsb=16)
    assert got == (WORKSPACE if status == OK else status)
    c = rf.raw_call("favor_causal", FAKE, FAKE, FAKE, FAKE, 2, 3, 100, d, dv, m, dt, 0, ctypes.c_float(0.0), 0, FAKE,
                    None, None, FAKE, ctypes.c_size_t(16), None)
    assert c == (WORKSPACE if status == OK else status)


def test_trig_only_on_exact_shapes():
    assert _bidir(d=64, dv=64, m=256, kind=2, wsb=16) == WORKSPACE
    assert _bidir(d=64, dv=128, m=256, kind=2, wsb=16) == UNSUPPORTED

    def causal(dv, m):
        return rf.raw_call("favor_causal", FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 64, dv, m, 1, 2, ctypes.c_float(0.0), 0,
                           FAKE, None, None, FAKE, ctypes.c_size_t(16), None)
    assert causal(64, 256) == WORKSPACE
    assert causal(128, 256) == UNSUPPORTED

