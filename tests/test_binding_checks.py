"""The Python binding's argument checks (no GPU needed).

The C ABI receives only pointers and the sizes read from q, so the binding must refuse any tensor whose shape or
dtype disagrees with them before a kernel could read or write outside a buffer. Every case below is built from
host tensors: each must fail on its shape or dtype, before the device-residence check is reached.
"""
import pytest
import torch

import random_feature_amd as rf

F, H16 = torch.float32, torch.bfloat16


def seq(B=2, H=3, L=40, d=16, dv=16, m=32, dtype=H16):
    q = torch.zeros(B, H, L, d, dtype=dtype)
    k = torch.zeros(B, H, L, d, dtype=dtype)
    v = torch.zeros(B, H, L, dv, dtype=dtype)
    om = torch.zeros(H, m, d, dtype=F)
    return q, k, v, om


def expect(msg, fn, *a, **kw):
    with pytest.raises(ValueError, match=msg):
        fn(*a, **kw)


@pytest.mark.parametrize("fn", [rf.bidir, rf.causal])
def test_sequence_inputs_must_agree_with_q(fn):
    q, k, v, om = seq()
    expect("k must have the length of q", fn, q, k[:, :, :39].contiguous(), v, om)
    expect(r"k must have shape \(2, 3, 40, 16\)", fn, q, torch.zeros(2, 2, 40, 16, dtype=H16), v, om)
    expect(r"k must have shape", fn, q, torch.zeros(2, 3, 40, 32, dtype=H16), v, om)
    expect("k must be torch.bfloat16", fn, q, k.float(), v, om)
    expect("v must be torch.bfloat16", fn, q, k, v.float(), om)
    expect(r"v must have shape \(2, 3, 40, 16\)", fn, q, k, torch.zeros(2, 3, 41, 16, dtype=H16), om)
    expect("omega must be torch.float32", fn, q, k, v, om.bfloat16())
    expect(r"omega must have shape \(3, 32, 16\)", fn, q, k, v, torch.zeros(2, 32, 16))
    expect(r"omega must have shape \(3, 32, 16\)", fn, q, k, v, torch.zeros(3, 32, 8))
    expect("omega must have 3 dimensions", fn, q, k, v, torch.zeros(32, 16))
    expect("q must have 4 dimensions", fn, q[0], k, v, om)
    expect("k must be contiguous", fn, q, k.transpose(0, 1), v, om)
    expect("q must be a device tensor", fn, q, k, v, om)  # everything consistent: only residence is left


def test_cross_attention_lengths():
    q, k, v, om = seq(L=40)
    expect(r"v must have shape \(2, 3, 40, 16\)", rf.bidir_cross, q[:, :, :10].contiguous(), k,
           v[:, :, :30].contiguous(), om)
    expect("q must be a device tensor", rf.bidir_cross, q[:, :, :10].contiguous(), k, v, om)


@pytest.mark.parametrize("fn", [rf.bidir_backward, rf.causal_backward])
def test_backward_inputs(fn):
    q, k, v, om = seq()
    expect(r"dout must have shape \(2, 3, 40, 16\)", fn, q, k, v, om, torch.zeros(2, 3, 40, 8, dtype=H16))
    expect("dout must be torch.bfloat16", fn, q, k, v, om, v.float())
    expect("k must be torch.bfloat16", fn, q, k.float(), v, om, v)


def decode_args(N=4, H=2, d=16, dv=32, m=48, dtype=H16):
    q = torch.zeros(N, H, d, dtype=dtype)
    k = torch.zeros(N, H, d, dtype=dtype)
    v = torch.zeros(N, H, dv, dtype=dtype)
    om = torch.zeros(H, m, d)
    S = torch.zeros(N, H, m, dv)
    z = torch.zeros(N, H, m)
    return q, k, v, om, S, z


def test_decode_state_and_output():
    q, k, v, om, S, z = decode_args()
    expect(r"S must have shape \(4, 2, 48, 32\)", rf.decode, q, k, v, om, S[:, :, :, :16].contiguous(), z)
    expect("S must be torch.float32", rf.decode, q, k, v, om, S.double(), z)
    expect(r"z must have shape \(4, 2, 48\)", rf.decode, q, k, v, om, S, z[:3].contiguous())
    expect("z must be torch.float32", rf.decode, q, k, v, om, S, z.bfloat16())
    expect(r"k must have shape \(4, 2, 16\)", rf.decode, q, k[:, :1].contiguous(), v, om, S, z)
    expect(r"omega must have shape \(2, 48, 16\)", rf.decode, q, k, v, torch.zeros(2, 48, 32), S, z)
    expect(r"out must have shape \(4, 2, 32\)", rf.decode, q, k, v, om, S, z, out=torch.zeros(4, 2, 16))
    expect("out must be torch.float32", rf.decode, q, k, v, om, S, z, out=torch.zeros(4, 2, 32, dtype=H16))
    expect("q must be a device tensor", rf.decode, q, k, v, om, S, z)


def test_decode_gated_gates():
    q, k, v, om, S, z = decode_args()
    expect(r"gate must have shape \(4, 2\)", rf.decode_gated, q, k, v, om, S, z, torch.zeros(2, 4))
    expect("gate must have 2 dimensions", rf.decode_gated, q, k, v, om, S, z, torch.zeros(8))
    expect("gate must be torch.float32", rf.decode_gated, q, k, v, om, S, z, torch.zeros(4, 2, dtype=H16))
    expect(r"in_weight must have shape \(4, 2\)", rf.decode_gated, q, k, v, om, S, z, torch.zeros(4, 2),
           torch.zeros(2, 4))


def test_features_omega():
    x = torch.zeros(2, 3, 40, 16, dtype=H16)
    expect(r"omega must have shape \(3, 32, 16\)", rf.features, x, torch.zeros(3, 32, 32))
    expect("omega must be torch.float32", rf.features, x, torch.zeros(3, 32, 16, dtype=H16))
    expect("x must be a device tensor", rf.features, x, torch.zeros(3, 32, 16))


def test_unsupported_dtype():
    q, k, v, om = seq(dtype=torch.float16)
    with pytest.raises(TypeError, match="unsupported dtype"):
        rf.bidir(q, k, v, om)


def test_prepared_omega_must_match_the_call():
    """A PreparedOmega is tied to (H, d, dv, m, dtype, kind); the binding refuses another combination before any
    library call."""
    prep = rf.PreparedOmega(None, 12, 64, 64, 256, torch.bfloat16, "prf")
    prep.check(12, 64, 64, 256, torch.bfloat16, "prf")
    for args in ((12, 64, 32, 256, torch.bfloat16, "prf"), (12, 64, 64, 256, torch.float32, "prf"),
                 (12, 64, 64, 256, torch.bfloat16, "relu"), (8, 64, 64, 256, torch.bfloat16, "prf")):
        with pytest.raises(ValueError):
            prep.check(*args)
