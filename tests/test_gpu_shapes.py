"""GPU parity over the boundary's shape set: d in {16, 32, 64, 128}, dv any multiple of 16 up to 256 (independent of
d), m any multiple of 16 up to 512 (the Performer paper's Algorithm 1 takes Q, K in R^{L x d} and V with its own
width). Shapes outside the exact kernels run on the general ones: features padded to a compiled capacity and masked,
values in column groups of 64. Every case against the fp64 oracle on the same seeded inputs, L = 300 (several 32-token
tiles and a ragged tail) unless stated."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import TOL, rel_err

pytestmark = pytest.mark.gpu

rf = pytest.importorskip("random_feature_amd")
DEV = "cuda"

# (d, dv, m): dv != d, m up to 512 and not a power of two, d = 128, dv up to 256, and one exact shape for reference
SHAPES = [(64, 128, 256), (128, 128, 256), (64, 64, 512), (16, 256, 32), (128, 64, 64), (32, 48, 48),
          (16, 80, 112), (128, 256, 512), (64, 208, 240), (32, 32, 96), (128, 16, 16), (64, 64, 256)]


def _fp32_built(d, m):
    return d <= 64 and m <= 256


def _inputs(B, H, L, d, dv, dtype, seed, scale=0.5):
    q = workloads.make_tensor((B, H, L, d), seed, scale, dtype)
    k = workloads.make_tensor((B, H, L, d), seed + 1, scale, dtype)
    v = workloads.make_tensor((B, H, L, dv), seed + 2, 1.0, dtype)
    return q, k, v


def _cases():
    for d, dv, m in SHAPES:
        for dt in (torch.bfloat16, torch.float32):
            if dt == torch.float32 and not _fp32_built(d, m):
                continue
            yield pytest.param(d, dv, m, dt, id=f"d{d}-dv{dv}-m{m}-{str(dt)[6:]}")


@pytest.mark.parametrize("d,dv,m,dtype", list(_cases()))
def test_bidir_shape_set(d, dv, m, dtype):
    B, H, L = 2, 2, 300
    print(f"bidir d{d} dv{dv} m{m} {dtype}", flush=True)
    q, k, v = _inputs(B, H, L, d, dv, dtype, 3000 + d + dv + m)
    om_dev = rf.make_omega(31 + m, H, m, d)
    om = om_dev.cpu().numpy()
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for kind, eps in (("prf", 0.0), ("relu", 1e-3)):
        ref = oracle.bidir(q, k, v, om, kind, eps)
        out = rf.bidir(qd, kd, vd, om_dev, kind=kind, eps=eps, out_f32=True)
        torch.cuda.synchronize()
        e = rel_err(out, ref)
        assert e < TOL[dtype], (kind, e)
    # the input-dtype output and cross attention with other lengths on the same kernels
    out = rf.bidir(qd, kd, vd, om_dev)
    torch.cuda.synchronize()
    assert out.dtype == dtype and rel_err(out, oracle.bidir(q, k, v, om)) < TOL[dtype]
    Lq = 97
    outx = rf.bidir_cross(qd[:, :, :Lq].contiguous(), kd, vd, om_dev, out_f32=True)
    torch.cuda.synchronize()
    assert rel_err(outx, oracle.bidir(q[:, :, :Lq], k, v, om)) < TOL[dtype]


@pytest.mark.parametrize("d,dv,m,dtype", list(_cases()))
def test_causal_shape_set(d, dv, m, dtype):
    B, H, L = 1, 2, 300
    print(f"causal d{d} dv{dv} m{m} {dtype}", flush=True)
    q, k, v = _inputs(B, H, L, d, dv, dtype, 4000 + d + dv + m)
    om_dev = rf.make_omega(41 + m, H, m, d)
    om = om_dev.cpu().numpy()
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    if d <= 64:  # the final state in canonical scale (fp32 range: d <= 64)
        ref, S_ref, z_ref = oracle.causal(q, k, v, om, return_state=True)
        out, S, z = rf.causal(qd, kd, vd, om_dev, out_f32=True, return_state=True)
        torch.cuda.synchronize()
        assert rel_err(out, ref) < TOL[dtype]
        assert rel_err(z, z_ref) < TOL[dtype]
        assert np.max(np.abs(S.cpu().double().numpy() - S_ref)) / np.max(np.abs(S_ref)) < TOL[dtype]
    else:
        out = rf.causal(qd, kd, vd, om_dev, out_f32=True)
        torch.cuda.synchronize()
        assert rel_err(out, oracle.causal(q, k, v, om)) < TOL[dtype]
    out = rf.causal(qd, kd, vd, om_dev, kind="relu", eps=1e-3, out_f32=True)
    torch.cuda.synchronize()
    assert rel_err(out, oracle.causal(q, k, v, om, "relu", 1e-3)) < TOL[dtype]


def test_one_hot_matrix_in_one_call():
    """The explicit L x L matrix D_hat^-1 A_hat (Performer appendix C.4: V = I_L) at the 256-token fp32 workload's
    shape (d = 16, m = 32), in one call with dv = L = 256; rows sum to 1 and match the oracle's matrix."""
    w = workloads.WORKLOADS["bidir_small"]
    q, k, _ = workloads.make_qkv(w)
    om_dev = rf.make_omega(w.seed, w.H, w.m, w.d)
    om = om_dev.cpu().numpy()
    eye = torch.eye(w.L, dtype=torch.float32).expand(w.B, w.H, w.L, w.L).contiguous()
    A = rf.bidir(q.to(DEV), k.to(DEV), eye.to(DEV), om_dev, out_f32=True)
    torch.cuda.synchronize()
    ref = oracle.attention_matrix(q, k, om)
    assert rel_err(A, ref) < TOL[torch.float32]
    assert np.allclose(A.sum(-1).cpu().double().numpy(), 1.0, atol=1e-5)


@pytest.mark.parametrize("d,m,dtype", [(128, 512, torch.bfloat16), (128, 512, torch.float32), (16, 48, torch.float32),
                                       (64, 400, torch.bfloat16), (128, 96, torch.float32), (32, 512, torch.float32)])
@pytest.mark.parametrize("kind", ["prf", "relu"])
def test_features_shape_set(d, m, dtype, kind):
    """The feature map alone: phi * exp(logscale) against the oracle's features (m > 256, or > 128 at large widths,
    runs as feature groups with every row's maximum taken over all groups first)."""
    x = workloads.make_tensor((2, 2, 100, d), 5000 + d + m, 0.5, dtype)
    om_dev = rf.make_omega(51, 2, m, d)
    om = om_dev.cpu().numpy()
    eps = 1e-3 if kind == "relu" else 0.0
    phi, ls = rf.features(x.to(DEV), om_dev, kind=kind, eps=eps)
    torch.cuda.synchronize()
    got = phi.cpu().double().numpy() * np.exp(ls.cpu().double().numpy())[..., None]
    ref = oracle.features(x, om, kind, eps)
    assert rel_err(got, ref) < TOL[dtype]
    if kind == "prf":  # each row's largest entry is 1/sqrt(m)
        assert np.allclose(phi.cpu().double().numpy().max(-1), 1 / np.sqrt(m), rtol=1e-6)


@pytest.mark.parametrize("d,dv,m", [(64, 48, 96), (16, 80, 512), (32, 208, 64), (64, 240, 256)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_value_widths(d, dv, m, dtype):
    """Decode with value widths that are multiples of 16 but not powers of two (the state rows of a
    workgroup then do not split evenly over its threads)."""
    N, H, T, P = 6, 2, 12, 30
    om_dev = rf.make_omega(61, H, m, d)
    om = om_dev.cpu().numpy()
    kp = workloads.make_tensor((N, H, P, d), 11, 1.0, dtype)
    vp = workloads.make_tensor((N, H, P, dv), 12, 1.0, dtype)
    S0, z0 = oracle.state_from_prior(kp, vp, om)
    S0, z0 = S0.astype(np.float32), z0.astype(np.float32)
    qs = workloads.make_tensor((T, N, H, d), 13, 1.0, dtype)
    ks = workloads.make_tensor((T, N, H, d), 14, 1.0, dtype)
    vs = workloads.make_tensor((T, N, H, dv), 15, 1.0, dtype)
    S_ref, z_ref, outs_ref = oracle.decode_run(S0, z0, qs, ks, vs, om)
    S = torch.from_numpy(S0).to(DEV)
    z = torch.from_numpy(z0).to(DEV)
    qd, kd, vd = qs.to(DEV), ks.to(DEV), vs.to(DEV)
    outs = torch.stack([rf.decode(qd[t], kd[t], vd[t], om_dev, S, z) for t in range(T)])
    torch.cuda.synchronize()
    assert rel_err(outs, outs_ref) < TOL[dtype]
    assert np.max(np.abs(S.cpu().double().numpy() - S_ref)) / np.max(np.abs(S_ref)) < 1e-5
    assert rel_err(z, z_ref) < 1e-5


@pytest.mark.parametrize("path", ["bidir", "causal"])
def test_bf16_values_beyond_fp16_range(path):
    """bf16 components of magnitude 65504 or more (here 1e6) in a few keys and one query: those keys' features are
    zero in exact arithmetic (exp(w.y - |y|^2/2) with |y|^2 ~ 1e11), and so they are in the kernels (the fp16
    projection copy is clamped, the norm is the true one). Every output stays finite; rows of the other queries
    match the oracle."""
    d, dv, m = 64, 64, 256
    B, H, L = 1, 2, 200
    q, k, v = _inputs(B, H, L, d, dv, torch.bfloat16, 6100)
    k[0, 0, 5, 3] = 1e6
    k[0, 1, 150, 0] = -2e6
    k[0, 1, 40, 10] = 7e4
    q[0, 0, 7, 1] = 1e6
    om_dev = rf.make_omega(71, H, m, d)
    om = om_dev.cpu().numpy()
    fn, ofn = (rf.bidir, oracle.bidir) if path == "bidir" else (rf.causal, oracle.causal)
    out = fn(q.cuda(), k.cuda(), v.cuda(), om_dev, out_f32=True).cpu()
    assert torch.isfinite(out).all()
    ref = ofn(q, k, v, om)
    keep = np.ones(L, bool)
    keep[7] = False  # the query beyond the range is projected along its clamped direction
    assert rel_err(out[:, :, keep], ref[:, :, keep]) < TOL[torch.bfloat16]
