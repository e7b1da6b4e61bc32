"""Approximation quality of the GPU path against exact softmax attention, in the shape of the Performer paper's
Figure 4 (section 4.2: mean squared error of the approximate attention output over 15 samples of random features,
orthogonal vs iid, positive vs trigonometric), on the fp32 workload of that figure's shape (B1 H8 L4096 d16 dv16,
m = 128 features, Q, K, V ~ N(0,1)). The paper prints no values; the test asserts the orderings the figure shows and
prints the table."""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

rf = pytest.importorskip("random_feature_amd")


def test_figure4_orthogonal_vs_iid_and_positive_vs_trig():
    w = workloads.WORKLOADS["bidir_fp32"]
    q, k, v = workloads.make_qkv(w)
    exact = oracle.softmax_attention(q, k, v)  # fp64, equation 1
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    mse = {"positive, orthogonal": [], "positive, iid": [], "trigonometric, orthogonal": []}
    for s in range(15):
        for name, kind, mode in (("positive, orthogonal", "prf", "ortho_chi"), ("positive, iid", "prf", "iid"),
                                 ("trigonometric, orthogonal", "trig", "trig_pairs")):
            om = rf.make_omega(100 + s, w.H, w.m, w.d, mode)
            out = rf.bidir(qd, kd, vd, om, kind=kind, out_f32=True)
            torch.cuda.synchronize()
            mse[name].append(float(np.mean((out.cpu().double().numpy() - exact) ** 2)))
    for name, vals in mse.items():
        print(f"{name:28s} MSE mean {np.mean(vals):.4e}  median {np.median(vals):.4e}  "
              f"range [{np.min(vals):.3e}, {np.max(vals):.3e}]")
    ortho, iid, trig = (np.mean(mse[n]) for n in mse)
    assert np.isfinite(ortho) and np.isfinite(iid)
    assert ortho < iid      # orthogonal features: lower error than iid ones (section 2.4, Theorem 2)
    assert ortho < trig     # positive features: lower error than trigonometric ones (Lemma 2)
