"""How precisely any fp32 computation can match the oracle's gradients at large input norms (no GPU).

At q, k ~ 2 N(0,1), d = 64 the exponents of the positive features reach about 100 in log2 units and attention is
nearly one-hot for many queries. Two consequences, measured here by evaluating the oracle's own formulas with every
step in fp32 (oracle work_dtype = np.float32) against the same formulas in fp64:

* dq rows whose attention is nearly one-hot nearly vanish (out ~ v_j whatever q is; causal row 0 is exactly 0), so
  a row-by-row relative error is meaningless for them: the fp32 evaluation misses those rows by 40 % to 1e9 relative.
  The GPU tests judge dq rows against at least 1 % of their (b,h) block's largest row.
* With that floor the fp32 evaluation still misses by up to about 1.2e-4 (dq) and 6e-5 (dk), above the 1e-4 used
  elsewhere for fp32 paths: the fp32 GPU gradients are held to 1e-3 in that regime, ten times the fp32 evaluation's
  own miss.

These are the figures the large-norm GPU parity test relies on; nothing here involves the HIP path.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads


def _errs(got, ref):
    out = {}
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        a = np.asarray(a, np.float64)
        num = np.max(np.abs(a - r), axis=-1)
        den = np.max(np.abs(r), axis=-1)
        floor = np.maximum(den, 1e-2 * np.max(np.abs(r), axis=(-2, -1), keepdims=True)[..., 0])
        out[name] = (float(np.max(num / den)), float(np.max(num / floor)))
    return out


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("fn", [oracle.bidir_backward, oracle.causal_backward])
def test_fp32_evaluation_of_the_gradients_at_large_norms(dtype, fn):
    d, dv, m = 64, 64, 256
    B, H, L = 1, 2, 300
    q = workloads.make_tensor((B, H, L, d), 2100, 2.0, dtype)
    k = workloads.make_tensor((B, H, L, d), 2101, 2.0, dtype)
    v = workloads.make_tensor((B, H, L, dv), 2102, 1.0, dtype)
    g = workloads.make_tensor((B, H, L, dv), 2101, 1.0, dtype)
    om = oracle.make_omega(49, H, m, d)
    ref = fn(q, k, v, om, g)
    got = fn(q, k, v, om, g, work_dtype=np.float32)
    e = _errs(got, ref)
    # dq row by row: some exact rows nearly vanish, so the relative error of a row is not a usable bound
    assert e["dq"][0] > 1e-2, e
    # with dq judged against 1 % of the block's scale (dk, dv are unaffected by the floor here) every gradient of
    # the fp32 evaluation is within 2.5e-4 of fp64: the 1e-3 bound leaves a factor four over the worst case
    worst = max(x[1] for x in e.values())
    assert 2e-5 < worst < 2.5e-4, e
    # the value gradient has no cancelling terms: it stays at the fp32 level
    assert e["dv"][0] < 2e-5, e
