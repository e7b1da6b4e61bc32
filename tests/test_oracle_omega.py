"""Pins for the oracle's Omega: orthogonality (Performer section 2.4), chi(d) lengths and N(0, I)
marginals (appendix F.4), independent blocks for m > d (appendix B.2), and the Gaussian stream itself."""
import math
import os

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle import make_omega, gaussians, stream_key


def test_gaussian_stream_is_standard_normal():
    g = np.array(gaussians(stream_key(7, 0, 0, 0), 40000))
    assert abs(g.mean()) < 4 / math.sqrt(len(g))
    assert g.var() == pytest.approx(1.0, abs=4 * math.sqrt(2.0 / len(g)))
    assert stats.kstest(g, "norm").pvalue > 1e-3
    # pairs (cos, sin) are independent: no correlation between consecutive draws
    assert abs(np.corrcoef(g[0::2], g[1::2])[0, 1]) < 4 / math.sqrt(len(g) / 2)


def test_streams_differ_by_seed_head_block_and_stream():
    keys = {stream_key(s, h, b, t) for s in (0, 1) for h in (0, 1) for b in (0, 1) for t in (0, 1)}
    assert len(keys) == 16
    a = make_omega(1, 2, 32, 16)
    assert not np.array_equal(a[0], a[1])
    assert not np.array_equal(a[0, :16], a[0, 16:])


def test_uniforms_strictly_inside_unit_interval():
    k = stream_key(3, 0, 0, 0)
    u = [oracle.uniform52(k, i) for i in range(2000)]
    assert 0.0 < min(u) and max(u) < 1.0


@pytest.mark.parametrize("d,m", [(16, 32), (16, 40), (8, 8), (32, 96)])
def test_rows_orthogonal_within_each_block(d, m):
    om = make_omega(5, 3, m, d).astype(np.float64)
    assert om.shape == (3, m, d)
    for h in range(3):
        for b0 in range(0, m, d):
            blk = om[h, b0:min(b0 + d, m)]
            n = np.linalg.norm(blk, axis=1)
            cos = (blk @ blk.T) / np.outer(n, n)
            off = cos - np.eye(len(blk))
            assert np.max(np.abs(off)) < 2e-6
        # different blocks are independent, not orthogonal to each other
        if m >= 2 * d:
            c = om[h, 0] @ om[h, d] / (np.linalg.norm(om[h, 0]) * np.linalg.norm(om[h, d]))
            assert abs(c) > 1e-4


def test_truncated_last_block_is_a_prefix_of_a_full_block():
    a = make_omega(9, 1, 40, 16)
    b = make_omega(9, 1, 48, 16)
    assert np.array_equal(a[0], b[0, :40])


def test_row_lengths_are_chi_d():
    """Appendix F.4: lengths independent of directions and chi(d)-distributed; moments of chi(d)."""
    d = 16
    om = make_omega(11, 64, 64, d).astype(np.float64)      # 256 blocks
    lens = np.linalg.norm(om.reshape(-1, d), axis=1)
    assert stats.kstest(lens, stats.chi(d).cdf).pvalue > 1e-3
    # chi moment mu_d(2) = d, mu_d(4) = d(d+2)
    assert np.mean(lens ** 2) == pytest.approx(d, rel=0.03)
    assert np.mean(lens ** 4) == pytest.approx(d * (d + 2), rel=0.06)


def test_orthogonal_rows_have_standard_normal_marginals():
    """Each orthogonal row is marginally N(0, I_d): zero mean, identity covariance."""
    d = 8
    om = make_omega(13, 256, 8, d).astype(np.float64).reshape(-1, d)   # 2048 rows
    assert np.max(np.abs(om.mean(axis=0))) < 4.5 / math.sqrt(len(om))
    cov = om.T @ om / len(om)
    assert np.max(np.abs(cov - np.eye(d))) < 0.15
    # every coordinate is N(0,1)
    assert stats.kstest(om[:, 3], "norm").pvalue > 1e-3


def test_sqrtd_mode_puts_rows_on_the_sphere():
    """Section 2.3 under Lemma 1 (SMREG): rows uniform on the sphere of radius sqrt(d)."""
    d = 16
    om = make_omega(17, 4, 32, d, "ortho_sqrtd").astype(np.float64)
    assert np.allclose(np.linalg.norm(om, axis=-1), math.sqrt(d), rtol=1e-6)


def test_iid_mode_is_the_gaussian_stream():
    d = 16
    om = make_omega(19, 1, 16, d, "iid")
    g = np.array(gaussians(stream_key(19, 0, 0, 0), d * d)).reshape(d, d).astype(np.float32)
    assert np.array_equal(om[0], g)


def test_omega_is_deterministic_and_matches_stored_spec_vector(golden_dir):
    """Stored bits were written by tests/golden/make_omega_golden.py, which calls only the oracle."""
    import json
    spec = json.load(open(os.path.join(golden_dir, "omega_spec.json")))
    for case in spec["cases"]:
        om = make_omega(case["seed"], case["H"], case["m"], case["d"], case["mode"])
        bits = om.view(np.uint32).reshape(-1)
        got = [int(bits[i]) for i in case["indices"]]
        assert got == case["bits"], case
