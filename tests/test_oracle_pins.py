"""Pins for the oracle: facts fixed by the pages or by mathematics, not by the oracle itself.

Each test names the passage it follows. A plausible slip in the oracle (a
dropped norm term, a missing d^(-1/4), a transposed contraction, an exclusive
instead of inclusive prefix, a wrong Gram-Schmidt step) fails at least one.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import features, bidir, bidir_from_features, causal, causal_bruteforce, decode_run, make_omega

RNG = np.random.default_rng(12345)


# ---------------------------------------------------------------- contraction

def test_worked_example_from_features(golden_dir):
    """Performer tutorial page, section 2 worked example: S=(3,10), z=(1,2), output 13/3."""
    g = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    phi_k = np.array(g["key_features"])
    v = np.array(g["values"])[:, None]
    phi_q = np.array([g["query_feature"]])
    out, S, z = bidir_from_features(phi_q, phi_k, v)
    assert np.array_equal(S[:, 0], np.array(g["S"]))
    assert np.array_equal(z, np.array(g["z"]))
    assert out[0, 0] == pytest.approx(g["output_numerator"] / g["output_denominator"], rel=1e-15)
    # the same number as a kernel-weighted average of the values
    w = phi_q @ phi_k.T
    assert np.allclose(w[0], g["kernel_weights"])


@pytest.mark.parametrize("d", [2, 16])
def test_worked_example_through_relu_feature_map(golden_dir, d):
    """Same example through the full path: ReLU features (Performer appendix A.4), Omega = I, eps = 0.

    With omega = identity, ReLU features are the positive parts of the scaled
    inputs; any common positive factor cancels in the ratio. Negative
    coordinates check that the ReLU clips them.
    """
    g = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    om = np.eye(d, dtype=np.float32)[None]
    t = 0.7
    k = np.zeros((1, 1, 2, d))
    k[0, 0, 0, :2] = np.array([1.0, -3.0]) * t        # ReLU -> (1, 0)
    k[0, 0, 1, :2] = np.array([0.0, 2.0]) * t         # -> (0, 2)
    k[0, 0, :, 2:] = -1.5                             # clipped away
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, :2] = t
    v = np.zeros((1, 1, 2, 4))
    v[0, 0, :, 0] = g["values"]
    pq = features(q, om, "relu", 0.0)
    pk = features(k, om, "relu", 0.0)
    out, _, _ = bidir_from_features(pq, pk, v)
    assert out[0, 0, 0, 0] == pytest.approx(13.0 / 3.0, rel=1e-14)
    assert np.all(out[0, 0, 0, 1:] == 0.0)


def test_four_token_toy_reassociation():
    """Tutorial page section 2: 4 tokens, feature width 3, value width 2: (Q'K'^T)V equals Q'(K'^T V)."""
    pq = RNG.random((4, 3)) + 0.1
    pk = RNG.random((4, 3)) + 0.1
    v = RNG.normal(size=(4, 2))
    explicit = pq @ pk.T                      # the 4 x 4 matrix the linear form avoids
    ref = (explicit @ v) / explicit.sum(axis=1, keepdims=True)
    out, S, z = bidir_from_features(pq, pk, v)
    assert S.shape == (3, 2) and z.shape == (3,)
    assert np.allclose(out, ref, rtol=1e-13, atol=0)


def test_bidir_equals_explicit_attention_matrix():
    """Equation 4 versus the explicit L x L matrix A_hat = Phi_Q Phi_K^T (equation 1 applied to A_hat)."""
    B, H, L, d, dv, m = 1, 2, 37, 16, 8, 32
    q = RNG.normal(size=(B, H, L, d)) * 0.5
    k = RNG.normal(size=(B, H, L, d)) * 0.5
    v = RNG.normal(size=(B, H, L, dv))
    om = make_omega(7, H, m, d)
    pq, pk = features(q, om), features(k, om)
    for h in range(H):
        A = pq[0, h] @ pk[0, h].T
        ref = np.diag(1.0 / A.sum(axis=1)) @ A @ v[0, h]
        assert np.max(np.abs(bidir(q, k, v, om)[0, h] - ref)) < 1e-12


def test_cross_and_unnormalised_bidir_equal_the_explicit_matrix():
    """Algorithm 1 with Lq != Lk (the RFA page's cross attention): Phi_Q (Phi_K^T V) equals the explicit
    Lq x Lk matrix A_hat = Phi_Q Phi_K^T applied to V, without D^-1 (renormalize off, appendix D.3) and with it
    (equation 1's normalisation applied to A_hat)."""
    B, H, Lq, Lk, d, dv, m = 1, 2, 5, 11, 16, 8, 32
    q = RNG.normal(size=(B, H, Lq, d)) * 0.5
    k = RNG.normal(size=(B, H, Lk, d)) * 0.5
    v = RNG.normal(size=(B, H, Lk, dv))
    om = make_omega(8, H, m, d)
    for kind, eps in (("prf", 0.0), ("relu", 1e-3)):
        A = np.einsum("bhim,bhjm->bhij", features(q, om, kind, eps), features(k, om, kind, eps))
        un = bidir(q, k, v, om, kind, eps, renormalize=False)
        assert np.max(np.abs(un - A @ v)) < 1e-12 * np.max(np.abs(A @ v))
        nrm = bidir(q, k, v, om, kind, eps)
        assert np.max(np.abs(nrm - (A @ v) / A.sum(-1, keepdims=True))) < 1e-12


def test_unnormalised_output_converges_to_the_softmax_numerator():
    """Lemma 1 under the unnormalised output: phi(q_i).S -> sum_j exp(q_i.k_j / sqrt(d)) v_j as m grows
    (the feature scale 1/sqrt(m) and the -|x|^2/2 term both matter here, unlike in the ratio)."""
    B, H, Lq, Lk, d, dv = 1, 1, 4, 9, 16, 3
    q = RNG.normal(size=(B, H, Lq, d)) * 0.4
    k = RNG.normal(size=(B, H, Lk, d)) * 0.4
    v = RNG.normal(size=(B, H, Lk, dv))
    exact = np.exp(np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(d)) @ v
    errs = []
    for m in (64, 4096, 65536):
        om = make_omega(90 + m, H, m, d)
        errs.append(np.max(np.abs(bidir(q, k, v, om, renormalize=False) - exact)) / np.max(np.abs(exact)))
    assert errs[-1] < 0.02 and errs[-1] < errs[0]


def test_one_hot_values_extract_the_normalised_matrix():
    """Performer appendix C.4: with V = I_L the output is D_hat^-1 A_hat; rows sum to one."""
    L, d, m = 24, 16, 32
    q = RNG.normal(size=(1, 1, L, d)) * 0.5
    k = RNG.normal(size=(1, 1, L, d)) * 0.5
    om = make_omega(3, 1, m, d)
    out = bidir(q, k, np.eye(L)[None, None], om)
    assert np.allclose(out.sum(axis=-1), 1.0, atol=1e-13)
    assert np.all(out > 0)
    assert np.allclose(out, oracle.attention_matrix(q, k, om), atol=1e-14)


# ---------------------------------------------------------------- causal

def test_causal_three_forms_agree():
    """Equation 11 (prefix sums, diagonal included) == masked brute force (equation 2 on A_hat) == decode recurrence."""
    B, H, L, d, dv, m = 2, 2, 29, 16, 8, 48
    q = RNG.normal(size=(B, H, L, d)) * 0.5
    k = RNG.normal(size=(B, H, L, d)) * 0.5
    v = RNG.normal(size=(B, H, L, dv))
    om = make_omega(11, H, m, d)
    rec = causal(q, k, v, om)
    brute = causal_bruteforce(q, k, v, om)
    assert np.max(np.abs(rec - brute)) < 1e-12
    # decode from the zero state: token t's output reads the state after adding token t
    S0 = np.zeros((B, H, m, dv))
    z0 = np.zeros((B, H, m))
    _, _, outs = decode_run(S0, z0, np.moveaxis(q, 2, 0), np.moveaxis(k, 2, 0), np.moveaxis(v, 2, 0), om)
    assert np.max(np.abs(np.moveaxis(outs, 0, 2) - rec)) < 1e-12
    # row 0 sees only token 0; the last row equals the bidirectional output
    assert np.allclose(rec[:, :, 0], v[:, :, 0], atol=1e-14)
    assert np.allclose(rec[:, :, -1], bidir(q, k, v, om)[:, :, -1], atol=1e-12)


def test_causal_state_matches_prior_state():
    B, H, L, d, dv, m = 1, 2, 40, 16, 16, 32
    k = RNG.normal(size=(B, H, L, d)) * 0.5
    v = RNG.normal(size=(B, H, L, dv))
    om = make_omega(5, H, m, d)
    _, S, z = causal(k, k, v, om, return_state=True)
    S2, z2 = oracle.state_from_prior(k, v, om)
    assert np.allclose(S, S2, rtol=1e-12) and np.allclose(z, z2, rtol=1e-12)


def test_gated_decode_recurrence_equals_unrolled_sum():
    """RFA page, section 3.2 (RFA-GATE): the step-by-step gated recurrence equals its unrolled form, in which
    token j enters step t with weight w_j * prod_{j<l<=t} g_l and the initial state with prod_{l<=t} g_l;
    with every g = w = 1 it is the ungated decode, and with g -> 0 a step sees only its own token."""
    N, H, T, d, dv, m = 2, 3, 9, 16, 8, 32
    om = make_omega(21, H, m, d)
    kp = RNG.normal(size=(N, H, 6, d)) * 0.5
    vp = RNG.normal(size=(N, H, 6, dv))
    S0, z0 = oracle.state_from_prior(kp, vp, om)
    q = RNG.normal(size=(T, N, H, d)) * 0.5
    k = RNG.normal(size=(T, N, H, d)) * 0.5
    v = RNG.normal(size=(T, N, H, dv))
    g = RNG.uniform(0.3, 1.0, size=(T, N, H))
    w = 1.0 - g
    for wt in (None, w):
        _, _, rec = oracle.decode_gated_run(S0, z0, q, k, v, om, g, wt)
        unrolled = oracle.decode_gated_unrolled(S0, z0, q, k, v, om, g, wt)
        assert np.max(np.abs(rec - unrolled)) < 1e-12
    ones = np.ones((T, N, H))
    S1, z1, o1 = oracle.decode_gated_run(S0, z0, q, k, v, om, ones)
    S2, z2, o2 = decode_run(S0, z0, q, k, v, om)
    assert np.max(np.abs(o1 - o2)) < 1e-13 and np.allclose(S1, S2, rtol=1e-14)
    _, _, tiny = oracle.decode_gated_run(S0, z0, q, k, v, om, np.full((T, N, H), 1e-30))
    assert np.max(np.abs(tiny - v)) < 1e-12


@pytest.mark.parametrize("kind,eps", [("prf", 0.0), ("relu", 1e-3)])
def test_bidir_backward_matches_finite_differences(kind, eps):
    """The chain-rule gradients of equation 4 against central differences of the forward estimator (fp64):
    every entry of dq, dk and dv for a random linear functional of the output."""
    B, H, L, d, dv, m = 1, 2, 6, 8, 4, 16
    rng = np.random.default_rng(3)
    q = rng.normal(size=(B, H, L, d)) * 0.6
    k = rng.normal(size=(B, H, L, d)) * 0.6
    v = rng.normal(size=(B, H, L, dv))
    g = rng.normal(size=(B, H, L, dv))
    om = make_omega(13, H, m, d)
    grads = oracle.bidir_backward(q, k, v, om, g, kind, eps)
    h = 1e-6
    for x, gx in zip((q, k, v), grads):
        num = np.empty_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[i] += h
            xm[i] -= h
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            fp = np.sum(g * bidir(*args_p, om, kind, eps))
            fm = np.sum(g * bidir(*args_m, om, kind, eps))
            num[i] = (fp - fm) / (2 * h)
        assert np.max(np.abs(num - gx)) < 1e-6 * max(1.0, np.max(np.abs(gx))), (kind, np.max(np.abs(num - gx)))


@pytest.mark.parametrize("kind,eps", [("prf", 0.0), ("relu", 1e-3)])
def test_causal_backward_matches_finite_differences(kind, eps):
    """The chain-rule gradients of the causal estimator (appendix B.1, equation 11, prefix sums including the
    diagonal) against central differences of the forward recurrence (fp64): every entry of dq, dk and dv for a
    random linear functional of the output. A key that only later queries see, a missing diagonal term or a
    prefix sum taken in the wrong direction fails it."""
    B, H, L, d, dv, m = 1, 2, 7, 8, 4, 16
    rng = np.random.default_rng(5)
    q = rng.normal(size=(B, H, L, d)) * 0.6
    k = rng.normal(size=(B, H, L, d)) * 0.6
    v = rng.normal(size=(B, H, L, dv))
    g = rng.normal(size=(B, H, L, dv))
    om = make_omega(17, H, m, d)
    grads = oracle.causal_backward(q, k, v, om, g, kind, eps)
    h = 1e-6
    for x, gx in zip((q, k, v), grads):
        num = np.empty_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[i] += h
            xm[i] -= h
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            fp = np.sum(g * causal(*args_p, om, kind, eps))
            fm = np.sum(g * causal(*args_m, om, kind, eps))
            num[i] = (fp - fm) / (2 * h)
        assert np.max(np.abs(num - gx)) < 1e-6 * max(1.0, np.max(np.abs(gx))), (kind, np.max(np.abs(num - gx)))


def test_causal_backward_last_position_and_single_token():
    """Two special cases: with L = 1 the causal and bidirectional estimators coincide, so do their gradients;
    and the last key is seen only by the last query, so with dout zero except at the last position its dv is
    the bidirectional one of that row (the last row of the causal output is the bidirectional output)."""
    B, H, d, dv, m = 1, 1, 8, 4, 16
    rng = np.random.default_rng(9)
    om = make_omega(21, H, m, d)
    q, k, v, g = (rng.normal(size=(B, H, 1, n)) * s for n, s in ((d, 0.6), (d, 0.6), (dv, 1.0), (dv, 1.0)))
    for a, b in zip(oracle.causal_backward(q, k, v, om, g), oracle.bidir_backward(q, k, v, om, g)):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-14)
    L = 9
    q, k, v = (rng.normal(size=(B, H, L, n)) * s for n, s in ((d, 0.6), (d, 0.6), (dv, 1.0)))
    g = np.zeros((B, H, L, dv))
    g[..., -1, :] = rng.normal(size=dv)
    c = oracle.causal_backward(q, k, v, om, g)
    # only the last query carries a gradient and it sees every key: dv_j = A_Lj g_L / sum_j A_Lj from the
    # explicit last row of A_hat = Phi_Q Phi_K^T
    pq = oracle.features(q, om)[..., -1, :]
    pk = oracle.features(k, om)
    A = np.einsum("...m,...jm->...j", pq, pk)
    dv_ref = A[..., :, None] / A.sum(axis=-1)[..., None, None] * g[..., -1, None, :]
    assert np.allclose(c[2], dv_ref, rtol=1e-12, atol=1e-14)


def test_bidir_backward_query_features_gradient_is_orthogonal_to_features():
    """The output is invariant to a per-row scale of the query features (it cancels in the ratio), so
    phi(q_i) . dPhi_Q_i = 0 for every row; hence dq has no |q|^2 term. Checked by rescaling q's features:
    the output and hence the gradients are unchanged."""
    B, H, L, d, dv, m = 1, 1, 9, 16, 8, 32
    rng = np.random.default_rng(4)
    q = rng.normal(size=(B, H, L, d)) * 0.5
    k = rng.normal(size=(B, H, L, d)) * 0.5
    v = rng.normal(size=(B, H, L, dv))
    g = rng.normal(size=(B, H, L, dv))
    om = make_omega(14, H, m, d)
    pq = features(q, om)
    pk = features(k, om)
    S = np.einsum("...lm,...le->...me", pk, v)
    z = pk.sum(-2)
    out, _, _ = bidir_from_features(pq, pk, v)
    D = np.einsum("...lm,...m->...l", pq, z)
    dpq = np.einsum("...le,...me->...lm", g / D[..., None], S) - (np.sum(g * out, -1) / D)[..., None] * z[..., None, :]
    assert np.max(np.abs(np.sum(pq * dpq, -1))) < 1e-12
    out2, _, _ = bidir_from_features(pq * rng.uniform(0.5, 2.0, size=(B, H, L, 1)), pk, v)
    assert np.max(np.abs(out2 - out)) < 1e-12


# ---------------------------------------------------------------- feature map

def _prf_single_estimates(x, y, om):
    """m * phi_r(x) phi_r(y) for every feature r: single-feature estimates of SM(x, y) (scaled inputs)."""
    d = x.shape[-1]
    s = float(d) ** 0.25  # undo the library-side scaling so that x, y are the scaled vectors
    m = om.shape[1]
    fx = features((x * s)[None, None, None], om)[0, 0, 0]
    fy = features((y * s)[None, None, None], om)[0, 0, 0]
    return m * fx * fy


def test_positive_features_unbiased_lemma1_with_lemma2_variance():
    """Lemma 1: E[phi(x).phi(y)] = exp(x.y); the iid estimator's MSE is Lemma 2's closed form.

    Lemma 2 (positive features): MSE = (1/m) exp(|z|^2) SM(x,y)^2 (1 - exp(-|z|^2)), z = x + y.
    """
    d, m = 16, 32768
    om = make_omega(2024, 1, m, d, "iid")
    for trial in range(3):
        x = RNG.normal(size=d) * 0.1
        y = RNG.normal(size=d) * 0.1
        sm = math.exp(float(x @ y))
        z2 = float((x + y) @ (x + y))
        mse1 = math.exp(z2) * sm ** 2 * (1.0 - math.exp(-z2))   # one feature
        est = _prf_single_estimates(x, y, om)
        mean = float(est.mean())
        assert abs(mean - sm) < 4.0 * math.sqrt(mse1 / m), (mean, sm)
        var = float(est.var())
        assert var == pytest.approx(mse1, rel=0.12), (var, mse1)
        # a feature map without the -|x|^2/2 term would be biased by exp((|x|^2+|y|^2)/2)
        bias = sm * (math.exp(0.5 * (float(x @ x) + float(y @ y))) - 1.0)
        assert bias > 8.0 * math.sqrt(mse1 / m)


def test_hyperbolic_features_unbiased_with_lemma2_variance():
    """Lemma 1 (second form): the hyperbolic features are unbiased for exp(x.y), and one random vector's
    estimate Lambda cosh(w.z) has variance m * MSE^hyp+ = (1/2)(1 - exp(-|z|^2)) exp(|z|^2) SM^2 (1 - exp(-|z|^2))
    (Lemma 2, equation 8, third line, with the second line for MSE^+)."""
    d, m = 16, 32768
    om = make_omega(2025, 1, m, d, "iid")
    s = float(d) ** 0.25
    for trial in range(3):
        x = RNG.normal(size=d) * 0.15
        y = RNG.normal(size=d) * 0.15
        sm = math.exp(float(x @ y))
        z2 = float((x + y) @ (x + y))
        var1 = 0.5 * (1.0 - math.exp(-z2)) * math.exp(z2) * sm ** 2 * (1.0 - math.exp(-z2))
        fx = oracle.features_hyperbolic((x * s)[None, None, None], om)[0, 0, 0]
        fy = oracle.features_hyperbolic((y * s)[None, None, None], om)[0, 0, 0]
        assert float(fx @ fy) == pytest.approx(sm, abs=4.0 * math.sqrt(var1 / m))
        est = m * (fx[:m] * fy[:m] + fx[m:] * fy[m:])   # one vector each
        assert float(est.var()) == pytest.approx(var1, rel=0.12)
        # the positive features' single-feature variance is larger by 2 / (1 - exp(-|z|^2))
        var_plus = math.exp(z2) * sm ** 2 * (1.0 - math.exp(-z2))
        assert float(_prf_single_estimates(x, y, om).var()) > 1.5 * var1 and var_plus > 2.0 * var1


def test_hyperbolic_omega_mode_gives_the_hyperbolic_features():
    """The hyperbolic Omega mode (the m/2 orthogonal chi(d) rows, then their negatives) under the plain
    positive feature map equals the hyperbolic features of those m/2 rows, in value and normaliser."""
    H, d, m = 2, 16, 64
    x = RNG.normal(size=(1, H, 7, d))
    om_h = make_omega(31, H, m, d, "hyperbolic")
    om_half = make_omega(31, H, m // 2, d, "ortho_chi")
    assert np.array_equal(om_h[:, :m // 2], om_half) and np.array_equal(om_h[:, m // 2:], -om_half)
    a = features(x, om_h)
    b = oracle.features_hyperbolic(x, om_half)
    assert np.max(np.abs(a - b) / b) < 1e-13


def test_trig_features_exact_on_the_diagonal_and_ordered_as_equation_5():
    """Equation 5 with h(x) = exp(|x|^2/2), l = 2, f1 = sin, f2 = cos (section 2.3, SM^trig): since
    sin^2 + cos^2 = 1, phi(x).phi(x) = exp(|x|^2) = SM(x, x) exactly for any omega (a dropped h, a wrong
    1/sqrt(m) or a missing cosine block fails this); the sine block comes first."""
    d, m = 16, 8
    s = float(d) ** 0.25
    om = make_omega(5, 1, m, d, "iid")
    for _ in range(3):
        x = RNG.normal(size=d) * 0.4
        f = oracle.features_trig((x * s)[None, None, None], om)[0, 0, 0]
        assert f.shape == (2 * m,)
        assert float(f @ f) == pytest.approx(math.exp(float(x @ x)), rel=1e-13)
    # one vector e_1 and x = (pi/2) e_1: sin = 1, cos = 0, h = exp((pi/2)^2 / 2)
    om1 = np.zeros((1, 1, d))
    om1[0, 0, 0] = 1.0
    x1 = np.zeros(d)
    x1[0] = math.pi / 2
    f1 = oracle.features_trig((x1 * s)[None, None, None], om1)[0, 0, 0]
    h = math.exp(0.5 * (math.pi / 2) ** 2)
    assert f1[0] == pytest.approx(h, rel=1e-14) and abs(f1[1]) < 1e-14 * h


def test_trig_features_unbiased_with_lemma2_variance():
    """SM^trig is unbiased for exp(x.y), and one vector's estimate exp((|x|^2+|y|^2)/2) cos(w.(x-y)) has
    variance m * MSE^trig = (1/2) exp(|x|^2 + |y|^2) (1 - exp(-|x-y|^2))^2 (Lemma 2, equation 8, first line,
    read with the squares of appendix F equations 13-15: exp(|z|^2) SM^-2 = exp(|x|^2 + |y|^2))."""
    d, m = 16, 32768
    om = make_omega(2026, 1, m, d, "iid")
    s = float(d) ** 0.25
    for trial in range(3):
        x = RNG.normal(size=d) * 0.15
        y = RNG.normal(size=d) * 0.15
        sm = math.exp(float(x @ y))
        dl2 = float((x - y) @ (x - y))
        var1 = 0.5 * math.exp(float(x @ x) + float(y @ y)) * (1.0 - math.exp(-dl2)) ** 2
        fx = oracle.features_trig((x * s)[None, None, None], om)[0, 0, 0]
        fy = oracle.features_trig((y * s)[None, None, None], om)[0, 0, 0]
        assert float(fx @ fy) == pytest.approx(sm, abs=4.0 * math.sqrt(var1 / m))
        est = m * (fx[:m] * fy[:m] + fx[m:] * fy[m:])   # one vector each
        assert float(est.var()) == pytest.approx(var1, rel=0.12)


def test_trig_pairs_omega_mode_repeats_the_rows():
    """The trig_pairs Omega mode: the m/2 orthogonal chi(d) rows, then the same rows again, so that the
    sine of the first m/2 projections and the cosine of the last m/2 are equation 5's 2(m/2) features."""
    H, d, m = 2, 16, 64
    x = RNG.normal(size=(1, H, 7, d))
    om_p = make_omega(31, H, m, d, "trig_pairs")
    om_half = make_omega(31, H, m // 2, d, "ortho_chi")
    assert np.array_equal(om_p[:, :m // 2], om_half) and np.array_equal(om_p[:, m // 2:], om_half)
    xs = x * d ** -0.25
    a = np.einsum("bhld,hmd->bhlm", xs, om_p.astype(np.float64))
    h = np.exp(0.5 * np.sum(xs * xs, axis=-1, keepdims=True)) / math.sqrt(m // 2)
    paired = np.concatenate([h * np.sin(a[..., :m // 2]), h * np.cos(a[..., m // 2:])], axis=-1)
    assert np.max(np.abs(paired - oracle.features_trig(x, om_half))) < 1e-13


def test_trig_attention_converges_to_softmax_attention():
    """With trigonometric features the ratio of equation 4 also approximates softmax attention (section
    2.3: SM^trig is unbiased; the per-key h(k) does not cancel) and improves with m."""
    B, H, L, d, dv = 1, 1, 24, 16, 8
    q = RNG.normal(size=(B, H, L, d)) * 0.3
    k = RNG.normal(size=(B, H, L, d)) * 0.3
    v = RNG.normal(size=(B, H, L, dv))
    exact = oracle.softmax_attention(q, k, v)
    errs = []
    for m in (16, 1024, 65536):
        approx = bidir(q, k, v, make_omega(3 + m, H, m, d, "iid"), kind="trig")
        errs.append(float(np.max(np.abs(approx - exact))))
    assert errs[2] < errs[0] and errs[2] < 0.02, errs


def test_features_apply_the_sqrt_d_temperature():
    """Section 2.3 under equation 6: raw q, k are scaled so that the kernel is exp(q.k / sqrt(d))."""
    d, m = 16, 16384
    om = make_omega(99, 1, m, d, "iid")
    rng = np.random.default_rng(7)  # its own draws: the bound below holds for any inputs, not for lucky ones
    q = rng.normal(size=d) * 0.3
    k = rng.normal(size=d) * 0.3
    est = float((features(q[None, None, None], om) * features(k[None, None, None], om)).sum())
    # Lemma 2 on the scaled vectors x = q d^-1/4, y = k d^-1/4: one feature's MSE is
    # exp(|x+y|^2) SM^2 (1 - exp(-|x+y|^2)); m iid features divide it by m
    sm = math.exp(float(q @ k) / math.sqrt(d))
    z2 = float((q + k) @ (q + k)) / math.sqrt(d)
    sigma = math.sqrt(math.exp(z2) * sm ** 2 * (1.0 - math.exp(-z2)) / m)
    assert abs(est - sm) < 4.0 * sigma
    # without the temperature the estimate would target exp(q.k), many standard deviations away
    assert abs(math.exp(float(q @ k)) - sm) > 8.0 * sigma


def test_orthogonal_features_reduce_mse_theorem2():
    """Theorem 2 (m <= d): MSE_ort <= MSE_iid - (1 - 1/m) * 2/(d+2) * (SM - Lambda)^2.

    The extracted statement lost its squares; the gap is read from appendix
    F.4 (equation 42 and its proof), with Lambda = exp(-(|x|^2 + |y|^2)/2).
    Monte Carlo over many independent Omega draws, small inputs.
    """
    d = m = 8
    R = 6000
    x = np.array([0.31, -0.12, 0.05, 0.22, -0.18, 0.09, 0.14, -0.07])
    y = np.array([0.11, 0.25, -0.16, 0.04, 0.13, -0.21, 0.08, 0.19])
    sm = math.exp(float(x @ y))
    z2 = float((x + y) @ (x + y))
    mse_iid = (1.0 / m) * math.exp(z2) * sm ** 2 * (1.0 - math.exp(-z2))
    lam = math.exp(-0.5 * (float(x @ x) + float(y @ y)))
    gap = (1.0 - 1.0 / m) * 2.0 / (d + 2) * (sm - lam) ** 2
    e_ort = np.array([_prf_single_estimates(x, y, make_omega(50000 + s, 1, m, d)).mean() for s in range(R)])
    e_iid = np.array([_prf_single_estimates(x, y, make_omega(50000 + s, 1, m, d, "iid")).mean() for s in range(R)])
    se = lambda e: float(np.std((e - sm) ** 2)) / math.sqrt(R)
    mse_ort = float(np.mean((e_ort - sm) ** 2))
    mse_iid_mc = float(np.mean((e_iid - sm) ** 2))
    assert abs(mse_iid_mc - mse_iid) < 4 * se(e_iid)          # Lemma 2 again, iid
    assert mse_ort < mse_iid - 3 * se(e_ort)                   # orthogonality helps
    assert mse_ort <= mse_iid - gap + 3 * se(e_ort)            # by at least the gap


def test_favor_converges_to_softmax_attention():
    """The estimator approximates equation 1 (exact softmax attention) and improves with m (section 4.2)."""
    B, H, L, d, dv = 1, 2, 64, 16, 16
    q = RNG.normal(size=(B, H, L, d)) * 0.6
    k = RNG.normal(size=(B, H, L, d)) * 0.6
    v = RNG.normal(size=(B, H, L, dv))
    exact = oracle.softmax_attention(q, k, v)
    errs = []
    for m in (16, 256, 4096):
        approx = bidir(q, k, v, make_omega(1, H, m, d))
        errs.append(float(np.sqrt(np.mean((approx - exact) ** 2))))
    assert errs[2] < errs[1] < errs[0]
    assert errs[2] < 0.02
    ex_c = oracle.softmax_attention(q, k, v, causal_mask=True)
    ap_c = causal(q, k, v, make_omega(1, H, 4096, d))
    assert float(np.sqrt(np.mean((ap_c - ex_c) ** 2))) < 0.03


def test_relu_features():
    """Equation 5 with f = ReLU: features are positive parts of omega.x scaled by 1/sqrt(m), plus eps."""
    d, m = 16, 32
    om = make_omega(4, 1, m, d)
    x = RNG.normal(size=(1, 1, 5, d))
    f0 = features(x, om, "relu", 0.0)
    f1 = features(x, om, "relu", 1e-3)
    assert np.all(f0 >= 0) and np.any(f0 == 0)
    assert np.allclose(f1 - f0, 1e-3, atol=1e-15)
    # positive rescaling of q (or k) cancels when eps = 0
    k = RNG.normal(size=(1, 1, 9, d))
    v = RNG.normal(size=(1, 1, 9, 4))
    a = bidir(x, k, v, om, "relu", 0.0)
    b = bidir(3.7 * x, 0.2 * k, v, om, "relu", 0.0)
    assert np.allclose(a, b, rtol=1e-12)


# ---------------------------------------------------------------- invariants

def test_invariants():
    B, H, L, d, dv, m = 1, 1, 31, 16, 8, 64
    q = RNG.normal(size=(B, H, L, d))
    k = RNG.normal(size=(B, H, L, d))
    v = RNG.normal(size=(B, H, L, dv))
    om = make_omega(21, H, m, d)
    out = bidir(q, k, v, om)
    # L = 1: the output is the single value
    assert np.allclose(bidir(q[:, :, :1], k[:, :, :1], v[:, :, :1], om), v[:, :, :1], atol=1e-15)
    # constant V gives that constant
    c = np.broadcast_to(RNG.normal(size=dv), v.shape)
    assert np.allclose(bidir(q, k, c, om), c, atol=1e-13)
    # identical keys: the mean of V
    kk = np.broadcast_to(k[:, :, :1], k.shape)
    assert np.allclose(bidir(q, kk, v, om), np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape), atol=1e-13)
    # linear in V
    v2 = RNG.normal(size=v.shape)
    assert np.allclose(bidir(q, k, 2.0 * v - v2, om), 2.0 * out - bidir(q, k, v2, om), atol=1e-12)
    # joint permutation of (K, V) rows leaves the bidirectional output unchanged
    p = RNG.permutation(L)
    assert np.allclose(bidir(q, k[:, :, p], v[:, :, p], om), out, atol=1e-13)
    # permuting the rows of Omega changes nothing
    pr = RNG.permutation(m)
    assert np.allclose(bidir(q, k, v, om[:, pr]), out, atol=1e-13)
    # outputs are convex combinations of values
    assert np.all(out <= v.max(axis=2, keepdims=True) + 1e-12)
    assert np.all(out >= v.min(axis=2, keepdims=True) - 1e-12)
