"""FAVOR+ attention, oracle side: fp64 NumPy, plain definitions, no stabiliser.

Shapes: q, k [B, H, L, d]; v [B, H, L, dv]; omega [H, m, d] (fp32 values).
Inputs may be fp32 or bf16 tensors/arrays; they are widened exactly to fp64.

Definitions followed (Performer paper, "Rethinking Attention with Performers",
unless stated otherwise):
  * scaling (section 2.3, under equation 6; also the Performer tutorial page,
    section 1): x = q * d^(-1/4), y = k * d^(-1/4), so x.y = q.k / sqrt(d);
  * positive random features (Lemma 1, equation 7, with the general form of
    equation 5, h(x) = exp(-|x|^2/2), f = exp):
        phi_r(x) = exp(omega_r . x - |x|^2 / 2) / sqrt(m);
  * ReLU features (equation 5 with h = 1, f = ReLU; the generalised-attention
    defaults of appendix A.4 add a small kernel epsilon to every feature):
        phi_r(x) = max(omega_r . x, 0) / sqrt(m) + eps;
  * trigonometric features (equation 5 with h(x) = exp(|x|^2/2), l = 2, f1 = sin,
    f2 = cos: the estimator SM^trig of section 2.3), m vectors -> 2m features:
        phi(x) = exp(|x|^2/2) / sqrt(m) (sin(w_1.x), ..., sin(w_m.x), cos(w_1.x), ..., cos(w_m.x));
  * bidirectional estimator (equation 4; Algorithm 1 with C = [V 1]):
        S = Phi_K^T V,  z = Phi_K^T 1,  out_i = (Phi_Q,i . S) / (Phi_Q,i . z);
  * causal estimator (appendix B.1, equation 11, prefix sums that include the
    diagonal; the same recurrence as the linear-attention blog's
    "Autoregressive Generation" section):
        S_i = S_{i-1} + phi(k_i) v_i^T,  z_i = z_{i-1} + phi(k_i),
        out_i = (phi(q_i) . S_i) / (phi(q_i) . z_i);
  * decode step (the same recurrence applied to one new token; RFA's
    recurrent form, appendix A.3 of the RFA summary page): the state is
    updated with token t first, and token t's output reads the updated state;
  * exact softmax attention (equations 1 and 2) for accuracy reports.
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x, work_dtype=np.float64) -> np.ndarray:
    """x widened exactly to fp64 (then rounded to work_dtype when that is narrower)."""
    if hasattr(x, "detach"):  # torch tensor (possibly bf16): widen exactly
        import torch
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(np.asarray(x, dtype=np.float64), dtype=work_dtype)


def features(x, omega, kind: str = "prf", eps: float = 0.0, work_dtype=np.float64) -> np.ndarray:
    """phi(x) for raw queries or keys x [B,H,L,d] and omega [H,m,d] -> [B,H,L,m] (fp64);
    kind "hyperbolic": the 2m hyperbolic features of the m rows (features_hyperbolic); kind "trig": the 2m
    trigonometric features of the m rows (features_trig). work_dtype = np.float32 evaluates the PRF and ReLU
    maps in fp32 instead (the same formulas; it shows what that precision loses, it is no reference)."""
    x = _f64(x, work_dtype)
    om = _f64(omega, work_dtype)
    d = x.shape[-1]
    m = om.shape[-2]
    xs = x * (float(d) ** -0.25)
    a = np.einsum("bhld,hmd->bhlm", xs, om)
    if kind == "prf":
        half_norm = 0.5 * np.sum(xs * xs, axis=-1, keepdims=True)
        return np.exp(a - half_norm) / math.sqrt(m)
    if kind == "relu":
        return np.maximum(a, 0.0) / math.sqrt(m) + eps
    if kind == "hyperbolic":  # the rows of omega are the random vectors; 2m features
        return features_hyperbolic(x, omega)
    if kind == "trig":  # likewise
        return features_trig(x, omega)
    raise ValueError(f"unknown feature kind {kind!r}")


def features_trig(x, omega) -> np.ndarray:
    """The trigonometric features (Performer paper, equation 5 with h(x) = exp(|x|^2/2), l = 2, f1 = sin,
    f2 = cos; section 2.3's SM^trig) for raw x [B,H,L,d] and the random vectors w_i = rows of omega [H,m,d]:
    with x scaled by d^-1/4,
        phi(x) = exp(|x|^2/2) / sqrt(m) * (sin(w_1.x), ..., sin(w_m.x), cos(w_1.x), ..., cos(w_m.x)),
    so phi(x).phi(y) = exp((|x|^2+|y|^2)/2) (1/m) sum_i cos(w_i.(x-y)). Returns [B,H,L,2m] (fp64)."""
    x = _f64(x)
    om = _f64(omega)
    d = x.shape[-1]
    m = om.shape[-2]
    xs = x * (float(d) ** -0.25)
    a = np.einsum("bhld,hmd->bhlm", xs, om)
    h = np.exp(0.5 * np.sum(xs * xs, axis=-1, keepdims=True)) / math.sqrt(m)
    return np.concatenate([h * np.sin(a), h * np.cos(a)], axis=-1)


def features_hyperbolic(x, omega) -> np.ndarray:
    """The hyperbolic positive features (Performer paper, Lemma 1, second form) for raw x [B,H,L,d] and the
    random vectors w_i = rows of omega [H,m,d]: with x scaled by d^-1/4,
        phi(x) = exp(-|x|^2/2) / sqrt(2m) * (exp(w_1.x), ..., exp(w_m.x), exp(-w_1.x), ..., exp(-w_m.x)),
    so phi(x).phi(y) = (1/m) sum_i exp(-(|x|^2+|y|^2)/2) cosh(w_i.(x+y)). Returns [B,H,L,2m] (fp64)."""
    x = _f64(x)
    om = _f64(omega)
    d = x.shape[-1]
    m = om.shape[-2]
    xs = x * (float(d) ** -0.25)
    a = np.einsum("bhld,hmd->bhlm", xs, om)
    h = np.exp(-0.5 * np.sum(xs * xs, axis=-1, keepdims=True)) / math.sqrt(2.0 * m)
    return np.concatenate([h * np.exp(a), h * np.exp(-a)], axis=-1)


def bidir_from_features(phi_q, phi_k, v):
    """Equation 4 from given features: returns (out, S, z)."""
    phi_q, phi_k, v = _f64(phi_q), _f64(phi_k), _f64(v)
    S = np.einsum("...lm,...le->...me", phi_k, v)
    z = np.sum(phi_k, axis=-2)
    num = np.einsum("...lm,...me->...le", phi_q, S)
    den = np.einsum("...lm,...m->...l", phi_q, z)
    return num / den[..., None], S, z


def bidir(q, k, v, omega, kind: str = "prf", eps: float = 0.0, renormalize: bool = True) -> np.ndarray:
    """Equation 4 (Algorithm 1): q [B,H,Lq,d] against k [B,H,Lk,d], v [B,H,Lk,dv] (Lq and Lk may differ: the
    RFA page's cross attention). renormalize=False drops D^-1 (Performer appendices A.3, D.3): the output is
    Phi_Q (Phi_K^T V) with the features in their own scale."""
    out, S, _ = bidir_from_features(features(q, omega, kind, eps), features(k, omega, kind, eps), v)
    if renormalize:
        return out
    return np.einsum("...lm,...me->...le", features(q, omega, kind, eps), S)


def _feature_backward(x, omega, phi, dphi, kind: str, work_dtype=np.float64):
    """d loss / d x (raw x) from d loss / d phi for the feature map of `features`.

    PRF: phi = exp(w.xs - |xs|^2/2)/sqrt(m), xs = d^-1/4 x, so
        d/dxs = Omega^T (phi * dphi) - xs * sum_r phi_r dphi_r;
    ReLU: phi = max(w.xs, 0)/sqrt(m) + eps, so d/dxs = Omega^T (1[w.xs > 0]/sqrt(m) * dphi).
    The chain rule through xs = d^-1/4 x multiplies by d^-1/4."""
    x = _f64(x, work_dtype)
    om = _f64(omega, work_dtype)
    d = x.shape[-1]
    m = om.shape[-2]
    s = float(d) ** -0.25
    xs = x * s
    if kind == "prf":
        pd = phi * dphi
        g = np.einsum("bhlm,hmd->bhld", pd, om) - xs * np.sum(pd, axis=-1, keepdims=True)
    elif kind == "relu":
        a = np.einsum("bhld,hmd->bhlm", xs, om)
        g = np.einsum("bhlm,hmd->bhld", (a > 0) * dphi / math.sqrt(m), om)
    else:
        raise ValueError(f"no backward for feature kind {kind!r}")
    return g * s


def bidir_backward(q, k, v, omega, dout, kind: str = "prf", eps: float = 0.0, work_dtype=np.float64):
    """Gradients of equation 4's output out = (Phi_Q S) / (Phi_Q z) (S = Phi_K^T V, z = Phi_K^T 1) with respect
    to the raw q, k and v, for the upstream gradient dout [B,H,L,dv]. By the chain rule, with N = Phi_Q S and
    D = Phi_Q z:
        dN = dout / D,  dD = -(dout . out) / D,
        dPhi_Q = dN S^T + dD z^T,  dS = Phi_Q^T dN,  dz = Phi_Q^T dD,
        dPhi_K = V dS^T + 1 dz^T,  dV = Phi_K dS,
    then through the feature map (_feature_backward). Returns (dq, dk, dv), fp64 (work_dtype = np.float32:
    every step in fp32 instead, to show what that precision loses; no reference)."""
    pq = features(q, omega, kind, eps, work_dtype)
    pk = features(k, omega, kind, eps, work_dtype)
    v = _f64(v, work_dtype)
    g = _f64(dout, work_dtype)
    S = np.einsum("...lm,...le->...me", pk, v)
    z = np.sum(pk, axis=-2)
    N = np.einsum("...lm,...me->...le", pq, S)
    D = np.einsum("...lm,...m->...l", pq, z)
    out = N / D[..., None]
    dN = g / D[..., None]
    dD = -np.sum(g * out, axis=-1) / D
    dpq = np.einsum("...le,...me->...lm", dN, S) + dD[..., None] * z[..., None, :]
    dS = np.einsum("...lm,...le->...me", pq, dN)
    dz = np.einsum("...lm,...l->...m", pq, dD)
    dpk = np.einsum("...le,...me->...lm", v, dS) + dz[..., None, :]
    dv = np.einsum("...lm,...me->...le", pk, dS)
    return (_feature_backward(q, omega, pq, dpq, kind, work_dtype), _feature_backward(k, omega, pk, dpk, kind, work_dtype),
            dv)


def causal(q, k, v, omega, kind: str = "prf", eps: float = 0.0, return_state: bool = False):
    """Causal estimator as the plain recurrence over positions (one token at a time)."""
    pq = features(q, omega, kind, eps)
    pk = features(k, omega, kind, eps)
    v = _f64(v)
    B, H, L, m = pq.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, m, dv))
    z = np.zeros((B, H, m))
    out = np.empty((B, H, L, dv))
    for i in range(L):
        S += pk[:, :, i, :, None] * v[:, :, i, None, :]
        z += pk[:, :, i, :]
        num = np.einsum("bhm,bhme->bhe", pq[:, :, i, :], S)
        den = np.einsum("bhm,bhm->bh", pq[:, :, i, :], z)
        out[:, :, i, :] = num / den[..., None]
    if return_state:
        return out, S, z
    return out


def causal_backward(q, k, v, omega, dout, kind: str = "prf", eps: float = 0.0, work_dtype=np.float64):
    """Gradients of the causal output (appendix B.1, equation 11: out_i = (Phi_Q,i . S_i) / (Phi_Q,i . z_i)
    with the prefix sums S_i = sum_{j<=i} phi(k_j) v_j^T, z_i = sum_{j<=i} phi(k_j)) with respect to the raw q,
    k and v, for the upstream gradient dout. By the chain rule, position by position:
        dN_i = dout_i / D_i,  dD_i = -(dout_i . out_i) / D_i,  dPhi_Q,i = S_i dN_i + z_i dD_i,
    and since S_i and z_i sum the keys j <= i, key j collects the suffix sums over i >= j:
        R_j = sum_{i>=j} Phi_Q,i dN_i^T,  r_j = sum_{i>=j} Phi_Q,i dD_i,
        dPhi_K,j = R_j v_j + r_j,  dV_j = R_j^T Phi_K,j,
    then through the feature map (_feature_backward). Returns (dq, dk, dv), fp64 (work_dtype as in
    bidir_backward)."""
    pq = features(q, omega, kind, eps, work_dtype)
    pk = features(k, omega, kind, eps, work_dtype)
    v = _f64(v, work_dtype)
    g = _f64(dout, work_dtype)
    # prefix states S_i [B,H,L,m,dv], z_i [B,H,L,m] (inclusive)
    S = np.cumsum(pk[..., :, None] * v[..., None, :], axis=-3)
    z = np.cumsum(pk, axis=-2)
    N = np.einsum("...lm,...lme->...le", pq, S)
    D = np.einsum("...lm,...lm->...l", pq, z)
    out = N / D[..., None]
    dN = g / D[..., None]
    dD = -np.sum(g * out, axis=-1) / D
    dpq = np.einsum("...lme,...le->...lm", S, dN) + z * dD[..., None]
    # suffix sums over i >= j (reverse cumulative sums)
    R = np.flip(np.cumsum(np.flip(pq[..., :, None] * dN[..., None, :], axis=-3), axis=-3), axis=-3)
    r = np.flip(np.cumsum(np.flip(pq * dD[..., None], axis=-2), axis=-2), axis=-2)
    dpk = np.einsum("...lme,...le->...lm", R, v) + r
    dv = np.einsum("...lme,...lm->...le", R, pk)
    return (_feature_backward(q, omega, pq, dpq, kind, work_dtype), _feature_backward(k, omega, pk, dpk, kind, work_dtype),
            dv)


def causal_bruteforce_from_features(phi_q, phi_k, v, rows: int | None = None):
    """Equation 2 applied to the explicit matrix A_hat = Phi_Q Phi_K^T, masked by tril."""
    phi_q, phi_k, v = _f64(phi_q), _f64(phi_k), _f64(v)
    L = phi_q.shape[-2]
    n = L if rows is None else min(rows, L)
    A = np.einsum("...im,...jm->...ij", phi_q[..., :n, :], phi_k)
    mask = np.tril(np.ones((n, L), dtype=bool))
    A = np.where(mask, A, 0.0)
    num = np.einsum("...ij,...je->...ie", A, v)
    den = np.sum(A, axis=-1)
    return num / den[..., None]


def causal_bruteforce(q, k, v, omega, kind: str = "prf", eps: float = 0.0, rows: int | None = None):
    return causal_bruteforce_from_features(features(q, omega, kind, eps), features(k, omega, kind, eps), v, rows)


def attention_matrix(q, k, omega, kind: str = "prf", eps: float = 0.0) -> np.ndarray:
    """The explicit normalised matrix D_hat^{-1} A_hat, A_hat = Phi_Q Phi_K^T ([B,H,L,L])."""
    A = np.einsum("bhim,bhjm->bhij", features(q, omega, kind, eps), features(k, omega, kind, eps))
    return A / np.sum(A, axis=-1, keepdims=True)


def decode_step(S, z, q, k, v, omega, kind: str = "prf", eps: float = 0.0):
    """One token for every (sequence, head): S [N,H,m,dv], z [N,H,m], q,k [N,H,d], v [N,H,dv].

    Returns (S', z', out) with the state updated first and out read from it.
    """
    S = _f64(S)
    z = _f64(z)
    pq = features(_f64(q)[:, :, None, :], omega, kind, eps)[:, :, 0, :]
    pk = features(_f64(k)[:, :, None, :], omega, kind, eps)[:, :, 0, :]
    v = _f64(v)
    S2 = S + pk[..., :, None] * v[..., None, :]
    z2 = z + pk
    num = np.einsum("nhm,nhme->nhe", pq, S2)
    den = np.einsum("nhm,nhm->nh", pq, z2)
    return S2, z2, num / den[..., None]


def decode_run(S, z, q_steps, k_steps, v_steps, omega, kind: str = "prf", eps: float = 0.0):
    """Several decode steps; q_steps [T,N,H,d] etc. Returns (S_T, z_T, outs [T,N,H,dv])."""
    q_steps, k_steps, v_steps = _f64(q_steps), _f64(k_steps), _f64(v_steps)
    S = _f64(S)
    z = _f64(z)
    outs = np.empty(q_steps.shape[:3] + (v_steps.shape[-1],))
    for t in range(q_steps.shape[0]):
        S, z, outs[t] = decode_step(S, z, q_steps[t], k_steps[t], v_steps[t], omega, kind, eps)
    return S, z, outs


def decode_gated_step(S, z, q, k, v, omega, gate, in_weight=None, kind: str = "prf", eps: float = 0.0):
    """One gated step (RFA page, section 3.2, RFA-GATE): the historical state of every (sequence, head)
    decays by its scalar gate g, in the value state and the normalisation state alike, and the new token
    enters with weight w (1 unless given; RFA's own choice is w = 1 - g):
        S' = g S + w phi(k) v^T,  z' = g z + w phi(k);  out = phi(q).S' / phi(q).z'.
    gate, in_weight: [N,H]. Returns (S', z', out)."""
    S = _f64(S)
    z = _f64(z)
    g = _f64(gate)
    w = np.ones_like(g) if in_weight is None else _f64(in_weight)
    pq = features(_f64(q)[:, :, None, :], omega, kind, eps)[:, :, 0, :]
    pk = features(_f64(k)[:, :, None, :], omega, kind, eps)[:, :, 0, :]
    v = _f64(v)
    S2 = g[..., None, None] * S + (w[..., None] * pk)[..., :, None] * v[..., None, :]
    z2 = g[..., None] * z + w[..., None] * pk
    num = np.einsum("nhm,nhme->nhe", pq, S2)
    den = np.einsum("nhm,nhm->nh", pq, z2)
    return S2, z2, num / den[..., None]


def decode_gated_run(S, z, q_steps, k_steps, v_steps, omega, gates, in_weights=None, kind: str = "prf",
                     eps: float = 0.0):
    """Several gated steps; gates (and in_weights) [T,N,H]. Returns (S_T, z_T, outs [T,N,H,dv])."""
    q_steps, k_steps, v_steps = _f64(q_steps), _f64(k_steps), _f64(v_steps)
    S = _f64(S)
    z = _f64(z)
    outs = np.empty(q_steps.shape[:3] + (v_steps.shape[-1],))
    for t in range(q_steps.shape[0]):
        w = None if in_weights is None else in_weights[t]
        S, z, outs[t] = decode_gated_step(S, z, q_steps[t], k_steps[t], v_steps[t], omega, gates[t], w, kind, eps)
    return S, z, outs


def decode_gated_unrolled(S0, z0, q_steps, k_steps, v_steps, omega, gates, in_weights=None, kind: str = "prf",
                          eps: float = 0.0):
    """The gated recurrence written out: at step t token j <= t carries the weight
    c_tj = w_j * prod_{j < l <= t} g_l and the initial state prod_{l <= t} g_l, so
    out_t = phi(q_t).(c_t0' S0 + sum_j c_tj phi(k_j) v_j^T) / phi(q_t).(c_t0' z0 + sum_j c_tj phi(k_j)).
    Returns outs [T,N,H,dv]."""
    S0, z0 = _f64(S0), _f64(z0)
    g = _f64(gates)
    T = g.shape[0]
    w = np.ones_like(g) if in_weights is None else _f64(in_weights)
    pq = np.stack([features(_f64(q_steps[t])[:, :, None, :], omega, kind, eps)[:, :, 0, :] for t in range(T)])
    pk = np.stack([features(_f64(k_steps[t])[:, :, None, :], omega, kind, eps)[:, :, 0, :] for t in range(T)])
    v = _f64(v_steps)
    outs = np.empty(v.shape)
    for t in range(T):
        c0 = np.prod(g[:t + 1], axis=0)                                   # [N,H]
        num = np.einsum("nhm,nhme->nhe", pq[t], S0) * c0[..., None]
        den = np.einsum("nhm,nhm->nh", pq[t], z0) * c0
        for j in range(t + 1):
            c = w[j] * np.prod(g[j + 1:t + 1], axis=0)                    # [N,H]
            a = np.einsum("nhm,nhm->nh", pq[t], pk[j]) * c
            num += a[..., None] * v[j]
            den += a
        outs[t] = num / den[..., None]
    return outs


def state_from_prior(k_prior, v_prior, omega, kind: str = "prf", eps: float = 0.0):
    """The canonical state after a prefix of tokens: S = sum_j phi(k_j) v_j^T, z = sum_j phi(k_j).

    k_prior [N,H,P,d], v_prior [N,H,P,dv] -> S [N,H,m,dv], z [N,H,m] (fp64).
    """
    pk = features(k_prior, omega, kind, eps)
    v = _f64(v_prior)
    return np.einsum("nhpm,nhpe->nhme", pk, v), np.sum(pk, axis=-2)


def softmax_attention(q, k, v, causal_mask: bool = False) -> np.ndarray:
    """Exact attention, equations 1 (bidirectional) and 2 (unidirectional)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    d = q.shape[-1]
    logits = np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(d)
    if causal_mask:
        L = logits.shape[-1]
        logits = np.where(np.tril(np.ones((L, L), dtype=bool)), logits, -np.inf)
    logits = logits - np.max(logits, axis=-1, keepdims=True)  # exact: cancels in the ratio
    A = np.exp(logits)
    return np.einsum("bhij,bhje->bhie", A, v) / np.sum(A, axis=-1)[..., None]


def row_norm_rel_err(out, ref) -> float:
    """max over rows of ||out_i - ref_i||_inf / ||ref_i||_inf (rows = last axis)."""
    out = _f64(out)
    ref = _f64(ref)
    num = np.max(np.abs(out - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return float(np.max(num / den))
