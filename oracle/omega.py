"""Random-feature matrix Omega, oracle side (pure Python, fp64).

What the pages fix (Performer paper, "Rethinking Attention with Performers"):
  * section 2.3 / Lemma 1: the rows omega_r of Omega are drawn from N(0, I_d);
  * section 2.4 (ORFs): the rows are made exactly orthogonal with the standard
    Gram-Schmidt procedure, which keeps each row's marginal distribution;
    this needs m <= d, so for m > d (appendix B.2) independent orthogonal
    blocks of d rows are stacked;
  * appendix F.4 (orthogonal Monte Carlo estimator): marginally each
    orthogonal row is still distributed as N(0, I_d), i.e. its direction is
    uniform and its length independent and chi(d)-distributed;
  * section 2.3 under Lemma 1: the regularised softmax kernel (SMREG) instead
    puts every row on the sphere of radius sqrt(d).

What the pages leave open, and the reading taken here (one recipe, so that the
library's host code and this oracle produce the same fp32 bits):
  * random stream: SplitMix64 (Steele, Lea and Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014) used as a counter-based
    generator: draw i of a stream with key K is mix(K + (i+1)*GAMMA) mod 2^64;
  * stream key for (seed, head h, block b, stream s):
        K = mix(seed XOR mix(h*2^40 + b*2^8 + s)),
    stream 0 fills the block's d x d Gaussian matrix G row by row, stream 1
    fills a second d x d Gaussian matrix N whose row norms are the chi(d)
    lengths;
  * uniforms: u = ((x >> 12) + 0.5) * 2^-52, strictly inside (0, 1);
  * Gaussians: Box-Muller on consecutive pairs (u1, u2):
        r = sqrt(-2 log u1),  g0 = r cos(2 pi u2),  g1 = r sin(2 pi u2),
    with the C library's log, cos, sin and a correctly rounded sqrt;
  * orthogonalisation: modified Gram-Schmidt over the rows of G in order,
    every dot product summed left to right from 0.0, no fused multiply-add,
    the normalisation a true division by the norm;
  * row r = b*d + i of Omega is ||N_i|| * q_i (mode "ortho_chi"), sqrt(d) * q_i
    (mode "ortho_sqrtd") or G_i unchanged (mode "iid"); rows beyond m are
    dropped (the last block is truncated when d does not divide m);
  * the fp64 row is rounded to fp32 with round-to-nearest-even.

Python floats are IEEE binary64 with round-to-nearest and `math.log`,
`math.cos`, `math.sin` call the platform C library, so this file follows the
recipe operation for operation. (NumPy's vectorised transcendentals are not
used because they may differ from the C library in the last bit.)
"""
from __future__ import annotations

import math
from functools import lru_cache

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
TWO_PI = 6.283185307179586  # the binary64 value nearest to 2*pi (== 2 * math.pi)
OMEGA_MODES = {"ortho_chi": 0, "iid": 1, "ortho_sqrtd": 2, "hyperbolic": 3, "trig_pairs": 4}


def splitmix64_mix(z: int) -> int:
    """SplitMix64 output function (the published variant-13 mixing constants)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, head: int, block: int, stream: int) -> int:
    tag = ((head << 40) + (block << 8) + stream) & MASK64
    return splitmix64_mix((seed & MASK64) ^ splitmix64_mix(tag))


def draw_u64(key: int, i: int) -> int:
    return splitmix64_mix((key + (i + 1) * GAMMA) & MASK64)


def uniform52(key: int, i: int) -> float:
    return (float(draw_u64(key, i) >> 12) + 0.5) * (2.0 ** -52)


def gaussians(key: int, n: int) -> list:
    """n standard normal draws of one stream (Box-Muller on consecutive uniform pairs)."""
    out = []
    for p in range((n + 1) // 2):
        u1 = uniform52(key, 2 * p)
        u2 = uniform52(key, 2 * p + 1)
        r = math.sqrt(-2.0 * math.log(u1))
        t = TWO_PI * u2
        out.append(r * math.cos(t))
        out.append(r * math.sin(t))
    return out[:n]


def _gram_schmidt_rows(G: list, d: int) -> list:
    """Modified Gram-Schmidt on the rows of G, in order (fp64, left-to-right sums)."""
    Q = []
    for i in range(d):
        v = list(G[i])
        for qj in Q:
            c = 0.0
            for t in range(d):
                c += v[t] * qj[t]
            for t in range(d):
                v[t] = v[t] - c * qj[t]
        s = 0.0
        for t in range(d):
            s += v[t] * v[t]
        nrm = math.sqrt(s)
        Q.append([v[t] / nrm for t in range(d)])
    return Q


def _block_rows(seed: int, head: int, block: int, d: int, mode: int) -> list:
    g = gaussians(stream_key(seed, head, block, 0), d * d)
    G = [g[i * d:(i + 1) * d] for i in range(d)]
    if mode == 1:  # iid: the Gaussian rows themselves
        return G
    Q = _gram_schmidt_rows(G, d)
    if mode == 2:  # regularised softmax kernel: every row has length sqrt(d)
        ln = math.sqrt(float(d))
        return [[ln * x for x in q] for q in Q]
    nvals = gaussians(stream_key(seed, head, block, 1), d * d)
    rows = []
    for i in range(d):
        s = 0.0
        for t in range(d):
            x = nvals[i * d + t]
            s += x * x
        ln = math.sqrt(s)
        rows.append([ln * x for x in Q[i]])
    return rows


@lru_cache(maxsize=64)
def _make_omega_cached(seed: int, H: int, m: int, d: int, mode: int) -> bytes:
    if mode == 3:
        # hyperbolic positive features (Performer paper, Lemma 1, second form): the m/2 vectors of the
        # orthogonal chi(d) mode, then their negatives, so that the positive feature map over these m rows
        # is exp(-|x|^2/2)/sqrt(m) (exp(w_i.x), exp(-w_i.x))
        if m % 2:
            raise ValueError("hyperbolic mode needs an even m")
        half = np.frombuffer(_make_omega_cached(seed, H, m // 2, d, 0), dtype=np.float32).reshape(H, m // 2, d)
        return np.concatenate([half, -half], axis=1).tobytes()
    if mode == 4:
        # trigonometric features (Performer paper, equation 5 with f1 = sin, f2 = cos): the m/2 vectors of the
        # orthogonal chi(d) mode, then the same rows again; a feature map that takes the sine of the first m/2
        # projections and the cosine of the last m/2 gives the 2(m/2) features of those m/2 vectors
        if m % 2:
            raise ValueError("trig_pairs mode needs an even m")
        half = np.frombuffer(_make_omega_cached(seed, H, m // 2, d, 0), dtype=np.float32).reshape(H, m // 2, d)
        return np.concatenate([half, half], axis=1).tobytes()
    out = np.empty((H, m, d), dtype=np.float32)
    nblocks = (m + d - 1) // d
    for h in range(H):
        r = 0
        for b in range(nblocks):
            rows = _block_rows(seed, h, b, d, mode)
            for i in range(d):
                if r >= m:
                    break
                out[h, r, :] = np.array(rows[i], dtype=np.float64).astype(np.float32)
                r += 1
    return out.tobytes()


def make_omega(seed: int, H: int, m: int, d: int, mode: str = "ortho_chi") -> np.ndarray:
    """Omega as fp32 [H, m, d]: head h's rows are the random features omega_r of that head."""
    mode_id = OMEGA_MODES[mode] if isinstance(mode, str) else int(mode)
    buf = _make_omega_cached(int(seed), int(H), int(m), int(d), mode_id)
    return np.frombuffer(buf, dtype=np.float32).reshape(H, m, d).copy()
