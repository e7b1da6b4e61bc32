"""FAVOR+ oracle: a plain, slow, fp64 CPU statement of what the GPU library computes.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this package: only `tests/`, the smoke check in `__graft_entry__.py`
and the CPU-baseline leg of `bench.py` use it. It shares no code with the HIP
library (`random_feature_amd`), and it imports nothing from it.

Contents
  omega.py  the random-feature matrix Omega: orthogonal Gaussian blocks built by
            Gram-Schmidt with chi(d) row lengths (Performer paper, section 2.4
            and appendix B.2), drawn from a counter-based SplitMix64 stream.
            The bit-level recipe is fixed so that two independent
            implementations produce identical fp32 bits.
  favor.py  the feature maps (positive softmax features, Lemma 1, and their
            hyperbolic form; trigonometric features, equation 5 with sin and
            cos; ReLU features, appendix A.4), the bidirectional estimator (equation 4 /
            Algorithm 1), the causal estimator as the prefix-sum recurrence
            (appendix B.1 equation 11; the RNN form in the linear-attention
            blog's "Autoregressive Generation" section), the single-token
            decode step, the gated decode step of the RFA page (section 3.2)
            with its unrolled form, and exact softmax attention (equations
            1-2) for accuracy reports.

Every floating-point quantity is computed in fp64 from inputs that are
exactly representable (fp32 or bf16 values widened to fp64). No stabiliser is
used: fp64 covers the exponent range of every supported shape.

Pinning: every function here is checked by `tests/test_oracle_*.py` against
facts fixed by the pages or by mathematics (a worked example, brute force on
the explicit attention matrix, Monte-Carlo unbiasedness against Lemma 1 with
the variance of Lemma 2, orthogonality and chi-length statistics of Omega,
convergence to exact softmax attention as m grows, invariants).
"""
from .omega import make_omega, splitmix64_mix, stream_key, uniform52, gaussians, OMEGA_MODES
from .favor import (
    features, features_hyperbolic, features_trig, bidir, bidir_from_features, bidir_backward, causal, causal_backward, causal_bruteforce, causal_bruteforce_from_features,
    decode_step, decode_run, decode_gated_step, decode_gated_run, decode_gated_unrolled, state_from_prior,
    softmax_attention, attention_matrix, row_norm_rel_err,
)

__all__ = [
    "make_omega", "splitmix64_mix", "stream_key", "uniform52", "gaussians", "OMEGA_MODES",
    "features", "features_hyperbolic", "features_trig", "bidir", "bidir_from_features", "bidir_backward", "causal", "causal_backward", "causal_bruteforce",
    "causal_bruteforce_from_features", "decode_step", "decode_run", "decode_gated_step", "decode_gated_run",
    "decode_gated_unrolled", "state_from_prior",
    "softmax_attention", "attention_matrix", "row_norm_rel_err",
]
