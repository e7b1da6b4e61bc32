"""What storing partial sums in bf16 costs, measured on the oracle's own features (no GPU).

For bf16 inputs the bidirectional path keeps each piece's partial S_aug = Phi_K^T [V 1] in bf16 and sums the
pieces in fp32, and the causal path keeps its carries (and, without a final state, its segment partials) in bf16;
either sum is then rounded to bf16 once more before any product uses it. The claim is that this adds less error to
an output row than rounding the output itself to bf16 does, and leaves the bf16 bound (2e-2) a wide margin. Here
the oracle's fp64 features of a headline-shaped (b,h) (L = 4096 keys in five pieces, m = 256, q, k ~
N(0,1)/sqrt(2)) give the exact output; the same output with S_aug rounded to bf16 once (fp32 partials), and with
S_aug summed from bf16-rounded partials and then rounded, are compared against it row-normwise, beside the bf16
rounding of the exact output (about 5.2e-3, 6.6e-3 and 3.8e-3). Nothing here involves the HIP path.
"""
import numpy as np
import torch

import oracle
import workloads


def _bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 (ties to even), back in fp64."""
    return torch.from_numpy(np.asarray(x, np.float32)).bfloat16().double().numpy()


def _rowerr(a, r):
    return float(np.max(np.max(np.abs(a - r), axis=-1) / np.max(np.abs(r), axis=-1)))


def test_bf16_partials_cost_less_than_the_bf16_output():
    d, dv, m, L, pieces = 64, 64, 256, 4096, 5
    q = workloads.make_tensor((1, 1, L, d), 31, 0.7071, torch.bfloat16)
    k = workloads.make_tensor((1, 1, L, d), 32, 0.7071, torch.bfloat16)
    v = workloads.make_tensor((1, 1, L, dv), 33, 1.0, torch.bfloat16)
    om = oracle.make_omega(2, 1, m, d)
    pq = oracle.features(q, om)[0, 0]
    pk = oracle.features(k, om)[0, 0]
    va = np.concatenate([np.asarray(v[0, 0].double()), np.ones((L, 1))], axis=1)  # [V 1]
    s_exact = pk.T @ va
    out_exact = pq @ s_exact[:, :dv] / (pq @ s_exact[:, dv:])
    cuts = np.linspace(0, L, pieces + 1).astype(int)
    # each piece's sums rescaled to a common maximum before rounding, as the kernels store them (the scale is a
    # power of two per piece, which bf16 represents exactly, so the test can leave it out)
    s_part = sum(_bf16(pk[a:b].T @ va[a:b]) for a, b in zip(cuts[:-1], cuts[1:]))
    s_used = _bf16(s_part)  # the contraction operand
    out_part = pq @ s_used[:, :dv] / (pq @ s_used[:, dv:])
    err_partials = _rowerr(out_part, out_exact)
    # reference points: S_aug rounded to bf16 once (the operand without bf16 partials), and the bf16 output
    s_once = _bf16(s_exact)
    err_once = _rowerr(pq @ s_once[:, :dv] / (pq @ s_once[:, dv:]), out_exact)
    err_output = _rowerr(_bf16(out_exact), out_exact)
    print(f"row-normwise error: bf16 partials {err_partials:.2e}, S_aug rounded once {err_once:.2e}, "
          f"bf16 output {err_output:.2e}")
    assert err_partials - err_once < err_output  # the partials' rounding adds less than the output's own
    assert err_partials < 1e-2                   # half the bf16 bound
