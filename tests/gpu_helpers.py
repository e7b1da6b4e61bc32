"""Shared helpers for the GPU parity tests (comparison metric and tolerances)."""
import numpy as np
import torch

# Tolerances on the row-normwise relative error  max_i ||o_i - ref_i||_inf / ||ref_i||_inf:
# fp32 paths 1e-4, bf16 inputs with fp32 accumulation 2e-2.
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def rel_err(out, ref) -> float:
    o = out.detach().float().cpu().double().numpy() if isinstance(out, torch.Tensor) else np.asarray(out, np.float64)
    r = ref.detach().cpu().double().numpy() if isinstance(ref, torch.Tensor) else np.asarray(ref, np.float64)
    assert o.shape == r.shape, (o.shape, r.shape)
    assert np.all(np.isfinite(o)), "non-finite output"
    num = np.max(np.abs(o - r), axis=-1)
    den = np.max(np.abs(r), axis=-1)
    return float(np.max(num / den))


def cuda_ok() -> bool:
    return torch.cuda.is_available()
