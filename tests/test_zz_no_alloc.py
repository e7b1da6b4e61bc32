"""favor_bidir_noalloc (the library's own device workspace array, no allocation) against favor_bidir, through the
C ABI: two calls in a row on one device, the second smaller, so the second runs over what the first left in the
shared array."""
import pytest
import torch

import oracle
import workloads
from tests.gpu_helpers import TOL, rel_err

pytestmark = pytest.mark.gpu

rf = pytest.importorskip("random_feature_amd")

# (B, H, L, d, dv, m, dtype, seed): the headline workload's shape, then a smaller fp32 case with a ragged tail
CASES = [(8, 12, 4096, 64, 64, 256, torch.bfloat16, 2), (2, 3, 1000, 16, 16, 32, torch.float32, 5)]


def test_noalloc_matches_bidir_on_two_calls_in_a_row():
    for B, H, L, d, dv, m, dt, seed in CASES:
        print(f"noalloc case B{B} H{H} L{L} d{d} dv{dv} m{m} {dt}", flush=True)
        q = workloads.make_tensor((B, H, L, d), seed, 0.5, dt)
        k = workloads.make_tensor((B, H, L, d), seed + 1, 0.5, dt)
        v = workloads.make_tensor((B, H, L, dv), seed + 2, 1.0, dt)
        om = rf.make_omega(seed, H, m, d)
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        got = rf.bidir_noalloc(qd, kd, vd, om)
        torch.cuda.synchronize()
        ref = rf.bidir(qd, kd, vd, om)
        torch.cuda.synchronize()
        # the same kernels and launch plan over a different workspace: bit-identical
        assert torch.equal(got, ref)
        # and within the parity bound of the oracle on one (b,h) pair
        sl = (slice(B - 1, B), slice(H - 1, H))
        r = oracle.bidir(q[sl], k[sl], v[sl], om.cpu().numpy()[H - 1:H])
        assert rel_err(got[sl].cpu(), r) < TOL[dt]


def test_noalloc_refuses_a_workspace_beyond_its_array():
    B, H, L, d, dv, m = 64, 16, 4096, 64, 64, 256
    assert rf.workspace_size(False, B, H, L, d, dv, m, torch.bfloat16) > rf.NOALLOC_MAX_BYTES
    q = torch.zeros((B, H, L, d), dtype=torch.bfloat16, device="cuda")
    om = rf.make_omega(1, H, m, d)
    with pytest.raises(rf.FavorError, match="workspace too small"):
        rf.bidir_noalloc(q, q, q, om)
