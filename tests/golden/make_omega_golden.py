"""Writes omega_spec.json: selected fp32 bit patterns of the oracle's Omega for a few seeds.

Calls only the oracle. Regenerate with `python tests/golden/make_omega_golden.py`
after a deliberate change of the Omega recipe (and say why in the commit).
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import make_omega  # noqa: E402

CASES = [
    dict(seed=0, H=1, m=32, d=16, mode="ortho_chi"),
    dict(seed=1, H=2, m=128, d=16, mode="ortho_chi"),
    dict(seed=2, H=2, m=256, d=64, mode="ortho_chi"),
    dict(seed=5, H=1, m=40, d=16, mode="ortho_sqrtd"),
    dict(seed=6, H=1, m=24, d=8, mode="iid"),
    dict(seed=2**64 - 1, H=1, m=16, d=16, mode="ortho_chi"),
]


def main():
    out = []
    for c in CASES:
        om = make_omega(c["seed"], c["H"], c["m"], c["d"], c["mode"])
        bits = om.view(np.uint32).reshape(-1)
        n = bits.size
        idx = sorted({0, 1, c["d"] - 1, c["d"], n // 3, n // 2, n - c["d"], n - 1})
        out.append(dict(c, indices=idx, bits=[int(bits[i]) for i in idx]))
    with open(os.path.join(HERE, "omega_spec.json"), "w") as f:
        json.dump({"source": "oracle/omega.py recipe (Performer section 2.4 and appendix B.2, F.4)",
                   "cases": out}, f, indent=1)


if __name__ == "__main__":
    main()
