"""Writes the stored expected values under tests/golden/ (calls only oracle/).

Run from the repository root:  python tests/golden/make_golden.py
The pages print no worked example for this path, so every stored value here is
the oracle's; the oracle itself is pinned in tests/test_oracle.py.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import schedule as S  # noqa: E402


def main():
    ab = S.alpha_bar(1000, 1e-4, 0.02)
    rows = []
    for t in [0, 1, 2, 19, 20, 21, 143, 286, 429, 500, 571, 714, 857, 999, 1000]:
        tp = S.prev_timestep(t, 20)
        c1, c2 = S.ddim_coefficients(t, tp, ab)
        rows.append({"t": t, "t_prev": tp, "c1": float(c1), "c2": float(c2)})
    out = {
        "_source": "oracle.schedule (DDPM linear betas 1e-4..0.02, T=1000; DDIM eta=0, stride 20); "
                   "written by tests/golden/make_golden.py",
        "schedule": {"T": 1000, "beta_start": 1e-4, "beta_end": 0.02, "stride": 20},
        "alpha_bar_1000": float(ab[1000]),
        "coefficients": rows,
    }
    with open(os.path.join(ROOT, "tests", "golden", "ddim_coefficients.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
