"""Derives the per-token verify cost of the high-concurrency workload with the oracle.

The workload asks for windows that shrink to 2-4 at B = 256, gamma = 16.  With the step
cost T(M) = 20 ms + theta * M (shape of the SGLang article's "Background" figure), this
script bisects theta on the seeded confidences until the oracle scheduler's mean window
is 3 (the middle of 2-4), and prints theta rounded to 4 significant digits.  The value is
stored as THETA_HIGH_CONCURRENCY in workloads/configs.py; test_workloads re-runs this
derivation and checks that the stored value still gives a mean window of 3.

Uses only oracle/ and the input generator.
"""

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

import oracle  # noqa: E402
from workloads import Inputs, get  # noqa: E402


def mean_window(a, gamma, B, theta_per_token, bias=20.0):
    theta = (np.float32(theta_per_token) * np.arange(B * gamma + 1, dtype=np.float32)).astype(np.float32)
    r = oracle.schedule_windows(a, gamma, bias, np.zeros(B + 1, np.float32), theta)
    return float(r["windows"].mean())


def derive():
    wl = get("high-conc-b256")
    inp = Inputs(wl)
    a = oracle.survival(inp.conf())
    lo, hi = 0.0, 1.0  # mean window(lo) > 3 >= mean window(hi)
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        if mean_window(a, wl.gamma, wl.B, mid) > 3.0:
            lo = mid
        else:
            hi = mid
    # 4 significant digits, rounded up so that the stored value is on the <= 3 side
    digits = 4 - 1 - int(np.floor(np.log10(hi)))
    theta = float(np.ceil(hi * 10 ** digits) / 10 ** digits)
    return round(theta, digits), mean_window(a, wl.gamma, wl.B, theta)


if __name__ == "__main__":
    th, mw = derive()
    print(f"THETA_HIGH_CONCURRENCY = {th}  (mean window {mw})")
