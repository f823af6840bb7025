"""Shared helpers of the GPU parity tests: run the HIP path (through the C
ABI) and the oracle on the same seeded inputs and compare.

Tolerances: rel-L2 <= 1e-4 for F32 models, 1e-2 for BF16 / Q8 models, per
tensor per step.  Greedy codes must match exactly; under teacher forcing a
decision may only differ from the oracle's where the oracle's top-1/top-2
margin is below 4x the measured logit error (a near-tie), and every such
case is reported.
"""
from __future__ import annotations

import numpy as np

TOL_F32 = 1e-4
TOL_BF16 = 1e-2


def tol_for(m):
    return TOL_F32 if (not m.act_bf16 and m.lin == 0) else TOL_BF16


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def margin(logits) -> float:
    s = np.sort(np.asarray(logits, np.float64))
    return float(s[-1] - s[-2])


def code_mismatches(gpu_codes, ref_codes, ref_logits, gpu_logits):
    """(f, b, j, margin, err) for every differing decision.

    ref_logits / gpu_logits: callables (f, b, j) -> logits deciding code j of
    frame f of stream b."""
    bad = []
    for f, b, j in zip(*np.nonzero(gpu_codes != ref_codes)):
        rl, gl = ref_logits(f, b, j), gpu_logits(f, b, j)
        bad.append((int(f), int(b), int(j), margin(rl), float(np.max(np.abs(rl - gl)))))
    return bad


def assert_near_ties_only(bad, label):
    for f, b, j, mg, err in bad:
        print(f"[{label}] code flip frame {f} stream {b} code {j}: oracle margin {mg:.3e}, "
              f"max |dlogit| {err:.3e}", flush=True)
        assert mg <= 4 * err, f"{label}: decision differs with margin {mg} > 4 x {err}"
