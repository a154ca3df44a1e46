"""Shared helpers of the GPU parity tests: device transfer of bf16 bits and the
comparison rules (output tolerances, the support rule with near ties)."""
from __future__ import annotations

import math
import sys

import numpy as np

import oracle

# Output tolerance for bf16 inputs (max-abs / mean-abs against the fp64 oracle).
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# Rows whose selection margin is within this of a boundary count as ties.
TIE_EPS = 1e-6


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_dev_to_f64(t) -> np.ndarray:
    import torch
    return oracle.bf16_to_f64(t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def compare_outputs(got: np.ndarray, ref: np.ndarray, what: str, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, mn = float(err.max()), float(err.mean())
    assert mx <= max_abs and mn <= mean_abs, f"{what}: max-abs {mx:.3e}, mean-abs {mn:.3e}"
    return mx, mn


def csr_rows(row_ptr: np.ndarray, col_idx: np.ndarray):
    return [col_idx[row_ptr[r]:row_ptr[r + 1]].tolist() for r in range(len(row_ptr) - 1)]


def tie_margin(mbar_row, q: int, eta: float) -> float:
    m = oracle.support_margins(mbar_row, q, eta)
    return min(2 * m["delta_rank"], m["delta_minus"], m["delta_plus"])


def support_ok(gpu_sup, mbar_row, q: int, eta: float, cap: int, tol_margin: float = TIE_EPS):
    """GPU support of one row against the oracle selection on the same masses.

    Equal supports pass.  A different support passes only for a near-tie row
    (a selection margin of Appendix A.1 within ``tol_margin``); it must still
    be ascending, hold the sink and the diagonal, and reach eta (up to
    ``tol_margin``) when no cap binds.
    """
    ref = oracle.select_support(mbar_row, q, eta, cap)
    if gpu_sup == ref:
        return True, False
    if tie_margin(mbar_row, q, eta) > tol_margin:
        return False, False
    valid = (gpu_sup == sorted(set(gpu_sup)) and 0 in gpu_sup and q in gpu_sup
             and all(0 <= b <= q for b in gpu_sup))
    if cap == 0:
        eta_part = [b for b in gpu_sup]
        valid = valid and sum(float(mbar_row[b]) for b in eta_part) >= eta - tol_margin
    return valid, True


def mass_tolerance(n_steps: int) -> float:
    """Absolute tolerance of accumulated fp32 block masses vs fp64.

    Each step's r_qb is a sum of fp32 probabilities normalised by an fp32 row
    sum; scores come from bf16 products accumulated in fp32 (relative error
    ~1e-6 on logits of size ~10, i.e. ~1e-5 relative on exp).  1e-5 per step
    bounds that with margin for r <= 1.
    """
    return 1e-5 * n_steps


def finite(x) -> bool:
    return bool(np.all(np.isfinite(x)))


def isclose_inf(a, b):
    return (math.isinf(a) and math.isinf(b)) or abs(a - b) < 1e-12
