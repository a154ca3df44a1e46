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


def run_trajectory(cfg, steps):
    """All four library calls over a list of (t, q, k, v) steps (bf16 bits)."""
    import torch
    import block_sparse_attention_wise_amd as wise
    nb = cfg.n_blocks
    mass = torch.zeros(cfg.batch, cfg.heads, nb, nb, dtype=torch.float32, device="cuda")
    outs = []
    row_ptr = col_idx = None
    for t, q, k, v in steps:
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        if t < cfg.td:
            outs.append(wise.wise_full_attn_accum(qd, kd, vd, mass, cfg.block))
        else:
            if row_ptr is None:
                row_ptr, col_idx = wise.wise_select_support(mass, cfg.td, cfg.eta, cfg.head_dim,
                                                            cfg.block, cfg.cap)
            outs.append(wise.wise_sparse_attn(qd, kd, vd, row_ptr, col_idx, cfg.block))
    torch.cuda.synchronize()
    return mass, row_ptr, col_idx, outs


def check_selection_every_row(cfg, gpu_mass, gpu_rows):
    """Every CSR row against the oracle's selection on the GPU's own masses.

    ``gpu_mass`` is the accumulated fp32 mass [batch, heads, nB, nB] and
    ``gpu_rows`` the CSR rows in (batch, head, query block) order.  Both
    sides select on the same fp32 masses divided by td, so the rows must be
    equal; only a row whose Appendix A.1 margin min(2 delta_rank,
    delta_minus, delta_plus) on those masses is within TIE_EPS may differ,
    and then it must still be a valid support.  Returns the number of such
    near-tie rows that differ.
    """
    nb, td = cfg.n_blocks, cfg.td
    ties = 0
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            for qb in range(nb):
                r = (b * cfg.heads + h) * nb + qb
                mbar = gpu_mass[b, h, qb].astype(np.float64) / td
                ok, tie = support_ok(gpu_rows[r], mbar, qb, cfg.eta, cfg.cap)
                assert ok, (b, h, qb, gpu_rows[r], oracle.select_support(mbar, qb, cfg.eta, cfg.cap))
                ties += int(tie)
    return ties


def check_trajectory_rows(cfg, gpu_mass, gpu_rows, gpu_outs, samples, head_steps_fn,
                          out_steps=None):
    """Compare sampled (b, h, q) rows of a GPU trajectory with the oracle.

    Masses within tolerance.  Supports equal to the oracle's (fp64 masses
    from the same bf16 inputs), except in a near-tie row: the oracle's
    Appendix A.1 margin min(2 delta_rank, delta_minus, delta_plus) within
    TIE_EPS of the selection threshold.  Such a row must then be the
    oracle's selection on the GPU's own masses.  Outputs within tolerance,
    recomputed with the GPU's support where it differs.
    """
    nb, td, B = cfg.n_blocks, cfg.td, cfg.block
    sc = oracle.default_scale(cfg.head_dim)
    by_head = {}
    for (b, h, qb) in samples:
        by_head.setdefault((b, h), []).append(qb)
    stats = {"rows": 0, "margin_rows": 0, "max_abs": 0.0, "mean_abs": []}
    for (b, h), qbs in by_head.items():
        steps = [(q, k, v) for _, (q, k, v) in head_steps_fn(b, h)]
        steps64 = [tuple(oracle.bf16_to_f64(x) for x in s) for s in steps]
        ref = oracle.trajectory_head(steps64, td, B, cfg.eta, cfg.cap, qblocks=qbs, out_rows=False)
        for i, qb in enumerate(qbs):
            r = (b * cfg.heads + h) * nb + qb
            gm = gpu_mass[b, h, qb].astype(np.float64)
            err = np.abs(gm - ref["mass_sum"][i])
            assert err.max() <= mass_tolerance(td), (b, h, qb, err.max())
            mbar_gpu = gm / td
            mbar_ref = ref["mass_mean"][i]
            sup_gpu = gpu_rows[r]
            sup_ref = ref["supports"][qb]
            if sup_gpu != sup_ref:
                margin = tie_margin(mbar_ref, qb, cfg.eta)
                assert margin <= TIE_EPS, (b, h, qb, sup_gpu, sup_ref, margin)
                assert sup_gpu == oracle.select_support(mbar_gpu, qb, cfg.eta, cfg.cap), (b, h, qb, sup_gpu)
                stats["margin_rows"] += 1
            stats["rows"] += 1
            rows = np.arange(qb * B, (qb + 1) * B)
            for t in (range(cfg.steps) if out_steps is None else out_steps):
                Q, K, V = steps64[t]
                if t < td:
                    want = oracle.dense_attention(Q, K, V, sc, rows)
                else:
                    want = oracle.masked_attention(Q, K, V, {qb: sup_gpu}, B, sc, rows)
                got = gpu_outs(t, b, h, rows)
                mx, mn = compare_outputs(got, want, f"O t{t} b{b}h{h}q{qb}")
                stats["max_abs"] = max(stats["max_abs"], mx)
                stats["mean_abs"].append(mn)
    return stats
