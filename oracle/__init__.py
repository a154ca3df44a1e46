"""fp64 CPU oracle of the WISE working-set attention path.

TEST INFRASTRUCTURE ONLY.  This package is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``,
and by nothing else.  It shares no code with the HIP library: it neither
imports it nor is imported by it.  The GPU path must never fall back to it.

What it computes is the plain definition from "Attention Routing Stabilizes
Early: Working-Set Inference for Recurrent Language Models" (WISE), written
out in float64 with numpy, in the order the paper states it:

* Section 3, Eq. (2): masked softmax attention A = softmax(Q K^T / sqrt(d_h) + M),
  O = A V, with M the causal mask (key j admissible for query i iff j <= i).
* Section 5.1, Eq. (5): block mass r_qb = (1/|I_q|) sum_{i in I_q} sum_{j in I_b} A_ij.
* Section 5.1, Eq. (6) (right-hand part) and Appendix A.1, Eq. (12): the
  cumulative-eta block support, the smallest set of admissible key blocks
  whose mass reaches eta.  Here it is applied once to the mean of the block
  masses over the discovery steps, then the sink block 0 and the diagonal
  block q are added (readings listed below).
* Section 5.2, Eq. (7)-(8): working-set mask R and late-step attention
  softmax(Q K^T / sqrt(d_h) + M + R) V.
* Appendix A.1, Eq. (13): identification margins delta_rank, delta_minus,
  delta_plus and Delta_q, used to tell near-tie rows from decided ones.
* Section 7 ("Evaluation metrics") and Appendix C.2, Eq. (23)-(25):
  retained future attention mass of a frozen support, the rolling working
  set and the Jaccard similarity of two working-set collections.

Readings where the paper leaves a step open (all of them also written out
with their reasons in the design notes):

1. Discovery steps are combined by averaging r over the td dense steps, then
   one selection runs on the mean (the temporal union of per-step supports is
   a separate variant).
2. Ties in the ranking are broken by the lower key-block index.
3. The threshold test is inclusive (mass >= eta), in float64.
4. Sink (block 0) and diagonal (block q) are added after the eta selection and
   do not count toward eta; the cap, if any, limits only the eta-ranked part.
5. Blocks are consecutive runs of B positions from position 0, so when S is
   not a multiple of B the last block is shorter (n_blocks = ceil(S / B)).
   |I_q| in Eq. (5) is the number of queries block q actually holds: B, or
   S - (n_blocks - 1) B for a short last block.  The diagonal block's mass
   counts only admissible keys j <= i.
6. If rounding leaves the total admissible mass below eta, every admissible
   block is kept.
7. Selection variants (Eq. (6) left / Eq. (18) temporal union; Appendix B
   controls Eq. (19)-(22)) take single-step block masses r^(t) and work on the
   eta-ranked part only; the sink and diagonal blocks are added to every
   variant's result afterwards, as for the main selection.  The union is over
   the steps passed in (the paper's window is the last four discovery steps);
   "the first recurrent step" of the controls is the first discovery step
   (0-based step 0).  m_q^WISE and K_q of Eq. (20) and (22) are taken over the
   union's eta-ranked part, and m_q^WISE is summed in float64.
8. Diagnostics use the working sets as the method builds them (sink and
   diagonal included); Eq. (23)'s window max(1, t-3)..t is max(0, t-3)..t
   with 0-based steps; the Jaccard of Eq. (24)/(25) pools the (row, key
   block) pairs of one example before dividing.

Inputs are float64 arrays (``bf16_to_f64`` widens bf16 bits exactly).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "bf16_to_f64", "default_scale", "n_blocks", "block_rows", "attention_weights", "attention_output",
    "dense_attention", "block_mass", "block_mass_rows", "mean_block_mass",
    "select_support", "support_margins", "working_set_mask",
    "eta_support", "topk_support", "select_union", "select_static",
    "select_mass_matched", "select_size_matched", "retained_mass",
    "rolling_working_set", "jaccard",
    "masked_attention_weights", "masked_attention", "trajectory_head",
]


def bf16_to_f64(bits) -> np.ndarray:
    """Widen raw bf16 bits (uint16) exactly to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def default_scale(head_dim: int) -> float:
    """1/sqrt(d_h), the softmax temperature of Eq. (2)."""
    return 1.0 / math.sqrt(head_dim)


def _rows(S: int, rows) -> np.ndarray:
    return np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)


def n_blocks(S: int, block: int) -> int:
    """Number of blocks of a length-S sequence, the last one possibly short (reading 5)."""
    return -(-S // block)


def block_rows(qb: int, block: int, S: int) -> np.ndarray:
    """Positions I_q of block qb: qb*B .. min(S, (qb+1)*B) - 1 (reading 5)."""
    return np.arange(qb * block, min(S, (qb + 1) * block))


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax of a logit matrix whose inadmissible entries are -inf."""
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def attention_weights(q, k, scale: float, rows=None) -> np.ndarray:
    """Rows ``rows`` of A = softmax(q k^T * scale + M), Eq. (2), causal M.

    q, k: float64 [S, D] of one (batch, head).  Returns [len(rows), S];
    entry (i, j) is zero for j > i.
    """
    S = k.shape[0]
    r = _rows(S, rows)
    s = (q[r] @ k.T) * scale
    causal = np.arange(S)[None, :] > r[:, None]          # M_ij = -inf for j > i
    s[causal] = -np.inf
    return _softmax_rows(s)


def attention_output(a, v) -> np.ndarray:
    """O = A V, Eq. (2)."""
    return a @ v


def dense_attention(q, k, v, scale: Optional[float] = None, rows=None) -> np.ndarray:
    """Dense causal attention output rows, Eq. (2)."""
    if scale is None:
        scale = default_scale(q.shape[1])
    return attention_output(attention_weights(q, k, scale, rows), v)


def block_mass_rows(a_q, block: int) -> np.ndarray:
    """Eq. (5) for one query block: r_qb for every key block b.

    ``a_q`` holds the |I_q| rows of A belonging to query block q
    ([|I_q|, S]); the result has n_blocks entries,
    r_qb = (1/|I_q|) sum_{i in I_q} sum_{j in I_b} A_ij.
    """
    B = block
    S = a_q.shape[1]
    nb = n_blocks(S, B)
    padded = np.zeros((a_q.shape[0], nb * B))
    padded[:, :S] = a_q                                              # a short last key block
    per_row_block = padded.reshape(a_q.shape[0], nb, B).sum(axis=2)  # sum over j in I_b
    return per_row_block.sum(axis=0) / a_q.shape[0]                  # (1/|I_q|) sum over i in I_q


def block_mass(q, k, scale: float, block: int, qblocks=None) -> np.ndarray:
    """Block-mass matrix r[q, b] of one (batch, head) at one step, Eq. (5).

    Returns [len(qblocks), n_blocks] (all query blocks by default).
    """
    S = k.shape[0]
    nb = n_blocks(S, block)
    qbs = range(nb) if qblocks is None else qblocks
    out = []
    for qb in qbs:
        rows = block_rows(qb, block, S)
        out.append(block_mass_rows(attention_weights(q, k, scale, rows), block))
    return np.array(out)


def mean_block_mass(step_masses: Sequence[np.ndarray]) -> np.ndarray:
    """Equal-weight mean of r over the discovery steps (reading 1)."""
    acc = np.zeros_like(np.asarray(step_masses[0], dtype=np.float64))
    for r in step_masses:
        acc = acc + r
    return acc / len(step_masses)


def _ranked(mbar_row, q: int) -> List[int]:
    """Admissible blocks 0..q ordered by mass descending, index ascending (reading 2)."""
    return sorted(range(q + 1), key=lambda b: (-float(mbar_row[b]), b))


def eta_support(mass_row, q: int, eta: float) -> List[int]:
    """The cumulative-eta block support of Eq. (6) (right-hand part) and
    Eq. (12): the k* highest-mass admissible blocks of query block q, where
    k* is the smallest k whose k largest masses sum to at least eta (reading
    3: inclusive; reading 6: all blocks if eta is never reached).  Ranked
    part only, ascending ids.  The same set is the B_q^(t,rho) of the
    controls in Appendix B."""
    order = _ranked(mass_row, q)
    prefix = 0.0
    k_star = len(order)
    for k, b in enumerate(order, start=1):
        prefix += float(mass_row[b])
        if prefix >= eta:
            k_star = k
            break
    return sorted(order[:k_star])


def topk_support(mass_row, q: int, k: int) -> List[int]:
    """TopK of Eq. (22): the k highest-mass admissible blocks (ties to the
    lower index, reading 2), ascending ids."""
    return sorted(_ranked(mass_row, q)[:max(0, k)])


def select_support(mbar_row, q: int, eta: float, cap: int = 0) -> List[int]:
    """Working set of query block q, ascending block ids.

    Eq. (6) / Eq. (12): k* is the smallest k whose k largest masses sum to at
    least eta; the top-k* blocks (capped at ``cap`` when cap > 0) are taken,
    then the sink block 0 and the diagonal block q are added (reading 4).
    """
    ranked = eta_support(mbar_row, q, eta)
    if cap > 0 and len(ranked) > cap:
        ranked = topk_support(mbar_row, q, cap)   # the cap keeps the top `cap` of the same order
    return sorted(set(ranked) | {0, q})


def _union_ranked(step_rows, q: int, eta: float) -> List[int]:
    out = set()
    for r in step_rows:
        out |= set(eta_support(r, q, eta))
    return sorted(out)


def select_union(step_rows, q: int, eta: float) -> List[int]:
    """WISE working set with temporal union, Eq. (6) (left) / Eq. (18):
    the union over the given discovery steps of each step's own eta-support
    of r^(t), plus sink and diagonal (reading 7)."""
    return sorted(set(_union_ranked(step_rows, q, eta)) | {0, q})


def select_static(first_row, q: int, eta: float) -> List[int]:
    """Static-95 control, Eq. (19): the eta-support of the first step's block
    masses (eta = 0.95 in the paper), plus sink and diagonal."""
    return sorted(set(eta_support(first_row, q, eta)) | {0, q})


def select_mass_matched(first_row, window_rows, q: int, eta: float) -> List[int]:
    """MassMatched control, Eq. (20)-(21): m = the first step's mass covered
    by the union working set W_q (Eq. 20, float64 sum in block order), then
    the smallest first-step-ranked prefix whose mass reaches m; plus sink and
    diagonal."""
    w = _union_ranked(window_rows, q, eta)
    m = 0.0
    for b in w:
        m += float(first_row[b])
    return sorted(set(eta_support(first_row, q, m)) | {0, q})


def select_size_matched(first_row, window_rows, q: int, eta: float) -> List[int]:
    """SizeMatched control, Eq. (22): the K_q = |W_q| highest first-step
    masses, plus sink and diagonal."""
    k = len(_union_ranked(window_rows, q, eta))
    return sorted(set(topk_support(first_row, q, k)) | {0, q})


def support_margins(mbar_row, q: int, eta: float) -> Dict[str, float]:
    """Identification margins of Appendix A.1, Eq. (13), for one row.

    delta_rank = (m_(k*) - m_(k*+1)) / 2 (inf when k* is the last block),
    delta_minus = eta - sum_{s<k*} m_(s), delta_plus = sum_{s<=k*} m_(s) - eta,
    Delta = min(delta_rank, delta_minus/(k*-1), delta_plus/k*).
    """
    order = _ranked(mbar_row, q)
    vals = [float(mbar_row[b]) for b in order]
    prefix = 0.0
    k_star = len(vals)
    for k, v in enumerate(vals, start=1):
        prefix += v
        if prefix >= eta:
            k_star = k
            break
    before = sum(vals[: k_star - 1])
    through = before + vals[k_star - 1]
    d_rank = (vals[k_star - 1] - vals[k_star]) / 2 if k_star < len(vals) else math.inf
    d_minus = eta - before
    d_plus = through - eta
    delta = min(d_rank, d_minus / (k_star - 1) if k_star > 1 else math.inf,
                d_plus / k_star)
    return {"k_star": k_star, "delta_rank": d_rank, "delta_minus": d_minus,
            "delta_plus": d_plus, "Delta": delta}


def retained_mass(mass_row, support_row: Sequence[int], q: int) -> float:
    """Retained attention mass (Section 7): the part of one step's block
    masses r_qb (Eq. 5; they sum to 1 over the admissible blocks) that falls
    inside the support; entries outside [0, q] and repeats are ignored."""
    total = 0.0
    for b in sorted(set(int(x) for x in support_row)):
        if 0 <= b <= q:
            total += float(mass_row[b])
    return total


def rolling_working_set(step_rows, t: int, q: int, eta: float) -> List[int]:
    """Eq. (23): the union of the per-step eta-supports of steps
    max(0, t-3)..t (0-based), plus sink and diagonal (reading 8)."""
    return select_union(list(step_rows)[max(0, t - 3):t + 1], q, eta)


def jaccard(rows_a: Sequence[Sequence[int]], rows_b: Sequence[Sequence[int]]) -> float:
    """Eq. (24)/(25) for one example: the working-set collections are the
    sets of (row, key block) pairs; |A & B| / |A | B| over all rows pooled."""
    inter = union = 0
    for a, b in zip(rows_a, rows_b):
        sa, sb = set(a), set(b)
        inter += len(sa & sb)
        union += len(sa | sb)
    return inter / union if union else 1.0


def working_set_mask(support_row: Sequence[int], S: int, block: int, rows) -> np.ndarray:
    """Eq. (7) restricted to query rows in one query block: 0 if b(j) in W, else -inf."""
    keep = np.zeros(n_blocks(S, block), dtype=bool)
    keep[list(support_row)] = True
    allowed = np.repeat(keep, block)[:S]              # b(j) in W_{q(i)}
    R = np.where(allowed, 0.0, -np.inf)
    return np.broadcast_to(R, (len(rows), S))


def masked_attention_weights(q, k, scale: float, block: int, supports: Dict[int, Sequence[int]],
                             rows) -> np.ndarray:
    """Rows of softmax(q k^T * scale + M + R), Eq. (8).

    ``supports`` maps query block -> key blocks kept for it.  A row whose
    support holds no admissible key returns zeros (no such row arises from
    ``select_support``, which always keeps the diagonal block).
    """
    S = k.shape[0]
    r = _rows(S, rows)
    s = (q[r] @ k.T) * scale
    s[np.arange(S)[None, :] > r[:, None]] = -np.inf                 # M
    for i, row in enumerate(r):
        s[i] += working_set_mask(supports[int(row) // block], S, block, [row])[0]   # R
    out = np.zeros_like(s)
    live = np.isfinite(s).any(axis=1)
    if live.any():
        out[live] = _softmax_rows(s[live])
    return out


def masked_attention(q, k, v, supports, block: int, scale: Optional[float] = None,
                     rows=None) -> np.ndarray:
    """Late-step output O~ = A~ V, Eq. (8)."""
    if scale is None:
        scale = default_scale(q.shape[1])
    return attention_output(masked_attention_weights(q, k, scale, block, supports, rows), v)


def trajectory_head(steps_qkv, td: int, block: int, eta: float, cap: int = 0,
                    qblocks=None, scale: Optional[float] = None, out_rows: bool = True):
    """Whole discover-early / reuse-late trajectory of one (batch, head).

    ``steps_qkv`` yields float64 (q, k, v) per recurrent step t = 0..T-1.
    Steps t < td are dense (Eq. 2) and contribute r^(t) (Eq. 5); the supports
    are chosen once from the mean mass (Eq. 6 + readings); steps t >= td
    recompute attention inside the frozen support (Eq. 7-8).  Only query
    blocks ``qblocks`` are evaluated (all by default).

    Returns dict with per-step outputs for the evaluated rows, the summed
    mass (the same quantity a caller accumulates over the td steps), the
    mean mass, the supports and their margins.
    """
    outputs, masses, supports, margins = [], [], {}, {}
    qbs = None
    for t, (q, k, v) in enumerate(steps_qkv):
        S, D = q.shape
        sc = default_scale(D) if scale is None else scale
        nb = n_blocks(S, block)
        if qbs is None:
            qbs = list(range(nb)) if qblocks is None else [int(x) for x in qblocks]
        per_block = [block_rows(qb, block, S) for qb in qbs]
        rows = np.concatenate(per_block)
        if t < td:
            a = attention_weights(q, k, sc, rows)
            ends = np.cumsum([len(r) for r in per_block])
            masses.append(np.array([block_mass_rows(a[e - len(r):e], block)
                                    for r, e in zip(per_block, ends)]))
            outputs.append(attention_output(a, v) if out_rows else None)
        else:
            if not supports:
                mbar = mean_block_mass(masses)
                for i, qb in enumerate(qbs):
                    supports[qb] = select_support(mbar[i], qb, eta, cap)
                    margins[qb] = support_margins(mbar[i], qb, eta)
            outputs.append(masked_attention(q, k, v, supports, block, sc, rows)
                           if out_rows else None)
    mass_sum = None
    if masses:
        mass_sum = np.zeros_like(masses[0])
        for r in masses:
            mass_sum = mass_sum + r
    return {"qblocks": qbs, "outputs": outputs, "mass_sum": mass_sum,
            "mass_mean": mean_block_mass(masses) if masses else None,
            "supports": supports, "margins": margins}
