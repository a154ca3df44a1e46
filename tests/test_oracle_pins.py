"""Pins of the fp64 oracle against what the WISE paper and mathematics fix.

Every check here is independent of the oracle's own code path: closed forms
(uniform attention, constant values, the logistic two-key case), invariants
(rows sum to one, logit shift invariance, full support reproduces dense
attention), brute-force subset enumeration for the selection rule, the
perturbation property of Appendix A.1, and hand-derived golden fixtures.
The mutation tests at the end plant typical mistakes into copies of the
oracle's functions and require at least one pin to fail for each.
"""
import contextlib
import inspect
import itertools
import json
import math
import os
import textwrap
from fractions import Fraction
from types import SimpleNamespace

import numpy as np
import pytest
from scipy.special import expit

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _impl(**over):
    ns = SimpleNamespace(attention_weights=oracle.attention_weights,
                         block_mass_rows=oracle.block_mass_rows,
                         select_support=oracle.select_support,
                         masked_attention_weights=oracle.masked_attention_weights,
                         eta_support=oracle.eta_support,
                         select_union=oracle.select_union,
                         select_static=oracle.select_static,
                         select_mass_matched=oracle.select_mass_matched,
                         select_size_matched=oracle.select_size_matched,
                         retained_mass=oracle.retained_mass,
                         rolling_working_set=oracle.rolling_working_set,
                         jaccard=oracle.jaccard,
                         default_scale=oracle.default_scale,
                         dense_attention=oracle.dense_attention,
                         mean_block_mass=oracle.mean_block_mass,
                         support_margins=oracle.support_margins,
                         trajectory_head=oracle.trajectory_head)
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


def _rand(seed, S, D):
    g = np.random.default_rng(seed)
    return (g.standard_normal((S, D)), g.standard_normal((S, D)), g.standard_normal((S, D)))


# --------------------------------------------------------------------------
# Pin functions (take an implementation namespace so mutants can be checked)
# --------------------------------------------------------------------------

def pin_uniform_when_q_zero(impl):
    """Eq. (2) with Q = 0: every admissible key gets weight 1/(i+1)."""
    S, D = 37, 8
    _, k, v = _rand(1, S, D)
    q = np.zeros((S, D))
    a = impl.attention_weights(q, k, 0.3)
    o = a @ v
    expect = np.cumsum(v, axis=0) / np.arange(1, S + 1)[:, None]
    np.testing.assert_allclose(o, expect, rtol=0, atol=1e-13)


def pin_constant_values(impl):
    S, D = 23, 5
    q, k, _ = _rand(2, S, D)
    v = np.full((S, D), 2.75)
    o = impl.attention_weights(q, k, 0.7) @ v
    np.testing.assert_allclose(o, 2.75, rtol=0, atol=1e-13)


def pin_single_position(impl):
    q, k, v = _rand(3, 1, 4)
    o = impl.attention_weights(q, k, 0.5) @ v
    np.testing.assert_allclose(o, v, rtol=0, atol=0)


def pin_logistic_two_keys(impl):
    """Row 1 over keys {0, 1}: A_11 = logistic((s_11 - s_10) * scale)."""
    q = np.array([[0.4], [1.3]])
    k = np.array([[-0.8], [0.6]])
    scale = 0.9
    a = impl.attention_weights(q, k, scale)
    expect = expit((q[1, 0] * k[1, 0] - q[1, 0] * k[0, 0]) * scale)
    assert abs(a[1, 1] - expect) < 1e-15
    assert abs(a[1, 0] - (1 - expect)) < 1e-15


def pin_causal_rows_sum_to_one(impl):
    S, D = 40, 6
    q, k, _ = _rand(4, S, D)
    a = impl.attention_weights(q, k, 0.4)
    np.testing.assert_allclose(a.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    assert np.all(a[np.triu_indices(S, 1)] == 0.0)
    assert np.all(a[np.tril_indices(S)] > 0.0)


def pin_key_shift_invariance(impl):
    """Adding one vector c to every key shifts row i's logits by q_i.c: A unchanged."""
    S, D = 29, 7
    q, k, _ = _rand(5, S, D)
    c = np.random.default_rng(6).standard_normal(D)
    a0 = impl.attention_weights(q, k, 0.35)
    a1 = impl.attention_weights(q, k + c, 0.35)
    np.testing.assert_allclose(a0, a1, rtol=0, atol=1e-12)


def pin_scale_is_a_temperature(impl):
    S, D = 19, 4
    q, k, _ = _rand(7, S, D)
    a0 = impl.attention_weights(q, k, 0.5)
    a1 = impl.attention_weights(2.0 * q, k, 0.25)
    np.testing.assert_allclose(a0, a1, rtol=0, atol=1e-13)
    a2 = impl.attention_weights(q, k, 1.0)
    assert np.max(np.abs(a2 - a0)) > 1e-3


def _frac(s):
    return float(Fraction(s))


def _golden_dense():
    with open(os.path.join(GOLDEN, "dense_closed_form.json")) as f:
        g = json.load(f)
    qmap = {"0": 0.0, "ln2": math.log(2.0), "ln3": math.log(3.0)}
    q = np.array([[qmap[x]] for x in g["q"]])
    k = np.array(g["k"])[:, None]
    v = np.array(g["v"])[:, None]
    A = np.array([[_frac(x) for x in row] for row in g["A"]])
    O = np.array([_frac(x) for x in g["O"]])
    r = np.array([[_frac(x) for x in row] for row in g["r"]])
    return g, q, k, v, A, O, r


def pin_golden_dense(impl):
    g, q, k, v, A, O, r = _golden_dense()
    a = impl.attention_weights(q, k, g["scale"])
    np.testing.assert_allclose(a, A, rtol=0, atol=1e-15)
    np.testing.assert_allclose((a @ v)[:, 0], O, rtol=0, atol=1e-14)
    B = g["block"]
    for qb in range(r.shape[0]):
        rows = a[qb * B:(qb + 1) * B]
        np.testing.assert_allclose(impl.block_mass_rows(rows, B), r[qb], rtol=0, atol=1e-15)


def pin_block_mass_sums_to_one(impl):
    S, D, B = 96, 8, 16
    q, k, _ = _rand(8, S, D)
    a = impl.attention_weights(q, k, 0.6)
    for qb in range(S // B):
        r = impl.block_mass_rows(a[qb * B:(qb + 1) * B], B)
        assert abs(r.sum() - 1.0) < 1e-13
        assert np.all(r[qb + 1:] == 0.0)
        assert np.all(r[:qb + 1] > 0.0)


def pin_block_mass_q_zero_closed_form(impl):
    """Q = 0: r_qb = (1/B) sum_{i in I_q} |{j in I_b : j <= i}| / (i + 1)."""
    S, D, B = 64, 4, 8
    _, k, _ = _rand(9, S, D)
    a = impl.attention_weights(np.zeros((S, D)), k, 1.0)
    for qb in range(S // B):
        r = impl.block_mass_rows(a[qb * B:(qb + 1) * B], B)
        expect = np.zeros(S // B)
        for i in range(qb * B, (qb + 1) * B):
            for b in range(S // B):
                n_adm = max(0, min(i, (b + 1) * B - 1) - b * B + 1)
                expect[b] += n_adm / (i + 1)
        np.testing.assert_allclose(r, expect / B, rtol=0, atol=1e-14)


def pin_block_mass_token_level(impl):
    """B = 1 reduces the block mass to the token attention distribution."""
    S, D = 17, 3
    q, k, _ = _rand(10, S, D)
    a = impl.attention_weights(q, k, 0.8)
    for i in range(S):
        np.testing.assert_allclose(impl.block_mass_rows(a[i:i + 1], 1), a[i], rtol=0, atol=1e-15)


def pin_block_mass_dominant_key(impl):
    """One key with a huge logit for every query pulls nearly all mass to its block."""
    S, D, B = 48, 2, 8
    g = np.random.default_rng(11)
    q = np.column_stack([np.ones(S), 0.01 * g.standard_normal(S)])
    k = 0.01 * g.standard_normal((S, D))
    k[3, 0] = 60.0                        # key 3 lies in block 0
    a = impl.attention_weights(q, k, 1.0)
    for qb in range(1, S // B):
        r = impl.block_mass_rows(a[qb * B:(qb + 1) * B], B)
        assert r[0] > 1 - 1e-12 and r[1:].max() < 1e-20 and abs(r.sum() - 1) < 1e-13


def _brute_force_support(mbar, q, eta):
    blocks = list(range(q + 1))
    for size in range(1, q + 2):
        feasible = [c for c in itertools.combinations(blocks, size)
                    if sum(mbar[b] for b in c) >= eta]
        if feasible:
            return size, feasible
    return q + 1, [tuple(blocks)]


def pin_selection_brute_force(impl):
    """Eq. (6): minimum cardinality equals k*, and the chosen set reaches eta."""
    g = np.random.default_rng(12)
    for trial in range(60):
        q = int(g.integers(1, 11))
        mbar = g.dirichlet(np.full(q + 1, 0.5))
        eta = float(g.choice([0.5, 0.8, 0.9, 0.95]))
        got = impl.select_support(mbar, q, eta)
        size, feasible = _brute_force_support(mbar, q, eta)
        eta_part = [b for b in got]
        # the eta-selected blocks are the top-k* by mass (distinct masses here)
        order = sorted(range(q + 1), key=lambda b: -mbar[b])
        top = set(order[:size])
        assert set(got) == top | {0, q}, (trial, got, top)
        assert sum(mbar[b] for b in top) >= eta
        assert tuple(sorted(top)) in [tuple(sorted(c)) for c in feasible]
        assert eta_part == sorted(eta_part)


def pin_selection_eta_one_keeps_all(impl):
    g = np.random.default_rng(13)
    for q in (0, 1, 5, 30):
        mbar = g.dirichlet(np.ones(q + 1))
        assert impl.select_support(mbar, q, 1.0) == list(range(q + 1))


def pin_selection_small_eta_keeps_argmax(impl):
    g = np.random.default_rng(14)
    for q in (3, 9, 20):
        mbar = g.dirichlet(np.ones(q + 1))
        got = impl.select_support(mbar, q, float(mbar.max()) * 0.999)
        assert got == sorted({int(np.argmax(mbar)), 0, q})


def pin_selection_golden(impl):
    with open(os.path.join(GOLDEN, "selection_dyadic.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        got = impl.select_support(np.array(case["mbar"]), case["q"], case["eta"], case["cap"])
        assert got == case["support"], (case, got)


def pin_selection_perturbation(impl):
    """Appendix A.1: a perturbation below Delta_q leaves the support unchanged."""
    g = np.random.default_rng(15)
    checked = 0
    for _ in range(200):
        q = int(g.integers(2, 25))
        mbar = g.dirichlet(np.full(q + 1, 0.7))
        eta = 0.9
        m = oracle.support_margins(mbar, q, eta)
        if not (m["Delta"] > 1e-9 and math.isfinite(m["Delta"])):
            continue
        base = impl.select_support(mbar, q, eta)
        for _ in range(5):
            eps = g.uniform(-1, 1, q + 1) * m["Delta"] * 0.999
            assert impl.select_support(mbar + eps, q, eta) == base
        checked += 1
    assert checked > 50


def pin_full_support_reproduces_dense(impl):
    S, D, B = 64, 8, 16
    q, k, _ = _rand(16, S, D)
    sup = {qb: list(range(qb + 1)) for qb in range(S // B)}
    a_dense = impl.attention_weights(q, k, 0.45)
    a_mask = impl.masked_attention_weights(q, k, 0.45, B, sup, np.arange(S))
    assert np.max(np.abs(a_dense - a_mask)) <= 1e-15


def pin_diagonal_only_support(impl):
    """W = {q}: block-local causal attention; with Q = 0 the mean of v over [qB, i]."""
    S, D, B = 48, 4, 8
    _, k, v = _rand(17, S, D)
    sup = {qb: [qb] for qb in range(S // B)}
    a = impl.masked_attention_weights(np.zeros((S, D)), k, 1.0, B, sup, np.arange(S))
    o = a @ v
    for i in range(S):
        lo = (i // B) * B
        np.testing.assert_allclose(o[i], v[lo:i + 1].mean(axis=0), rtol=0, atol=1e-13)


def pin_sink_and_diagonal_support(impl):
    S, D, B = 48, 4, 8
    _, k, v = _rand(18, S, D)
    sup = {qb: sorted({0, qb}) for qb in range(S // B)}
    a = impl.masked_attention_weights(np.zeros((S, D)), k, 1.0, B, sup, np.arange(S))
    o = a @ v
    for i in range(B, S):
        lo = (i // B) * B
        idx = list(range(0, B)) + list(range(lo, i + 1))
        np.testing.assert_allclose(o[i], v[idx].mean(axis=0), rtol=0, atol=1e-13)


def pin_masked_rows_normalised(impl):
    S, D, B = 64, 5, 8
    q, k, _ = _rand(19, S, D)
    g = np.random.default_rng(20)
    sup = {qb: sorted(set(g.choice(qb + 1, size=min(qb + 1, 3), replace=False).tolist()) | {qb})
           for qb in range(S // B)}
    a = impl.masked_attention_weights(q, k, 0.5, B, sup, np.arange(S))
    np.testing.assert_allclose(a.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    for i in range(S):
        allowed = np.zeros(S, dtype=bool)
        for b in sup[i // B]:
            allowed[b * B:(b + 1) * B] = True
        allowed[i + 1:] = False
        assert np.all(a[i, ~allowed] == 0) and np.all(a[i, allowed] > 0)


def pin_variants_golden(impl):
    """Hand-worked dyadic cases of Eq. (6)/(18), (19), (20)-(21), (22)."""
    with open(os.path.join(GOLDEN, "selection_variants_dyadic.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        q, eta = case["q"], case["eta"]
        first = np.array(case["first"])
        window = [np.array(w) for w in case["window"]]
        assert impl.eta_support(first, q, eta) == case["first_support"], case["note"]
        assert [impl.eta_support(w, q, eta) for w in window] == case["window_supports"], case["note"]
        assert impl.select_union(window, q, eta) == case["union"], case["note"]
        assert impl.select_static(first, q, eta) == case["static"], case["note"]
        assert impl.select_mass_matched(first, window, q, eta) == case["mass_matched"], case["note"]
        assert impl.select_size_matched(first, window, q, eta) == case["size_matched"], case["note"]


def pin_eta_support_brute_force(impl):
    """Eq. (6) right: the per-step support is a minimum-cardinality set
    reaching eta and consists of the highest masses (distinct masses)."""
    g = np.random.default_rng(21)
    for trial in range(60):
        q = int(g.integers(0, 10))
        r = g.dirichlet(np.full(q + 1, 0.5))
        eta = float(g.choice([0.5, 0.8, 0.95]))
        got = impl.eta_support(r, q, eta)
        size, feasible = _brute_force_support(r, q, eta)
        assert len(got) == size, (trial, got, size)
        assert tuple(got) in [tuple(sorted(c)) for c in feasible]
        assert min(r[got]) >= max([r[b] for b in range(q + 1) if b not in got], default=-1.0)


def pin_union_structure(impl):
    """Eq. (18): the union contains every step's own support and nothing
    else (besides sink/diagonal); one step gives that step's support; equal
    steps give the single-step selection."""
    g = np.random.default_rng(22)
    for trial in range(40):
        q = int(g.integers(1, 30))
        steps = [g.dirichlet(np.full(q + 1, 0.4)) for _ in range(int(g.integers(1, 5)))]
        eta = float(g.choice([0.6, 0.9, 0.95]))
        got = set(impl.select_union(steps, q, eta))
        parts = [set(impl.eta_support(r, q, eta)) for r in steps]
        assert got == set().union(*parts) | {0, q}, trial
        assert impl.select_union(steps[:1], q, eta) == sorted(parts[0] | {0, q})
        assert impl.select_union([steps[0]] * 3, q, eta) == impl.select_support(steps[0], q, eta)
        assert impl.select_static(steps[0], q, eta) == impl.select_support(steps[0], q, eta)


def pin_matched_controls(impl):
    """Eq. (20)-(22) on random rows: MassMatched is the shortest first-step
    prefix reaching the union's first-step mass; SizeMatched keeps exactly
    |union| first-step-ranked blocks."""
    g = np.random.default_rng(23)
    for trial in range(60):
        q = int(g.integers(2, 40))
        first = g.dirichlet(np.full(q + 1, 0.5))
        window = [g.dirichlet(np.full(q + 1, 0.3)) for _ in range(4)]
        eta = float(g.choice([0.7, 0.9, 0.95]))
        union = set().union(*[set(impl.eta_support(r, q, eta)) for r in window])
        order = sorted(range(q + 1), key=lambda b: (-first[b], b))
        m = sum(first[b] for b in sorted(union))
        mm = impl.select_mass_matched(first, window, q, eta)
        k = 1
        while sum(first[b] for b in order[:k]) < m and k <= q:
            k += 1
        assert mm == sorted(set(order[:k]) | {0, q}), (trial, mm, k)
        sm = impl.select_size_matched(first, window, q, eta)
        assert sm == sorted(set(order[:len(union)]) | {0, q}), (trial, sm)


def pin_retained_mass(impl):
    """Section 7: the full admissible support retains all of a step's mass
    (Eq. 5 rows sum to 1); at Q = 0 the sink + diagonal support retains the
    closed-form r_q0 + r_qq; invalid and repeated entries change nothing."""
    S, D, B = 128, 8, 16
    nb = S // B
    q0 = np.zeros((S, D))
    k0 = np.random.default_rng(31).standard_normal((S, D))
    r = oracle.block_mass(q0, k0, 1.0, B)
    for qb in range(nb):
        assert abs(impl.retained_mass(r[qb], list(range(qb + 1)), qb) - 1.0) < 1e-12
        i = np.arange(qb * B, (qb + 1) * B)
        closed_sink = float(np.mean([min(B, ii + 1) / (ii + 1) for ii in i]))
        closed_diag = float(np.mean([(ii - qb * B + 1) / (ii + 1) for ii in i]))
        want = closed_sink if qb == 0 else closed_sink + closed_diag
        assert abs(impl.retained_mass(r[qb], [0, qb], qb) - want) < 1e-12, qb
        assert impl.retained_mass(r[qb], [qb, 0, 0, -1, qb + 1, qb], qb) == impl.retained_mass(r[qb], [0, qb], qb)


def pin_rolling_and_jaccard(impl):
    """Eq. (23)-(24): rolling sets from the dyadic fixture's windows, and a
    hand-worked pooled Jaccard (per-row averaging would give 0.75)."""
    with open(os.path.join(GOLDEN, "selection_variants_dyadic.json")) as f:
        case = json.load(f)["cases"][0]
    q, eta = case["q"], case["eta"]
    steps = [np.array(case["first"])] + [np.array(w) for w in case["window"]]
    assert impl.rolling_working_set(steps, 0, q, eta) == sorted(set(case["first_support"]) | {0, q})
    assert impl.rolling_working_set(steps, 2, q, eta) == sorted(set(case["first_support"]) | {2, 4, 5, 0, q})
    assert impl.rolling_working_set(steps[1:], 1, q, eta) == case["union"]
    # t = 4: the window is steps 1..4 (four steps), so the first step drops out
    five = steps + steps[1:]
    assert impl.rolling_working_set(five, 4, q, eta) == case["union"]
    a = [[0, 1, 2, 5], [0, 3]]
    b = [[0, 2], [0, 3]]
    assert abs(impl.jaccard(a, b) - 4 / 6) < 1e-15
    assert impl.jaccard(a, a) == 1.0
    assert impl.jaccard([[1, 2]], [[3]]) == 0.0


def pin_short_last_block_mass(impl):
    """S not a multiple of B: the last block holds S - (nB - 1) B queries and
    keys.  Q = 0 gives r_qb = (1/|I_q|) sum_{i in I_q} |{j in I_b : j <= i}| / (i + 1)
    with |I_q| counted from the block's real extent, and every row of r,
    the short one included, sums to one."""
    S, D, B = 45, 4, 8
    nb = 6                                   # blocks [0,8) ... [40,45)
    _, k, _ = _rand(31, S, D)
    a = impl.attention_weights(np.zeros((S, D)), k, 1.0)
    for qb in range(nb):
        lo, hi = qb * B, min(S, qb * B + B)
        r = impl.block_mass_rows(a[lo:hi], B)
        assert r.shape == (nb,)
        expect = np.zeros(nb)
        for i in range(lo, hi):
            for b in range(nb):
                n_adm = max(0, min(i, b * B + B - 1, S - 1) - b * B + 1)
                expect[b] += n_adm / (i + 1)
        np.testing.assert_allclose(r, expect / (hi - lo), rtol=0, atol=1e-14)
    q, k, _ = _rand(32, S, D)
    a = impl.attention_weights(q, k, 0.7)
    for qb in range(nb):
        r = impl.block_mass_rows(a[qb * B:min(S, qb * B + B)], B)
        assert abs(r.sum() - 1.0) < 1e-13 and np.all(r[qb + 1:] == 0.0)


def pin_short_last_block_prefix(impl):
    """Causality: positions past S never reach the first S queries.  A
    length-S problem (S not a multiple of B) therefore matches the first S
    rows of a longer one that extends it to whole blocks: weights, the masses
    of the whole query blocks, and late-step attention on any support."""
    S, L, D, B = 53, 64, 6, 16
    q, k, _ = _rand(33, L, D)
    a_s = impl.attention_weights(q[:S], k[:S], 0.5)
    a_l = impl.attention_weights(q, k, 0.5)
    np.testing.assert_allclose(a_s, a_l[:S, :S], rtol=0, atol=1e-15)
    assert np.all(a_l[:S, S:] == 0.0)
    for qb in range(S // B):
        rows = slice(qb * B, qb * B + B)
        np.testing.assert_allclose(impl.block_mass_rows(a_s[rows], B),
                                   impl.block_mass_rows(a_l[rows], B), rtol=0, atol=1e-15)
    g = np.random.default_rng(34)
    sup = {qb: sorted({0, qb} | set(g.integers(0, qb + 1, 2).tolist())) for qb in range(L // B)}
    m_s = impl.masked_attention_weights(q[:S], k[:S], 0.5, B, sup, np.arange(S))
    m_l = impl.masked_attention_weights(q, k, 0.5, B, sup, np.arange(L))
    np.testing.assert_allclose(m_s, m_l[:S, :S], rtol=0, atol=1e-15)
    full = {qb: list(range(qb + 1)) for qb in range(-(-S // B))}
    assert np.max(np.abs(impl.masked_attention_weights(q[:S], k[:S], 0.5, B, full, np.arange(S))
                         - a_s)) <= 1e-15


def pin_default_scale(impl):
    """Eq. (2): the softmax temperature is 1/sqrt(d_h).  Exact values at
    d_h = 4, 16, 64, 256, and through dense attention with no scale given:
    two keys whose dot products with q differ by 4x at d_h = 4 give
    A_11 = logistic(4x / 2)."""
    for d, want in ((4, 0.5), (16, 0.25), (64, 0.125), (256, 0.0625)):
        assert impl.default_scale(d) == want, (d, impl.default_scale(d))
    x = 0.3
    q = np.ones((2, 4))
    k = np.vstack([np.zeros(4), np.full(4, x)])
    v = np.array([[0.0] * 4, [1.0] * 4])
    o = impl.dense_attention(q, k, v)
    assert abs(o[1, 0] - expit(4 * x / 2)) < 1e-15, o[1, 0]


def pin_mean_block_mass_closed_form(impl):
    """The discovery steps' masses combine as their equal-weight mean
    (dyadic rows, exact), and the mean of rows that each sum to one sums to
    one."""
    rows = [np.array([1.0, 0.0, 0.0]), np.array([0.5, 0.5, 0.0]), np.array([0.0, 0.25, 0.75])]
    got = impl.mean_block_mass(rows)
    assert np.array_equal(got, np.array([0.5, 0.25, 0.25])), got
    g = np.random.default_rng(35)
    steps = [g.dirichlet(np.ones(9), size=4) for _ in range(5)]
    np.testing.assert_allclose(impl.mean_block_mass(steps).sum(axis=1), 1.0, rtol=0, atol=1e-14)
    one = impl.mean_block_mass([steps[2]])
    np.testing.assert_allclose(one, steps[2], rtol=0, atol=0)


def _golden_discovery():
    with open(os.path.join(GOLDEN, "discovery_mean_dyadic.json")) as f:
        g = json.load(f)
    S = g["seq_len"]
    qkv = []
    for w in g["weights_x64"]:
        q = np.ones((S, 1))
        k = np.log(np.array(w, dtype=np.float64) / 64.0)[:, None]
        v = np.array(g["values"], dtype=np.float64)[:, None]
        qkv.append((q, k, v))
    return g, qkv


def pin_trajectory_selects_on_mean(impl):
    """Section 5.1-5.2 on a hand-worked trajectory: the support is chosen on
    the mean of the discovery masses (not on the last or first step, their
    union or their sum), and the late step attends inside it."""
    g, qkv = _golden_discovery()
    qb = g["query_block"]
    out = impl.trajectory_head(qkv, g["td"], g["block"], g["eta"], qblocks=[qb], scale=1.0)
    assert out["supports"][qb] == g["support"], out["supports"][qb]
    np.testing.assert_allclose(out["mass_sum"][0], np.array(g["mass_sum_x64"]) / 64.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(out["mass_mean"][0], np.array(g["mass_mean_x128"]) / 128.0, rtol=0, atol=1e-15)
    late = out["outputs"][g["td"]]
    assert abs(late[0, 0] - _frac(g["late_output"])) < 1e-14, late


def pin_margins_golden(impl):
    """Appendix A.1, Eq. (13), hand-derived on dyadic rows with k* = 3, one
    where delta_minus / (k* - 1) is the binding term and one where
    delta_plus / k* is."""
    with open(os.path.join(GOLDEN, "margins_dyadic.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        m = impl.support_margins(np.array(case["mbar_x32"]) / 32.0, case["q"], case["eta_x64"] / 64.0)
        assert m["k_star"] == case["k_star"], (case["note"], m)
        for key in ("delta_rank", "delta_minus", "delta_plus", "Delta"):
            assert abs(m[key] - _frac(case[key])) < 1e-16, (case["note"], key, m[key])


PINS = [pin_uniform_when_q_zero, pin_constant_values, pin_single_position,
        pin_logistic_two_keys, pin_causal_rows_sum_to_one, pin_key_shift_invariance,
        pin_scale_is_a_temperature, pin_golden_dense, pin_block_mass_sums_to_one,
        pin_block_mass_q_zero_closed_form, pin_block_mass_token_level,
        pin_block_mass_dominant_key, pin_selection_brute_force,
        pin_selection_eta_one_keeps_all, pin_selection_small_eta_keeps_argmax,
        pin_selection_golden, pin_selection_perturbation,
        pin_full_support_reproduces_dense, pin_diagonal_only_support,
        pin_sink_and_diagonal_support, pin_masked_rows_normalised,
        pin_variants_golden, pin_eta_support_brute_force, pin_union_structure,
        pin_matched_controls, pin_retained_mass, pin_rolling_and_jaccard,
        pin_short_last_block_mass, pin_short_last_block_prefix, pin_default_scale,
        pin_mean_block_mass_closed_form, pin_trajectory_selects_on_mean, pin_margins_golden]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(_impl())


# --------------------------------------------------------------------------
# Other pins that do not fit the namespace form
# --------------------------------------------------------------------------

def test_margins_match_definition():
    mbar = np.array([0.0625, 0.5, 0.1875, 0.1875, 0.0625])
    m = oracle.support_margins(mbar, 4, 0.6)
    assert m["k_star"] == 2
    assert m["delta_rank"] == 0.0                  # 0.1875 tie at the boundary
    assert abs(m["delta_minus"] - 0.1) < 1e-15
    assert abs(m["delta_plus"] - 0.0875) < 1e-15


def test_trajectory_dense_only_equals_dense():
    S, D, B = 64, 8, 16
    steps = [_rand(30 + t, S, D) for t in range(3)]
    out = oracle.trajectory_head(steps, td=3, block=B, eta=0.9)
    for t in range(3):
        q, k, v = steps[t]
        np.testing.assert_allclose(out["outputs"][t], oracle.dense_attention(q, k, v),
                                   rtol=0, atol=0)
        assert out["mass_sum"].shape == (S // B, S // B)


@pytest.mark.parametrize("S", [64, 61])
def test_trajectory_eta_one_late_equals_dense(S):
    D, B = 8, 16
    steps = [_rand(40 + t, S, D) for t in range(4)]
    out = oracle.trajectory_head(steps, td=2, block=B, eta=1.0)
    for qb, sup in out["supports"].items():
        assert sup == list(range(qb + 1))
    for t in (2, 3):
        q, k, v = steps[t]
        assert np.max(np.abs(out["outputs"][t] - oracle.dense_attention(q, k, v))) <= 1e-15
    row_sums = out["mass_sum"].sum(axis=1)
    assert out["mass_sum"].shape == (4, 4)
    np.testing.assert_allclose(row_sums, 2.0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("S", [128, 123])
def test_trajectory_supports_keep_sink_and_diagonal(S):
    D, B = 8, 16
    steps = [_rand(50 + t, S, D) for t in range(4)]
    out = oracle.trajectory_head(steps, td=2, block=B, eta=0.5, cap=1)
    assert sorted(out["supports"]) == list(range(8))
    np.testing.assert_allclose(out["mass_sum"].sum(axis=1), 2.0, rtol=0, atol=1e-13)
    for qb, sup in out["supports"].items():
        assert 0 in sup and qb in sup and sup == sorted(sup)
        assert len(sup) <= 3


def test_bf16_widening_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x7F7F], dtype=np.uint16)
    got = oracle.bf16_to_f64(bits)
    assert got[0] == 1.0 and got[1] == -1.0 and got[3] == 0.0
    assert got[2] == 3.140625
    assert got[4] == float(np.float32(3.3895313892515355e38))


# --------------------------------------------------------------------------
# Mutation tests: each planted mistake must be caught by some pin
# --------------------------------------------------------------------------

def _caught(impl):
    for pin in PINS:
        try:
            pin(impl)
        except Exception:        # a failed assertion, or a planted mistake that crashes
            return True
    return False


def _mut_transposed(q, k, scale, rows=None):
    S = k.shape[0]
    r = np.arange(S) if rows is None else np.asarray(rows)
    s = (k[r] @ q.T) * scale
    s[np.arange(S)[None, :] > r[:, None]] = -np.inf
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def _mut_no_scale(q, k, scale, rows=None):
    return oracle.attention_weights(q, k, 1.0, rows)


def _mut_mask_off_by_one(q, k, scale, rows=None):
    S = k.shape[0]
    r = np.arange(S) if rows is None else np.asarray(rows)
    s = (q[r] @ k.T) * scale
    s[np.arange(S)[None, :] >= r[:, None] + 2] = -np.inf      # lets j = i + 1 through
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def _mut_mass_no_norm(a_q, block):
    return oracle.block_mass_rows(a_q, block) * a_q.shape[0]


def _mut_mass_divides_by_block(a_q, block):
    return oracle.block_mass_rows(a_q, block) * a_q.shape[0] / block


def _mut_mass_wrong_axis(a_q, block):
    nb = a_q.shape[1] // block
    return a_q.reshape(a_q.shape[0], nb, block).sum(axis=(0, 2))[::-1] / a_q.shape[0]


def _mut_select_exclusive(mbar, q, eta, cap=0):
    order = sorted(range(q + 1), key=lambda b: (-float(mbar[b]), b))
    prefix, k_star = 0.0, q + 1
    for kk, b in enumerate(order, 1):
        prefix += float(mbar[b])
        if prefix > eta:
            k_star = kk
            break
    k = min(k_star, cap) if cap > 0 else k_star
    return sorted(set(order[:k]) | {0, q})


def _mut_select_tie_high(mbar, q, eta, cap=0):
    order = sorted(range(q + 1), key=lambda b: (-float(mbar[b]), -b))
    prefix, k_star = 0.0, q + 1
    for kk, b in enumerate(order, 1):
        prefix += float(mbar[b])
        if prefix >= eta:
            k_star = kk
            break
    k = min(k_star, cap) if cap > 0 else k_star
    return sorted(set(order[:k]) | {0, q})


def _mut_select_one_short(mbar, q, eta, cap=0):
    full = oracle.select_support(mbar, q, eta, cap)
    order = sorted(range(q + 1), key=lambda b: (-float(mbar[b]), b))
    prefix, k_star = 0.0, q + 1
    for kk, b in enumerate(order, 1):
        prefix += float(mbar[b])
        if prefix >= eta:
            k_star = kk
            break
    k = max(1, k_star - 1)
    return sorted(set(order[:k]) | {0, q}) if full else full


def _mut_select_no_sink(mbar, q, eta, cap=0):
    return [b for b in oracle.select_support(mbar, q, eta, cap) if b != 0 or q == 0
            or b in sorted(range(q + 1), key=lambda c: (-float(mbar[c]), c))[:1]]


def _mut_masked_ignores_support(q, k, scale, block, supports, rows):
    full = {qb: list(range(qb + 1)) for qb in supports}
    return oracle.masked_attention_weights(q, k, scale, block, full, rows)


def _mut_union_is_intersection(steps, q, eta):
    parts = [set(oracle.eta_support(r, q, eta)) for r in steps]
    return sorted(set.intersection(*parts) | {0, q})


def _mut_union_of_mean(steps, q, eta):
    return oracle.select_support(oracle.mean_block_mass(steps), q, eta)


def _mut_static_uses_last_step(first, q, eta):
    return oracle.select_static(np.roll(first, 1), q, eta)


def _mut_mass_matched_counts_sink(first, window, q, eta):
    w = set(oracle.select_union(window, q, eta))        # includes sink and diagonal
    m = sum(float(first[b]) for b in sorted(w))
    return sorted(set(oracle.eta_support(first, q, m)) | {0, q})


def _mut_mass_matched_uses_window_ranking(first, window, q, eta):
    return oracle.select_mass_matched(window[0], window, q, eta)


def _mut_size_matched_one_more(first, window, q, eta):
    k = len(oracle.select_union(window, q, eta)) - 1    # sink/diagonal counted, minus one
    return sorted(set(oracle.topk_support(first, q, k)) | {0, q})


def _mut_eta_support_exclusive(r, q, eta):
    order = sorted(range(q + 1), key=lambda b: (-float(r[b]), b))
    prefix, k_star = 0.0, q + 1
    for kk, b in enumerate(order, 1):
        prefix += float(r[b])
        if prefix > eta:
            k_star = kk
            break
    return sorted(order[:k_star])


def _mut_jaccard_per_row_mean(rows_a, rows_b):
    vals = [len(set(a) & set(b)) / len(set(a) | set(b)) for a, b in zip(rows_a, rows_b)]
    return float(np.mean(vals))


def _mut_rolling_window_five(step_rows, t, q, eta):
    return oracle.select_union(list(step_rows)[max(0, t - 4):t + 1], q, eta)


def _mut_retained_counts_repeats(mass_row, support_row, q):
    return float(sum(mass_row[b] for b in support_row if 0 <= b <= q))


MUTANTS = {
    "jaccard_per_row_mean": dict(jaccard=_mut_jaccard_per_row_mean),
    "rolling_window_five_steps": dict(rolling_working_set=_mut_rolling_window_five),
    "retained_counts_repeats": dict(retained_mass=_mut_retained_counts_repeats),
    "union_is_intersection": dict(select_union=_mut_union_is_intersection),
    "union_selects_on_mean": dict(select_union=_mut_union_of_mean),
    "static_wrong_step": dict(select_static=_mut_static_uses_last_step),
    "mass_matched_counts_sink": dict(select_mass_matched=_mut_mass_matched_counts_sink),
    "mass_matched_wrong_ranking": dict(select_mass_matched=_mut_mass_matched_uses_window_ranking),
    "size_matched_off_by_one": dict(select_size_matched=_mut_size_matched_one_more),
    "eta_support_exclusive": dict(eta_support=_mut_eta_support_exclusive),
    "transposed_operand": dict(attention_weights=_mut_transposed),
    "missing_scale": dict(attention_weights=_mut_no_scale),
    "causal_off_by_one": dict(attention_weights=_mut_mask_off_by_one),
    "mass_missing_1_over_B": dict(block_mass_rows=_mut_mass_no_norm),
    "mass_wrong_axis": dict(block_mass_rows=_mut_mass_wrong_axis),
    "mass_short_block_over_B": dict(block_mass_rows=_mut_mass_divides_by_block),
    "select_exclusive_threshold": dict(select_support=_mut_select_exclusive),
    "select_tie_to_higher_index": dict(select_support=_mut_select_tie_high),
    "select_one_block_short": dict(select_support=_mut_select_one_short),
    "select_drops_sink": dict(select_support=_mut_select_no_sink),
    "masked_ignores_support": dict(masked_attention_weights=_mut_masked_ignores_support),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    assert _caught(_impl(**MUTANTS[name])), name


# Mistakes planted into the oracle's own source: a copy of the function with
# one edit, compiled against the oracle module's namespace and swapped into
# the module while every pin runs, so that the oracle's internal calls (the
# trajectory calling the mean, dense attention calling the default scale)
# reach the mutant too.

def _source_mutant(func, old, new):
    src = textwrap.dedent(inspect.getsource(func))
    assert src.count(old) == 1, (func.__name__, old)
    local = {}
    exec(compile(src.replace(old, new), f"<mutant of {func.__name__}>", "exec"), vars(oracle), local)
    return local[func.__name__]


@contextlib.contextmanager
def _swapped(name, fn):
    saved = getattr(oracle, name)
    setattr(oracle, name, fn)
    try:
        yield
    finally:
        setattr(oracle, name, saved)


SOURCE_MUTANTS = {
    "mean_divides_by_steps_plus_one": (oracle.mean_block_mass, "acc / len(step_masses)",
                                       "acc / (len(step_masses) + 1)"),
    "trajectory_selects_on_last_step": (oracle.trajectory_head, "mbar = mean_block_mass(masses)",
                                        "mbar = masses[-1]"),
    "trajectory_selects_on_first_step": (oracle.trajectory_head, "mbar = mean_block_mass(masses)",
                                         "mbar = masses[0]"),
    "trajectory_selects_on_sum": (oracle.trajectory_head, "mbar = mean_block_mass(masses)",
                                  "mbar = sum(masses)"),
    "trajectory_late_step_dense": (oracle.trajectory_head,
                                   "outputs.append(masked_attention(q, k, v, supports, block, sc, rows)",
                                   "outputs.append(dense_attention(q, k, v, sc, rows)"),
    "default_scale_one_over_d": (oracle.default_scale, "1.0 / math.sqrt(head_dim)", "1.0 / head_dim"),
    "margins_minus_over_k": (oracle.support_margins, "d_minus / (k_star - 1)", "d_minus / k_star"),
    "margins_plus_over_k_minus_1": (oracle.support_margins, "d_plus / k_star)", "d_plus / max(1, k_star - 1))"),
    "margins_rank_not_halved": (oracle.support_margins, "(vals[k_star - 1] - vals[k_star]) / 2",
                                "(vals[k_star - 1] - vals[k_star])"),
}


@pytest.mark.parametrize("name", sorted(SOURCE_MUTANTS))
def test_pins_catch_mistake_in_oracle_source(name):
    func, old, new = SOURCE_MUTANTS[name]
    mutant = _source_mutant(func, old, new)
    with _swapped(func.__name__, mutant):
        assert _caught(_impl()), name
    assert getattr(oracle, func.__name__) is func


def test_unmutated_source_copy_passes_every_pin():
    """The mutant harness itself: an unedited copy of each function, swapped
    in the same way, passes every pin."""
    for func in {m[0] for m in SOURCE_MUTANTS.values()}:
        src = textwrap.dedent(inspect.getsource(func))
        first = src.splitlines()[0]
        copy = _source_mutant(func, first, first)
        with _swapped(func.__name__, copy):
            impl = _impl()
            for pin in PINS:
                pin(impl)
