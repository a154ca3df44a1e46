"""GPU parity of the selection variants behind wise_select_variant:
temporal union (Eq. 6 left / Eq. 18) and the early-static controls of
Appendix B (Static-95 Eq. 19, MassMatched Eq. 20-21, SizeMatched Eq. 22),
against the fp64 oracle on the same fp32 step masses, and one short
trajectory that discovers per-step masses on the GPU, selects the union and
runs the reuse steps on it."""
import numpy as np
import pytest

import oracle
from wise_inputs import CONFIGS, Workload
from wise_testlib import TIE_EPS, bf16_dev_to_f64, compare_outputs, csr_rows, say, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
wise = pytest.importorskip("block_sparse_attention_wise_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wise.load_library()


def _step_masses(rng, n_mass, b_, h_, nb, kind):
    """[n_mass, b, h, nb, nb] fp32 single-step masses (rows sum to 1 over 0..q)."""
    m = np.zeros((n_mass, b_, h_, nb, nb), dtype=np.float32)
    for w in range(n_mass):
        for b in range(b_):
            for h in range(h_):
                for q in range(nb):
                    if kind == "dyadic":
                        x = rng.integers(0, 6, q + 1).astype(np.float64)
                        x[q] += 1.0
                        x = np.round(x / x.sum() * 256) / 256
                    else:
                        x = rng.dirichlet(np.full(q + 1, 0.4))
                    m[w, b, h, q, :q + 1] = x.astype(np.float32)
    return m


def _oracle_row(kind, rows, q, eta):
    if kind == wise.SELECT_UNION:
        return oracle.select_union(rows, q, eta)
    if kind == wise.SELECT_STATIC:
        return oracle.select_static(rows[0], q, eta)
    if kind == wise.SELECT_MASS_MATCHED:
        return oracle.select_mass_matched(rows[0], rows[1:], q, eta)
    return oracle.select_size_matched(rows[0], rows[1:], q, eta)


def _near_tie(kind, rows, q, eta):
    """Is any eta decision of this row within TIE_EPS of a boundary (Appendix
    A.1 margins), so that float64 summation order may legitimately flip it?"""
    window = rows if kind in (wise.SELECT_UNION, wise.SELECT_STATIC) else rows[1:]
    for r in window:
        m = oracle.support_margins(r, q, eta)
        if min(2 * m["delta_rank"], m["delta_minus"], m["delta_plus"]) <= TIE_EPS:
            return True
    if kind == wise.SELECT_MASS_MATCHED:
        w = set()
        for r in window:
            w |= set(oracle.eta_support(r, q, eta))
        mm = sum(float(rows[0][b]) for b in sorted(w))
        m = oracle.support_margins(rows[0], q, min(mm, 1.0))
        if min(2 * m["delta_rank"], m["delta_minus"], m["delta_plus"]) <= TIE_EPS:
            return True
    return False


CASES = [
    (wise.SELECT_UNION, 4, 33, "dirichlet", 0.95),
    (wise.SELECT_UNION, 1, 64, "dirichlet", 0.9),
    (wise.SELECT_UNION, 4, 130, "dyadic", 0.75),
    (wise.SELECT_STATIC, 1, 70, "dirichlet", 0.95),
    (wise.SELECT_STATIC, 1, 64, "dyadic", 0.5),
    (wise.SELECT_MASS_MATCHED, 5, 40, "dirichlet", 0.95),
    (wise.SELECT_MASS_MATCHED, 5, 200, "dyadic", 0.9),
    (wise.SELECT_SIZE_MATCHED, 5, 40, "dirichlet", 0.95),
    (wise.SELECT_SIZE_MATCHED, 3, 257, "dyadic", 0.8),
    (wise.SELECT_SIZE_MATCHED, 5, 1, "dirichlet", 0.9),
]


@pytest.mark.parametrize("kind,n_mass,nb,dist,eta", CASES,
                         ids=[f"k{c[0]}_n{c[1]}_nb{c[2]}_{c[3]}_eta{c[4]}" for c in CASES])
def test_select_variant_matches_oracle(kind, n_mass, nb, dist, eta):
    b_, h_ = 2, 2
    say(f"select variant kind {kind} n_mass {n_mass} nb {nb} {dist} eta {eta}")
    rng = np.random.default_rng(1000 + 7 * kind + nb + n_mass)
    m = _step_masses(rng, n_mass, b_, h_, nb, dist)
    rp, ci = wise.wise_select_variant(kind, torch.from_numpy(m).cuda(), eta, 64, 32)
    torch.cuda.synchronize()
    rows = csr_rows(rp.cpu().numpy(), ci.cpu().numpy())
    near = 0
    for b in range(b_):
        for h in range(h_):
            for q in range(nb):
                r = (b * h_ + h) * nb + q
                steps = [m[w, b, h, q].astype(np.float64) for w in range(n_mass)]
                want = _oracle_row(kind, steps, q, eta)
                got = rows[r]
                if got == want:
                    continue
                assert _near_tie(kind, steps, q, eta), (b, h, q, got, want)
                assert got == sorted(set(got)) and 0 in got and q in got and max(got) <= q
                near += 1
    say(f"  rows {b_ * h_ * nb}, near-tie differences {near}")


def test_union_trajectory_end_to_end():
    """Per-step discovery masses from the GPU, the union of the last discovery
    steps' supports, then reuse steps on that union (Eq. 18 with Eq. 7-8)."""
    cfg = CONFIGS["tiny"].with_(steps=8, td=4, index=205)
    nb, B = cfg.n_blocks, cfg.block
    say(f"union trajectory: {cfg.batch}x{cfg.heads} heads, S {cfg.seq_len}, td {cfg.td}")
    steps = list(Workload(cfg, threads=4).steps())
    step_mass = torch.zeros(cfg.td, cfg.batch, cfg.heads, nb, nb, dtype=torch.float32, device="cuda")
    outs = {}
    rp = ci = None
    for t, q, k, v in steps:
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        if t < cfg.td:
            wise.wise_full_attn_accum(qd, kd, vd, step_mass[t], B)
        else:
            if rp is None:
                rp, ci = wise.wise_select_variant(wise.SELECT_UNION, step_mass, cfg.eta, cfg.head_dim, B)
            outs[t] = bf16_dev_to_f64(wise.wise_sparse_attn(qd, kd, vd, rp, ci, B))
    torch.cuda.synchronize()
    gm = step_mass.cpu().numpy().astype(np.float64)
    rows = csr_rows(rp.cpu().numpy(), ci.cpu().numpy())
    sc = oracle.default_scale(cfg.head_dim)
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            heads = [tuple(oracle.bf16_to_f64(x[b, h]) for x in (q, k, v)) for _, q, k, v in steps]
            per_step = [oracle.block_mass(Q, K, sc, B) for (Q, K, V) in heads[:cfg.td]]
            for t in range(cfg.td):
                assert np.abs(gm[t, b, h] - per_step[t]).max() <= 1e-5
            sup = {}
            for qb in range(nb):
                r = (b * cfg.heads + h) * nb + qb
                want = oracle.select_union([gm[t, b, h, qb] for t in range(cfg.td)], qb, cfg.eta)
                assert rows[r] == want or _near_tie(wise.SELECT_UNION,
                                                    [gm[t, b, h, qb] for t in range(cfg.td)], qb, cfg.eta)
                sup[qb] = rows[r]
            for t in range(cfg.td, cfg.steps):
                Q, K, V = heads[t]
                compare_outputs(outs[t][b, h], oracle.masked_attention(Q, K, V, sup, B, sc),
                                f"O t{t} b{b}h{h}")
