"""GPU parity of the working-set diagnostics (Section 7 "Evaluation metrics";
Appendix C.2, Eq. 23-25): retained future attention mass of a support and
the per-row overlap behind the Jaccard similarity, against the oracle."""
import numpy as np
import pytest

import oracle
from wise_inputs import CONFIGS, Workload
from wise_testlib import TIE_EPS, csr_rows, say, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
wise = pytest.importorskip("block_sparse_attention_wise_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wise.load_library()


def _random_csr(rng, n_rows, nb, messy):
    rows = []
    for r in range(n_rows):
        q = r % nb
        k = int(rng.integers(1, q + 2))
        row = list(rng.choice(q + 1, size=k, replace=False))
        if messy:   # repeats, out-of-range entries, any order
            row += list(rng.choice(q + 1, size=2)) + [-1, q + 1, nb + 5]
            rng.shuffle(row)
        rows.append([int(x) for x in row])
    rp = np.concatenate([[0], np.cumsum([len(x) for x in rows])]).astype(np.int32)
    ci = np.array([c for x in rows for c in x] or [0], dtype=np.int32)
    return rows, torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()


@pytest.mark.parametrize("nb,messy", [(8, False), (65, True), (300, True), (1, False)])
def test_support_mass_matches_oracle(nb, messy):
    b_, h_ = 2, 3
    say(f"support mass nb {nb} messy {messy}")
    rng = np.random.default_rng(400 + nb)
    m = np.zeros((b_, h_, nb, nb), dtype=np.float32)
    for idx in np.ndindex(b_, h_, nb):
        q = idx[2]
        m[idx][:q + 1] = rng.dirichlet(np.full(q + 1, 0.5)).astype(np.float32)
    rows, rp, ci = _random_csr(rng, b_ * h_ * nb, nb, messy)
    got = wise.wise_support_mass(torch.from_numpy(m).cuda(), rp, ci, 64, 32).cpu().numpy()
    torch.cuda.synchronize()
    for r in range(b_ * h_ * nb):
        b, h, q = r // (h_ * nb), (r // nb) % h_, r % nb
        want = oracle.retained_mass(m[b, h, q].astype(np.float64), rows[r], q)
        assert abs(float(got[r]) - want) <= 1e-6, (r, got[r], want)


@pytest.mark.parametrize("nb", [7, 130, 2048])
def test_support_overlap_matches_sets(nb):
    b_, h_ = 1, 2
    say(f"support overlap nb {nb}")
    rng = np.random.default_rng(500 + nb)
    n_rows = b_ * h_ * nb
    rows_a, rpa, cia = _random_csr(rng, n_rows, nb, True)
    rows_b, rpb, cib = _random_csr(rng, n_rows, nb, nb != 130)
    inter, uni = wise.wise_support_overlap((rpa, cia), (rpb, cib), b_, h_, nb, 64, 32)
    inter, uni = inter.cpu().numpy(), uni.cpu().numpy()
    for r in range(n_rows):
        q = r % nb
        sa = {c for c in rows_a[r] if 0 <= c <= q}
        sb = {c for c in rows_b[r] if 0 <= c <= q}
        assert inter[r] == len(sa & sb) and uni[r] == len(sa | sb), r


def test_diagnostics_on_a_trajectory():
    """Retained future mass of the frozen support and the rolling-set Jaccard
    (Eq. 23-25) on a short GPU trajectory, against the oracle on the GPU's
    own supports."""
    cfg = CONFIGS["tiny"].with_(steps=8, td=4, index=301)
    nb, B = cfg.n_blocks, cfg.block
    say(f"diagnostics trajectory {cfg.batch}x{cfg.heads}, S {cfg.seq_len}")
    steps = list(Workload(cfg, threads=4).steps())
    sm = torch.zeros(cfg.steps, cfg.batch, cfg.heads, nb, nb, dtype=torch.float32, device="cuda")
    for t, q, k, v in steps:       # unrestricted masses at every step (diagnostic mode)
        wise.wise_full_attn_accum(to_dev(q), to_dev(k), to_dev(v), sm[t], B)
    frozen = wise.wise_select_variant(wise.SELECT_UNION, sm[cfg.td - 4:cfg.td].contiguous(), cfg.eta,
                                      cfg.head_dim, B)
    late = [wise.wise_support_mass(sm[t], *frozen, cfg.head_dim, B) for t in range(cfg.td, cfg.steps)]
    w_prev = wise.wise_select_variant(wise.SELECT_UNION, sm[max(0, cfg.td - 5):cfg.td - 1].contiguous(), cfg.eta,
                                      cfg.head_dim, B)
    w_final = wise.wise_select_variant(wise.SELECT_UNION, sm[cfg.steps - 4:].contiguous(), cfg.eta,
                                       cfg.head_dim, B)
    ov_roll = wise.wise_support_overlap(frozen, w_prev, cfg.batch, cfg.heads, nb, cfg.head_dim, B)
    ov_fin = wise.wise_support_overlap(frozen, w_final, cfg.batch, cfg.heads, nb, cfg.head_dim, B)
    torch.cuda.synchronize()
    gm = sm.cpu().numpy().astype(np.float64)
    rows_f = csr_rows(*(x.cpu().numpy() for x in frozen))
    rows_p = csr_rows(*(x.cpu().numpy() for x in w_prev))
    rows_z = csr_rows(*(x.cpu().numpy() for x in w_final))
    for i, t in enumerate(range(cfg.td, cfg.steps)):
        got = late[i].cpu().numpy()
        for r in range(len(rows_f)):
            b, h, q = r // (cfg.heads * nb), (r // nb) % cfg.heads, r % nb
            assert abs(float(got[r]) - oracle.retained_mass(gm[t, b, h, q], rows_f[r], q)) <= 1e-6
    # the GPU's rolling sets are the oracle's on the same masses (Eq. 23),
    # up to Appendix A.1 near-ties of the per-step supports
    def near_tie(rows, q):
        for r in rows:
            m = oracle.support_margins(r, q, cfg.eta)
            if min(2 * m["delta_rank"], m["delta_minus"], m["delta_plus"]) <= TIE_EPS:
                return True
        return False
    for r in range(len(rows_f)):
        b, h, q = r // (cfg.heads * nb), (r // nb) % cfg.heads, r % nb
        per_step = [gm[t, b, h, q] for t in range(cfg.steps)]
        for got, t in ((rows_p[r], cfg.td - 2), (rows_z[r], cfg.steps - 1)):
            want = oracle.rolling_working_set(per_step, t, q, cfg.eta)
            assert got == want or near_tie(per_step[max(0, t - 3):t + 1], q), (r, t, got, want)
    j_roll = ov_roll[0].sum().item() / ov_roll[1].sum().item()
    j_fin = ov_fin[0].sum().item() / ov_fin[1].sum().item()
    assert j_roll == oracle.jaccard(rows_f, rows_p) and j_fin == oracle.jaccard(rows_f, rows_z)
    say(f"  retained future mass {np.mean([x.cpu().numpy().mean() for x in late]):.4f}, "
        f"J_roll {j_roll:.4f}, J(switch, final) {j_fin:.4f}")
