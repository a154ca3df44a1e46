"""GPU parity at the full workload sizes, in the launch configuration that
bench.py times (the same four library calls on whole tensors).

The oracle cannot evaluate whole 4K-32K trajectories, so each test checks
sampled (batch, head, query block) rows one by one (block masses, supports
against the oracle's fp64 selection with only 1e-6 near ties allowed to
differ, and the attention outputs of every evaluated step), plus, for every
row: block masses sum to the number of discovery steps, each CSR row equals
the oracle's selection on the GPU's own masses (bit-exact but for 1e-6 near
ties), is ascending inside [0, q], holds the sink and the diagonal, and the
cap is respected.

For the larger workloads only the first two reuse steps are run (the
discovery steps, the selection and the late-step kernel are exercised in
full; later reuse steps repeat the same launch on new inputs)."""
import numpy as np
import pytest

from wise_inputs import CONFIGS, Workload
from wise_testlib import (bf16_dev_to_f64, check_selection_every_row, check_trajectory_rows, csr_rows,
                          say, to_dev)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
wise = pytest.importorskip("block_sparse_attention_wise_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wise.load_library()


def _samples(cfg, rng):
    nb = cfg.n_blocks
    heads = {(0, 0), (cfg.batch - 1, cfg.heads - 1), (cfg.batch // 2, cfg.heads // 2)}
    out = []
    for (b, h) in sorted(heads):
        qbs = {0, 1, nb // 2, nb - 1} | set(int(x) for x in rng.integers(0, nb, 3))
        out += [(b, h, qb) for qb in sorted(qbs)]
    return out


@pytest.mark.parametrize("name", ["ctx4k", "ctx8k", "ctx16k", "ctx32k", "wide", "long", "gqa4k", "ctx4k_eta06"])
def test_full_size_trajectory(name):
    cfg = CONFIGS[name]
    n_steps = cfg.steps if name == "ctx4k" else cfg.td + 2
    rng = np.random.default_rng(cfg.seed)
    samples = _samples(cfg, rng)
    say(f"full-size {name}: {cfg.batch}x{cfg.heads} heads, S {cfg.seq_len}, D {cfg.head_dim}, "
        f"B {cfg.block}, {n_steps} steps, {len(samples)} sampled rows")
    nb, B = cfg.n_blocks, cfg.block
    mass = torch.zeros(cfg.batch, cfg.heads, nb, nb, dtype=torch.float32, device="cuda")
    # the discovery steps run as bench.py runs them: block-mass partials in a workspace
    ws = torch.empty(max(wise.wise_accum_workspace_bytes(cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, B), 16),
                     dtype=torch.uint8, device="cuda")
    rows_idx = {(b, h, qb): (b, h, np.arange(qb * B, (qb + 1) * B)) for (b, h, qb) in samples}
    got = {}
    row_ptr = col_idx = None
    for t, q, k, v in Workload(cfg, threads=16).steps(n_steps):
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        del q, k, v
        if t < cfg.td:
            o = wise.wise_full_attn_accum_ws(qd, kd, vd, mass, B, workspace=ws)
        else:
            if row_ptr is None:
                row_ptr, col_idx = wise.wise_select_support(mass, cfg.td, cfg.eta, cfg.head_dim, B, cfg.cap)
            o = wise.wise_sparse_attn(qd, kd, vd, row_ptr, col_idx, B)
        for key, (b, h, r) in rows_idx.items():
            got[(t,) + key] = bf16_dev_to_f64(o[b, h, r[0]:r[-1] + 1])
        del qd, kd, vd, o
    torch.cuda.synchronize()
    say(f"  GPU trajectory done, nnz {int(row_ptr[-1])}")

    gm = mass.cpu().numpy()
    # Every row: masses sum to td; nothing written above the diagonal.
    sums = gm.sum(axis=-1)
    assert np.abs(sums - cfg.td).max() < 1e-3 * cfg.td, np.abs(sums - cfg.td).max()
    iu = np.triu_indices(nb, 1)
    assert np.all(gm[..., iu[0], iu[1]] == 0.0)
    rp, ci = row_ptr.cpu().numpy(), col_idx.cpu().numpy()
    rows = csr_rows(rp, ci)
    for r, sup in enumerate(rows):
        qb = r % nb
        assert sup[0] == 0 and sup[-1] == qb and all(a < b for a, b in zip(sup, sup[1:])), (r, sup)
        if cfg.cap > 0:
            assert len(sup) <= cfg.cap + 2
    dens = rp[-1] / (cfg.batch * cfg.heads * nb * (nb + 1) / 2)
    say(f"  realised density (admissible) {dens:.4f}")
    ties = check_selection_every_row(cfg, gm, rows)
    say(f"  all {len(rows)} CSR rows equal the oracle's selection on the GPU's masses; "
        f"near-tie rows that differ: {ties}")

    wl = Workload(cfg, threads=4)
    stats = check_trajectory_rows(
        cfg, gm, rows, lambda t, b, h, r: got[(t, b, h, int(r[0]) // B)], samples,
        lambda b, h: wl.head_steps(b, h, n_steps), out_steps=range(n_steps))
    say(f"  {stats['rows']} sampled rows, {stats['margin_rows']} near-margin supports, "
        f"max-abs {stats['max_abs']:.2e}, mean-abs {np.mean(stats['mean_abs']):.2e}")


# Largest sizes the library accepts: 65536 keys (the descriptor limit), 2048
# key blocks per row (the selection limit) at block 32 and at block 16.
MAX_SHAPES = [(65536, 128, 64), (65536, 64, 32), (32768, 96, 16)]


@pytest.mark.parametrize("shape", MAX_SHAPES, ids=[f"s{s[0]}d{s[1]}B{s[2]}" for s in MAX_SHAPES])
def test_maximum_sizes(shape):
    s_, d_, blk = shape
    cfg = CONFIGS["tiny"].with_(batch=1, heads=1, seq_len=s_, head_dim=d_, block=blk, steps=3, td=2,
                                planted=(8, 8), beta=2.0, sigma=0.02, index=900 + blk)
    nb = cfg.n_blocks
    rng = np.random.default_rng(cfg.seed)
    qbs = sorted({0, 1, nb // 2, nb - 2, nb - 1} | set(int(x) for x in rng.integers(0, nb, 2)))
    samples = [(0, 0, qb) for qb in qbs]
    say(f"maximum size {shape}: {nb} blocks, sampled rows {qbs}")
    mass = torch.zeros(1, 1, nb, nb, dtype=torch.float32, device="cuda")
    got = {}
    row_ptr = col_idx = None
    for t, q, k, v in Workload(cfg, threads=16).steps():
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        if t < cfg.td:
            o = wise.wise_full_attn_accum(qd, kd, vd, mass, blk)
        else:
            row_ptr, col_idx = wise.wise_select_support(mass, cfg.td, cfg.eta, d_, blk)
            o = wise.wise_sparse_attn(qd, kd, vd, row_ptr, col_idx, blk)
        for qb in qbs:
            got[(t, qb)] = bf16_dev_to_f64(o[0, 0, qb * blk:(qb + 1) * blk])
        del qd, kd, vd, o
    torch.cuda.synchronize()
    gm = mass.cpu().numpy()
    np.testing.assert_allclose(gm.sum(axis=-1), cfg.td, atol=1e-3 * cfg.td)
    rows = csr_rows(row_ptr.cpu().numpy(), col_idx.cpu().numpy())
    assert all(r[0] == 0 and r[-1] == i for i, r in enumerate(rows))
    wl = Workload(cfg, threads=4)
    ties = check_selection_every_row(cfg, gm, rows)
    stats = check_trajectory_rows(cfg, gm, rows, lambda t, b, h, r: got[(t, int(r[0]) // blk)], samples,
                                  lambda b, h: wl.head_steps(b, h, cfg.steps), out_steps=range(cfg.steps))
    say(f"  {stats['rows']} rows, {ties} near-tie CSR rows, max-abs {stats['max_abs']:.2e}")
