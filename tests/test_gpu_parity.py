"""GPU parity: every HIP kernel behind the C ABI against the fp64 oracle.

Sizes are chosen so the oracle finishes in seconds while still spanning
several key tiles, all three head dims, all three block sizes, several heads
and batches, and odd block counts (a ragged tail of the longest-first grid).
"""
import numpy as np
import pytest

import oracle
from wise_inputs import CONFIGS, Workload
from wise_testlib import (MAX_ABS, MEAN_ABS, bf16_dev_to_f64, check_trajectory_rows,
                          compare_outputs, csr_rows, mass_tolerance, run_trajectory, say,
                          support_ok, to_dev)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

wise = pytest.importorskip("block_sparse_attention_wise_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wise.load_library()


# (batch, heads, seq, head_dim, block): small shapes covering every built kernel.
SHAPES = [
    (1, 2, 256, 64, 16),      # block 16: two logical blocks per 32 x 32 tile
    (2, 1, 160, 128, 16),     # 10 logical blocks; the mass runs in two passes
    (1, 2, 192, 96, 16),
    (1, 2, 256, 64, 32),
    (2, 1, 160, 96, 32),      # 5 blocks
    (1, 2, 320, 128, 64),     # 5 blocks
    (2, 2, 448, 96, 64),      # 7 blocks
    (1, 3, 512, 64, 64),
    (1, 2, 640, 128, 128),    # 5 blocks, two 64-key tiles per block
    (1, 1, 384, 96, 128),
    (1, 1, 256, 128, 32),
]


def _cfg(b, h, s, d, blk, **kw):
    base = CONFIGS["tiny"].with_(batch=b, heads=h, seq_len=s, head_dim=d, block=blk,
                                 steps=4, td=2, planted=(2, 2), index=100 + s + d + blk)
    return base.with_(**kw) if kw else base


def _steps(cfg, n=None):
    return list(Workload(cfg, threads=4).steps(n))


def _oracle_head(bits, b, h):
    return oracle.bf16_to_f64(bits[b, h])


# The two entry points of the discovery step: block-mass partials on chip
# (wise_full_attn_accum) or in a device workspace (wise_full_attn_accum_ws).
ENTRIES = ["lds", "ws"]


def _accum(entry):
    return wise.wise_full_attn_accum if entry == "lds" else wise.wise_full_attn_accum_ws


@pytest.mark.parametrize("shape", SHAPES, ids=[f"b{s[0]}h{s[1]}s{s[2]}d{s[3]}B{s[4]}" for s in SHAPES])
def test_dense_matches_oracle(shape):
    b_, h_, s_, d_, blk = shape
    say(f"dense {shape}")
    _, q, k, v = _steps(_cfg(*shape), 1)[0]
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    lse = torch.empty(b_, h_, s_, dtype=torch.float32, device="cuda")
    o = wise.wise_full_attn(qd, kd, vd, blk, lse=lse)
    torch.cuda.synchronize()
    got = bf16_dev_to_f64(o)
    lse_h = lse.cpu().numpy()
    sc = oracle.default_scale(d_)
    for b in range(b_):
        for h in range(h_):
            Q, K, V = (_oracle_head(x, b, h) for x in (q, k, v))
            ref = oracle.dense_attention(Q, K, V, sc)
            compare_outputs(got[b, h], ref, f"O b{b}h{h}")
            s = (Q @ K.T) * sc
            s[np.triu_indices(s_, 1)] = -np.inf
            m = s.max(axis=1)
            ref_lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
            # The row sum adds the bf16-rounded probabilities that the PV product
            # uses (8 significant bits, round to nearest: relative error <= 2^-8
            # each), so log(l) moves by at most -log(1 - 2^-8) = 3.91e-3.
            assert np.max(np.abs(lse_h[b, h] - ref_lse)) < 4e-3


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("d_,blk", [(64, 32), (128, 64), (96, 128)])
def test_dense_large_logits_rescale_path(d_, blk, entry):
    """Logits spanning hundreds of units: the reference max jumps by more than
    the 64 log2-unit slack on about half of the non-first wave tiles, so the
    rescale of O, l and the mass partials runs many times."""
    say(f"dense large logits d{d_} B{blk} {entry}")
    s_ = 4 * blk
    g = np.random.default_rng(7)
    from wise_inputs import round_to_bf16_bits
    q = round_to_bf16_bits(3.0 * g.standard_normal((1, 2, s_, d_)).astype(np.float32))
    k = round_to_bf16_bits(3.0 * g.standard_normal((1, 2, s_, d_)).astype(np.float32))
    v = round_to_bf16_bits(g.standard_normal((1, 2, s_, d_)).astype(np.float32))
    # later keys grow, so the max rises along the key walk
    o = wise.wise_full_attn(to_dev(q), to_dev(k), to_dev(v), blk, softmax_scale=1.0)
    mass = torch.zeros(1, 2, s_ // blk, s_ // blk, dtype=torch.float32, device="cuda")
    o2 = _accum(entry)(to_dev(q), to_dev(k), to_dev(v), mass, blk, softmax_scale=1.0)
    torch.cuda.synchronize()
    got, got2 = bf16_dev_to_f64(o), bf16_dev_to_f64(o2)
    mass_h = mass.cpu().numpy().astype(np.float64)
    for h in range(2):
        Q, K, V = (oracle.bf16_to_f64(x[0, h]) for x in (q, k, v))
        compare_outputs(got[0, h], oracle.dense_attention(Q, K, V, 1.0), f"O h{h}")
        compare_outputs(got2[0, h], oracle.dense_attention(Q, K, V, 1.0), f"O(accum) h{h}")
        r = oracle.block_mass(Q, K, 1.0, blk)
        # peaked softmax: bf16 score rounding matters more, allow 1e-3
        assert np.max(np.abs(mass_h[0, h] - np.tril(r))) < 1e-3


# (heads, seq, head_dim, block, seed).  Q and K at 4x amplitude give rows
# whose softmax is dominated by one or two keys, and outputs near |O| = 4,
# where bf16 output rounding alone is up to 2^-6.  P enters the PV product
# rounded to bf16; if O is divided by a sum that counts the dominant weight
# unrounded (the fp32 sum of p, or p/l rounded as the operand), that
# weight's rounding error reaches O undamped.  For each case a CPU emulation
# of the roundings puts the earlier forms above the 2e-2 bound: the p/l
# operand of the two-pass mass launch (blocks 16 and 32) at 2.1-2.3e-2, the
# plain fp32 divisor of the one-pass launch (blocks 64 and 128) at
# 2.4-2.9e-2.  Counting the dominant weight as rounded keeps every mode at
# the output rounding floor (about 1.5e-2 at worst).
PEAKED = [(8, 256, 128, 32, 2), (8, 256, 64, 32, 7), (8, 256, 96, 16, 1),
          (8, 256, 128, 64, 30), (4, 512, 128, 128, 20)]


@pytest.mark.parametrize("shape", PEAKED, ids=[f"h{s[0]}s{s[1]}d{s[2]}B{s[3]}seed{s[4]}" for s in PEAKED])
def test_peaked_rows_every_mode(shape):
    h_, s_, d_, blk, seed = shape
    say(f"peaked rows {shape}")
    from wise_inputs import round_to_bf16_bits
    g = np.random.default_rng(seed)
    q = round_to_bf16_bits((4.0 * g.standard_normal((1, h_, s_, d_))).astype(np.float32))
    k = round_to_bf16_bits((4.0 * g.standard_normal((1, h_, s_, d_))).astype(np.float32))
    v = round_to_bf16_bits(g.standard_normal((1, h_, s_, d_)).astype(np.float32))
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    nb = s_ // blk
    o = wise.wise_full_attn(qd, kd, vd, blk)
    mass = torch.zeros(1, h_, nb, nb, dtype=torch.float32, device="cuda")
    oa = wise.wise_full_attn_accum(qd, kd, vd, mass, blk)
    mass_ws = torch.zeros_like(mass)
    oa_ws = wise.wise_full_attn_accum_ws(qd, kd, vd, mass_ws, blk)
    # full causal support through the sparse kernel
    rows = [list(range(r % nb + 1)) for r in range(h_ * nb)]
    rp = np.zeros(len(rows) + 1, dtype=np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ci = np.array([c for r in rows for c in r], dtype=np.int32)
    os_ = wise.wise_sparse_attn(qd, kd, vd, torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda(), blk)
    torch.cuda.synchronize()
    got, got_a, got_s = bf16_dev_to_f64(o), bf16_dev_to_f64(oa), bf16_dev_to_f64(os_)
    got_w = bf16_dev_to_f64(oa_ws)
    mass_h = mass.cpu().numpy().astype(np.float64)
    mass_w = mass_ws.cpu().numpy().astype(np.float64)
    sc = oracle.default_scale(d_)
    for h in range(h_):
        Q, K, V = (oracle.bf16_to_f64(x[0, h]) for x in (q, k, v))
        ref = oracle.dense_attention(Q, K, V, sc)
        compare_outputs(got[0, h], ref, f"O(dense) h{h}")
        compare_outputs(got_a[0, h], ref, f"O(accum) h{h}")
        compare_outputs(got_s[0, h], ref, f"O(sparse) h{h}")
        compare_outputs(got_w[0, h], ref, f"O(accum, workspace) h{h}")
        # logits reach ~60 here; fp32 accumulation of the scores then moves
        # p by up to ~5e-4 relative in the worst case
        mref = np.tril(oracle.block_mass(Q, K, sc, blk))
        assert np.max(np.abs(mass_h[0, h] - mref)) < 1e-3
        assert np.max(np.abs(mass_w[0, h] - mref)) < 1e-3


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("shape", SHAPES[:9], ids=[f"b{s[0]}h{s[1]}s{s[2]}d{s[3]}B{s[4]}" for s in SHAPES[:9]])
def test_accum_mass_matches_oracle(shape, entry):
    b_, h_, s_, d_, blk = shape
    say(f"accum {shape} {entry}")
    steps = _steps(_cfg(*shape), 2)
    nb = s_ // blk
    mass = torch.zeros(b_, h_, nb, nb, dtype=torch.float32, device="cuda")
    outs = []
    dense_outs = []
    for _, q, k, v in steps:
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        outs.append(_accum(entry)(qd, kd, vd, mass, blk))
        dense_outs.append(wise.wise_full_attn(qd, kd, vd, blk))
    torch.cuda.synchronize()
    mass_h = mass.cpu().numpy().astype(np.float64)
    sc = oracle.default_scale(d_)
    for t in range(2):
        # Same attention output as the dense kernel up to one bf16 rounding
        # step: the mass launch divides by the fp32 row sum (its largest term
        # as rounded), the dense one by the sum of the bf16 operands, and the
        # two may walk the keys in tiles of different sizes.
        diff = (outs[t].float() - dense_outs[t].float()).abs().max().item()
        assert diff <= 2 ** -6, diff
    for b in range(b_):
        for h in range(h_):
            ref = np.zeros((nb, nb))
            for t, (_, q, k, v) in enumerate(steps):
                Q, K, V = (_oracle_head(x, b, h) for x in (q, k, v))
                ref += oracle.block_mass(Q, K, sc, blk)
                compare_outputs(bf16_dev_to_f64(outs[t])[b, h], oracle.dense_attention(Q, K, V, sc),
                                f"O t{t} b{b}h{h}")
            err = np.abs(mass_h[b, h] - ref)
            assert err.max() <= mass_tolerance(2), err.max()
            np.testing.assert_allclose(mass_h[b, h].sum(axis=1), 2.0, atol=1e-4)
            # entries above the diagonal are never written (still zero)
            assert np.all(mass_h[b, h][np.triu_indices(nb, 1)] == 0.0)


def _random_masses(rng, b_, h_, nb, n_steps, kind):
    m = np.zeros((b_, h_, nb, nb), dtype=np.float32)
    for b in range(b_):
        for h in range(h_):
            for q in range(nb):
                if kind == "dirichlet":
                    w = rng.dirichlet(np.full(q + 1, 0.4))
                elif kind == "dyadic":      # exact ties on a 1/64 grid
                    w = rng.integers(0, 5, q + 1).astype(np.float64)
                    w[q] += 1.0
                    w = w / w.sum()
                    w = np.round(w * 64) / 64
                else:                      # zeros and equal masses
                    w = np.zeros(q + 1)
                    idx = rng.choice(q + 1, size=min(q + 1, 3), replace=False)
                    w[idx] = 1.0 / len(idx)
                m[b, h, q, :q + 1] = (w * n_steps).astype(np.float32)
    return m


@pytest.mark.parametrize("nb,kind,eta,cap,n_steps", [
    (8, "dirichlet", 0.9, 0, 2), (33, "dirichlet", 0.95, 0, 8), (64, "dirichlet", 0.9, 0, 8),
    (64, "dyadic", 0.75, 0, 4), (64, "ties", 0.5, 0, 3), (130, "dirichlet", 0.9, 5, 8),
    (256, "dirichlet", 0.9, 64, 4), (512, "dirichlet", 0.9, 0, 8), (100, "dirichlet", 1.0, 0, 8),
    (70, "dyadic", 0.9, 2, 1), (1, "dirichlet", 0.9, 0, 2), (1100, "dirichlet", 0.95, 0, 8),
])
def test_select_matches_oracle(nb, kind, eta, cap, n_steps):
    say(f"select nb{nb} {kind} eta{eta} cap{cap}")
    rng = np.random.default_rng(nb * 7 + cap)
    b_, h_, blk = 1, 2, 32
    mass = _random_masses(rng, b_, h_, nb, n_steps, kind)
    row_ptr, col_idx = wise.wise_select_support(torch.from_numpy(mass).cuda(), n_steps, eta, 64,
                                                blk, cap)
    torch.cuda.synchronize()
    rp, ci = row_ptr.cpu().numpy(), col_idx.cpu().numpy()
    assert rp[0] == 0 and np.all(np.diff(rp) >= 1)
    rows = csr_rows(rp, ci)
    ties = 0
    for r, sup in enumerate(rows):
        q = r % nb
        mbar = mass.reshape(-1, nb)[r].astype(np.float64) / n_steps
        ok, tie = support_ok(sup, mbar, q, eta, cap)
        assert ok, (r, q, sup, oracle.select_support(mbar, q, eta, cap))
        ties += tie
    say(f"  rows {len(rows)} near-tie differences {ties}")


def _csr_from_supports(sup_rows):
    rp = np.zeros(len(sup_rows) + 1, dtype=np.int32)
    for i, s in enumerate(sup_rows):
        rp[i + 1] = rp[i] + len(s)
    ci = np.array([c for s in sup_rows for c in s] or [0], dtype=np.int32)
    return rp, ci


@pytest.mark.parametrize("shape", SHAPES, ids=[f"b{s[0]}h{s[1]}s{s[2]}d{s[3]}B{s[4]}" for s in SHAPES])
def test_sparse_matches_oracle(shape):
    b_, h_, s_, d_, blk = shape
    say(f"sparse {shape}")
    _, q, k, v = _steps(_cfg(*shape), 1)[0]
    nb = s_ // blk
    rng = np.random.default_rng(s_ + d_)
    sups = []
    for r in range(b_ * h_ * nb):
        qb = r % nb
        kind = r % 4
        if kind == 0:
            sup = sorted(set(rng.choice(qb + 1, size=rng.integers(1, qb + 2), replace=False).tolist()) | {qb})
        elif kind == 1:
            sup = sorted(set(rng.choice(qb + 1, size=rng.integers(1, qb + 2), replace=False).tolist()) | {0})
        elif kind == 2:
            sup = [qb]
        else:
            sup = list(range(qb + 1))
        sups.append(sup)
    rp, ci = _csr_from_supports(sups)
    o = wise.wise_sparse_attn(to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(rp).cuda(),
                              torch.from_numpy(ci).cuda(), blk)
    torch.cuda.synchronize()
    got = bf16_dev_to_f64(o)
    sc = oracle.default_scale(d_)
    for b in range(b_):
        for h in range(h_):
            Q, K, V = (_oracle_head(x, b, h) for x in (q, k, v))
            base = (b * h_ + h) * nb
            supports = {qb: sups[base + qb] for qb in range(nb)}
            ref = oracle.masked_attention(Q, K, V, supports, blk, sc)
            compare_outputs(got[b, h], ref, f"sparse O b{b}h{h}")


def test_sparse_ignores_invalid_entries():
    """CSR rows are read as sets: out-of-range entries are skipped (never
    read), repeats count once, order does not matter."""
    b_, h_, s_, d_, blk = 1, 1, 320, 128, 64
    say("sparse invalid entries")
    _, q, k, v = _steps(_cfg(b_, h_, s_, d_, blk), 1)[0]
    raw = [[0, 0], [1, -3, 0, 1], [7, 0, 2, 2, 1], [0, 1, 3, 9], [2, 4, 3, 100, -1]]
    clean = [sorted({c for c in row if 0 <= c <= qb}) for qb, row in enumerate(raw)]
    assert clean == [[0], [0, 1], [0, 1, 2], [0, 1, 3], [2, 3, 4]]
    rp, ci = _csr_from_supports(raw)
    o = wise.wise_sparse_attn(to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(rp).cuda(),
                              torch.from_numpy(ci).cuda(), blk)
    torch.cuda.synchronize()
    Q, K, V = (_oracle_head(x, 0, 0) for x in (q, k, v))
    ref = oracle.masked_attention(Q, K, V, {i: c for i, c in enumerate(clean)}, blk)
    compare_outputs(bf16_dev_to_f64(o)[0, 0], ref, "sparse O (cleaned CSR)")


def test_sparse_empty_rows_give_zeros():
    b_, h_, s_, d_, blk = 1, 1, 256, 64, 64
    _, q, k, v = _steps(_cfg(b_, h_, s_, d_, blk), 1)[0]
    rp, ci = _csr_from_supports([[0], [], [0, 2], []])
    o = wise.wise_sparse_attn(to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(rp).cuda(),
                              torch.from_numpy(ci).cuda(), blk)
    torch.cuda.synchronize()
    got = bf16_dev_to_f64(o)[0, 0]
    assert np.all(got[64:128] == 0) and np.all(got[192:256] == 0)
    Q, K, V = (_oracle_head(x, 0, 0) for x in (q, k, v))
    ref = oracle.masked_attention(Q, K, V, {0: [0], 1: [], 2: [0, 2], 3: []}, blk)
    compare_outputs(got, ref, "sparse O with empty rows")


@pytest.mark.parametrize("shape", [SHAPES[3], SHAPES[5], SHAPES[8], SHAPES[6], SHAPES[0], SHAPES[1]],
                         ids=["d64B32", "d128B64", "d128B128", "d96B64b2", "d64B16", "d128B16b2"])
def test_sparse_full_support_equals_dense_bitwise(shape):
    """Same backend on every causal block: the sparse kernel reproduces the
    dense kernel exactly (same tiles in the same order)."""
    b_, h_, s_, d_, blk = shape
    _, q, k, v = _steps(_cfg(*shape), 1)[0]
    nb = s_ // blk
    rp, ci = _csr_from_supports([list(range(r % nb + 1)) for r in range(b_ * h_ * nb)])
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o_s = wise.wise_sparse_attn(qd, kd, vd, torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda(), blk)
    o_d = wise.wise_full_attn(qd, kd, vd, blk)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_d)


def test_deterministic_repeat():
    shape = SHAPES[5]
    b_, h_, s_, d_, blk = shape
    _, q, k, v = _steps(_cfg(*shape), 1)[0]
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    nb = s_ // blk
    m1 = torch.zeros(b_, h_, nb, nb, device="cuda")
    m2 = torch.zeros(b_, h_, nb, nb, device="cuda")
    o1 = wise.wise_full_attn_accum(qd, kd, vd, m1, blk)
    o2 = wise.wise_full_attn_accum(qd, kd, vd, m2, blk)
    r1, c1 = wise.wise_select_support(m1, 1, 0.9, d_, blk)
    r2, c2 = wise.wise_select_support(m2, 1, 0.9, d_, blk)
    s1 = wise.wise_sparse_attn(qd, kd, vd, r1, c1, blk)
    s2 = wise.wise_sparse_attn(qd, kd, vd, r2, c2, blk)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(m1, m2) and torch.equal(r1, r2)
    n = int(r1[-1])
    assert torch.equal(c1[:n], c2[:n]) and torch.equal(s1, s2)


def test_tiny_trajectory_end_to_end():
    """The tiny workload (4 heads, d 64, seq 256, B 32, T 4, td 2, eta 0.9)
    through all four calls, every row checked."""
    cfg = CONFIGS["tiny"]
    say("tiny trajectory")
    steps = _steps(cfg)
    mass, row_ptr, col_idx, outs = run_trajectory(cfg, steps)
    gm = mass.cpu().numpy()
    rows = csr_rows(row_ptr.cpu().numpy(), col_idx.cpu().numpy())
    outs_h = [bf16_dev_to_f64(o) for o in outs]
    wl = Workload(cfg)
    samples = [(0, h, qb) for h in range(cfg.heads) for qb in range(cfg.n_blocks)]
    stats = _check(cfg, gm, rows, outs_h, samples, wl)
    say(f"  {stats['rows']} rows, margin rows {stats['margin_rows']}, max-abs {stats['max_abs']:.2e}")


def _check(cfg, gm, rows, outs_h, samples, wl, out_steps=None):
    return check_trajectory_rows(cfg, gm, rows, lambda t, b, h, r: outs_h[t][b, h][r], samples,
                                 lambda b, h: wl.head_steps(b, h), out_steps=out_steps)


def test_small_trajectories_end_to_end():
    """Scaled-down versions of the 4K, wide-head and long-context workloads."""
    for cfg in (CONFIGS["ctx4k"].with_(heads=2, seq_len=1024, steps=6, td=3),
                CONFIGS["wide"].with_(batch=2, heads=3, seq_len=768, steps=5, td=2),
                CONFIGS["long"].with_(heads=2, seq_len=2048, steps=4, td=2, cap=6),
                CONFIGS["ctx4k"].with_(heads=2, seq_len=1024, block=16, steps=5, td=2, index=77)):
        say(f"trajectory {cfg.name} {cfg.batch}x{cfg.heads} S{cfg.seq_len}")
        steps = _steps(cfg)
        mass, row_ptr, col_idx, outs = run_trajectory(cfg, steps)
        gm = mass.cpu().numpy()
        rows = csr_rows(row_ptr.cpu().numpy(), col_idx.cpu().numpy())
        outs_h = [bf16_dev_to_f64(o) for o in outs]
        wl = Workload(cfg)
        samples = [(b, h, qb) for b in range(cfg.batch) for h in range(cfg.heads)
                   for qb in range(cfg.n_blocks)]
        stats = _check(cfg, gm, rows, outs_h, samples, wl)
        say(f"  {stats['rows']} rows, margin rows {stats['margin_rows']}, "
            f"max-abs {stats['max_abs']:.2e}, mean-abs {np.mean(stats['mean_abs']):.2e}")


# Long rows: the on-chip mass launch switches to its two-pass form (row max
# and sum first, then P, O and the mass) when one-pass LDS partials would
# leave too few resident waves; the workspace launch keeps one pass with
# its partials in device memory.  (batch, heads, seq, head_dim, block)
LONG_SHAPES = [
    (1, 1, 32768, 128, 64),
    (1, 2, 8192, 64, 32),
    (1, 1, 40960, 96, 128),
]


@pytest.mark.parametrize("entry", ENTRIES)
@pytest.mark.parametrize("shape", LONG_SHAPES, ids=[f"b{s[0]}h{s[1]}s{s[2]}d{s[3]}B{s[4]}" for s in LONG_SHAPES])
def test_accum_long_rows_matches_oracle(shape, entry):
    b_, h_, s_, d_, blk = shape
    say(f"accum long rows {shape} {entry}")
    steps = _steps(_cfg(*shape), 2)
    nb = s_ // blk
    mass = torch.zeros(b_, h_, nb, nb, dtype=torch.float32, device="cuda")
    qbs = sorted({0, 1, nb // 3, nb - 2, nb - 1})
    outs = []
    for _, q, k, v in steps:
        o = _accum(entry)(to_dev(q), to_dev(k), to_dev(v), mass, blk)
        outs.append({qb: bf16_dev_to_f64(o[:, :, qb * blk:(qb + 1) * blk]) for qb in qbs})
    torch.cuda.synchronize()
    mass_h = mass.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(mass_h.sum(axis=-1), 2.0, atol=1e-4)
    iu = np.triu_indices(nb, 1)
    assert np.all(mass_h[..., iu[0], iu[1]] == 0.0)
    sc = oracle.default_scale(d_)
    for b in range(b_):
        for h in range(h_):
            ref = np.zeros((len(qbs), nb))
            for t, (_, q, k, v) in enumerate(steps):
                Q, K, V = (_oracle_head(x, b, h) for x in (q, k, v))
                ref += oracle.block_mass(Q, K, sc, blk, qblocks=qbs)
                for qb in qbs:
                    rows = np.arange(qb * blk, (qb + 1) * blk)
                    compare_outputs(outs[t][qb][b, h], oracle.dense_attention(Q, K, V, sc, rows),
                                    f"O t{t} b{b}h{h}q{qb}")
            err = np.abs(mass_h[b, h][qbs] - ref)
            assert err.max() <= mass_tolerance(2), err.max()


# Grouped-query attention: (batch, heads, kv_heads, seq, head_dim, block).
GQA_SHAPES = [
    (1, 8, 2, 320, 128, 64),
    (2, 4, 1, 256, 64, 32),
    (1, 6, 3, 384, 96, 128),
]


@pytest.mark.parametrize("shape", GQA_SHAPES, ids=[f"b{s[0]}h{s[1]}kv{s[2]}s{s[3]}d{s[4]}B{s[5]}" for s in GQA_SHAPES])
def test_gqa_all_calls_match_oracle(shape):
    """Every attention call with K/V shared by groups of query heads: query
    head h reads K/V head h // (heads / kv_heads); mass and CSR rows stay per
    query head."""
    b_, h_, kv_, s_, d_, blk = shape
    say(f"gqa {shape}")
    cfg = _cfg(b_, h_, s_, d_, blk).with_(kv_heads=kv_, td=2, steps=3)
    steps = _steps(cfg)
    G, nb = h_ // kv_, s_ // blk
    assert steps[0][2].shape[1] == kv_
    mass = torch.zeros(b_, h_, nb, nb, dtype=torch.float32, device="cuda")
    dense, accum = [], []
    for t, q, k, v in steps[:2]:
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        dense.append(bf16_dev_to_f64(wise.wise_full_attn(qd, kd, vd, blk)))
        accum.append(bf16_dev_to_f64(wise.wise_full_attn_accum(qd, kd, vd, mass, blk)))
    rp, ci = wise.wise_select_support(mass, 2, cfg.eta, d_, blk)
    _, q, k, v = steps[2]
    sparse = bf16_dev_to_f64(wise.wise_sparse_attn(to_dev(q), to_dev(k), to_dev(v), rp, ci, blk))
    torch.cuda.synchronize()
    rows = csr_rows(rp.cpu().numpy(), ci.cpu().numpy())
    mass_h = mass.cpu().numpy().astype(np.float64)
    sc = oracle.default_scale(d_)
    for b in range(b_):
        for h in range(h_):
            ref_mass = np.zeros((nb, nb))
            for t in range(2):
                _, q, k, v = steps[t]
                Q, K, V = _oracle_head(q, b, h), _oracle_head(k, b, h // G), _oracle_head(v, b, h // G)
                ref = oracle.dense_attention(Q, K, V, sc)
                compare_outputs(dense[t][b, h], ref, f"dense t{t} b{b}h{h}")
                compare_outputs(accum[t][b, h], ref, f"accum t{t} b{b}h{h}")
                ref_mass += oracle.block_mass(Q, K, sc, blk)
            assert np.abs(mass_h[b, h] - ref_mass).max() <= mass_tolerance(2)
            _, q, k, v = steps[2]
            Q, K, V = _oracle_head(q, b, h), _oracle_head(k, b, h // G), _oracle_head(v, b, h // G)
            sup = {qb: rows[(b * h_ + h) * nb + qb] for qb in range(nb)}
            compare_outputs(sparse[b, h], oracle.masked_attention(Q, K, V, sup, blk, sc), f"sparse b{b}h{h}")
