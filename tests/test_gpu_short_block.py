"""GPU parity when seq_len is not a multiple of the block size.

The sequence is then cut into ceil(S / B) blocks and the last one is short
(Section 5.1 of the WISE paper with |I_q| counted from the block's real
extent).  Every entry point is compared with the fp64 oracle on seeded
normal bf16 inputs: dense attention and its log-sum-exp, the discovery step
with both mass entry points (on-chip partials and the workspace form), the
selection on the GPU's masses, and sparse attention on random supports that
list the short block.  The shapes put the sequence end inside a 32-query
wave, right after a wave boundary, inside the first 64-key tile of a
128-key block (the second tile then lies wholly past the end), inside the
second tile, and below one block.
"""
import numpy as np
import pytest

import oracle
from wise_inputs import round_to_bf16_bits
from wise_testlib import bf16_dev_to_f64, compare_outputs, mass_tolerance, say, support_ok, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

wise = pytest.importorskip("block_sparse_attention_wise_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wise.load_library()


# (batch, heads, seq, head_dim, block, kv_heads)
SHAPES = [
    (1, 2, 100, 64, 32, 0),     # 4 blocks, the last holds 4 queries (mass in two passes)
    (1, 2, 200, 128, 64, 0),    # 4 blocks, last 8; the last two rows share a workgroup
    (2, 1, 161, 96, 64, 0),     # last block 33: its second wave holds one query
    (1, 2, 300, 128, 128, 0),   # last block 44: second 64-key tile wholly past the end
    (1, 1, 1000, 64, 128, 0),   # last block 104: the second tile holds 40 keys
    (1, 2, 40, 128, 64, 0),     # one block, shorter than the block size
    (1, 4, 230, 128, 64, 2),    # grouped-query attention, last block 38
]
IDS = [f"b{s[0]}h{s[1]}s{s[2]}d{s[3]}B{s[4]}kv{s[5]}" for s in SHAPES]


def _inputs(b, h, s, d, kv, seed, n_steps=1):
    g = np.random.default_rng(seed)
    kvh = kv or h
    out = []
    for _ in range(n_steps):
        q = round_to_bf16_bits(g.standard_normal((b, h, s, d)).astype(np.float32))
        k = round_to_bf16_bits(g.standard_normal((b, kvh, s, d)).astype(np.float32))
        v = round_to_bf16_bits(g.standard_normal((b, kvh, s, d)).astype(np.float32))
        out.append((q, k, v))
    return out


def _heads(q, k, v, b, h, group):
    return oracle.bf16_to_f64(q[b, h]), oracle.bf16_to_f64(k[b, h // group]), oracle.bf16_to_f64(v[b, h // group])


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_short_last_block_dense_and_accum(shape):
    b_, h_, s_, d_, blk, kv = shape
    group = h_ // (kv or h_)
    nb = -(-s_ // blk)
    say(f"short block dense/accum {shape}")
    steps = _inputs(b_, h_, s_, d_, kv, seed=s_ + d_ + blk, n_steps=2)
    mass_l = torch.zeros(b_, h_, nb, nb, dtype=torch.float32, device="cuda")
    mass_w = torch.zeros_like(mass_l)
    lse = torch.empty(b_, h_, s_, dtype=torch.float32, device="cuda")
    outs = []
    for t, (q, k, v) in enumerate(steps):
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        o_d = wise.wise_full_attn(qd, kd, vd, blk, lse=lse if t == 0 else None)
        o_l = wise.wise_full_attn_accum(qd, kd, vd, mass_l, blk)
        o_w = wise.wise_full_attn_accum_ws(qd, kd, vd, mass_w, blk)
        outs.append((o_d, o_l, o_w))
    torch.cuda.synchronize()
    lse_h = lse.cpu().numpy()
    sc = oracle.default_scale(d_)
    for b in range(b_):
        for h in range(h_):
            ref_mass = np.zeros((nb, nb))
            for t, (q, k, v) in enumerate(steps):
                Q, K, V = _heads(q, k, v, b, h, group)
                ref = oracle.dense_attention(Q, K, V, sc)
                for name, o in zip(("dense", "accum", "accum_ws"), outs[t]):
                    compare_outputs(bf16_dev_to_f64(o)[b, h], ref, f"{name} O t{t} b{b}h{h}")
                ref_mass += oracle.block_mass(Q, K, sc, blk)
                if t == 0:
                    s = (Q @ K.T) * sc
                    s[np.triu_indices(s_, 1)] = -np.inf
                    m = s.max(axis=1)
                    ref_lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
                    assert np.max(np.abs(lse_h[b, h] - ref_lse)) < 4e-3
            for name, mass in (("lds", mass_l), ("ws", mass_w)):
                got = mass.cpu().numpy().astype(np.float64)[b, h]
                err = np.abs(got - ref_mass)
                assert err.max() <= mass_tolerance(2), (name, err.max())
                # every row, the short one included, sums to the number of steps
                np.testing.assert_allclose(got.sum(axis=1), 2.0, atol=1e-4)
                assert np.all(got[np.triu_indices(nb, 1)] == 0.0)


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_short_last_block_select_and_sparse(shape):
    b_, h_, s_, d_, blk, kv = shape
    group = h_ // (kv or h_)
    nb = -(-s_ // blk)
    say(f"short block select/sparse {shape}")
    (q, k, v), = _inputs(b_, h_, s_, d_, kv, seed=7 * s_ + d_)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    mass = torch.zeros(b_, h_, nb, nb, dtype=torch.float32, device="cuda")
    wise.wise_full_attn_accum_ws(qd, kd, vd, mass, blk)
    eta = 0.8
    rp_s, ci_s = wise.wise_select_support(mass, 1, eta, d_, blk)
    # random supports, every other row listing the (possibly short) diagonal block
    rng = np.random.default_rng(s_ + blk)
    sups = []
    for r in range(b_ * h_ * nb):
        qb = r % nb
        sup = set(rng.choice(qb + 1, size=rng.integers(1, qb + 2), replace=False).tolist())
        if r % 2 == 0:
            sup.add(qb)
        sups.append(sorted(sup))
    rp = np.zeros(len(sups) + 1, dtype=np.int32)
    rp[1:] = np.cumsum([len(x) for x in sups])
    ci = np.array([c for x in sups for c in x], dtype=np.int32)
    o_r = wise.wise_sparse_attn(qd, kd, vd, torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda(), blk)
    o_s = wise.wise_sparse_attn(qd, kd, vd, rp_s, ci_s, blk)
    torch.cuda.synchronize()
    mass_h = mass.cpu().numpy().astype(np.float64)
    rp_h, ci_h = rp_s.cpu().numpy(), ci_s.cpu().numpy()
    got_r, got_s = bf16_dev_to_f64(o_r), bf16_dev_to_f64(o_s)
    sc = oracle.default_scale(d_)
    for b in range(b_):
        for h in range(h_):
            Q, K, V = _heads(q, k, v, b, h, group)
            base = (b * h_ + h) * nb
            sel = {}
            for qb in range(nb):
                r = base + qb
                row = ci_h[rp_h[r]:rp_h[r + 1]].tolist()
                ok, _ = support_ok(row, mass_h[b, h, qb], qb, eta, 0)
                assert ok, (b, h, qb, row)
                sel[qb] = row
            ref = oracle.masked_attention(Q, K, V, {qb: sups[base + qb] for qb in range(nb)}, blk, sc)
            compare_outputs(got_r[b, h], ref, f"sparse O b{b}h{h}")
            compare_outputs(got_s[b, h], oracle.masked_attention(Q, K, V, sel, blk, sc),
                            f"sparse O (selected) b{b}h{h}")


def test_short_last_block_full_support_equals_dense_bitwise():
    """With every admissible block listed, the sparse launch walks the same
    tiles as the dense one, the short last tile included."""
    b_, h_, s_, d_, blk = 1, 2, 200, 128, 64
    nb = -(-s_ // blk)
    (q, k, v), = _inputs(b_, h_, s_, d_, 0, seed=5)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    sups = [list(range(r % nb + 1)) for r in range(b_ * h_ * nb)]
    rp = np.zeros(len(sups) + 1, dtype=np.int32)
    rp[1:] = np.cumsum([len(x) for x in sups])
    ci = np.array([c for x in sups for c in x], dtype=np.int32)
    o_s = wise.wise_sparse_attn(qd, kd, vd, torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda(), blk)
    o_d = wise.wise_full_attn(qd, kd, vd, blk)
    torch.cuda.synchronize()
    assert torch.equal(o_s.view(torch.int16), o_d.view(torch.int16))


def test_block16_attention_needs_whole_32_tiles():
    """Block 16 runs two logical blocks per 32-key tile: its attention calls
    keep requiring seq_len % 32 == 0, while selection accepts any length."""
    (q, k, v), = _inputs(1, 1, 48, 64, 0, seed=9)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    with pytest.raises(wise.WiseError) as e:
        wise.wise_full_attn(qd, kd, vd, 16)
    assert e.value.status == wise.WISE_ERR_UNSUPPORTED
    mass = torch.full((1, 1, 3, 3), 1.0 / 3, dtype=torch.float32, device="cuda")
    rp, ci = wise.wise_select_support(torch.tril(mass), 1, 0.5, 64, 16)
    torch.cuda.synchronize()
    assert rp.cpu().tolist()[0] == 0 and rp.numel() == 4
