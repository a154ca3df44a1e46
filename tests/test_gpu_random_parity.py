"""Randomised GPU parity: every attention launch on random small problems.

Each case draws, from its own seed: the head dim (64, 96, 128), the block
size (16, 32, 64, 128), 1-10 query blocks, 1-2 batches, 1-2 KV heads with
1, 2 or 4 query heads each (grouped-query attention), the default or a
random softmax scale, and Q and K at unit or 4x amplitude (4x makes rows
whose softmax is dominated by one or two keys).  It runs the dense launch
(with LSE), both mass launches (partials on chip and in a workspace) and
the sparse launch on messy CSR rows (empty,
the full causal row, random entries with repeats, entries outside [0, q]
that the kernel must ignore, unsorted), and checks each against the fp64
oracle: O to the output tolerance, the LSE to bf16-operand accuracy, the
block mass to fp32 accuracy.  Cases from N_CASES on also cut the sequence
short of a whole last block (block sizes 32-128; block 16 attention needs
whole 32-key tiles), so that block holds between 1 and B - 1 positions.
"""
import numpy as np
import pytest

import oracle
from wise_inputs import round_to_bf16_bits
from wise_testlib import bf16_dev_to_f64, compare_outputs, mass_tolerance, say, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

wise = pytest.importorskip("block_sparse_attention_wise_amd")

N_CASES = 48
N_SHORT = 16


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wise.load_library()


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    d = int(rng.choice([64, 96, 128]))
    blk = int(rng.choice([16, 32, 64, 128]))
    nb = int(rng.integers(1, 11))
    if blk == 16 and nb % 2:
        nb += 1                                   # block 16 needs an even block count
    b = int(rng.integers(1, 3))
    kvh = int(rng.choice([1, 2]))
    grp = int(rng.choice([1, 2, 4]))
    scale = 0.0 if rng.random() < 0.5 else float(rng.uniform(0.02, 0.3))   # 0: 1/sqrt(d)
    amp = float(rng.choice([1.0, 4.0]))
    s = nb * blk
    if seed >= N_CASES:
        if blk == 16:
            blk = 32
            s = nb * blk
        s -= int(rng.integers(1, blk))            # a short last block of 1..B-1 positions
    return rng, dict(d=d, blk=blk, nb=nb, s=s, b=b, kvh=kvh, h=kvh * grp, grp=grp,
                     scale=scale, amp=amp)


def _messy_rows(rng, n_rows, nb):
    rows = []
    for r in range(n_rows):
        qb = r % nb
        kind = int(rng.integers(0, 5))
        if kind == 0:
            row = []
        elif kind == 1:
            row = list(range(qb + 1))
        else:
            row = rng.integers(-2, qb + 3, size=int(rng.integers(1, qb + 4))).tolist()
            if kind == 3:
                row = row + row[:2]               # repeats
        rows.append(row)
    return rows


@pytest.mark.parametrize("seed", range(N_CASES + N_SHORT))
def test_random_case(seed):
    rng, c = _case(seed)
    say(f"random case {seed}: {c}")
    b, h, kvh, s, d, blk, nb = c["b"], c["h"], c["kvh"], c["s"], c["d"], c["blk"], c["nb"]
    q = round_to_bf16_bits((c["amp"] * rng.standard_normal((b, h, s, d))).astype(np.float32))
    k = round_to_bf16_bits((c["amp"] * rng.standard_normal((b, kvh, s, d))).astype(np.float32))
    v = round_to_bf16_bits(rng.standard_normal((b, kvh, s, d)).astype(np.float32))
    rows = _messy_rows(rng, b * h * nb, nb)
    rp = np.zeros(len(rows) + 1, dtype=np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ci = np.array([x for r in rows for x in r] or [0], dtype=np.int32)

    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    lse = torch.empty(b, h, s, dtype=torch.float32, device="cuda")
    o = wise.wise_full_attn(qd, kd, vd, blk, lse=lse, softmax_scale=c["scale"])
    mass = torch.zeros(b, h, nb, nb, dtype=torch.float32, device="cuda")
    oa = wise.wise_full_attn_accum(qd, kd, vd, mass, blk, softmax_scale=c["scale"])
    mass_w = torch.zeros_like(mass)
    ow = wise.wise_full_attn_accum_ws(qd, kd, vd, mass_w, blk, softmax_scale=c["scale"])
    osp = wise.wise_sparse_attn(qd, kd, vd, torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda(), blk,
                                softmax_scale=c["scale"])
    torch.cuda.synchronize()
    got_o, got_a, got_s = bf16_dev_to_f64(o), bf16_dev_to_f64(oa), bf16_dev_to_f64(osp)
    got_w, got_mass_w = bf16_dev_to_f64(ow), mass_w.cpu().numpy().astype(np.float64)
    got_lse, got_mass = lse.cpu().numpy().astype(np.float64), mass.cpu().numpy().astype(np.float64)

    sc = c["scale"] if c["scale"] > 0 else oracle.default_scale(d)
    for bb in range(b):
        for hh in range(h):
            tag = f"b{bb}h{hh}"
            Q = oracle.bf16_to_f64(q[bb, hh])
            K = oracle.bf16_to_f64(k[bb, hh // c["grp"]])
            V = oracle.bf16_to_f64(v[bb, hh // c["grp"]])
            ref = oracle.dense_attention(Q, K, V, sc)
            compare_outputs(got_o[bb, hh], ref, f"dense O {tag}")
            compare_outputs(got_a[bb, hh], ref, f"mass-launch O {tag}")
            compare_outputs(got_w[bb, hh], ref, f"workspace mass-launch O {tag}")
            # log-sum-exp of the scaled causal scores; the kernel's row sum adds
            # bf16-rounded probabilities (relative error <= 2^-8 each, so log(l)
            # moves by at most -log(1 - 2^-8) = 3.91e-3)
            sco = (Q @ K.T) * sc
            sco[np.triu_indices(s, 1)] = -np.inf
            mx = sco.max(axis=1)
            ref_lse = mx + np.log(np.exp(sco - mx[:, None]).sum(axis=1))
            assert np.max(np.abs(got_lse[bb, hh] - ref_lse)) < 4e-3, f"lse {tag}"
            mref = np.tril(oracle.block_mass(Q, K, sc, blk))
            assert np.max(np.abs(got_mass[bb, hh] - mref)) <= mass_tolerance(1), f"mass {tag}"
            assert np.max(np.abs(got_mass_w[bb, hh] - mref)) <= mass_tolerance(1), f"workspace mass {tag}"
            base = (bb * h + hh) * nb
            sups = {qb: sorted({x for x in rows[base + qb] if 0 <= x <= qb}) for qb in range(nb)}
            refs = oracle.masked_attention(Q, K, V, sups, blk, sc)
            compare_outputs(got_s[bb, hh], refs, f"sparse O {tag}")
