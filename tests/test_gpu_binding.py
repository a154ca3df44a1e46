"""GPU checks of the Python binding's argument handling and of the sparse
kernel's reading of malformed CSR pointers.

The error cases are rejected before any launch (by the binding or by the C
ABI's host-side validation).  The malformed-pointer case launches the sparse
kernel on a row_ptr whose values all stay within col_idx once a negative
start is read as 0, which is what the kernel does; its output is compared
with the oracle on the rows that reading implies.
"""
import numpy as np
import pytest

import oracle
from wise_inputs import round_to_bf16_bits
from wise_testlib import bf16_dev_to_f64, check_trajectory_rows, compare_outputs, say, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

wise = pytest.importorskip("block_sparse_attention_wise_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wise.load_library()


def _qkv(b=1, h=2, s=256, d=64, seed=3):
    g = np.random.default_rng(seed)
    mk = lambda: round_to_bf16_bits(g.standard_normal((b, h, s, d)).astype(np.float32))
    q, k, v = mk(), mk(), mk()
    return (q, k, v), (to_dev(q), to_dev(k), to_dev(v))


def test_binding_rejects_bad_arguments():
    say("binding argument checks")
    _, (q, k, v) = _qkv()
    with pytest.raises(ValueError):
        wise.wise_full_attn(q, k, v, 0)                       # block size 0
    with pytest.raises(ValueError):
        wise.wise_full_attn(q, k, v, -32)
    with pytest.raises(wise.WiseError) as e:
        wise.wise_full_attn(q, k, v, 48)                      # not a built block size
    assert e.value.status == wise.WISE_ERR_UNSUPPORTED
    with pytest.raises(wise.WiseError) as e:
        wise.wise_full_attn(q, k, v, 32, o=q)                 # o aliases q
    assert e.value.status == wise.WISE_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        wise.wise_full_attn(q.transpose(2, 3), k, v, 32)      # not contiguous
    with pytest.raises(TypeError):
        wise.wise_full_attn(q.float(), k, v, 32)              # wrong dtype
    with pytest.raises(ValueError):
        wise.wise_full_attn(q, k[:, :, :128].contiguous(), v, 32)   # seq mismatch
    mass = torch.zeros(1, 2, 4, 4, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        wise.wise_full_attn_accum(q, k, v, mass, 32)          # mass shape for block 64, not 32
    rp = torch.zeros(5, dtype=torch.int32, device="cuda")
    ci = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        wise.wise_sparse_attn(q, k, v, rp, ci, 32)            # row_ptr length
    with pytest.raises(wise.WiseError) as e:
        wise.wise_select_support(torch.zeros(1, 2, 8, 8, device="cuda"), 1, 1.5, 64, 32)   # eta > 1
    assert e.value.status == wise.WISE_ERR_INVALID_ARG
    torch.cuda.synchronize()


def test_sparse_malformed_row_pointers_read_in_bounds():
    """row 0 starts at -7 (read from 0), row 1 ends below its start (empty),
    and the remaining rows are ordinary; every pointer stays within col_idx."""
    b, h, s, d, blk = 1, 2, 256, 64, 32
    nb = s // blk
    say("sparse malformed row_ptr")
    (qh, kh, vh), (q, k, v) = _qkv(b, h, s, d, seed=11)
    g = np.random.default_rng(5)
    rows = [sorted(set(g.integers(0, r % nb + 1, size=3).tolist()) | {r % nb}) for r in range(b * h * nb)]
    rp = np.zeros(len(rows) + 1, dtype=np.int64)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ci = np.array([x for r in rows for x in r], dtype=np.int32)
    rp_bad = rp.copy()
    rp_bad[0] = -7                      # row 0 reads col_idx[0:rp[1]]
    rp_bad[2] = rp_bad[1] - 1           # row 1: end below start -> empty
    assert rp_bad[2] >= 0 and rp_bad.max() <= len(ci)
    sup_rows = [list(ci[max(rp_bad[r], 0):max(rp_bad[r + 1], max(rp_bad[r], 0))]) for r in range(len(rows))]
    assert sup_rows[1] == []
    o = wise.wise_sparse_attn(q, k, v, torch.from_numpy(rp_bad.astype(np.int32)).cuda(),
                              torch.from_numpy(ci).cuda(), blk)
    torch.cuda.synchronize()
    got = bf16_dev_to_f64(o)
    sc = oracle.default_scale(d)
    for hh in range(h):
        Q, K, V = (oracle.bf16_to_f64(x[0, hh]) for x in (qh, kh, vh))
        sups = {qb: sorted({int(x) for x in sup_rows[hh * nb + qb] if 0 <= x <= qb}) for qb in range(nb)}
        ref = oracle.masked_attention(Q, K, V, sups, blk, sc)
        compare_outputs(got[0, hh], ref, f"h{hh}")
    # the empty row gives zeros
    assert np.all(got[0, 0, blk:2 * blk] == 0.0)


@pytest.mark.parametrize("shape", [(0, 2, 256, 64), (1, 0, 256, 64), (1, 2, 0, 64)],
                         ids=["batch0", "heads0", "seq0"])
def test_empty_inputs_are_no_ops(shape):
    """Zero batch, heads or sequence length: every call succeeds and computes
    nothing; the selection calls write the CSR of zero rows, row_ptr = [0]."""
    b, h, s, d = shape
    blk = 64
    nb = -(-s // blk)
    say(f"empty inputs {shape}")
    q, k, v = (torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    assert wise.wise_full_attn(q, k, v, blk).shape == shape
    mass = torch.zeros(b, h, nb, nb, dtype=torch.float32, device="cuda")
    wise.wise_full_attn_accum(q, k, v, mass, blk)
    wise.wise_full_attn_accum_ws(q, k, v, mass, blk)
    rp = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    rp, ci = wise.wise_select_support(mass, 1, 0.9, d, blk, row_ptr=rp)
    rp_u = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    rp_u, ci_u = wise.wise_select_variant(wise.SELECT_UNION, torch.stack([mass, mass]).contiguous(), 0.9, d, blk,
                                          row_ptr=rp_u)
    o = wise.wise_sparse_attn(q, k, v, rp, ci, blk)
    ret = wise.wise_support_mass(mass, rp, ci, d, blk)
    inter, uni = wise.wise_support_overlap((rp, ci), (rp_u, ci_u), b, h, nb, d, blk)
    torch.cuda.synchronize()
    assert rp.cpu().tolist() == [0] and rp_u.cpu().tolist() == [0]
    assert o.shape == shape and ret.numel() == 0 and inter.numel() == 0 and uni.numel() == 0


def test_diagnostics_malformed_row_pointers_read_in_bounds():
    """The diagnostics read malformed CSR pointers as the sparse kernel does:
    a negative start as 0, an end below its start as an empty row; every
    pointer stays within col_idx once read that way."""
    b, h, s, d, blk = 1, 2, 256, 64, 32
    nb = s // blk
    say("diagnostics malformed row_ptr")
    g = np.random.default_rng(6)
    rows = [sorted(set(g.integers(0, r % nb + 1, size=3).tolist()) | {r % nb}) for r in range(b * h * nb)]
    rp = np.zeros(len(rows) + 1, dtype=np.int64)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ci = np.array([x for r in rows for x in r], dtype=np.int32)
    rp_bad = rp.copy()
    rp_bad[0] = -5                      # row 0 reads col_idx[0:rp[1]]
    rp_bad[4] = rp_bad[3] - 2           # row 3: end below start -> empty
    assert rp_bad.max() <= len(ci) and rp_bad[4] >= 0
    read = [list(ci[max(rp_bad[r], 0):max(rp_bad[r + 1], max(rp_bad[r], 0))]) for r in range(len(rows))]
    assert read[3] == [] and read[0] == rows[0]
    mass = np.tril(g.dirichlet(np.ones(nb), size=(b, h, nb))).astype(np.float32)
    rp_d, ci_d = torch.from_numpy(rp_bad.astype(np.int32)).cuda(), torch.from_numpy(ci).cuda()
    rp_ok, ci_ok = torch.from_numpy(rp.astype(np.int32)).cuda(), torch.from_numpy(ci).cuda()
    ret = wise.wise_support_mass(torch.from_numpy(mass).cuda(), rp_d, ci_d, d, blk)
    inter, uni = wise.wise_support_overlap((rp_d, ci_d), (rp_ok, ci_ok), b, h, nb, d, blk)
    torch.cuda.synchronize()
    ret, inter, uni = ret.cpu().numpy(), inter.cpu().numpy(), uni.cpu().numpy()
    for r in range(len(rows)):
        qb = r % nb
        m_row = mass.reshape(-1, nb)[r].astype(np.float64)
        want = oracle.retained_mass(m_row, read[r], qb)
        assert abs(ret[r] - want) <= 1e-6, (r, ret[r], want)
        a = {x for x in read[r] if 0 <= x <= qb}
        bset = {x for x in rows[r] if 0 <= x <= qb}
        assert (inter[r], uni[r]) == (len(a & bset), len(a | bset)), r


def test_trajectory_on_a_side_stream():
    """The discovery, selection (with the device nnz output) and reuse calls
    issued on a non-default stream, with every output and the workspace
    allocated by the binding: results equal, bit for bit, those of the same
    calls on the current stream, and the oracle's."""
    from wise_inputs import CONFIGS, Workload
    cfg = CONFIGS["tiny"].with_(block=64, seq_len=512, heads=3, index=970)
    say(f"side stream trajectory {cfg.batch}x{cfg.heads} S {cfg.seq_len} B {cfg.block}")
    steps = list(Workload(cfg).steps())
    nb = cfg.n_blocks

    def run(stream):
        mass = torch.zeros(cfg.batch, cfg.heads, nb, nb, dtype=torch.float32, device="cuda")
        nnz = torch.zeros(1, dtype=torch.int64, device="cuda")
        dev = [tuple(to_dev(x) for x in (q, k, v)) for _, q, k, v in steps]
        if stream is not None:
            stream.wait_stream(torch.cuda.current_stream())   # inputs are ready on the current stream
        outs, rp, ci = [], None, None
        for t, (q, k, v) in enumerate(dev):
            if t < cfg.td:
                outs.append(wise.wise_full_attn_accum_ws(q, k, v, mass, cfg.block, stream=stream))
            else:
                if rp is None:
                    rp, ci = wise.wise_select_support(mass, cfg.td, cfg.eta, cfg.head_dim, cfg.block, cfg.cap,
                                                      nnz=nnz, stream=stream)
                outs.append(wise.wise_sparse_attn(q, k, v, rp, ci, cfg.block, stream=stream))
        if stream is not None:
            stream.synchronize()
        torch.cuda.synchronize()
        return mass.cpu(), rp.cpu(), ci.cpu(), int(nnz.cpu()), [o.cpu() for o in outs]

    side = torch.cuda.Stream()
    assert side.cuda_stream != torch.cuda.current_stream().cuda_stream
    m0, rp0, ci0, n0, o0 = run(None)
    m1, rp1, ci1, n1, o1 = run(side)
    assert n0 == int(rp0[-1]) and n1 == int(rp1[-1])
    assert torch.equal(m0, m1) and torch.equal(rp0, rp1) and torch.equal(ci0[:n0], ci1[:n1])
    for a, b_ in zip(o0, o1):
        assert torch.equal(a.view(torch.int16), b_.view(torch.int16))
    rows = [ci1[rp1[r]:rp1[r + 1]].tolist() for r in range(len(rp1) - 1)]
    outs = [oracle.bf16_to_f64(o.view(torch.int16).numpy().view(np.uint16)) for o in o1]
    samples = [(0, h, qb) for h in range(cfg.heads) for qb in range(nb)]
    wl = Workload(cfg)
    stats = check_trajectory_rows(cfg, m1.numpy(), rows, lambda t, b, h, r: outs[t][b, h][r], samples,
                                  lambda b, h: wl.head_steps(b, h, cfg.steps))
    say(f"  {stats['rows']} rows, max-abs {stats['max_abs']:.2e}")


def test_trace_prints_one_line_per_launch():
    """WISE_TRACE=1 (read once per process, so in a child process): one
    stderr line per kernel launch naming the kernel, grid and parameters."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys, torch; sys.path.insert(0, %r)\n"
            "import block_sparse_attention_wise_amd as w\n"
            "q = torch.randn(1, 2, 256, 64, device='cuda').to(torch.bfloat16)\n"
            "m = torch.zeros(1, 2, 4, 4, device='cuda')\n"
            "w.wise_full_attn_accum(q, q, q, m, 64)\n"
            "rp, ci = w.wise_select_support(m, 1, 0.9, 64, 64)\n"
            "w.wise_sparse_attn(q, q, q, rp, ci, 64)\n"
            "torch.cuda.synchronize()\n") % root
    say("WISE_TRACE child process")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, WISE_TRACE="1"))
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("[wise] ")]
    assert len(lines) == 3, lines
    assert "mode=dense+mass" in lines[0] and "grid=" in lines[0] and "lds=" in lines[0]
    assert lines[1].startswith("[wise] select_count/scan/fill") and "rows=8" in lines[1]
    assert "mode=sparse" in lines[2] and "head_dim=64 block=64" in lines[2]
