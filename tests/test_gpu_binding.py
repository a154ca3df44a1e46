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
from wise_testlib import bf16_dev_to_f64, compare_outputs, say, to_dev

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
