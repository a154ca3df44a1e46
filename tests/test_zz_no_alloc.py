"""The no-allocation discovery call (wise_full_attn_accum_noalloc) against
the workspace call it mirrors (wise_full_attn_accum_ws), through the C ABI.

Two calls in a row on one GPU: first at the largest size the fixed buffer
holds (64 heads x 4096 keys x head_dim 128 at block 64: exactly its 64 MiB
of block-mass partials), then a smaller one (short last block, head_dim 96,
block 128) that finds the first call's contents in the buffer.  Each must
equal the workspace call bitwise (same kernels), and the second is also
checked against the oracle on sampled rows.  A size one head beyond the
buffer is refused before any launch.
"""
import ctypes

import numpy as np
import pytest

import oracle
from wise_inputs import round_to_bf16_bits
from wise_testlib import compare_outputs, mass_tolerance, say, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
wise = pytest.importorskip("block_sparse_attention_wise_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wise.load_library()


def _abi_call(lib, name, d, *ptrs):
    st = getattr(lib, name)(ctypes.byref(d), *ptrs, torch.cuda.current_stream().cuda_stream)
    assert st == wise.WISE_OK, (name, st, lib.wise_last_error())


def _both(b, h, s, dh, blk, q, k, v):
    """Run the no-alloc call and the workspace call on the same inputs;
    return (o, mass) of each."""
    lib = wise.load_library()
    nb = -(-s // blk)
    d = wise.WiseDesc(b, h, s, dh, blk, 0.0, 0)
    need = lib.wise_full_attn_accum_workspace_bytes(ctypes.byref(d))
    assert 0 < need <= lib.wise_full_attn_accum_noalloc_max_bytes()
    o_n = torch.empty_like(q)
    m_n = torch.zeros(b, h, nb, nb, dtype=torch.float32, device="cuda")
    _abi_call(lib, "wise_full_attn_accum_noalloc", d, q.data_ptr(), k.data_ptr(), v.data_ptr(),
              o_n.data_ptr(), m_n.data_ptr())
    o_w = torch.empty_like(q)
    m_w = torch.zeros_like(m_n)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    _abi_call(lib, "wise_full_attn_accum_ws", d, q.data_ptr(), k.data_ptr(), v.data_ptr(),
              o_w.data_ptr(), m_w.data_ptr(), ws.data_ptr(), ctypes.c_int64(need))
    torch.cuda.synchronize()
    return (o_n, m_n), (o_w, m_w)


def test_noalloc_matches_workspace_call_twice():
    lib = wise.load_library()
    # 1: the largest shape the buffer holds
    b, h, s, dh, blk = 1, 64, 4096, 128, 64
    d = wise.WiseDesc(b, h, s, dh, blk, 0.0, 0)
    assert lib.wise_full_attn_accum_workspace_bytes(ctypes.byref(d)) == lib.wise_full_attn_accum_noalloc_max_bytes()
    say(f"no-alloc call 1: {b}x{h} heads, S {s}, D {dh}, B {blk} (the full buffer)")
    g = torch.Generator(device="cuda").manual_seed(7)
    q, k, v = (torch.randn(b, h, s, dh, generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    (o_n, m_n), (o_w, m_w) = _both(b, h, s, dh, blk, q, k, v)
    assert torch.equal(o_n.view(torch.int16), o_w.view(torch.int16))
    assert torch.equal(m_n, m_w)
    assert float((m_n.sum(-1) - 1.0).abs().max()) < 1e-3
    del q, k, v, o_n, o_w

    # 2: smaller, short last block, head_dim 96, block 128; the buffer still
    # holds call 1's partials
    b, h, s, dh, blk = 2, 3, 1000, 96, 128
    nb = -(-s // blk)
    say(f"no-alloc call 2: {b}x{h} heads, S {s}, D {dh}, B {blk}")
    rng = np.random.default_rng(11)
    qh, kh, vh = (round_to_bf16_bits(rng.standard_normal((b, h, s, dh)).astype(np.float32)) for _ in range(3))
    q, k, v = to_dev(qh), to_dev(kh), to_dev(vh)
    (o_n, m_n), (o_w, m_w) = _both(b, h, s, dh, blk, q, k, v)
    assert torch.equal(o_n.view(torch.int16), o_w.view(torch.int16))
    assert torch.equal(m_n, m_w)
    got_o = oracle.bf16_to_f64(o_n.view(torch.int16).cpu().numpy().view(np.uint16))
    got_m = m_n.cpu().numpy().astype(np.float64)
    sc = oracle.default_scale(dh)
    for (bb, hh) in ((0, 0), (1, 2)):
        Q, K, V = (oracle.bf16_to_f64(x[bb, hh]) for x in (qh, kh, vh))
        compare_outputs(got_o[bb, hh], oracle.dense_attention(Q, K, V, sc), f"O b{bb}h{hh}")
        ref_m = oracle.block_mass(Q, K, sc, blk)
        assert np.abs(got_m[bb, hh] - ref_m).max() <= mass_tolerance(1), (bb, hh)
    assert m_n.shape == (b, h, nb, nb)


def test_noalloc_refuses_more_than_the_buffer():
    lib = wise.load_library()
    d = wise.WiseDesc(1, 65, 4096, 128, 64, 0.0, 0)
    x = torch.empty(16, dtype=torch.uint8, device="cuda")
    st = lib.wise_full_attn_accum_noalloc(ctypes.byref(d), x.data_ptr(), x.data_ptr(), x.data_ptr(),
                                          x.data_ptr(), x.data_ptr(), None)
    assert st == wise.WISE_ERR_CAPACITY
    assert b"fixed buffer" in lib.wise_last_error()
