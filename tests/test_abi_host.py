"""Host-only checks of the C ABI: the library loads, exports every function the
header declares, and rejects invalid arguments before touching the device.

No call here passes validation, so nothing is ever launched (these tests run
without a GPU)."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_wise_amd as wise

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HEADER = os.path.join(ROOT, "include", "wise.h")

FAKE = 0x10000        # 16-byte aligned, never dereferenced: every call below fails validation first


def _lib():
    if not os.path.exists(wise.library_path()):
        pytest.skip("libwise.so not built")
    return wise.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(wise_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_calls():
    names = _declared_functions()
    for n in ("wise_full_attn", "wise_full_attn_accum", "wise_select_support", "wise_select_variant",
              "wise_sparse_attn", "wise_select_max_nnz", "wise_status_string", "wise_last_error",
              "wise_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    lib = _lib()
    assert lib.wise_abi_version() == 5
    assert lib.wise_status_string(0) == b"WISE_OK"
    assert lib.wise_status_string(3) == b"WISE_ERR_CAPACITY"
    assert lib.wise_status_string(5) == b"WISE_ERR_OVERFLOW"
    assert lib.wise_status_string(99) == b"WISE_ERR_UNKNOWN"


def _desc(b=1, h=2, s=256, d=64, blk=32, scale=0.0):
    return wise.WiseDesc(b, h, s, d, blk, scale)


@pytest.mark.parametrize("nb,cap", [(8, 0), (8, 2), (64, 0), (64, 10), (1, 0)])
def test_select_max_nnz_closed_form(nb, cap):
    _lib()
    blk = 32
    per_head = sum(min(q + 1, cap + 2) if cap > 0 else q + 1 for q in range(nb))
    assert wise.wise_select_max_nnz(2, 3, nb * blk, 64, blk, cap) == 6 * per_head


@pytest.mark.parametrize("seq,blk,nb", [(250, 32, 8), (16, 32, 1), (4097, 64, 65), (300, 128, 3), (256, 64, 4)])
def test_short_last_block_counts(seq, blk, nb):
    """n_blocks = ceil(seq_len / block_size): sizes that depend on it follow."""
    _lib()
    assert wise.wise_select_max_nnz(1, 2, seq, 64, blk, 0) == 2 * nb * (nb + 1) // 2
    want = 2 * nb * nb * blk * 4 if blk >= 32 else 0
    assert wise.wise_accum_workspace_bytes(1, 2, seq, 64, blk) == want


@pytest.mark.parametrize("b,h,s", [(0, 2, 256), (1, 0, 256), (1, 2, 0)])
def test_empty_calls_are_no_ops(b, h, s):
    """batch * heads * n_blocks == 0: every call except the selection ones
    returns WISE_OK without launching anything, its pointers NULL (so no
    GPU is needed here); the sizes that depend on the shape are 0."""
    lib = _lib()
    for blk in (32, 64, 128):
        d = _desc(b=b, h=h, s=s, d=128, blk=blk)
        r = ctypes.byref(d)
        assert lib.wise_full_attn(r, None, None, None, None, None, None) == wise.WISE_OK
        assert lib.wise_full_attn_accum(r, None, None, None, None, None, None) == wise.WISE_OK
        assert lib.wise_full_attn_accum_ws(r, None, None, None, None, None, None, 0, None) == wise.WISE_OK
        assert lib.wise_sparse_attn(r, None, None, None, None, None, None, None) == wise.WISE_OK
        assert lib.wise_support_mass(r, None, None, None, None, None) == wise.WISE_OK
        assert lib.wise_support_overlap(r, None, None, None, None, None, None, None) == wise.WISE_OK
        assert lib.wise_full_attn_accum_workspace_bytes(r) == 0
        assert lib.wise_select_max_nnz(r, 0) == 0
        # the selection calls still need row_ptr (they write its one entry)
        assert lib.wise_select_support(r, None, 1, 0.9, 0, None, None, 0, None, None) == wise.WISE_ERR_INVALID_ARG
        assert lib.wise_select_support(r, None, 0, 0.9, 0, FAKE, None, 0, None, None) == wise.WISE_ERR_INVALID_ARG


def _status(fn, *args):
    return fn(*args)


def test_invalid_descriptors_rejected():
    lib = _lib()
    f = lib.wise_full_attn
    assert f(None, FAKE, FAKE, FAKE, FAKE + 4096, None, None) == wise.WISE_ERR_INVALID_ARG
    for d, want in [(_desc(b=-1), wise.WISE_ERR_INVALID_ARG), (_desc(h=-1), wise.WISE_ERR_INVALID_ARG),
                    (_desc(d=80), wise.WISE_ERR_UNSUPPORTED), (_desc(blk=48), wise.WISE_ERR_UNSUPPORTED),
                    (_desc(s=-1), wise.WISE_ERR_INVALID_ARG), (_desc(s=-32), wise.WISE_ERR_INVALID_ARG),
                    (_desc(s=131072), wise.WISE_ERR_UNSUPPORTED),
                    (_desc(scale=float("nan")), wise.WISE_ERR_INVALID_ARG)]:
        # bad desc, null o: the desc check must fire first or the pointer check; either way no launch
        st = f(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, None)
        assert st == want, (d.batch, d.heads, d.seq_len, d.head_dim, d.block_size, st)
        assert lib.wise_last_error() != b""


def test_invalid_pointers_rejected():
    lib = _lib()
    d = _desc()
    f = lib.wise_full_attn
    assert f(ctypes.byref(d), None, FAKE, FAKE, FAKE + 4096, None, None) == wise.WISE_ERR_INVALID_ARG
    assert f(ctypes.byref(d), FAKE + 2, FAKE, FAKE, FAKE + 4096, None, None) == wise.WISE_ERR_INVALID_ARG
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None) == wise.WISE_ERR_INVALID_ARG  # o aliases q
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE + 4096, FAKE + 4098, None) == wise.WISE_ERR_INVALID_ARG
    assert lib.wise_full_attn_accum(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE + 4096, None, None) \
        == wise.WISE_ERR_INVALID_ARG
    assert lib.wise_sparse_attn(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, FAKE + 4096, None) \
        == wise.WISE_ERR_INVALID_ARG
    assert lib.wise_sparse_attn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE + 4096, None) \
        == wise.WISE_ERR_INVALID_ARG


def test_select_arguments_rejected():
    lib = _lib()
    d = _desc(s=256, blk=32)
    sel = lib.wise_select_support
    need = lib.wise_select_max_nnz(ctypes.byref(d), 0)
    assert need == 2 * sum(range(1, 9))
    # eta outside (0, 1]
    for eta in (0.0, -0.5, 1.0000001, float("nan")):
        assert sel(ctypes.byref(d), FAKE, 2, eta, 0, FAKE, FAKE, need, None, None) == wise.WISE_ERR_INVALID_ARG
    assert sel(ctypes.byref(d), FAKE, 0, 0.9, 0, FAKE, FAKE, need, None, None) == wise.WISE_ERR_INVALID_ARG
    assert sel(ctypes.byref(d), FAKE, 2, 0.9, -1, FAKE, FAKE, need, None, None) == wise.WISE_ERR_INVALID_ARG
    assert sel(ctypes.byref(d), None, 2, 0.9, 0, FAKE, FAKE, need, None, None) == wise.WISE_ERR_INVALID_ARG
    assert sel(ctypes.byref(d), FAKE + 2, 2, 0.9, 0, FAKE, FAKE, need, None, None) == wise.WISE_ERR_INVALID_ARG
    # capacity below the worst case is refused before any launch
    assert sel(ctypes.byref(d), FAKE, 2, 0.9, 0, FAKE, FAKE, need - 1, None, None) == wise.WISE_ERR_CAPACITY
    capped = lib.wise_select_max_nnz(ctypes.byref(d), 1)
    assert capped == 2 * sum(min(q + 1, 3) for q in range(8))
    assert sel(ctypes.byref(d), FAKE, 2, 0.9, 1, FAKE, FAKE, capped - 1, None, None) == wise.WISE_ERR_CAPACITY
    assert lib.wise_select_max_nnz(None, 0) == -1
    assert lib.wise_select_max_nnz(ctypes.byref(d), -3) == -1
    # the optional device nnz output must be 8-byte aligned
    assert sel(ctypes.byref(d), FAKE, 2, 0.9, 0, FAKE, FAKE, need, FAKE + 4, None) == wise.WISE_ERR_INVALID_ARG
    assert lib.wise_select_variant(ctypes.byref(d), wise.SELECT_UNION, FAKE, 2, 0.9, FAKE, FAKE, need,
                                   FAKE + 4, None) == wise.WISE_ERR_INVALID_ARG


def test_gqa_descriptor_rejected_when_heads_do_not_split():
    lib = _lib()
    for kv in (3, -1, 5):
        d = _desc(h=4)
        d.kv_heads = kv
        assert lib.wise_full_attn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None) \
            == wise.WISE_ERR_INVALID_ARG, kv
    assert lib.wise_abi_version() == 5


def test_select_variant_arguments_rejected():
    lib = _lib()
    d = _desc(s=256, blk=32)
    sel = lib.wise_select_variant
    need = lib.wise_select_max_nnz(ctypes.byref(d), 0)
    ok_args = dict(union=(wise.SELECT_UNION, 4), static=(wise.SELECT_STATIC, 1),
                   mass=(wise.SELECT_MASS_MATCHED, 5), size=(wise.SELECT_SIZE_MATCHED, 2))
    for kind, n_mass in ok_args.values():
        for eta in (0.0, 1.5, float("nan")):
            assert sel(ctypes.byref(d), kind, FAKE, n_mass, eta, FAKE, FAKE, need, None, None) \
                == wise.WISE_ERR_INVALID_ARG
        assert sel(ctypes.byref(d), kind, None, n_mass, 0.9, FAKE, FAKE, need, None, None) \
            == wise.WISE_ERR_INVALID_ARG
        assert sel(ctypes.byref(d), kind, FAKE, n_mass, 0.9, FAKE, FAKE, need - 1, None, None) \
            == wise.WISE_ERR_CAPACITY
    # unknown kinds (0 is the main selection, which has its own call) and bad step counts
    for kind in (0, 5, -1):
        assert sel(ctypes.byref(d), kind, FAKE, 2, 0.9, FAKE, FAKE, need, None, None) == wise.WISE_ERR_INVALID_ARG
    assert sel(ctypes.byref(d), wise.SELECT_UNION, FAKE, 0, 0.9, FAKE, FAKE, need, None, None) \
        == wise.WISE_ERR_INVALID_ARG
    assert sel(ctypes.byref(d), wise.SELECT_STATIC, FAKE, 2, 0.9, FAKE, FAKE, need, None, None) \
        == wise.WISE_ERR_INVALID_ARG
    for kind in (wise.SELECT_MASS_MATCHED, wise.SELECT_SIZE_MATCHED):
        assert sel(ctypes.byref(d), kind, FAKE, 1, 0.9, FAKE, FAKE, need, None, None) == wise.WISE_ERR_INVALID_ARG


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    _lib()
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        wise.wise_full_attn(q, q, q, 32)


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(wise, "_lib", None)
    with pytest.raises(ImportError):
        wise.load_library(str(tmp_path / "missing.so"))


def test_m0_only_feeds_the_direct_lds_loads():
    """The attention kernels write M0 from inline assembly right before each
    buffer_load ... lds (the compiler is not told about those LDS writes).
    That is only sound while nothing else in the kernels uses M0: check the
    generated gfx950 assembly."""
    import shutil
    import subprocess
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    hipcc = "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    csrc = os.path.join(ROOT, "block_sparse_attention_wise_amd", "csrc")
    tmp = tempfile.mkdtemp()

    def asm(name):
        out = os.path.join(tmp, name + ".s")
        subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++20", "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops", "-S", "--cuda-device-only",
                        os.path.join(csrc, name + ".hip"), "-o", out],
                       check=True, capture_output=True)
        return open(out).read().splitlines()
    try:
        with ThreadPoolExecutor(3) as pool:
            listings = list(pool.map(asm, ["wise_attn_d64", "wise_attn_d96", "wise_attn_d128"]))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    n_dma = 0
    for lines in listings:
        body = [l.strip() for l in lines if l.strip() and not l.strip().startswith(";")]
        for i, l in enumerate(body):
            if re.search(r"\bm0\b", l):
                assert re.fullmatch(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)", l), l   # from a scalar register
                assert body[i + 1].startswith("buffer_load_dwordx4") and body[i + 1].endswith(" lds"), body[i + 1]
                n_dma += 1
    assert n_dma > 0


def test_accum_workspace_size_and_arguments():
    lib = _lib()
    for blk, nb in ((64, 8), (128, 4), (32, 8), (16, 16)):
        d = _desc(b=2, h=3, s=blk * nb, d=64, blk=blk)
        want = 2 * 3 * nb * nb * blk * 4 if blk >= 32 else 0
        assert lib.wise_full_attn_accum_workspace_bytes(ctypes.byref(d)) == want
        assert wise.wise_accum_workspace_bytes(2, 3, blk * nb, 64, blk) == want
    assert lib.wise_full_attn_accum_workspace_bytes(None) == -1
    d = _desc(s=512, blk=64)
    need = lib.wise_full_attn_accum_workspace_bytes(ctypes.byref(d))
    f = lib.wise_full_attn_accum_ws
    O = FAKE + 65536
    # no workspace, misaligned, too small, aliasing an argument: refused before any launch
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, O, FAKE + 4096, None, need, None) == wise.WISE_ERR_INVALID_ARG
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, O, FAKE + 4096, (FAKE << 8) + 4, need, None) \
        == wise.WISE_ERR_INVALID_ARG
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, O, FAKE + 4096, FAKE << 8, need - 1, None) == wise.WISE_ERR_CAPACITY
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, O, FAKE + 4096, O, need, None) == wise.WISE_ERR_INVALID_ARG
    # mass is still required
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, O, None, FAKE << 8, need, None) == wise.WISE_ERR_INVALID_ARG
    assert lib.wise_last_error() != b""


def test_noalloc_call_refuses_sizes_beyond_its_buffer():
    """wise_full_attn_accum_noalloc checks its fixed buffer's limit and its
    arguments on the host, before any device call."""
    lib = _lib()
    assert lib.wise_full_attn_accum_noalloc_max_bytes() == 64 << 20
    big = wise.WiseDesc(1, 65, 4096, 128, 64, 0.0)
    assert lib.wise_full_attn_accum_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE + 4096, FAKE, None) \
        == wise.WISE_ERR_CAPACITY
    fits = wise.WiseDesc(1, 64, 4096, 128, 64, 0.0)
    assert lib.wise_full_attn_accum_workspace_bytes(ctypes.byref(fits)) == 64 << 20
    assert lib.wise_full_attn_accum_noalloc(ctypes.byref(fits), None, FAKE, FAKE, FAKE, FAKE, None) \
        == wise.WISE_ERR_INVALID_ARG
    assert lib.wise_full_attn_accum_noalloc(ctypes.byref(fits), FAKE, FAKE, FAKE, FAKE + 4096, None, None) \
        == wise.WISE_ERR_INVALID_ARG
    empty = wise.WiseDesc(0, 4, 4096, 128, 64, 0.0)
    assert lib.wise_full_attn_accum_noalloc(ctypes.byref(empty), None, None, None, None, None, None) \
        == wise.WISE_OK


def test_host_validation_under_sanitizers(tmp_path):
    """The C ABI's host-side validation built with the host address and
    undefined-behaviour sanitizers (device code unchanged) and run without a
    GPU: every invalid call is refused, every empty call succeeds, and the
    sanitizers report nothing."""
    import shutil
    import subprocess
    root = os.path.dirname(HERE)
    pkg = os.path.join(root, "block_sparse_attention_wise_amd")
    objs = [os.path.join(pkg, "_build", f"{n}.o") for n in
            ("wise_select", "wise_diag", "wise_attn_d64", "wise_attn_d96", "wise_attn_d128")]
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not (shutil.which(hipcc) or os.path.exists(hipcc)) or not all(os.path.exists(o) for o in objs):
        pytest.skip("needs hipcc and the library's built objects")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++20", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops"]
    capi_o = str(tmp_path / "wise_capi_san.o")
    check_o = str(tmp_path / "abi_check_san.o")
    exe = str(tmp_path / "abi_check_san")
    for src, out in ((os.path.join(pkg, "csrc", "wise_capi.hip"), capi_o),
                     (os.path.join(HERE, "abi_sanitize_check.cpp"), check_o)):
        r = subprocess.run([hipcc, *common, *san, "-c", src, "-o", out], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([hipcc, "--offload-arch=gfx950", *san, check_o, capi_o, *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-3000:])
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
