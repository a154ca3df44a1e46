"""Python binding of libwise, the WISE working-set attention library (gfx950).

Thin argument marshalling over the C ABI in ``include/wise.h``: every
function here checks tensor dtypes/shapes/devices (all on one GPU), makes
that GPU current for the call, passes raw device pointers and the stream
(default: that GPU's current HIP stream), and turns a non-zero status into
``WiseError``.  All computation runs in the HIP kernels of ``libwise.so``;
there is no fallback path.  Build the library with
``python -m block_sparse_attention_wise_amd.build``.

Layouts (see the header for the full contract):
  q, o         bf16  [batch, heads, seq_len, head_dim], contiguous, on the GPU
  k, v         bf16  [batch, kv_heads, seq_len, head_dim] (kv_heads divides heads)
  mass         fp32  [batch, heads, n_blocks, n_blocks], n_blocks = ceil(seq_len / block_size)
  row_ptr      int32 [batch * heads * n_blocks + 1]
  col_idx      int32 [>= wise_select_max_nnz(...)]
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Tuple

__all__ = ["WiseError", "WiseDesc", "load_library", "library_path", "wise_full_attn",
           "wise_full_attn_accum", "wise_full_attn_accum_ws", "wise_accum_workspace_bytes",
           "wise_full_attn_accum_noalloc", "wise_noalloc_max_bytes",
           "wise_select_support", "wise_select_variant", "wise_sparse_attn",
           "SELECT_UNION", "SELECT_STATIC", "SELECT_MASS_MATCHED", "SELECT_SIZE_MATCHED",
           "wise_support_mass", "wise_support_overlap",
           "wise_select_max_nnz", "wise_abi_version", "WISE_OK", "WISE_ERR_INVALID_ARG",
           "WISE_ERR_UNSUPPORTED", "WISE_ERR_CAPACITY", "WISE_ERR_HIP", "WISE_ERR_OVERFLOW"]

WISE_OK = 0
WISE_ERR_INVALID_ARG = 1
WISE_ERR_UNSUPPORTED = 2
WISE_ERR_CAPACITY = 3
WISE_ERR_HIP = 4
WISE_ERR_OVERFLOW = 5   # reserved by the ABI, never returned

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.environ.get("WISE_LIBRARY", os.path.join(_HERE, "libwise.so"))


class WiseError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: status {status} ({_status_name(status)}): {detail}")


class WiseDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("kv_heads", ctypes.c_int32)]


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libwise.so once; raises if it is missing (no fallback exists)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path()
    if not os.path.exists(p):
        raise ImportError(f"libwise.so not found at {p}; build it with "
                          "`python -m block_sparse_attention_wise_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    dp = ctypes.POINTER(WiseDesc)
    sigs = {
        "wise_full_attn": ([dp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
        "wise_full_attn_accum": ([dp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
        "wise_full_attn_accum_ws": ([dp, vp, vp, vp, vp, vp, vp, i64, vp], ctypes.c_int),
        "wise_full_attn_accum_workspace_bytes": ([dp], i64),
        "wise_full_attn_accum_noalloc": ([dp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
        "wise_full_attn_accum_noalloc_max_bytes": ([], i64),
        "wise_select_support": ([dp, vp, i32, ctypes.c_double, i32, vp, vp, i64, vp, vp], ctypes.c_int),
        "wise_select_variant": ([dp, i32, vp, i32, ctypes.c_double, vp, vp, i64, vp, vp], ctypes.c_int),
        "wise_support_mass": ([dp, vp, vp, vp, vp, vp], ctypes.c_int),
        "wise_support_overlap": ([dp, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
        "wise_sparse_attn": ([dp, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
        "wise_select_max_nnz": ([dp, i32], i64),
        "wise_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "wise_last_error": ([], ctypes.c_char_p),
        "wise_abi_version": ([], i32),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _lib = lib
    return lib


def _status_name(status: int) -> str:
    return {0: "WISE_OK", 1: "WISE_ERR_INVALID_ARG", 2: "WISE_ERR_UNSUPPORTED",
            3: "WISE_ERR_CAPACITY", 4: "WISE_ERR_HIP", 5: "WISE_ERR_OVERFLOW"}.get(status, "?")


def _check(status: int, func: str) -> None:
    if status != WISE_OK:
        detail = load_library().wise_last_error().decode(errors="replace")
        raise WiseError(status, func, detail)


def _call(func: str, device, stream, *args) -> None:
    """Run one library call with ``device`` current (the library launches on
    the current device) on ``stream`` (default: that device's current
    stream), and raise on a non-zero status."""
    torch = _torch()
    lib = load_library()
    with torch.cuda.device(device):
        st = getattr(lib, func)(*args, _stream_ptr(stream))
        if st != WISE_OK:
            _check(st, func)


def _torch():
    import torch
    return torch


def _stream_ptr(stream) -> Optional[int]:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _alloc_on(stream):
    """Context for the tensors this binding allocates (outputs, workspace):
    with a caller's ``stream`` they are allocated on that stream, so torch's
    caching allocator does not hand their memory to other work before the
    kernels that use them on that stream have run."""
    if stream is None:
        return contextlib.nullcontext()
    return _torch().cuda.stream(stream)


def _need(t, name, dtype, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def _same_device(*named):
    """Every tensor on the first one's device; returns that device."""
    dev = named[0][0].device
    for t, n in named[1:]:
        if t.device != dev:
            raise ValueError(f"{n} is on {t.device}, {named[0][1]} on {dev}: all tensors must share one GPU")
    return dev


def _block(block_size) -> int:
    b = int(block_size)
    if b <= 0:
        raise ValueError(f"block_size must be positive, got {block_size}")
    return b


def _desc(q, block_size: int, softmax_scale: float, k=None) -> WiseDesc:
    b, h, s, d = q.shape
    kv = int(k.shape[1]) if k is not None else 0
    return WiseDesc(b, h, s, d, int(block_size), float(softmax_scale), kv)


def _qkv(q, k, v):
    """q [batch, heads, S, D]; k, v [batch, kv_heads, S, D] with kv_heads
    dividing heads (grouped-query attention when smaller)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, 4)
    b, h, s, d = q.shape
    kvh = k.shape[1]
    if (k.shape != v.shape or k.shape[0] != b or k.shape[2:] != q.shape[2:]
            or not ((kvh >= 1 and h % kvh == 0) or (h == 0 and kvh == 0))):
        raise ValueError(f"q/k/v shapes do not match: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")


def _out(o, q, stream=None):
    torch = _torch()
    if o is None:
        with _alloc_on(stream):
            return torch.empty_like(q)
    _need(o, "o", torch.bfloat16, 4)
    if o.shape != q.shape:
        raise ValueError("o must have q's shape")
    return o


def wise_full_attn(q, k, v, block_size: int, o=None, lse=None, softmax_scale: float = 0.0,
                   stream=None):
    """Dense causal attention (Eq. 2).  Returns o (bf16)."""
    torch = _torch()
    block_size = _block(block_size)
    _qkv(q, k, v)
    o = _out(o, q, stream)
    lse_ptr = None
    named = [(q, "q"), (k, "k"), (v, "v"), (o, "o")]
    if lse is not None:
        _need(lse, "lse", torch.float32, 3)
        if tuple(lse.shape) != tuple(q.shape[:3]):
            raise ValueError("lse must be [batch, heads, seq_len]")
        lse_ptr = lse.data_ptr()
        named.append((lse, "lse"))
    dev = _same_device(*named)
    d = _desc(q, block_size, softmax_scale, k)
    _call("wise_full_attn", dev, stream, ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(),
          o.data_ptr(), lse_ptr)
    return o


def _mass_shape(q, block_size):
    b, h, s, _ = q.shape
    nb = -(-s // block_size)          # the last block is short when s % block_size != 0
    return (b, h, nb, nb)


def wise_full_attn_accum(q, k, v, mass, block_size: int, o=None, softmax_scale: float = 0.0,
                         stream=None):
    """Discovery step: dense attention + block mass (Eq. 2, 5) added into ``mass``."""
    torch = _torch()
    block_size = _block(block_size)
    _qkv(q, k, v)
    _need(mass, "mass", torch.float32, 4)
    if tuple(mass.shape) != _mass_shape(q, block_size):
        raise ValueError(f"mass must be {_mass_shape(q, block_size)}, got {tuple(mass.shape)}")
    o = _out(o, q, stream)
    dev = _same_device((q, "q"), (k, "k"), (v, "v"), (o, "o"), (mass, "mass"))
    d = _desc(q, block_size, softmax_scale, k)
    _call("wise_full_attn_accum", dev, stream, ctypes.byref(d), q.data_ptr(), k.data_ptr(),
          v.data_ptr(), o.data_ptr(), mass.data_ptr())
    return o


def wise_accum_workspace_bytes(batch: int, heads: int, seq_len: int, head_dim: int, block_size: int) -> int:
    """Bytes of workspace wise_full_attn_accum_ws needs (0 for block 16)."""
    d = WiseDesc(batch, heads, seq_len, head_dim, _block(block_size), 0.0)
    n = load_library().wise_full_attn_accum_workspace_bytes(ctypes.byref(d))
    if n < 0:
        raise WiseError(WISE_ERR_INVALID_ARG, "wise_full_attn_accum_workspace_bytes", "invalid shape")
    return int(n)


def wise_full_attn_accum_ws(q, k, v, mass, block_size: int, o=None, workspace=None,
                            softmax_scale: float = 0.0, stream=None):
    """Discovery step as wise_full_attn_accum, with the block-mass partials
    in a device workspace (a uint8 tensor of at least
    wise_accum_workspace_bytes(...) bytes on the tensors' GPU; allocated here
    when None).  Returns o."""
    torch = _torch()
    block_size = _block(block_size)
    _qkv(q, k, v)
    _need(mass, "mass", torch.float32, 4)
    if tuple(mass.shape) != _mass_shape(q, block_size):
        raise ValueError(f"mass must be {_mass_shape(q, block_size)}, got {tuple(mass.shape)}")
    o = _out(o, q, stream)
    b, h, s, dh = q.shape
    need = wise_accum_workspace_bytes(b, h, s, dh, block_size)
    if workspace is None and need > 0:
        with _alloc_on(stream):     # freed on return: its block must stay with `stream`
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    named = [(q, "q"), (k, "k"), (v, "v"), (o, "o"), (mass, "mass")]
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1)
        named.append((workspace, "workspace"))
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    dev = _same_device(*named)
    d = _desc(q, block_size, softmax_scale, k)
    _call("wise_full_attn_accum_ws", dev, stream, ctypes.byref(d), q.data_ptr(), k.data_ptr(),
          v.data_ptr(), o.data_ptr(), mass.data_ptr(), ws_ptr, ws_bytes)
    return o


def wise_noalloc_max_bytes() -> int:
    """Size of the fixed device buffer behind wise_full_attn_accum_noalloc."""
    return int(load_library().wise_full_attn_accum_noalloc_max_bytes())


def wise_full_attn_accum_noalloc(q, k, v, mass, block_size: int, o, softmax_scale: float = 0.0, stream=None):
    """Discovery step as wise_full_attn_accum_ws, with the block-mass partials
    in the library's fixed per-GPU buffer: no device memory is allocated,
    here or in the library (``o`` must therefore be given).  Calls on one
    GPU that overlap in time race on that buffer."""
    torch = _torch()
    block_size = _block(block_size)
    _qkv(q, k, v)
    _need(mass, "mass", torch.float32, 4)
    if tuple(mass.shape) != _mass_shape(q, block_size):
        raise ValueError(f"mass must be {_mass_shape(q, block_size)}, got {tuple(mass.shape)}")
    if o is None:
        raise ValueError("o must be given: this call allocates nothing")
    o = _out(o, q)
    dev = _same_device((q, "q"), (k, "k"), (v, "v"), (o, "o"), (mass, "mass"))
    d = _desc(q, block_size, softmax_scale, k)
    _call("wise_full_attn_accum_noalloc", dev, stream, ctypes.byref(d), q.data_ptr(), k.data_ptr(),
          v.data_ptr(), o.data_ptr(), mass.data_ptr())
    return o


def wise_select_max_nnz(batch: int, heads: int, seq_len: int, head_dim: int, block_size: int,
                        max_blocks: int = 0) -> int:
    d = WiseDesc(batch, heads, seq_len, head_dim, block_size, 0.0)
    n = load_library().wise_select_max_nnz(ctypes.byref(d), int(max_blocks))
    if n < 0:
        raise WiseError(WISE_ERR_INVALID_ARG, "wise_select_max_nnz", "invalid shape")
    return int(n)


def _nnz_ptr(nnz, dev):
    if nnz is None:
        return None
    torch = _torch()
    _need(nnz, "nnz", torch.int64, 1)
    if nnz.numel() != 1 or nnz.device != dev:
        raise ValueError("nnz must be one int64 on the mass tensor's GPU")
    return nnz.data_ptr()


def wise_select_support(mass, n_steps: int, eta: float, head_dim: int, block_size: int,
                        max_blocks: int = 0, row_ptr=None, col_idx=None, nnz=None,
                        stream=None) -> Tuple[object, object]:
    """Working-set selection (Eq. 6 + sink/diagonal) -> (row_ptr, col_idx) CSR.

    ``col_idx`` is sized to the worst case; its first ``row_ptr[-1]`` entries
    are meaningful.  ``nnz`` (optional, int64 [1] on the GPU) receives that
    count on the device.
    """
    torch = _torch()
    block_size = _block(block_size)
    _need(mass, "mass", torch.float32, 4)
    b, h, nb, nb2 = mass.shape
    if nb != nb2:
        raise ValueError("mass must be [batch, heads, n_blocks, n_blocks]")
    seq = nb * block_size
    d = WiseDesc(b, h, seq, head_dim, block_size, 0.0)
    cap = wise_select_max_nnz(b, h, seq, head_dim, block_size, max_blocks)
    n_rows = b * h * nb
    with _alloc_on(stream):
        if row_ptr is None:
            row_ptr = torch.empty(n_rows + 1, dtype=torch.int32, device=mass.device)
        if col_idx is None:
            col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=mass.device)
    _need(row_ptr, "row_ptr", torch.int32, 1)
    _need(col_idx, "col_idx", torch.int32, 1)
    if row_ptr.numel() != n_rows + 1:
        raise ValueError(f"row_ptr must have {n_rows + 1} entries")
    dev = _same_device((mass, "mass"), (row_ptr, "row_ptr"), (col_idx, "col_idx"))
    _call("wise_select_support", dev, stream, ctypes.byref(d), mass.data_ptr(), int(n_steps),
          float(eta), int(max_blocks), row_ptr.data_ptr(), col_idx.data_ptr(), col_idx.numel(),
          _nnz_ptr(nnz, dev))
    return row_ptr, col_idx


SELECT_UNION, SELECT_STATIC, SELECT_MASS_MATCHED, SELECT_SIZE_MATCHED = 1, 2, 3, 4


def wise_select_variant(kind: int, step_mass, eta: float, head_dim: int, block_size: int,
                        row_ptr=None, col_idx=None, nnz=None, stream=None) -> Tuple[object, object]:
    """Selection variants (temporal union, Static, MassMatched, SizeMatched)
    over single-step masses ``step_mass`` [n_mass, batch, heads, nB, nB]
    -> (row_ptr, col_idx) CSR."""
    torch = _torch()
    block_size = _block(block_size)
    _need(step_mass, "step_mass", torch.float32, 5)
    n_mass, b, h, nb, nb2 = step_mass.shape
    if nb != nb2:
        raise ValueError("step_mass must be [n_mass, batch, heads, n_blocks, n_blocks]")
    seq = nb * block_size
    d = WiseDesc(b, h, seq, head_dim, block_size, 0.0)
    cap = wise_select_max_nnz(b, h, seq, head_dim, block_size, 0)
    n_rows = b * h * nb
    with _alloc_on(stream):
        if row_ptr is None:
            row_ptr = torch.empty(n_rows + 1, dtype=torch.int32, device=step_mass.device)
        if col_idx is None:
            col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=step_mass.device)
    _need(row_ptr, "row_ptr", torch.int32, 1)
    _need(col_idx, "col_idx", torch.int32, 1)
    if row_ptr.numel() != n_rows + 1:
        raise ValueError(f"row_ptr must have {n_rows + 1} entries")
    dev = _same_device((step_mass, "step_mass"), (row_ptr, "row_ptr"), (col_idx, "col_idx"))
    _call("wise_select_variant", dev, stream, ctypes.byref(d), int(kind), step_mass.data_ptr(), int(n_mass),
          float(eta), row_ptr.data_ptr(), col_idx.data_ptr(), col_idx.numel(), _nnz_ptr(nnz, dev))
    return row_ptr, col_idx


def wise_support_mass(mass, row_ptr, col_idx, head_dim: int, block_size: int, retained=None, stream=None):
    """Per-row mass of ``mass`` [batch, heads, nB, nB] inside the CSR support
    -> fp32 [batch * heads * nB] (retained future attention mass)."""
    torch = _torch()
    block_size = _block(block_size)
    _need(mass, "mass", torch.float32, 4)
    _need(row_ptr, "row_ptr", torch.int32, 1)
    _need(col_idx, "col_idx", torch.int32, 1)
    b, h, nb, _ = mass.shape
    n_rows = b * h * nb
    if row_ptr.numel() != n_rows + 1:
        raise ValueError(f"row_ptr must have {n_rows + 1} entries")
    if retained is None:
        with _alloc_on(stream):
            retained = torch.empty(n_rows, dtype=torch.float32, device=mass.device)
    _need(retained, "retained", torch.float32, 1)
    if retained.numel() != n_rows:
        raise ValueError(f"retained must have {n_rows} entries")
    dev = _same_device((mass, "mass"), (row_ptr, "row_ptr"), (col_idx, "col_idx"), (retained, "retained"))
    d = WiseDesc(b, h, nb * block_size, head_dim, block_size, 0.0)
    _call("wise_support_mass", dev, stream, ctypes.byref(d), mass.data_ptr(), row_ptr.data_ptr(),
          col_idx.data_ptr(), retained.data_ptr())
    return retained


def wise_support_overlap(csr_a, csr_b, batch: int, heads: int, n_blocks: int, head_dim: int,
                         block_size: int, stream=None):
    """Per-row |A & B| and |A | B| of two CSR supports -> (n_inter, n_union) int32."""
    torch = _torch()
    block_size = _block(block_size)
    (ra, ca), (rb, cb) = csr_a, csr_b
    for t, n in ((ra, "row_ptr_a"), (ca, "col_idx_a"), (rb, "row_ptr_b"), (cb, "col_idx_b")):
        _need(t, n, torch.int32, 1)
    n_rows = batch * heads * n_blocks
    if ra.numel() != n_rows + 1 or rb.numel() != n_rows + 1:
        raise ValueError(f"row_ptr arrays must have {n_rows + 1} entries")
    dev = _same_device((ra, "row_ptr_a"), (ca, "col_idx_a"), (rb, "row_ptr_b"), (cb, "col_idx_b"))
    with _alloc_on(stream):
        inter = torch.empty(n_rows, dtype=torch.int32, device=dev)
        uni = torch.empty(n_rows, dtype=torch.int32, device=dev)
    d = WiseDesc(batch, heads, n_blocks * block_size, head_dim, block_size, 0.0)
    _call("wise_support_overlap", dev, stream, ctypes.byref(d), ra.data_ptr(), ca.data_ptr(), rb.data_ptr(),
          cb.data_ptr(), inter.data_ptr(), uni.data_ptr())
    return inter, uni


def wise_sparse_attn(q, k, v, row_ptr, col_idx, block_size: int, o=None,
                     softmax_scale: float = 0.0, stream=None):
    """Reuse step: attention restricted to the CSR block support (Eq. 7-8)."""
    torch = _torch()
    block_size = _block(block_size)
    _qkv(q, k, v)
    _need(row_ptr, "row_ptr", torch.int32, 1)
    _need(col_idx, "col_idx", torch.int32, 1)
    b, h, s, _ = q.shape
    if row_ptr.numel() != b * h * -(-s // block_size) + 1:
        raise ValueError("row_ptr must have batch*heads*n_blocks + 1 entries")
    o = _out(o, q, stream)
    dev = _same_device((q, "q"), (k, "k"), (v, "v"), (o, "o"), (row_ptr, "row_ptr"), (col_idx, "col_idx"))
    d = _desc(q, block_size, softmax_scale, k)
    _call("wise_sparse_attn", dev, stream, ctypes.byref(d), q.data_ptr(), k.data_ptr(),
          v.data_ptr(), row_ptr.data_ptr(), col_idx.data_ptr(), o.data_ptr())
    return o


def wise_abi_version() -> int:
    return int(load_library().wise_abi_version())
