"""Sparse-BitLinear forward path on AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libsbl.so`` (C ABI in ``include/sbl.h``).  Every
function here only marshals arguments: it checks tensor dtypes and devices,
allocates outputs with torch on the input's device, passes raw device
pointers and torch's current HIP stream, and raises ``SblError`` on a non-zero
status.  Every step of the computation runs in the HIP kernels of libsbl;
there is no CPU or PyTorch fallback, and importing a function when the
library is missing raises.

Function names match the C entry points.  Tensors are torch.Tensors on a
ROCm device:
  W float32 [rows, cols]; x bfloat16 [tokens, cols]; masks uint8 bits;
  packed uint8 [rows, cols/4]; scales float32 [rows] and bf16 bits (uint16
  stored in int16 tensors, or torch.bfloat16 tensors).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "SblError", "lib_path", "load", "nm_mask_create", "ternary_quant_pack",
    "nm_mask_quant_pack", "nm_mask_quant_pack_grouped", "act_quant_i8",
    "sparse_bitlinear_gemm", "sparse24_bytes", "sparse24_compress",
    "sparse_bitlinear_gemm_sparse24", "sparse_bitlinear_gemv",
    "sparse_bitlinear_gemv_grouped", "GemvDesc", "RefreshDesc", "refresh_descs", "gemv_descs",
    "SCALE_FROM_MASKED", "SCALE_PER_TENSOR", "SCALE_F32", "SCALE_BF16", "GEMV_MAX_TOKENS",
    "rmsnorm_act_quant_i8", "nm_mask_stats", "packed_codes_check", "sparse_bitlinear_ste_backward",
    "sparse_bitlinear_ste_workspace_bytes", "sparse_bitlinear_ste_backward_noalloc",
    "STE_SCRATCH_BYTES",
]

SCALE_FROM_MASKED = 1
SCALE_PER_TENSOR = 2
SCALE_F32 = 0
SCALE_BF16 = 1
GEMV_MAX_TOKENS = 16
GEMV_MAX_ROWS = 1 << 28
STE_SCRATCH_BYTES = 64 << 20  # library-owned workspace of the allocation-free backward

_HERE = os.path.dirname(os.path.abspath(__file__))
# SBL_SANITIZE=1 loads the build whose host code carries ASan/UBSan
# (sparse_linear_layers_amd.build); device code is the same.
_LIB = os.path.join(_HERE, "libsbl_san.so" if os.environ.get("SBL_SANITIZE") == "1" else "libsbl.so")
_lib = None


class SblError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


def lib_path() -> str:
    return _LIB


class RefreshDesc(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("mask_bits", ctypes.c_void_p),
                ("packed", ctypes.c_void_p), ("row_scale", ctypes.c_void_p),
                ("row_scale_bf16", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64)]


class GemvDesc(ctypes.Structure):
    _fields_ = [("xq", ctypes.c_void_p), ("beta", ctypes.c_void_p),
                ("packed", ctypes.c_void_p), ("row_scale", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("acc", ctypes.c_void_p), ("K", ctypes.c_int64),
                ("N", ctypes.c_int64), ("scale_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


def load() -> ctypes.CDLL:
    """Load libsbl.so (built in-tree by ``sparse_linear_layers_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        raise RuntimeError(
            f"{_LIB} is not built; run `python -m sparse_linear_layers_amd.build` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(_LIB)
    P, I64, I, U = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint
    sig = {
        "nm_mask_create": [P, I64, I64, I, I, P, P],
        "ternary_quant_pack": [P, P, I64, I64, U, P, P, P, P],
        "nm_mask_quant_pack": [P, I64, I64, I, I, U, P, P, P, P, P],
        "nm_mask_quant_pack_grouped": [P, P, I, I, I, U, P],
        "act_quant_i8": [P, I64, I64, P, P, P],
        "rmsnorm_act_quant_i8": [P, P, ctypes.c_float, I64, I64, P, P, P],
        "nm_mask_stats": [P, P, I64, I64, I, I, P, P],
        "packed_codes_check": [P, I64, I64, I, I, P, P],
        "sparse_bitlinear_ste_backward": [P, P, P, P, P, I64, I64, I64, P, P, P,
                                          ctypes.c_size_t, P],
        "sparse_bitlinear_ste_backward_noalloc": [P, P, P, P, P, I64, I64, I64, P, P, P],
        "sparse_bitlinear_gemm": [P, P, P, P, I, I64, I64, I64, P, P, P],
        "sparse24_compress": [P, I64, I64, P, P, P],
        "sparse_bitlinear_gemm_sparse24": [P, P, P, P, I, I64, I64, I64, P, P, P],
        "sparse_bitlinear_gemv": [P, P, P, P, I, I64, I64, I64, P, P, P],
        "sparse_bitlinear_gemv_grouped": [P, P, I, I64, P],
        "sbl_probe_mfma_i8": [I64, I, P, P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.sparse_bitlinear_ste_workspace_bytes.argtypes = [I64, I64, I64]
    lib.sparse_bitlinear_ste_workspace_bytes.restype = ctypes.c_size_t
    lib.sparse24_bytes.argtypes = [I64, I64]
    lib.sparse24_bytes.restype = ctypes.c_size_t
    lib.sbl_status_str.argtypes = [I]
    lib.sbl_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise SblError(fn, status, load().sbl_status_str(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, name, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must live on a ROCm device, got {t.device}")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


def _shape(t, shape, dtype, name):
    """A caller-provided tensor must match the size the kernels write or
    read exactly: the C ABI only sees its pointer."""
    _need(t, dtype, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


_BF16_BITS = (torch.bfloat16, torch.int16, torch.uint16) if hasattr(torch, "uint16") \
    else (torch.bfloat16, torch.int16)


def nm_mask_create(W: torch.Tensor, n: int, m: int, out: torch.Tensor | None = None):
    _need(W, torch.float32, "W", 2)
    rows, cols = W.shape
    if out is None:
        out = torch.empty(rows * cols // 8, dtype=torch.uint8, device=W.device)
    _shape(out, (rows * cols // 8,), torch.uint8, "out")
    _check("nm_mask_create", load().nm_mask_create(_ptr(W), rows, cols, n, m, _ptr(out),
                                                   _stream(W.device)))
    return out


def ternary_quant_pack(W: torch.Tensor, mask_bits: torch.Tensor | None = None,
                       flags: int = 0, want_bf16: bool = True):
    """-> (packed uint8 [rows, cols/4], scale float32 [rows], scale_bf16 int16 bits or None)."""
    _need(W, torch.float32, "W", 2)
    rows, cols = W.shape
    if mask_bits is not None:
        _shape(mask_bits, (rows * cols // 8,), torch.uint8, "mask_bits")
    dev = W.device
    packed = torch.empty((rows, cols // 4), dtype=torch.uint8, device=dev)
    scale = torch.empty(rows, dtype=torch.float32, device=dev)
    sb = torch.empty(rows, dtype=torch.int16, device=dev) if want_bf16 else None
    _check("ternary_quant_pack", load().ternary_quant_pack(
        _ptr(W), _ptr(mask_bits), rows, cols, flags, _ptr(packed), _ptr(scale), _ptr(sb),
        _stream(dev)))
    return packed, scale, sb


def nm_mask_quant_pack(W: torch.Tensor, n: int, m: int, flags: int = 0,
                       want_mask: bool = True, want_bf16: bool = True, out=None):
    """-> (mask bits or None, packed, scale, scale_bf16 or None); `out` may
    pass that tuple preallocated."""
    _need(W, torch.float32, "W", 2)
    rows, cols = W.shape
    dev = W.device
    if out is not None:
        mask, packed, scale, sb = out
        if mask is not None:
            _shape(mask, (rows * cols // 8,), torch.uint8, "mask")
        _shape(packed, (rows, cols // 4), torch.uint8, "packed")
        _shape(scale, (rows,), torch.float32, "scale")
        if sb is not None:
            _shape(sb, (rows,), _BF16_BITS, "scale_bf16")
    else:
        mask = torch.empty(rows * cols // 8, dtype=torch.uint8, device=dev) if want_mask else None
        packed = torch.empty((rows, cols // 4), dtype=torch.uint8, device=dev)
        scale = torch.empty(rows, dtype=torch.float32, device=dev)
        sb = torch.empty(rows, dtype=torch.int16, device=dev) if want_bf16 else None
    _check("nm_mask_quant_pack", load().nm_mask_quant_pack(
        _ptr(W), rows, cols, n, m, flags, _ptr(mask), _ptr(packed), _ptr(scale), _ptr(sb),
        _stream(dev)))
    return mask, packed, scale, sb


def _desc_array(descs, cls, device):
    n = len(descs)
    host = (cls * n)(*descs)
    raw = torch.frombuffer(bytearray(bytes(host)), dtype=torch.uint8)
    dev = raw.to(device)  # synchronous host->device copy
    return host, dev


def refresh_descs(jobs):
    """(host array, device tensor) descriptors for nm_mask_quant_pack_grouped
    from dicts with preallocated W, packed, scale and optional mask and
    scale_bf16 tensors."""
    ds = []
    for j in jobs:
        W = _need(j["W"], torch.float32, "W", 2)
        mask, sb = j.get("mask"), j.get("scale_bf16")
        rows, cols = W.shape
        _shape(j["packed"], (rows, cols // 4), torch.uint8, "packed")
        _shape(j["scale"], (rows,), torch.float32, "scale")
        if mask is not None:
            _shape(mask, (rows * cols // 8,), torch.uint8, "mask")
        if sb is not None:
            _shape(sb, (rows,), _BF16_BITS, "scale_bf16")
        ds.append(RefreshDesc(W.data_ptr(), mask.data_ptr() if mask is not None else None,
                              j["packed"].data_ptr(), j["scale"].data_ptr(),
                              sb.data_ptr() if sb is not None else None,
                              W.shape[0], W.shape[1]))
    return _desc_array(ds, RefreshDesc, jobs[0]["W"].device)


def nm_mask_quant_pack_grouped(host, devbuf, count: int, n: int, m: int, flags: int,
                               device) -> None:
    """One launch of mask + quantise + pack over every descriptor (see
    refresh_descs).  The device descriptors must stay alive until the stream
    passes the launch."""
    _check("nm_mask_quant_pack_grouped", load().nm_mask_quant_pack_grouped(
        ctypes.cast(host, ctypes.c_void_p), _ptr(devbuf), count, n, m, flags, _stream(device)))


def rmsnorm_act_quant_i8(x: torch.Tensor, norm_weight: torch.Tensor, eps: float = 1e-6,
                         xq: torch.Tensor | None = None, beta: torch.Tensor | None = None):
    """RMSNorm (per-channel float32 weight [cols], eps) then per-token absmax
    int8: x bfloat16 [tokens, cols] -> (xq int8 [tokens, cols], beta float32
    [tokens])."""
    _need(x, _BF16_BITS, "x", 2)
    T, K = x.shape
    _shape(norm_weight, (K,), torch.float32, "norm_weight")
    if xq is None:
        xq = torch.empty((T, K), dtype=torch.int8, device=x.device)
    if beta is None:
        beta = torch.empty(T, dtype=torch.float32, device=x.device)
    _shape(xq, (T, K), torch.int8, "xq")
    _shape(beta, (T,), torch.float32, "beta")
    _check("rmsnorm_act_quant_i8", load().rmsnorm_act_quant_i8(
        _ptr(x), _ptr(norm_weight), ctypes.c_float(eps), T, K, _ptr(xq), _ptr(beta),
        _stream(x.device)))
    return xq, beta


def nm_mask_stats(old_bits: torch.Tensor | None, new_bits: torch.Tensor, rows: int, cols: int,
                  n: int, m: int, stats: torch.Tensor | None = None) -> torch.Tensor:
    """Mask monitor counts as an int64 device tensor [2]: weights whose mask
    bit changed from old_bits (0 without it) and m-groups of new_bits not
    keeping exactly n."""
    nbytes = rows * cols // 8
    _shape(new_bits, (nbytes,), torch.uint8, "new_bits")
    if old_bits is not None:
        _shape(old_bits, (nbytes,), torch.uint8, "old_bits")
    if stats is None:
        stats = torch.empty(2, dtype=torch.int64, device=new_bits.device)
    _shape(stats, (2,), torch.int64, "stats")
    _check("nm_mask_stats", load().nm_mask_stats(
        _ptr(old_bits), _ptr(new_bits), rows, cols, n, m, _ptr(stats), _stream(new_bits.device)))
    return stats


def packed_codes_check(packed: torch.Tensor, n: int, m: int,
                       stats: torch.Tensor | None = None) -> torch.Tensor:
    """Validator of packed codes [rows, cols/4] as an int64 device tensor
    [2]: 2-bit fields equal to 11 (not a code), and m-groups of a row holding
    more than n nonzero codes."""
    _need(packed, torch.uint8, "packed", 2)
    rows, cols = packed.shape[0], packed.shape[1] * 4
    if stats is None:
        stats = torch.empty(2, dtype=torch.int64, device=packed.device)
    _shape(stats, (2,), torch.int64, "stats")
    _check("packed_codes_check", load().packed_codes_check(
        _ptr(packed), rows, cols, n, m, _ptr(stats), _stream(packed.device)))
    return stats


def sparse_bitlinear_ste_workspace_bytes(T: int, K: int, N: int) -> int:
    return int(load().sparse_bitlinear_ste_workspace_bytes(T, K, N))


def sparse_bitlinear_ste_backward(dy, xq, beta, packed, scale, want_dx: bool = True,
                                  want_dw: bool = True, workspace: torch.Tensor | None = None):
    """Straight-through backward: dy float32 [T, N], xq int8 [T, K], beta
    float32 [T], packed uint8 [N, K/4], scale float32 [N] -> (dx float32
    [T, K] or None, dw float32 [N, K] or None).  `workspace` (uint8 device
    tensor) is allocated here when not given."""
    _need(dy, torch.float32, "dy", 2)
    _need(xq, torch.int8, "xq", 2)
    _need(packed, torch.uint8, "packed", 2)
    T, N = dy.shape
    K = xq.shape[1]
    _shape(xq, (T, K), torch.int8, "xq")
    _shape(beta, (T,), torch.float32, "beta")
    _shape(packed, (N, K // 4), torch.uint8, "packed")
    _shape(scale, (N,), torch.float32, "scale")
    dev = dy.device
    dx = torch.empty((T, K), dtype=torch.float32, device=dev) if want_dx else None
    dw = torch.empty((N, K), dtype=torch.float32, device=dev) if want_dw else None
    need = sparse_bitlinear_ste_workspace_bytes(T, K, N) if want_dw else 0
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need(workspace, torch.uint8, "workspace", 1)
    _check("sparse_bitlinear_ste_backward", load().sparse_bitlinear_ste_backward(
        _ptr(dy), _ptr(xq), _ptr(beta), _ptr(packed), _ptr(scale), T, K, N, _ptr(dx), _ptr(dw),
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(dev)))
    return dx, dw


def sparse_bitlinear_ste_backward_noalloc(dy, xq, beta, packed, scale,
                                          dx: torch.Tensor | None = None,
                                          dw: torch.Tensor | None = None):
    """The straight-through backward through the allocation-free entry
    point: the library computes in its own fixed device workspace, and the
    outputs are the caller's (dx float32 [T, K], dw float32 [N, K]; at least
    one of them).  Returns (dx, dw)."""
    _need(dy, torch.float32, "dy", 2)
    _need(xq, torch.int8, "xq", 2)
    T, N = dy.shape
    K = xq.shape[1]
    _shape(xq, (T, K), torch.int8, "xq")
    _shape(beta, (T,), torch.float32, "beta")
    _shape(packed, (N, K // 4), torch.uint8, "packed")
    _shape(scale, (N,), torch.float32, "scale")
    if dx is None and dw is None:
        raise ValueError("dx, dw: pass at least one output")
    if dx is not None:
        _shape(dx, (T, K), torch.float32, "dx")
    if dw is not None:
        _shape(dw, (N, K), torch.float32, "dw")
    _check("sparse_bitlinear_ste_backward_noalloc", load().sparse_bitlinear_ste_backward_noalloc(
        _ptr(dy), _ptr(xq), _ptr(beta), _ptr(packed), _ptr(scale), T, K, N, _ptr(dx), _ptr(dw),
        _stream(dy.device)))
    return dx, dw


def probe_mfma_i8(iters: int, blocks: int, sink: torch.Tensor) -> int:
    """Launch the int8 matrix-core probe (measurement only) on the current
    stream; returns the int8 operations it performs."""
    _shape(sink, (blocks * 4,), torch.int32, "sink")
    _check("sbl_probe_mfma_i8", load().sbl_probe_mfma_i8(iters, blocks, _ptr(sink),
                                                          _stream(sink.device)))
    return blocks * 4 * 4 * iters * 65536


def act_quant_i8(x: torch.Tensor, xq: torch.Tensor | None = None,
                 beta: torch.Tensor | None = None):
    """x bfloat16 [tokens, cols] -> (xq int8 [tokens, cols], beta float32 [tokens])."""
    _need(x, _BF16_BITS, "x", 2)
    T, K = x.shape
    if xq is None:
        xq = torch.empty((T, K), dtype=torch.int8, device=x.device)
    if beta is None:
        beta = torch.empty(T, dtype=torch.float32, device=x.device)
    _shape(xq, (T, K), torch.int8, "xq")
    _shape(beta, (T,), torch.float32, "beta")
    _check("act_quant_i8", load().act_quant_i8(_ptr(x), T, K, _ptr(xq), _ptr(beta),
                                               _stream(x.device)))
    return xq, beta


def _scale_dtype(scale):
    if scale.dtype == torch.float32:
        return SCALE_F32
    if scale.dtype in _BF16_BITS:
        return SCALE_BF16
    raise TypeError(f"row scale: float32 or bf16 bits, got {scale.dtype}")


def sparse_bitlinear_gemm(xq, beta, packed, scale, want_acc: bool = False,
                          y: torch.Tensor | None = None):
    # (y may be preallocated [T, N] float32)
    """-> (y float32 [T, N], acc int32 [T, N] or None)."""
    _need(xq, torch.int8, "xq", 2)
    _need(beta, torch.float32, "beta", 1)
    _need(packed, torch.uint8, "packed", 2)
    _need(scale, None, "scale", 1)
    T, K = xq.shape
    N = packed.shape[0]
    if packed.shape[1] * 4 != K:
        raise ValueError("packed must be [N, K/4]")
    _shape(beta, (T,), torch.float32, "beta")
    _shape(scale, (N,), None, "scale")
    dev = xq.device
    if y is None:
        y = torch.empty((T, N), dtype=torch.float32, device=dev)
    _shape(y, (T, N), torch.float32, "y")
    acc = torch.empty((T, N), dtype=torch.int32, device=dev) if want_acc else None
    _check("sparse_bitlinear_gemm", load().sparse_bitlinear_gemm(
        _ptr(xq), _ptr(beta), _ptr(packed), _ptr(scale), _scale_dtype(scale), T, K, N,
        _ptr(y), _ptr(acc), _stream(dev)))
    return y, acc


def sparse24_bytes(N: int, K: int) -> int:
    return int(load().sparse24_bytes(N, K))


def sparse24_compress(packed: torch.Tensor, bad_groups: torch.Tensor | None = None,
                      out: torch.Tensor | None = None):
    """packed uint8 [N, K/4] (2:4 codes) -> private smfmac operand image
    (uint8, at least sparse24_bytes(N, K) bytes).  `bad_groups` (int32 [>= 1]
    on the same device, zeroed by the caller) counts groups of 4 codes that
    hold more than 2 nonzeros."""
    _need(packed, torch.uint8, "packed", 2)
    N, K = packed.shape[0], packed.shape[1] * 4
    if out is None:
        out = torch.empty(max(sparse24_bytes(N, K), 16), dtype=torch.uint8, device=packed.device)
    _need(out, torch.uint8, "out")
    if out.device != packed.device:
        raise ValueError(f"out: must live on {packed.device}, got {out.device}")
    if out.numel() < sparse24_bytes(N, K):
        raise ValueError("out: smaller than sparse24_bytes(N, K)")
    if bad_groups is not None:
        _need(bad_groups, torch.int32, "bad_groups")
        if bad_groups.device != packed.device:
            raise ValueError(f"bad_groups: must live on {packed.device}, got {bad_groups.device}")
        if bad_groups.numel() < 1:
            raise ValueError("bad_groups: needs at least one element")
    _check("sparse24_compress", load().sparse24_compress(
        _ptr(packed), N, K, _ptr(out), _ptr(bad_groups), _stream(packed.device)))
    return out


def sparse_bitlinear_gemm_sparse24(xq, beta, sp24, N: int, scale, want_acc: bool = False,
                                   y: torch.Tensor | None = None):
    _need(xq, torch.int8, "xq", 2)
    _need(beta, torch.float32, "beta", 1)
    _need(sp24, torch.uint8, "sparse24")
    _need(scale, None, "scale", 1)
    T, K = xq.shape
    _shape(beta, (T,), torch.float32, "beta")
    _shape(scale, (N,), None, "scale")
    if sp24.numel() < sparse24_bytes(N, K):
        raise ValueError("sparse24: image smaller than sparse24_bytes(N, K)")
    dev = xq.device
    if y is None:
        y = torch.empty((T, N), dtype=torch.float32, device=dev)
    _shape(y, (T, N), torch.float32, "y")
    acc = torch.empty((T, N), dtype=torch.int32, device=dev) if want_acc else None
    _check("sparse_bitlinear_gemm_sparse24", load().sparse_bitlinear_gemm_sparse24(
        _ptr(xq), _ptr(beta), _ptr(sp24), _ptr(scale), _scale_dtype(scale), T, K, N,
        _ptr(y), _ptr(acc), _stream(dev)))
    return y, acc


def sparse_bitlinear_gemv(xq, beta, packed, scale, y: torch.Tensor | None = None,
                          want_acc: bool = False):
    """Decode product, 1 <= T <= 16 tokens -> y float32 [T, N] (and the
    int32 accumulators [T, N] when want_acc: then a tuple (y, acc))."""
    _need(xq, torch.int8, "xq", 2)
    _need(beta, torch.float32, "beta", 1)
    _need(packed, torch.uint8, "packed", 2)
    _need(scale, None, "scale", 1)
    T, K = xq.shape
    N = packed.shape[0]
    if packed.shape[1] * 4 != K:
        raise ValueError("packed must be [N, K/4]")
    _shape(beta, (T,), torch.float32, "beta")
    _shape(scale, (N,), None, "scale")
    dev = xq.device
    if y is None:
        y = torch.empty((T, N), dtype=torch.float32, device=dev)
    _shape(y, (T, N), torch.float32, "y")
    acc = torch.empty((T, N), dtype=torch.int32, device=dev) if want_acc else None
    _check("sparse_bitlinear_gemv", load().sparse_bitlinear_gemv(
        _ptr(xq), _ptr(beta), _ptr(packed), _ptr(scale), _scale_dtype(scale), T, K, N,
        _ptr(y), _ptr(acc), _stream(dev)))
    return (y, acc) if want_acc else y


def gemv_descs(jobs):
    """Build (host array, device tensor) descriptors for
    sparse_bitlinear_gemv_grouped from dicts with xq, beta, packed, scale, y
    and an optional int32 acc [T, N]."""
    dev = jobs[0]["xq"].device
    ds = []
    if len({j["xq"].shape[0] for j in jobs}) > 1:
        raise ValueError("gemv_descs: every job of a grouped launch has the same token count")
    for j in jobs:
        xq, packed, scale = j["xq"], j["packed"], j["scale"]
        _need(xq, torch.int8, "xq", 2)
        _need(packed, torch.uint8, "packed", 2)
        T, K = xq.shape
        N = packed.shape[0]
        if packed.shape[1] * 4 != K:
            raise ValueError("packed must be [N, K/4]")
        _shape(j["beta"], (T,), torch.float32, "beta")
        _shape(scale, (N,), None, "scale")
        _shape(j["y"], (T, N), torch.float32, "y")
        acc = j.get("acc")
        if acc is not None:
            _shape(acc, (T, N), torch.int32, "acc")
        ds.append(GemvDesc(xq.data_ptr(), j["beta"].data_ptr(), packed.data_ptr(),
                           scale.data_ptr(), j["y"].data_ptr(),
                           acc.data_ptr() if acc is not None else None, xq.shape[1],
                           packed.shape[0], _scale_dtype(scale), 0))
    return _desc_array(ds, GemvDesc, dev)


def sparse_bitlinear_gemv_grouped(host, devbuf, count: int, T: int, device) -> None:
    _check("sparse_bitlinear_gemv_grouped", load().sparse_bitlinear_gemv_grouped(
        ctypes.cast(host, ctypes.c_void_p), _ptr(devbuf), count, T, _stream(device)))
