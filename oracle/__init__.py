"""Plain CPU oracle for the Sparse-BitLinear forward path (ctypes over numpy).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library (``sparse_linear_layers_amd``) and does
not import it.

Each function wraps the C routine of the same name in ``sbl_oracle.c``, which
cites the passage it follows.  Pins (what fixes each function against
something other than itself; the tests named are under ``tests/``):

* ``nm_mask``        brute-force subset enumeration on tiny groups with forced
                     ties; the worked 2:4 example of the guide's "Hardware
                     Mechanics of 2:4 Sparsity" figure (golden file);
                     n == m gives all ones; ``torch.topk`` on tie-free data;
                     exactly-n-per-group and min-kept >= max-dropped
                     invariants (test_oracle_mask.py).
* ``row_scale``      exact rational mean (``fractions.Fraction``) rounded to
                     float by an independent exact rounding routine; bf16 copy
                     checked against an exact rational nearest-even rounding
                     (test_oracle_quant.py).
* ``ternary_codes``  closed form sign(w) * [|w| > gamma/2], checked on
                     boundary-dense inputs (values at and one ulp around
                     gamma/2 and 3*gamma/2); exact rational rounding of
                     w/gamma away from ties (test_oracle_quant.py).
* ``pack_codes``     hand-encoded golden bytes from the model card's code
                     table; round trip; total size of the 0.5B skeleton's
                     packed state matching the card's 346 MB
                     (test_oracle_pack.py).
* ``packed_check``   pure-Python bit loops over every byte value; codes
                     packed from n:m-masked ternary weights validate clean;
                     planted 11 fields and over-full groups counted exactly;
                     a hand-decoded byte (test_oracle_pack.py).
* ``act_quant``      exact rational |x~ - x*127/beta| <= 1/2 (+ float slack);
                     argmax element maps to +-127; zero token; scaling x by
                     a power of two leaves x~ unchanged (test_oracle_act.py).
* ``gemm_acc``       numpy int64 matmul of the unpacked operands; pure Python
                     brute force on tiny shapes (test_oracle_gemm.py).
* ``rmsnorm_act_quant``  each float step re-derived exactly (exact rational
                     mean, high-precision decimal square root, exact
                     rounding) on small rows; a float64 statement of
                     RMSNorm within float rounding; power-of-two scaling
                     invariance at eps = 0; zero and constant rows
                     (test_oracle_next.py).
* ``mask_stats``     pure-Python bit-by-bit count on random masks; masks
                     from ``nm_mask`` verify clean; single flips
                     (test_oracle_next.py).
* ``tensor_scale``   exact rational mean over the tensor rounded to float;
                     one-row tensors equal ``row_scale`` (test_oracle_next.py).
* ``ste_backward``   exact rational sums on tiny shapes; numpy float64
                     matmul of the same float factors; linearity of the
                     forward (the change of sum(dy * y) for a one-step change
                     of a code or of x~, through gemm_acc) equals the
                     gradient entry (test_oracle_ste.py).
* ``dequant``        exact rational product rounded to float
                     (test_oracle_gemm.py); whole-layer cross-check against
                     a numpy statement of the guide's formulation (stable-sort
                     mask, closed-form codes, int64 product) with per-row
                     gamma and no RMSNorm (test_oracle_layer.py).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sbl_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# SBL_SANITIZE=1: built with clang, AddressSanitizer and
# UndefinedBehaviorSanitizer into liboracle_san.so (same arithmetic flags),
# for a test run with the clang ASan runtime preloaded.
_SANITIZE = os.environ.get("SBL_SANITIZE") == "1"
if _SANITIZE:
    _LIB_PATH = os.path.join(_HERE, "liboracle_san.so")
# A test that plants a mistake in a scratch copy of the oracle points here.
_LIB_OVERRIDE = os.environ.get("SBL_ORACLE_LIB")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile ``sbl_oracle.c`` into ``liboracle.so`` (plain gcc, OpenMP).

    -ffp-contract=off keeps every float operation a separately rounded IEEE
    operation (no fused multiply-add), and no fast-math flag is used.
    """
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        _SRC, "-o", _LIB_PATH + ".tmp", "-lm",
    ]
    if _SANITIZE:
        cmd[0:1] = ["/opt/rocm/llvm/bin/clang", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.oracle_nm_mask.argtypes = [P, I64, I64, I, I, P]
    lib.oracle_row_scale.argtypes = [P, P, I, I64, I64, P, P]
    lib.oracle_ternary_codes.argtypes = [P, P, P, I64, I64, P]
    lib.oracle_pack_codes.argtypes = [P, I64, I64, P]
    lib.oracle_unpack_codes.argtypes = [P, I64, I64, P]
    lib.oracle_act_quant.argtypes = [P, I64, I64, P, P]
    lib.oracle_gemm_acc.argtypes = [P, P, I64, I64, I64, P]
    lib.oracle_dequant.argtypes = [P, P, P, I64, I64, P]
    lib.oracle_rmsnorm_act_quant.argtypes = [P, P, ctypes.c_float, I64, I64, P, P, P]
    lib.oracle_mask_stats.argtypes = [P, P, I64, I64, I, I, P]
    lib.oracle_packed_check.argtypes = [P, I64, I64, I, I, P]
    lib.oracle_tensor_scale.argtypes = [P, P, I, I64, I64]
    lib.oracle_tensor_scale.restype = ctypes.c_float
    lib.oracle_ste_backward.argtypes = [P, P, P, P, P, I64, I64, I64, P, P]
    lib.oracle_bf16_rne.argtypes = [ctypes.c_float]
    lib.oracle_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = I
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def nm_mask(W: np.ndarray, n: int, m: int) -> np.ndarray:
    """Bit-packed N:M mask of fp32 W [rows, cols] -> uint8 [rows*cols/8]."""
    W = _c(W, np.float32)
    rows, cols = W.shape
    assert cols % m == 0 and 0 <= n <= m
    out = np.zeros((rows * cols + 7) // 8, dtype=np.uint8)
    _load().oracle_nm_mask(_ptr(W), rows, cols, n, m, _ptr(out))
    return out


def row_scale(W: np.ndarray, mask_bits: np.ndarray | None = None,
              from_masked: bool = False):
    """(gamma fp32 [rows], gamma bf16 bits uint16 [rows])."""
    W = _c(W, np.float32)
    rows, cols = W.shape
    if from_masked:
        assert mask_bits is not None
        mask_bits = _c(mask_bits, np.uint8)
    g = np.empty(rows, dtype=np.float32)
    gb = np.empty(rows, dtype=np.uint16)
    _load().oracle_row_scale(_ptr(W), _ptr(mask_bits) if from_masked else None,
                             1 if from_masked else 0, rows, cols, _ptr(g), _ptr(gb))
    return g, gb


def ternary_codes(W: np.ndarray, mask_bits: np.ndarray | None,
                  gamma: np.ndarray) -> np.ndarray:
    """int8 codes in {-1, 0, 1}, [rows, cols]."""
    W = _c(W, np.float32)
    rows, cols = W.shape
    gamma = _c(gamma, np.float32)
    assert gamma.shape == (rows,)
    if mask_bits is not None:
        mask_bits = _c(mask_bits, np.uint8)
    out = np.empty((rows, cols), dtype=np.int8)
    _load().oracle_ternary_codes(_ptr(W), _ptr(mask_bits), _ptr(gamma), rows, cols,
                                 _ptr(out))
    return out


def pack_codes(codes: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.int8)
    rows, cols = codes.shape
    assert cols % 4 == 0
    out = np.empty((rows, cols // 4), dtype=np.uint8)
    _load().oracle_pack_codes(_ptr(codes), rows, cols, _ptr(out))
    return out


def unpack_codes(packed: np.ndarray, cols: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    rows = packed.shape[0]
    assert packed.shape == (rows, cols // 4)
    out = np.empty((rows, cols), dtype=np.int8)
    _load().oracle_unpack_codes(_ptr(packed), rows, cols, _ptr(out))
    return out


def packed_check(packed: np.ndarray, cols: int, n: int, m: int) -> tuple[int, int]:
    """(fields equal to 11, m-groups with more than n nonzero codes)."""
    p = _c(packed, np.uint8)
    rows = p.shape[0]
    out = np.zeros(2, np.int64)
    _load().oracle_packed_check(_ptr(p), rows, cols, n, m, _ptr(out))
    return int(out[0]), int(out[1])


def act_quant(x_bf16: np.ndarray):
    """x bf16 bits uint16 [T, K] -> (x~ int8 [T, K], beta fp32 [T])."""
    x_bf16 = _c(x_bf16, np.uint16)
    T, K = x_bf16.shape
    xq = np.empty((T, K), dtype=np.int8)
    beta = np.empty(T, dtype=np.float32)
    _load().oracle_act_quant(_ptr(x_bf16), T, K, _ptr(xq), _ptr(beta))
    return xq, beta


def gemm_acc(xq: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """int32 acc [T, N] = x~ [T, K] . codes [N, K]^T."""
    xq = _c(xq, np.int8)
    codes = _c(codes, np.int8)
    T, K = xq.shape
    N, K2 = codes.shape
    assert K == K2
    out = np.empty((T, N), dtype=np.int32)
    _load().oracle_gemm_acc(_ptr(xq), _ptr(codes), T, K, N, _ptr(out))
    return out


def dequant(acc: np.ndarray, beta: np.ndarray, gamma: np.ndarray) -> np.ndarray:
    acc = _c(acc, np.int32)
    beta = _c(beta, np.float32)
    gamma = _c(gamma, np.float32)
    T, N = acc.shape
    assert beta.shape == (T,) and gamma.shape == (N,)
    y = np.empty((T, N), dtype=np.float32)
    _load().oracle_dequant(_ptr(acc), _ptr(beta), _ptr(gamma), T, N, _ptr(y))
    return y


def rmsnorm_act_quant(x_bf16: np.ndarray, weight: np.ndarray, eps: float,
                      want_normed: bool = False):
    """RMSNorm with per-channel weight, then per-token absmax int8:
    x bf16 bits [T, K], weight fp32 [K] -> (x~ int8 [T, K], beta fp32 [T],
    normalised fp32 [T, K] or None)."""
    x_bf16 = _c(x_bf16, np.uint16)
    T, K = x_bf16.shape
    weight = _c(weight, np.float32)
    assert weight.shape == (K,)
    xq = np.empty((T, K), dtype=np.int8)
    beta = np.empty(T, dtype=np.float32)
    normed = np.empty((T, K), dtype=np.float32) if want_normed else None
    _load().oracle_rmsnorm_act_quant(_ptr(x_bf16), _ptr(weight), ctypes.c_float(eps), T, K,
                                     _ptr(xq), _ptr(beta), _ptr(normed))
    return xq, beta, normed


def mask_stats(old_bits: np.ndarray | None, new_bits: np.ndarray, rows: int, cols: int,
               n: int, m: int) -> tuple[int, int]:
    """(weights whose mask state changed, M-groups not keeping exactly n)."""
    new_bits = _c(new_bits, np.uint8)
    if old_bits is not None:
        old_bits = _c(old_bits, np.uint8)
    assert new_bits.size * 8 >= rows * cols and cols % m == 0
    st = np.zeros(2, dtype=np.int64)
    _load().oracle_mask_stats(_ptr(old_bits), _ptr(new_bits), rows, cols, n, m, _ptr(st))
    return int(st[0]), int(st[1])


def tensor_scale(W: np.ndarray, mask_bits: np.ndarray | None = None,
                 from_masked: bool = False) -> np.float32:
    """Per-tensor absmean scale (one float for the whole matrix)."""
    W = _c(W, np.float32)
    rows, cols = W.shape
    if from_masked:
        mask_bits = _c(mask_bits, np.uint8)
    return np.float32(_load().oracle_tensor_scale(_ptr(W), _ptr(mask_bits) if from_masked else None,
                                                  1 if from_masked else 0, rows, cols))


def ste_backward(dy: np.ndarray, xq: np.ndarray, beta: np.ndarray, codes: np.ndarray,
                 gamma: np.ndarray, want_dx: bool = True, want_dw: bool = True):
    """Straight-through backward of the layer: dy fp32 [T, N], x~ int8
    [T, K], beta fp32 [T], codes int8 [N, K], gamma fp32 [N] ->
    (dx fp32 [T, K] or None, dw fp32 [N, K] or None)."""
    dy = _c(dy, np.float32)
    xq = _c(xq, np.int8)
    beta = _c(beta, np.float32)
    codes = _c(codes, np.int8)
    gamma = _c(gamma, np.float32)
    T, N = dy.shape
    N2, K = codes.shape
    assert N2 == N and xq.shape == (T, K) and beta.shape == (T,) and gamma.shape == (N,)
    dx = np.empty((T, K), dtype=np.float32) if want_dx else None
    dw = np.empty((N, K), dtype=np.float32) if want_dw else None
    _load().oracle_ste_backward(_ptr(dy), _ptr(xq), _ptr(beta), _ptr(codes), _ptr(gamma),
                                T, K, N, _ptr(dx), _ptr(dw))
    return dx, dw


def bf16_rne(f: float) -> int:
    return int(_load().oracle_bf16_rne(ctypes.c_float(f)))


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def forward_layer(W: np.ndarray, x_bf16: np.ndarray, n: int, m: int,
                  scale_bf16: bool = False, from_masked: bool = False) -> dict:
    """The whole forward path in the guide's order: mask, scale, codes, pack,
    activation quantisation, integer product, rescale."""
    mask = nm_mask(W, n, m)
    gamma, gamma_bf16 = row_scale(W, mask, from_masked)
    codes = ternary_codes(W, mask, gamma)
    packed = pack_codes(codes)
    xq, beta = act_quant(x_bf16)
    acc = gemm_acc(xq, codes)
    g_used = bf16_bits_to_float(gamma_bf16) if scale_bf16 else gamma
    y = dequant(acc, beta, g_used)
    return dict(mask=mask, gamma=gamma, gamma_bf16=gamma_bf16, codes=codes,
                packed=packed, xq=xq, beta=beta, acc=acc, y=y)
