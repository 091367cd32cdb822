"""C ABI checks that need no GPU: the library loads, exports every function
declared in include/sbl.h, and rejects bad arguments before touching HIP.
The fake device pointers below are never dereferenced: validation returns
first."""
import ctypes
import os
import re

import pytest

import sparse_linear_layers_amd as sbl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sbl.h")

OK, ARG, SHAPE, ALIGN, UNSUP = 0, -1, -2, -3, -4
P = 0x10000          # aligned fake pointer
MIS = 0x10004        # misaligned fake pointer


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s+([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sbl.lib_path()):
        from sparse_linear_layers_amd import build
        build.build()
    return sbl.load()


def test_exports_every_declared_function(lib):
    names = _declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in (OK, ARG, SHAPE, ALIGN, UNSUP, -5, 99):
        assert lib.sbl_status_str(s)


def test_mask_validation(lib):
    f = lib.nm_mask_create
    assert f(None, 4, 64, 2, 4, P, None) == ARG
    assert f(P, -1, 64, 2, 4, P, None) == ARG
    assert f(P, 4, 60, 2, 4, P, None) == SHAPE
    assert f(P, 4, 0, 2, 4, P, None) == SHAPE
    assert f(P, 4, 65536 + 64, 2, 4, P, None) == SHAPE
    assert f(P, 4, 64, 2, 3, P, None) == UNSUP
    assert f(P, 4, 64, 5, 4, P, None) == UNSUP
    assert f(P, 4, 64, -1, 8, P, None) == UNSUP
    assert f(MIS, 4, 64, 2, 4, P, None) == ALIGN
    assert f(P, 4, 64, 2, 4, MIS, None) == ALIGN
    assert f(P, 0, 64, 2, 4, P, None) == OK  # empty: nothing launched


def test_quant_validation(lib):
    f = lib.ternary_quant_pack
    assert f(P, None, 4, 64, 0, None, P, None, None) == ARG
    assert f(P, None, 4, 64, 1, P, P, None, None) == ARG       # from-masked needs a mask
    assert f(P, None, 4, 64, 4, P, P, None, None) == UNSUP     # unknown flag
    assert f(P, None, 4, 96, 0, P, P, None, None) == SHAPE
    assert f(P, None, 4, 64, 0, P, P, MIS, None) == ALIGN
    assert f(P, None, 0, 64, 0, P, P, None, None) == OK
    g = lib.nm_mask_quant_pack
    assert g(P, 4, 64, 2, 6, 0, None, P, P, None, None) == UNSUP
    assert g(P, 4, 64, 2, 4, 0, MIS, P, P, None, None) == ALIGN
    assert g(P, 0, 64, 6, 8, 1, None, P, P, None, None) == OK


def test_product_validation(lib):
    f = lib.sparse_bitlinear_gemm
    assert f(P, P, P, P, 0, 8, 64, 8, None, None, None) == ARG
    assert f(P, P, P, P, 2, 8, 64, 8, P, None, None) == UNSUP   # scale dtype
    assert f(P, P, P, P, 0, 8, 100, 8, P, None, None) == SHAPE
    assert f(P, P, P, P, 0, 8, 64, 8, P, MIS, None) == ALIGN
    assert f(P, P, P, P, 0, 0, 64, 8, P, None, None) == OK
    assert f(P, P, P, P, 0, 8, 64, 0, P, None, None) == OK
    v = lib.sparse_bitlinear_gemv
    assert v(P, P, P, P, 0, 0, 64, 8, P, None, None) == UNSUP
    assert v(P, P, P, P, 0, 17, 64, 8, P, None, None) == UNSUP
    assert v(P, P, P, P, 1, 1, 64, 0, P, None, None) == OK
    assert v(P, P, P, P, 1, 1, 64, 8, P, MIS, None) == ALIGN      # int32 accumulators
    assert v(P, P, P, P, 1, 1, 64, (1 << 28) + 1, P, None, None) == SHAPE
    s = lib.sparse_bitlinear_gemm_sparse24
    assert s(P, P, None, P, 0, 8, 64, 8, P, None, None) == ARG
    assert lib.sparse24_compress(P, 8, 64, P, MIS + 2, None) == ALIGN
    assert lib.sparse24_compress(P, 0, 64, P, None, None) == OK
    assert lib.sparse24_bytes(896, 4864) == 896 * 4864 // 4


def test_grouped_validation(lib):
    d = (sbl.GemvDesc * 2)(sbl.GemvDesc(P, P, P, P, P, None, 64, 8, 0, 0),
                           sbl.GemvDesc(P, P, P, P, P, None, 96, 8, 0, 0))
    hp = ctypes.cast(d, ctypes.c_void_p)
    assert lib.sparse_bitlinear_gemv_grouped(hp, P, 2, 1, None) == SHAPE
    assert lib.sparse_bitlinear_gemv_grouped(hp, P, 0, 1, None) == OK
    assert lib.sparse_bitlinear_gemv_grouped(hp, None, 2, 1, None) == ARG
    assert lib.sparse_bitlinear_gemv_grouped(hp, P, 1, 20, None) == UNSUP
    d[0].acc = MIS
    assert lib.sparse_bitlinear_gemv_grouped(hp, P, 1, 1, None) == ALIGN
    d[0].acc, d[0].N = None, (1 << 28) + 4
    assert lib.sparse_bitlinear_gemv_grouped(hp, P, 1, 1, None) == SHAPE
    d[0].N, d[0].reserved = 8, 1
    assert lib.sparse_bitlinear_gemv_grouped(hp, P, 1, 1, None) == ARG
    r = (sbl.RefreshDesc * 1)(sbl.RefreshDesc(P, None, P, P, MIS, 4, 64))
    assert lib.nm_mask_quant_pack_grouped(ctypes.cast(r, ctypes.c_void_p), P, 1, 3, 4, 0, None) == ALIGN
    assert lib.nm_mask_quant_pack_grouped(ctypes.cast(r, ctypes.c_void_p), P, 1, 3, 5, 0, None) == UNSUP


def test_product_path_does_not_touch_the_oracle():
    """The HIP package must not import or load anything under oracle/."""
    pkg = os.path.join(ROOT, "sparse_linear_layers_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in text and "liboracle" not in text, fn
                assert "sbl_oracle" not in text, fn


def test_rmsnorm_act_quant_validation(lib):
    f = lib.rmsnorm_act_quant_i8
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert f(P, P, 1e-6, 0, 64, P, P, None) == OK          # empty: nothing launched
    assert f(P, P, -1.0, 4, 64, P, P, None) == ARG         # negative eps
    assert f(P, P, float("nan"), 4, 64, P, P, None) == ARG
    assert f(P, P, float("inf"), 4, 64, P, P, None) == ARG
    assert f(P, None, 1e-6, 4, 64, P, P, None) == ARG      # the norm weight is required
    assert f(P, P, 1e-6, 4, 96, P, P, None) == SHAPE
    assert f(P, MIS, 1e-6, 4, 64, P, P, None) == ALIGN
    assert f(P, P, 1e-6, -2, 64, P, P, None) == ARG


def test_mask_stats_validation(lib):
    f = lib.nm_mask_stats
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert f(P, None, 4, 64, 3, 4, P, None) == ARG         # new mask required
    assert f(P, P, 4, 64, 3, 4, None, None) == ARG         # counters required
    assert f(P, P, 4, 96, 3, 4, P, None) == SHAPE
    assert f(P, P, 4, 64, 3, 6, P, None) == UNSUP
    assert f(P, P, 4, 64, 5, 4, P, None) == UNSUP
    assert f(MIS, P, 4, 64, 3, 4, P, None) == ALIGN
    assert f(P, P, 4, 64, 3, 4, P + 4, None) == ALIGN     # int64 counters: 8-byte aligned


def test_per_tensor_flag(lib):
    tq = lib.ternary_quant_pack
    assert tq(P, None, 0, 64, 2, P, P, None, None) == OK   # SBL_SCALE_PER_TENSOR accepted
    assert tq(P, None, 0, 64, 3, P, P, None, None) == OK   # with SBL_SCALE_FROM_MASKED
    assert tq(P, None, 4, 64, 3, P, P, None, None) == ARG  # from-masked needs a mask
    assert tq(P, None, 0, 64, 4, P, P, None, None) == UNSUP
    mq = lib.nm_mask_quant_pack
    assert mq(P, 0, 64, 3, 4, 2, None, P, P, None, None) == OK
    assert mq(P, 0, 64, 3, 4, 8, None, P, P, None, None) == UNSUP
    # the grouped refresh keeps per-row scales only
    g = lib.nm_mask_quant_pack_grouped
    assert g(P, P, 1, 3, 4, 2, None) == UNSUP


def test_ste_backward_validation(lib):
    f = lib.sparse_bitlinear_ste_backward
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 3 + \
        [ctypes.c_size_t, ctypes.c_void_p]
    wsb = lib.sparse_bitlinear_ste_workspace_bytes
    wsb.argtypes = [ctypes.c_int64] * 3
    wsb.restype = ctypes.c_size_t
    need = wsb(32768, 896, 896)
    assert need > 0 and wsb(0, 896, 896) == 0 and wsb(16, 128, 16) == 64   # 16 token scales
    assert f(P, P, P, P, P, 64, 128, (1 << 22) + 1, P, None, None, 0, None) == SHAPE
    # nothing requested / empty: no-op
    assert f(P, P, P, P, P, 64, 128, 64, None, None, None, 0, None) == OK
    assert f(P, P, P, P, P, 0, 128, 64, P, None, None, 0, None) == OK   # empty dx
    assert f(P, P, P, P, P, 64, 128, 0, None, P, None, 0, None) == OK   # empty dw
    assert f(None, None, None, None, None, 0, 128, 64, None, P, None, 0, None) == ARG  # gamma
    assert f(None, P, P, P, P, 64, 128, 64, P, None, None, 0, None) == ARG
    assert f(P, P, P, None, P, 64, 128, 64, P, None, None, 0, None) == ARG     # dx needs codes
    assert f(P, None, P, P, P, 64, 128, 64, None, P, P, 1 << 30, None) == ARG  # dw needs x~
    assert f(P, P, P, P, P, 32768, 896, 896, None, P, P, need - 1, None) == ARG  # small workspace
    assert f(P, P, P, P, P, 32768, 896, 896, None, P, None, need, None) == ARG
    assert f(P, P, P, P, P, 64, 100, 64, P, None, None, 0, None) == SHAPE
    assert f(MIS, P, P, P, P, 64, 128, 64, P, None, None, 0, None) == ALIGN


def test_packed_codes_check_validation(lib):
    f = lib.packed_codes_check
    assert f(None, 4, 64, 3, 4, P, None) == ARG            # codes required
    assert f(P, 4, 64, 3, 4, None, None) == ARG            # counters required
    assert f(P, -1, 64, 3, 4, P, None) == ARG
    assert f(P, 4, 96, 3, 4, P, None) == SHAPE
    assert f(P, 4, 64, 3, 5, P, None) == UNSUP
    assert f(P, 4, 64, 9, 8, P, None) == UNSUP
    assert f(MIS, 4, 64, 3, 4, P, None) == ALIGN
    assert f(P, 4, 64, 3, 4, P + 4, None) == ALIGN        # int64 counters: 8-byte aligned


def test_gemv_desc_layout_matches_header():
    """The ctypes mirror of sbl_gemv_desc has the header's field order and
    size (six pointers, two int64, two int32)."""
    text = open(HEADER).read()
    body = text[text.index("typedef struct sbl_gemv_desc"):text.index("} sbl_gemv_desc;")]
    names = re.findall(r"\b([A-Za-z_]+);", re.sub(r"/\*.*?\*/", "", body, flags=re.S))
    assert names == [n for n, _ in sbl.GemvDesc._fields_]
    assert ctypes.sizeof(sbl.GemvDesc) == 6 * 8 + 2 * 8 + 2 * 4


def test_ste_backward_noalloc_validation(lib):
    f = lib.sparse_bitlinear_ste_backward_noalloc
    wsb = lib.sparse_bitlinear_ste_workspace_bytes
    wsb.argtypes = [ctypes.c_int64] * 3
    wsb.restype = ctypes.c_size_t
    assert f(P, P, P, P, P, 64, 128, 64, None, None, None) == OK          # nothing requested
    assert f(P, P, P, P, P, 0, 128, 64, P, None, None) == OK              # empty dx
    assert f(None, P, P, P, P, 64, 128, 64, P, None, None) == ARG
    assert f(P, P, P, None, P, 64, 128, 64, P, None, None) == ARG         # dx needs codes
    assert f(P, P, P, P, P, 64, 100, 64, P, None, None) == SHAPE
    assert f(MIS, P, P, P, P, 64, 128, 64, P, None, None) == ALIGN
    # a dw whose workspace exceeds the fixed scratch is refused before any launch
    big = (1 << 25, 128, 64)                 # beta/127 alone is 128 MiB
    assert wsb(*big) > sbl.STE_SCRATCH_BYTES
    assert f(P, P, P, P, P, *big, None, P, None) == -6
    assert lib.sbl_status_str(-6)
