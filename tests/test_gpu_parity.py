"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Bit-exact for masks, packed codes, row scales (float and
bf16), int8 activations, beta and int32 accumulators; y within 1e-6
relative (three float roundings of an exact integer product are at most
~1.8e-7 apart from the exactly rounded value)."""
import numpy as np
import pytest

import oracle
from brute import unpack_bits

from sparse_linear_layers_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

Y_RTOL = 1e-6


@pytest.fixture(scope="module")
def sbl():
    import sparse_linear_layers_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load()
    return m


DEV = "cuda:0"


def dev(a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t, dtype=None):
    a = t.cpu().numpy()
    return a.view(dtype) if dtype is not None else a


def assert_y_close(got, want):
    got = got.astype(np.float64)
    want = want.astype(np.float64)
    nz = want != 0
    assert (got[~nz] == 0).all()
    rel = np.abs(got[nz] - want[nz]) / np.abs(want[nz])
    assert rel.size == 0 or rel.max() <= Y_RTOL, rel.max()


def assert_product_full(acc_d, y_d, xq, beta, codes, g, chunk=4096):
    """Every token of a product against the oracle: acc bit-exact, y within
    Y_RTOL.  Token chunks bound the host memory of the comparison."""
    T = xq.shape[0]
    assert tuple(acc_d.shape) == (T, codes.shape[0]) and tuple(y_d.shape) == (T, codes.shape[0])
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        acc_ref = oracle.gemm_acc(xq[t0:t1], codes)
        assert np.array_equal(host(acc_d[t0:t1]), acc_ref), f"acc, tokens {t0}..{t1}"
        assert_y_close(host(y_d[t0:t1]), oracle.dequant(acc_ref, beta[t0:t1], g))


def tie_heavy(tag, rows, cols):
    r = synth.rng(tag)
    alphabet = np.array([0.0, -0.0, 0.01, -0.01, 0.02, -0.02, 0.03], dtype=np.float32)
    return r.choice(alphabet, size=(rows, cols)).astype(np.float32)


# --------------------------------------------------------------------- mask
@pytest.mark.parametrize("n,m", [(3, 4), (2, 4), (1, 4), (4, 4), (0, 4), (2, 8), (4, 8), (6, 8)])
@pytest.mark.parametrize("rows,cols", [(1, 64), (37, 256), (512, 896), (33, 4864)])
def test_nm_mask(sbl, n, m, rows, cols):
    W = synth.latent_weight(f"gpu/mask/{rows}x{cols}", rows, cols)
    got = host(sbl.nm_mask_create(dev(W), n, m))
    assert np.array_equal(got, oracle.nm_mask(W, n, m))


@pytest.mark.parametrize("n,m", [(3, 4), (2, 4), (6, 8)])
def test_nm_mask_ties(sbl, n, m):
    W = tie_heavy("gpu/mask/ties", 64, 512)
    got = host(sbl.nm_mask_create(dev(W), n, m))
    assert np.array_equal(got, oracle.nm_mask(W, n, m))


# ------------------------------------------------------------ quant + pack
def _check_quant(W, mask, flags, packed, scale, sb):
    from_masked = bool(flags & 1)
    g_ref, gb_ref = oracle.row_scale(W, mask, from_masked)
    g = host(scale)
    # the decision given the device's scale is bit-exact
    codes_given = oracle.ternary_codes(W, mask, g)
    assert np.array_equal(host(packed), oracle.pack_codes(codes_given))
    # and the scale itself equals the oracle's (both are the mean rounded
    # once to float)
    assert np.array_equal(g, g_ref)
    if sb is not None:
        assert np.array_equal(host(sb, np.uint16), gb_ref)


@pytest.mark.parametrize("rows,cols", [(1, 64), (5, 256), (37, 896), (64, 4864), (9, 7168), (3, 9216)])
@pytest.mark.parametrize("mode", ["dense", "mask", "mask_from_masked"])
def test_ternary_quant_pack(sbl, rows, cols, mode):
    W = synth.latent_weight(f"gpu/quant/{rows}x{cols}", rows, cols)
    mask = None if mode == "dense" else oracle.nm_mask(W, 3, 4)
    flags = 1 if mode == "mask_from_masked" else 0
    packed, scale, sb = sbl.ternary_quant_pack(dev(W), None if mask is None else dev(mask), flags)
    _check_quant(W, mask, flags, packed, scale, sb)


@pytest.mark.parametrize("n,m", [(3, 4), (2, 4), (4, 8), (6, 8)])
@pytest.mark.parametrize("rows,cols", [(1, 64), (21, 896), (16, 4864), (4, 9216)])
@pytest.mark.parametrize("flags", [0, 1])
def test_nm_mask_quant_pack_fused(sbl, n, m, rows, cols, flags):
    W = synth.latent_weight(f"gpu/fused/{rows}x{cols}", rows, cols)
    mask_d, packed, scale, sb = sbl.nm_mask_quant_pack(dev(W), n, m, flags)
    mask = oracle.nm_mask(W, n, m)
    assert np.array_equal(host(mask_d), mask)
    _check_quant(W, mask, flags, packed, scale, sb)


@pytest.mark.parametrize("n", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("rows,cols", [(24, 896), (5, 7168)])
@pytest.mark.parametrize("flags", [0, 1])
def test_nm_mask_quant_pack_fused_every_n4(sbl, n, rows, cols, flags):
    """Every n of 4 on rows full of equal magnitudes and signed zeros, where
    the rank rule's tie-break decides: n = 3 and 2 run the kernels that keep
    their decisions as lane masks, the other n the kernel that keeps bits."""
    W = tie_heavy(f"gpu/fused_ties/{n}/{rows}x{cols}", rows, cols)
    mask_d, packed, scale, sb = sbl.nm_mask_quant_pack(dev(W), n, 4, flags)
    mask = oracle.nm_mask(W, n, 4)
    assert np.array_equal(host(mask_d), mask)
    _check_quant(W, mask, flags, packed, scale, sb)


def test_quant_edge_rows(sbl):
    W = synth.latent_weight("gpu/quant/edge", 6, 256)
    W[0] = 0.0                       # all-zero row: gamma clamps to 1e-5
    W[1] = 1e-9                      # mean below the clamp
    W[2, :] = 0.02                   # all equal: every |w| > gamma/2
    W[3] = tie_heavy("gpu/quant/edge3", 1, 256)
    W[4, ::2] = 0.0
    mask_d, packed, scale, sb = sbl.nm_mask_quant_pack(dev(W), 3, 4)
    mask = oracle.nm_mask(W, 3, 4)
    assert np.array_equal(host(mask_d), mask)
    _check_quant(W, mask, 0, packed, scale, sb)
    assert host(scale)[0] == np.float32(1e-5) and host(scale)[1] == np.float32(1e-5)


def test_quant_exact_half_boundaries(sbl):
    """Rows whose scale is known exactly: half the magnitudes v, half 3v, so
    gamma = 2v and |w| = v sits exactly on gamma/2 (rounds to 0) and 3v on
    1.5 gamma (rounds to 2, clipped to 1).  Pairs v+u, v-u (u one ulp) keep
    the mean exact and put weights one ulp either side of the boundary."""
    rows, cols = 8, 256
    v = np.float32(3 * 2.0 ** -9)
    up, dn = np.nextafter(v, np.float32(1)), np.nextafter(v, np.float32(0))
    assert np.float64(up) - v == v - np.float64(dn)
    rng = synth.rng("gpu/quant/exact-half")
    W = np.empty((rows, cols), np.float32)
    for r in range(rows):
        mags = np.concatenate([np.full(cols // 2 - 16, v), np.repeat([up, dn], 8),
                               np.full(cols // 2, np.float32(3) * v)]).astype(np.float32)
        signs = rng.choice(np.array([-1, 1], np.float32), cols)
        W[r] = rng.permutation(mags * signs)
    g_ref, _ = oracle.row_scale(W)
    assert (g_ref == np.float32(2) * v).all()
    packed, scale, sb = sbl.ternary_quant_pack(dev(W))
    _check_quant(W, None, 0, packed, scale, sb)
    codes = oracle.unpack_codes(host(packed), cols)
    assert (codes[np.abs(W) == v] == 0).all() and (codes[np.abs(W) == up] != 0).all()
    assert (codes[np.abs(W) == dn] == 0).all() and (np.abs(codes[np.abs(W) == 3 * v]) == 1).all()


def test_grouped_refresh(sbl):
    shapes = [(896, 896), (128, 896), (4864, 896), (896, 4864), (64, 256)]
    jobs, refs = [], []
    for i, (r, c) in enumerate(shapes):
        W = synth.latent_weight(f"gpu/grouped/{i}", r, c)
        Wd = dev(W)
        jobs.append(dict(W=Wd, mask=torch.empty(r * c // 8, dtype=torch.uint8, device=DEV),
                         packed=torch.empty((r, c // 4), dtype=torch.uint8, device=DEV),
                         scale=torch.empty(r, dtype=torch.float32, device=DEV),
                         scale_bf16=torch.empty(r, dtype=torch.int16, device=DEV)))
        refs.append(W)
    hostd, devd = sbl.refresh_descs(jobs)
    sbl.nm_mask_quant_pack_grouped(hostd, devd, len(jobs), 3, 4, 0, DEV)
    torch.cuda.synchronize()
    for W, j in zip(refs, jobs):
        mask = oracle.nm_mask(W, 3, 4)
        assert np.array_equal(host(j["mask"]), mask)
        _check_quant(W, mask, 0, j["packed"], j["scale"], j["scale_bf16"])



def test_grouped_refresh_wide_stack_as_benchmarked(sbl):
    """The 2048/7168 stack's refresh as the benchmark launches it: all 112
    latent matrices (16 layers x q, k, v, o, gate, up, down; 973M weights)
    in one grouped 3:4 call with fp32 row scales and no mask output; the
    packed codes and scales of a sample of matrices (each shape class, the
    first and the last) compared in full with the oracle."""
    jobs, keep = [], {}
    sample = {(0, "q"), (0, "down"), (7, "gate"), (11, "v"), (15, "up"), (15, "down")}
    for layer in range(synth.WIDE_LAYERS):
        for name, N, K in synth.WIDE_LINEARS:
            W = synth.latent_weight(f"gpu/widestack/L{layer}/{name}", N, K)
            jobs.append(dict(W=dev(W), packed=torch.empty((N, K // 4), dtype=torch.uint8, device=DEV),
                             scale=torch.empty(N, dtype=torch.float32, device=DEV)))
            if (layer, name) in sample:
                keep[len(jobs) - 1] = W
    assert sum(j["W"].numel() for j in jobs) == 973078528
    hostd, devd = sbl.refresh_descs(jobs)
    sbl.nm_mask_quant_pack_grouped(hostd, devd, len(jobs), 3, 4, 0, DEV)
    torch.cuda.synchronize()
    for i, W in keep.items():
        _check_quant(W, oracle.nm_mask(W, 3, 4), 0, jobs[i]["packed"], jobs[i]["scale"], None)


@pytest.mark.parametrize("n,m,flags", [(3, 4, 0), (6, 8, 0), (3, 4, 1), (4, 8, 1), (2, 4, 1), (1, 4, 0)])
def test_grouped_refresh_mixed_row_classes(sbl, n, m, flags):
    """One grouped call over rows of every footprint: short rows (a wave
    each), rows of 2049..32768 columns (a block each, in one launch with the
    short ones when no class exceeds 8 chunks, else per class) and rows
    longer than that (the two-pass path), n:4 and n:8 masks."""
    shapes = [(33, 9216), (3, 40960), (64, 256), (17, 2112), (100, 896), (7, 4864), (1, 64)]
    jobs, refs = [], []
    for i, (r, c) in enumerate(shapes):
        W = synth.latent_weight(f"gpu/grouped_mixed/{n}{m}/{i}", r, c)
        jobs.append(dict(W=dev(W), mask=torch.empty(r * c // 8, dtype=torch.uint8, device=DEV),
                         packed=torch.empty((r, c // 4), dtype=torch.uint8, device=DEV),
                         scale=torch.empty(r, dtype=torch.float32, device=DEV),
                         scale_bf16=torch.empty(r, dtype=torch.int16, device=DEV)))
        refs.append(W)
    hostd, devd = sbl.refresh_descs(jobs)
    sbl.nm_mask_quant_pack_grouped(hostd, devd, len(jobs), n, m, flags, DEV)
    torch.cuda.synchronize()
    for W, j in zip(refs, jobs):
        mask = oracle.nm_mask(W, n, m)
        assert np.array_equal(host(j["mask"]), mask)
        _check_quant(W, mask, flags, j["packed"], j["scale"], j["scale_bf16"])


@pytest.mark.parametrize("n,m", [(3, 4), (2, 8)])
def test_grouped_refresh_merged_launch(sbl, n, m):
    """A group whose widest rows need at most 8 chunks per thread (both
    benchmark stacks' shapes, scaled down): a single launch with whole-block
    rows first."""
    shapes = [(40, 2048), (9, 7168), (21, 896), (5, 4864), (2, 2112)]
    jobs, refs = [], []
    for i, (r, c) in enumerate(shapes):
        W = synth.latent_weight(f"gpu/grouped_merged/{n}{m}/{i}", r, c)
        jobs.append(dict(W=dev(W), packed=torch.empty((r, c // 4), dtype=torch.uint8, device=DEV),
                         scale=torch.empty(r, dtype=torch.float32, device=DEV)))
        refs.append(W)
    hostd, devd = sbl.refresh_descs(jobs)
    sbl.nm_mask_quant_pack_grouped(hostd, devd, len(jobs), n, m, 0, DEV)
    torch.cuda.synchronize()
    for W, j in zip(refs, jobs):
        _check_quant(W, oracle.nm_mask(W, n, m), 0, j["packed"], j["scale"], None)


# -------------------------------------------------------------- act quant
@pytest.mark.parametrize("T,K", [(1, 64), (3, 256), (128, 896), (77, 4864), (5, 8192), (4, 9216)])
def test_act_quant(sbl, T, K):
    x = synth.activations_bf16(f"gpu/act/{T}x{K}", T, K)
    x[0, : min(K, 8)] = 0  # a few exact zeros
    xq, beta = sbl.act_quant_i8(dev(x))
    xq_ref, b_ref = oracle.act_quant(x)
    assert np.array_equal(host(xq), xq_ref)
    assert np.array_equal(host(beta), b_ref)


def test_act_quant_edge_tokens(sbl):
    x = synth.activations_bf16("gpu/act/edge", 4, 256)
    x[0] = 0                            # zero token: beta = 1e-5
    x[1] = 0x8000                       # all -0.0
    vals = np.array([127, 0.5, 1.5, 2.5, -0.5, -2.5, 3.5, -126.5], dtype=np.float32)
    x[2, :8] = synth.float_to_bf16_bits(vals)  # beta = 127: exact .5 ties
    x[2, 8:] = 0
    x[3] = synth.float_to_bf16_bits(np.full(256, -3.0, np.float32))
    xq, beta = sbl.act_quant_i8(dev(x))
    xq_ref, b_ref = oracle.act_quant(x)
    assert np.array_equal(host(xq), xq_ref)
    assert np.array_equal(host(beta), b_ref)
    assert host(xq)[2, :8].tolist() == [127, 0, 2, 2, 0, -2, 4, -126]


# -------------------------------------------------------------- products
def _operands(tag, T, K, N, n=3, m=4):
    W = synth.latent_weight(f"{tag}/W", N, K)
    x = synth.activations_bf16(f"{tag}/x", T, K)
    mask = oracle.nm_mask(W, n, m)
    g, gb = oracle.row_scale(W)
    codes = oracle.ternary_codes(W, mask, g)
    packed = oracle.pack_codes(codes)
    xq, beta = oracle.act_quant(x)
    return dict(codes=codes, packed=packed, g=g, gb=gb, xq=xq, beta=beta)


GEMM_SHAPES = [(128, 256, 512), (300, 896, 200), (257, 448, 1152), (33, 64, 4), (1, 64, 1),
               (5, 128, 7), (130, 896, 128), (129, 4864, 260), (64, 2048, 2048)]


@pytest.mark.parametrize("T,K,N", GEMM_SHAPES)
@pytest.mark.parametrize("bf16_scale", [False, True])
def test_gemm(sbl, T, K, N, bf16_scale):
    o = _operands(f"gpu/gemm/{T}x{K}x{N}", T, K, N)
    scale = dev(o["gb"]) if bf16_scale else dev(o["g"])
    y, acc = sbl.sparse_bitlinear_gemm(dev(o["xq"]), dev(o["beta"]), dev(o["packed"]), scale,
                                       want_acc=True)
    acc_ref = oracle.gemm_acc(o["xq"], o["codes"])
    assert np.array_equal(host(acc), acc_ref)
    g_used = oracle.bf16_bits_to_float(o["gb"]) if bf16_scale else o["g"]
    assert_y_close(host(y), oracle.dequant(acc_ref, o["beta"], g_used))


def test_gemm_extreme_operands(sbl):
    """All-127 / all -128 activations against all +-1 codes: the largest
    accumulators the contract allows at this K."""
    T, K, N = 64, 4864, 64
    xq = np.full((T, K), 127, np.int8)
    xq[1::2] = -128
    codes = np.ones((N, K), np.int8)
    codes[1::2] = -1
    codes[2::4, ::3] = 0
    packed = oracle.pack_codes(codes)
    beta = np.ones(T, np.float32)
    g = np.full(N, 0.02, np.float32)
    y, acc = sbl.sparse_bitlinear_gemm(dev(xq), dev(beta), dev(packed), dev(g), want_acc=True)
    acc_ref = oracle.gemm_acc(xq, codes)
    assert np.array_equal(host(acc), acc_ref)
    assert_y_close(host(y), oracle.dequant(acc_ref, beta, g))


@pytest.mark.parametrize("T,K,N,bf16_scale", [(16400, 320, 1000, False), (16400, 192, 1002, True),
                                                (8292, 896, 4864, False), (16385, 4864, 896, True),
                                                (8192, 448, 7100, False), (100, 192, 65539, True),
                                                (300, 320, 30001, False)])
def test_gemm_large_tiles(sbl, T, K, N, bf16_scale):
    """Sizes that take the warp-specialised kernel (on 256 CUs): ragged
    token and row edges, K % 128 == 64, N % 4 != 0; acc and y compared on
    every token.  On 256 x 256 tiles the HBM-bound shapes run their last
    round as half tiles, over ragged last token rows (an empty second half)
    and over whole ones with a ragged feature edge (8192 x 7100); 16385 x
    4864 x 896 and the few-token, many-feature shapes (one 100-token row;
    128 + 128 + 44 tokens) take 256 x 128 tiles."""
    o = _operands(f"gpu/gemm_big/{T}x{K}x{N}", T, K, N)
    scale = dev(o["gb"]) if bf16_scale else dev(o["g"])
    y, acc = sbl.sparse_bitlinear_gemm(dev(o["xq"]), dev(o["beta"]), dev(o["packed"]), scale,
                                       want_acc=True)
    g_used = oracle.bf16_bits_to_float(o["gb"]) if bf16_scale else o["g"]
    assert_product_full(acc, y, o["xq"], o["beta"], o["codes"], g_used)


@pytest.mark.parametrize("T,K,N", [(16400, 320, 1000), (8193, 896, 896), (300, 896, 200)])
def test_gemm_stores_stay_in_bounds(sbl, T, K, N):
    """y (and the int32 hook) sit inside larger buffers filled with a
    sentinel: rows past T, and the columns past N of a partial feature tile,
    must never be written."""
    o = _operands(f"gpu/gemm_guard/{T}x{K}x{N}", T, K, N)
    pad = 300
    ybig = torch.full(((T + pad) * N + 64,), float("nan"), dtype=torch.float32, device=DEV)
    y = ybig[:T * N].view(T, N)
    y, _ = sbl.sparse_bitlinear_gemm(dev(o["xq"]), dev(o["beta"]), dev(o["packed"]), dev(o["g"]), y=y)
    tail = host(ybig[T * N:])
    assert np.isnan(tail).all(), "stores past the end of y"
    acc_ref = oracle.gemm_acc(o["xq"], o["codes"])
    assert_y_close(host(y), oracle.dequant(acc_ref, o["beta"], o["g"]))


@pytest.mark.parametrize("name,N,K", [("q", 896, 896), ("k", 128, 896), ("gate", 4864, 896),
                                      ("down", 896, 4864), ("wide_o", 2048, 2048),
                                      ("wide_up", 7168, 2048), ("wide_down", 2048, 7168)])
def test_full_size_layer(sbl, name, N, K):
    """Full-size prefill shapes (32768 tokens for the 0.5B skeleton, 8192 for
    the 2048/7168 stack), run end to end on the GPU; masks, codes, scales,
    x~ and beta compared in full, and acc and y on every token."""
    T = 8192 if name.startswith("wide") else 32768
    W = synth.latent_weight(f"cfg/full/{name}/W", N, K)
    x = synth.activations_bf16(f"cfg/full/{name}/x", T, K)
    mask_d, packed_d, scale_d, sb_d = sbl.nm_mask_quant_pack(dev(W), 3, 4)
    xq_d, beta_d = sbl.act_quant_i8(dev(x))
    y_d, acc_d = sbl.sparse_bitlinear_gemm(xq_d, beta_d, packed_d, scale_d, want_acc=True)
    mask = oracle.nm_mask(W, 3, 4)
    g, gb = oracle.row_scale(W)
    codes = oracle.ternary_codes(W, mask, g)
    assert np.array_equal(host(mask_d), mask)
    assert np.array_equal(host(packed_d), oracle.pack_codes(codes))
    assert np.array_equal(host(scale_d), g)
    xq, beta = oracle.act_quant(x)
    assert np.array_equal(host(xq_d), xq)
    assert np.array_equal(host(beta_d), beta)
    assert_product_full(acc_d, y_d, xq, beta, codes, g)


def test_full_size_fused_projection_step(sbl):
    """The benchmark's layer step as it launches it: the 7 latent matrices of
    the 0.5B skeleton refreshed in one grouped launch into the row ranges of
    four projection buffers (q/k/v, o, gate/up, down), the 4 activation
    inputs quantised, and 4 products at 32768 tokens.  Codes and scales of
    every linear, x~ / beta, and acc and y of every token compared against
    the oracle; the k and gate column slices equal the products launched on
    their own."""
    T = synth.QWEN05B_PREFILL_TOKENS
    dims = {name: (N, K) for name, N, K in synth.QWEN05B_LINEARS}
    groups = (("qkv", ("q", "k", "v"), "attn_in", 896), ("o", ("o",), "attn_out", 896),
              ("gate_up", ("gate", "up"), "mlp_in", 896), ("down", ("down",), "mlp_hidden", 4864))
    W = {name: synth.latent_weight(f"gpu/fused/{name}/W", N, K) for name, (N, K) in dims.items()}
    packed_f, scale_f, packed, scale = {}, {}, {}, {}
    for gname, members, _, K in groups:
        N = sum(dims[mn][0] for mn in members)
        packed_f[gname] = torch.empty((N, K // 4), dtype=torch.uint8, device=DEV)
        scale_f[gname] = torch.empty(N, dtype=torch.float32, device=DEV)
        r0 = 0
        for mn in members:
            packed[mn] = packed_f[gname][r0:r0 + dims[mn][0]]
            scale[mn] = scale_f[gname][r0:r0 + dims[mn][0]]
            r0 += dims[mn][0]
    Wd = {name: dev(w) for name, w in W.items()}
    jobs = [dict(W=Wd[name], packed=packed[name], scale=scale[name]) for name in dims]
    h, d = sbl.refresh_descs(jobs)
    sbl.nm_mask_quant_pack_grouped(h, d, len(jobs), 3, 4, 0, torch.device(DEV))
    codes = {}
    for name, w in W.items():
        g, _ = oracle.row_scale(w)
        codes[name] = oracle.ternary_codes(w, oracle.nm_mask(w, 3, 4), g)
        assert np.array_equal(host(packed[name]), oracle.pack_codes(codes[name])), name
        assert np.array_equal(host(scale[name]), g), name
    for gname, members, xn, K in groups:
        x = synth.activations_bf16(f"gpu/fused/{xn}/x", T, K)
        xq_d, beta_d = sbl.act_quant_i8(dev(x))
        xq, beta = oracle.act_quant(x)
        assert np.array_equal(host(xq_d), xq), xn
        assert np.array_equal(host(beta_d), beta), xn
        y_d, acc_d = sbl.sparse_bitlinear_gemm(xq_d, beta_d, packed_f[gname], scale_f[gname],
                                               want_acc=True)
        c = np.concatenate([codes[mn] for mn in members])
        g = host(scale_f[gname])
        assert_product_full(acc_d, y_d, xq, beta, c, g)
        for mn in members:
            if mn in ("k", "gate"):
                r0 = sum(dims[o][0] for o in members[:members.index(mn)])
                alone = sbl.sparse_bitlinear_gemm(xq_d, beta_d, packed[mn], scale[mn])[0]
                assert torch.equal(y_d[:, r0:r0 + dims[mn][0]], alone), mn
        del y_d, acc_d


# ------------------------------------------------------------------ 2:4
@pytest.mark.parametrize("T,K,N", [(128, 256, 512), (300, 896, 200), (65, 4864, 896), (7, 64, 36)])
def test_sparse24_matches_dense(sbl, T, K, N):
    o = _operands(f"gpu/sp24/{T}x{K}x{N}", T, K, N, n=2, m=4)
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    sp = sbl.sparse24_compress(dev(o["packed"]), bad)
    y, acc = sbl.sparse_bitlinear_gemm_sparse24(dev(o["xq"]), dev(o["beta"]), sp, N, dev(o["g"]),
                                                want_acc=True)
    yd, accd = sbl.sparse_bitlinear_gemm(dev(o["xq"]), dev(o["beta"]), dev(o["packed"]),
                                         dev(o["g"]), want_acc=True)
    assert int(bad.item()) == 0
    acc_ref = oracle.gemm_acc(o["xq"], o["codes"])
    assert np.array_equal(host(acc), acc_ref)
    assert np.array_equal(host(accd), acc_ref)
    assert np.array_equal(host(y), host(yd))
    assert_y_close(host(y), oracle.dequant(acc_ref, o["beta"], o["g"]))


@pytest.mark.parametrize("name,N,K", [("q", 896, 896), ("gate", 4864, 896), ("down", 896, 4864),
                                      ("qkv", 1152, 896), ("gate_up", 9728, 896)])
def test_sparse24_full_size(sbl, name, N, K):
    """The 2:4 product at the 0.5B skeleton's prefill size (32768 tokens),
    per linear and on the fused projections the benchmark times: acc and y
    of every token against the oracle, and y equal to the dense product's
    everywhere."""
    T = synth.QWEN05B_PREFILL_TOKENS
    W = synth.latent_weight(f"gpu/sp24full/{name}/W", N, K)
    x = synth.activations_bf16(f"gpu/sp24full/{name}/x", T, K)
    mask = oracle.nm_mask(W, 2, 4)
    g, _ = oracle.row_scale(W)
    codes = oracle.ternary_codes(W, mask, g)
    xq, beta = oracle.act_quant(x)
    packed = dev(oracle.pack_codes(codes))
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    sp = sbl.sparse24_compress(packed, bad)
    y, acc = sbl.sparse_bitlinear_gemm_sparse24(dev(xq), dev(beta), sp, N, dev(g), want_acc=True)
    yd = sbl.sparse_bitlinear_gemm(dev(xq), dev(beta), packed, dev(g))[0]
    assert int(bad.item()) == 0
    assert torch.equal(y, yd)
    assert_product_full(acc, y, xq, beta, codes, g)


@pytest.mark.parametrize("T,K,N,bf16_scale", [(16400, 320, 1000, False), (16400, 192, 1004, True),
                                                (8292, 896, 4864, False), (16385, 4864, 896, True),
                                                (16400, 192, 1002, False), (8192, 448, 7100, True)])
def test_sparse24_large_tiles(sbl, T, K, N, bf16_scale):
    """Sizes that take the large-tile smfmac kernel (at least one 256 x 256
    tile per CU, N % 4 == 0): ragged token and row edges, K % 128 == 64,
    bf16 row scales; N % 4 != 0 takes the small-tile kernel.  y equal to the
    dense product's everywhere (which runs its last round of tiles as half
    tiles at the HBM-bound sizes here); acc and y of every token against
    the oracle."""
    o = _operands(f"gpu/sp24_big/{T}x{K}x{N}", T, K, N, n=2, m=4)
    scale = dev(o["gb"]) if bf16_scale else dev(o["g"])
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    sp = sbl.sparse24_compress(dev(o["packed"]), bad)
    y, acc = sbl.sparse_bitlinear_gemm_sparse24(dev(o["xq"]), dev(o["beta"]), sp, N, scale,
                                                want_acc=True)
    yd = sbl.sparse_bitlinear_gemm(dev(o["xq"]), dev(o["beta"]), dev(o["packed"]), scale)[0]
    assert int(bad.item()) == 0
    assert torch.equal(y, yd)
    g_used = oracle.bf16_bits_to_float(o["gb"]) if bf16_scale else o["g"]
    assert_product_full(acc, y, o["xq"], o["beta"], o["codes"], g_used)


def test_sparse24_stores_stay_in_bounds(sbl):
    """y and the int32 hook of the large-tile smfmac kernel sit inside larger
    buffers filled with a sentinel: rows past T and the columns past N of the
    partial feature tile must never be written."""
    T, K, N = 16400, 320, 1000
    o = _operands(f"gpu/sp24_guard/{T}x{K}x{N}", T, K, N, n=2, m=4)
    pad = 300
    ybig = torch.full(((T + pad) * N + 64,), float("nan"), dtype=torch.float32, device=DEV)
    abig = torch.full(((T + pad) * N + 64,), -7, dtype=torch.int32, device=DEV)
    sp = sbl.sparse24_compress(dev(o["packed"]))
    xq, beta, g = dev(o["xq"]), dev(o["beta"]), dev(o["g"])
    y, acc = ybig[:T * N].view(T, N), abig[:T * N].view(T, N)
    st = sbl.load().sparse_bitlinear_gemm_sparse24(
        sbl._ptr(xq), sbl._ptr(beta), sbl._ptr(sp), sbl._ptr(g), sbl._scale_dtype(g), T, K, N,
        sbl._ptr(y), sbl._ptr(acc), sbl._stream(xq.device))
    assert st == 0
    torch.cuda.synchronize()
    assert np.isnan(host(ybig[T * N:])).all(), "stores past the end of y"
    assert (host(abig[T * N:]) == -7).all(), "stores past the end of acc"
    assert_product_full(acc, y, o["xq"], o["beta"], o["codes"], o["g"])


def test_sparse24_counts_groups_that_are_not_2of4(sbl):
    o = _operands("gpu/sp24/bad", 16, 256, 64, n=3, m=4)
    nz = (o["codes"].reshape(64, -1, 4) != 0).sum(-1)
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    sbl.sparse24_compress(dev(o["packed"]), bad)
    assert int(bad.item()) == int((nz > 2).sum())


# ---------------------------------------------------------------- decode
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 16])
@pytest.mark.parametrize("N,K", [(512, 256), (896, 896), (128, 896), (4864, 896), (896, 4864),
                                 (100, 192), (2048, 7168), (33, 64), (31, 576)])
@pytest.mark.parametrize("bf16_scale", [True, False])
def test_gemv(sbl, T, N, K, bf16_scale):
    """The decode product on every kernel it has: vector ALU for 1, 2 and up
    to 4 tokens, matrix cores above; acc bit-exact and y within Y_RTOL on
    every output (row counts not a multiple of the 32-row unit, K not a
    multiple of the 512-code step)."""
    o = _operands(f"gpu/gemv/{N}x{K}", T, K, N)
    scale = dev(o["gb"]) if bf16_scale else dev(o["g"])
    y, acc = sbl.sparse_bitlinear_gemv(dev(o["xq"]), dev(o["beta"]), dev(o["packed"]), scale,
                                       want_acc=True)
    acc_ref = oracle.gemm_acc(o["xq"], o["codes"])
    assert np.array_equal(host(acc), acc_ref)
    g = oracle.bf16_bits_to_float(o["gb"]) if bf16_scale else o["g"]
    assert_y_close(host(y), oracle.dequant(acc_ref, o["beta"], g))


@pytest.mark.parametrize("T", [1, 2, 4, 16])
def test_gemv_stores_stay_in_bounds(sbl, T):
    """y and acc of the decode product sit inside larger buffers filled with
    a sentinel: nothing past T x N is written (N = 1000 is not a multiple
    of the 32- or 64-row unit)."""
    N, K = 1000, 896
    o = _operands("gpu/gemv_guard", T, K, N)
    ybig = torch.full((T * N + 256,), float("nan"), dtype=torch.float32, device=DEV)
    abig = torch.full((T * N + 256,), -7, dtype=torch.int32, device=DEV)
    xq, beta, packed, g = dev(o["xq"]), dev(o["beta"]), dev(o["packed"]), dev(o["gb"])
    y, acc = ybig[:T * N].view(T, N), abig[:T * N].view(T, N)
    st = sbl.load().sparse_bitlinear_gemv(
        sbl._ptr(xq), sbl._ptr(beta), sbl._ptr(packed), sbl._ptr(g), sbl.SCALE_BF16, T, K, N,
        sbl._ptr(y), sbl._ptr(acc), sbl._stream(xq.device))
    assert st == 0
    torch.cuda.synchronize()
    assert np.isnan(host(ybig[T * N:])).all(), "stores past the end of y"
    assert (host(abig[T * N:]) == -7).all(), "stores past the end of acc"
    acc_ref = oracle.gemm_acc(o["xq"], o["codes"])
    assert np.array_equal(host(acc), acc_ref)
    assert_y_close(host(y), oracle.dequant(acc_ref, o["beta"], oracle.bf16_bits_to_float(o["gb"])))


@pytest.mark.parametrize("T", [1, 2, 4, 16])
def test_gemv_grouped(sbl, T):
    shapes = [("q", 896, 896), ("k", 128, 896), ("v", 128, 896), ("o", 896, 896),
              ("gate", 4864, 896), ("up", 4864, 896), ("down", 896, 4864), ("tiny", 36, 64)]
    jobs, refs = [], []
    for name, N, K in shapes:
        o = _operands(f"gpu/gemvg/{name}", T, K, N, n=2 if name == "o" else 3)
        jobs.append(dict(xq=dev(o["xq"]), beta=dev(o["beta"]), packed=dev(o["packed"]),
                         scale=dev(o["gb"]) if name != "v" else dev(o["g"]),
                         y=torch.full((T, N), float("nan"), device=DEV),
                         acc=torch.full((T, N), -7, dtype=torch.int32, device=DEV)
                         if name != "k" else None))
        refs.append(o)
    hostd, devd = sbl.gemv_descs(jobs)
    sbl.sparse_bitlinear_gemv_grouped(hostd, devd, len(jobs), T, DEV)
    torch.cuda.synchronize()
    for (name, N, K), j, o in zip(shapes, jobs, refs):
        g = o["g"] if name == "v" else oracle.bf16_bits_to_float(o["gb"])
        acc_ref = oracle.gemm_acc(o["xq"], o["codes"])
        if j["acc"] is not None:
            assert np.array_equal(host(j["acc"]), acc_ref), name
        assert_y_close(host(j["y"]), oracle.dequant(acc_ref, o["beta"], g))


@pytest.mark.parametrize("T,n", [(1, 3), (4, 3), (16, 3), (1, 2), (4, 2), (16, 2)])
def test_gemv_grouped_full_sweep(sbl, T, n):
    """The decode sweep as the benchmark launches it: all 168 linears of the
    0.5B skeleton (24 layers x 7) in one grouped call, bf16 row scales, one
    x~ per input width, at 3:4 and at 2:4 and at every token count the
    benchmark times; every int32 accumulator (bit-exact) and every y
    against the oracle."""
    K_in = {"q": 896, "k": 896, "v": 896, "o": 896, "gate": 896, "up": 896, "down": 4864}
    xs = {}
    for K in (896, 4864):
        x = synth.activations_bf16(f"gpu/gemvsweep/x/{K}/{T}", T, K)
        xs[K] = oracle.act_quant(x)
    xd = {K: (dev(v[0]), dev(v[1])) for K, v in xs.items()}
    jobs, refs = [], []
    for layer in range(synth.QWEN05B_LAYERS):
        for name, N, K in synth.QWEN05B_LINEARS:
            W = synth.latent_weight(f"gpu/gemvsweep/L{layer}/{name}", N, K)
            g, gb = oracle.row_scale(W)
            codes = oracle.ternary_codes(W, oracle.nm_mask(W, n, 4), g)
            jobs.append(dict(xq=xd[K][0], beta=xd[K][1], packed=dev(oracle.pack_codes(codes)),
                             scale=dev(gb), y=torch.full((T, N), float("nan"), device=DEV),
                             acc=torch.full((T, N), -7, dtype=torch.int32, device=DEV)))
            refs.append((codes, oracle.bf16_bits_to_float(gb), K))
    hostd, devd = sbl.gemv_descs(jobs)
    sbl.sparse_bitlinear_gemv_grouped(hostd, devd, len(jobs), T, DEV)
    torch.cuda.synchronize()
    for j, (codes, g, K) in zip(jobs, refs):
        xq, beta = xs[K]
        acc_ref = oracle.gemm_acc(xq, codes)
        assert np.array_equal(host(j["acc"]), acc_ref)
        assert_y_close(host(j["y"]), oracle.dequant(acc_ref, beta, g))


# ------------------------------------------------- stray 11 fields, validator
def _with_stray_fields(packed, tag, frac=0.1):
    """The packed codes with a seeded share of their zero fields (00) set to
    the non-code 11 (model card "Packed vs raw" lists 00, 01, 10 only):
    every decoder reads 11 as 0, so products and their accumulators must
    not change."""
    rng = synth.rng(tag)
    p = packed.copy()
    for r in range(4):
        f = (p >> (2 * r)) & 3
        hit = (f == 0) & (rng.random(p.shape) < frac)
        p[hit] |= np.uint8(3 << (2 * r))
    return p


@pytest.mark.parametrize("T,K,N", [(300, 896, 200), (8192, 896, 2048), (33, 64, 4)])
def test_stray_fields_read_as_zero_gemm(sbl, T, K, N):
    """Small-tile and large-tile (at least one 256 x 256 tile per CU)
    prefill kernels on codes carrying stray 11 fields."""
    o = _operands(f"gpu/stray/gemm/{T}x{K}x{N}", T, K, N)
    dirty = _with_stray_fields(o["packed"], f"gpu/stray/gemm/{T}x{K}x{N}/f")
    assert ((dirty >> 6) == 3).any() or ((dirty & 3) == 3).any()
    assert np.array_equal(oracle.unpack_codes(dirty, K), o["codes"])
    y, acc = sbl.sparse_bitlinear_gemm(dev(o["xq"]), dev(o["beta"]), dev(dirty), dev(o["g"]),
                                       want_acc=True)
    assert_product_full(acc, y, o["xq"], o["beta"], oracle.unpack_codes(dirty, K), o["g"])


@pytest.mark.parametrize("T", [1, 2, 4, 16])
def test_stray_fields_read_as_zero_gemv(sbl, T):
    N, K = 896, 4864
    o = _operands("gpu/stray/gemv", T, K, N)
    dirty = _with_stray_fields(o["packed"], "gpu/stray/gemv/f")
    y, acc = sbl.sparse_bitlinear_gemv(dev(o["xq"]), dev(o["beta"]), dev(dirty), dev(o["gb"]),
                                       want_acc=True)
    acc_ref = oracle.gemm_acc(o["xq"], oracle.unpack_codes(dirty, K))
    assert np.array_equal(host(acc), acc_ref)
    assert_y_close(host(y), oracle.dequant(acc_ref, o["beta"], oracle.bf16_bits_to_float(o["gb"])))


@pytest.mark.parametrize("T,K,N", [(300, 896, 200), (8192, 896, 2048)])
def test_stray_fields_read_as_zero_sparse24(sbl, T, K, N):
    """2:4 codes whose zero slots carry stray 11 fields: the compressor
    counts no bad group and the smfmac product equals the oracle's."""
    o = _operands(f"gpu/stray/sp24/{T}x{K}x{N}", T, K, N, n=2, m=4)
    dirty = _with_stray_fields(o["packed"], f"gpu/stray/sp24/{T}x{K}x{N}/f")
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    img = sbl.sparse24_compress(dev(dirty), bad)
    y, acc = sbl.sparse_bitlinear_gemm_sparse24(dev(o["xq"]), dev(o["beta"]), img, N, dev(o["g"]),
                                                want_acc=True)
    assert int(bad.item()) == 0
    assert_product_full(acc, y, o["xq"], o["beta"], oracle.unpack_codes(dirty, K), o["g"])


@pytest.mark.parametrize("n,m", [(3, 4), (2, 4), (1, 4), (6, 8), (4, 8), (0, 4), (8, 8)])
@pytest.mark.parametrize("rows,cols", [(1, 64), (37, 896), (300, 4864)])
def test_packed_codes_check(sbl, n, m, rows, cols):
    """The validator against the oracle on clean codes (an n:m mask) and on
    codes with stray 11 fields and over-full groups planted."""
    W = synth.latent_weight(f"gpu/pcheck/{rows}x{cols}", rows, cols)
    mask = oracle.nm_mask(W, max(n, 1) if n < m else m, m)
    g, _ = oracle.row_scale(W)
    packed = oracle.pack_codes(oracle.ternary_codes(W, mask, g))
    dirty = _with_stray_fields(packed, f"gpu/pcheck/{rows}x{cols}/f", 0.02)
    rng = synth.rng(f"gpu/pcheck/{rows}x{cols}/full")
    full = rng.random(dirty.shape) < 0.01
    dirty[full] = 0x55                      # four +1 codes: a full group of 4
    for arr in (packed, dirty):
        st = host(sbl.packed_codes_check(dev(arr), n, m))
        assert tuple(st.tolist()) == oracle.packed_check(arr, cols, n, m)


def test_packed_codes_check_of_the_full_layer(sbl):
    """The codes the grouped refresh writes for a 0.5B-skeleton layer (3:4)
    validate clean: no 11 field, no group of 4 with more than 3 nonzeros."""
    for name, N, K in synth.QWEN05B_LINEARS:
        W = dev(synth.latent_weight(f"gpu/pcheck/layer/{name}", N, K))
        _, packed, _, _ = sbl.nm_mask_quant_pack(W, 3, 4)
        assert host(sbl.packed_codes_check(packed, 3, 4)).tolist() == [0, 0], name
        assert host(sbl.packed_codes_check(packed, 2, 4))[1] > 0, name


# ------------------------------------------------------------- plumbing
def test_empty_inputs_are_noops(sbl):
    x = torch.empty((0, 64), dtype=torch.int16, device=DEV)
    xq, beta = sbl.act_quant_i8(x)
    assert xq.shape == (0, 64)
    W = torch.empty((0, 64), dtype=torch.float32, device=DEV)
    _, packed, scale, _ = sbl.nm_mask_quant_pack(W, 3, 4)
    assert packed.shape == (0, 16)
    y, _ = sbl.sparse_bitlinear_gemm(torch.empty((0, 64), dtype=torch.int8, device=DEV),
                                     torch.empty(0, device=DEV),
                                     torch.zeros((8, 16), dtype=torch.uint8, device=DEV),
                                     torch.ones(8, device=DEV))
    assert y.shape == (0, 8)


def test_errors_raise(sbl):
    W = torch.zeros((4, 96), dtype=torch.float32, device=DEV)
    with pytest.raises(sbl.SblError):
        sbl.nm_mask_create(W, 2, 4)
    x = torch.zeros((20, 64), dtype=torch.int8, device=DEV)
    with pytest.raises(sbl.SblError):
        sbl.sparse_bitlinear_gemv(x, torch.ones(20, device=DEV),
                                  torch.zeros((8, 16), dtype=torch.uint8, device=DEV),
                                  torch.ones(8, device=DEV))


def test_binding_rejects_mis_sized_buffers(sbl):
    """The C ABI sees only pointers: the binding checks every buffer it is
    handed against the sizes the kernels will touch."""
    xq = torch.zeros((20, 64), dtype=torch.int8, device=DEV)
    packed = torch.zeros((8, 16), dtype=torch.uint8, device=DEV)
    ok = dict(beta=torch.ones(20, device=DEV), scale=torch.ones(8, device=DEV))
    with pytest.raises(ValueError):
        sbl.sparse_bitlinear_gemm(xq, ok["beta"], packed, ok["scale"],
                                  y=torch.empty((20, 7), device=DEV))
    with pytest.raises(ValueError):
        sbl.sparse_bitlinear_gemm(xq, torch.ones(19, device=DEV), packed, ok["scale"])
    with pytest.raises(ValueError):
        sbl.sparse_bitlinear_gemm(xq, ok["beta"], packed, torch.ones(9, device=DEV))
    with pytest.raises(ValueError):
        sbl.act_quant_i8(torch.zeros((4, 64), dtype=torch.int16, device=DEV),
                         torch.empty((4, 63), dtype=torch.int8, device=DEV))
    p24 = torch.zeros((8, 64), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):       # image smaller than sparse24_bytes
        sbl.sparse24_compress(p24, out=torch.empty(8 * 256 // 4 - 16, dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError):       # image on the host
        sbl.sparse24_compress(p24, out=torch.empty(8 * 256 // 4, dtype=torch.uint8))
    with pytest.raises(TypeError):        # image of another dtype
        sbl.sparse24_compress(p24, out=torch.empty(8 * 256 // 16, dtype=torch.int32, device=DEV))
    with pytest.raises(TypeError):        # counter of another dtype
        sbl.sparse24_compress(p24, torch.zeros(1, dtype=torch.int64, device=DEV))
    with pytest.raises(ValueError):       # counter on the host
        sbl.sparse24_compress(p24, torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError):       # no counter element
        sbl.sparse24_compress(p24, torch.zeros(0, dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError):       # GEMV accumulators of the wrong shape
        sbl.gemv_descs([dict(xq=xq[:2].contiguous(), beta=ok["beta"][:2].contiguous(), packed=packed,
                             scale=ok["scale"], y=torch.empty((2, 8), device=DEV),
                             acc=torch.empty((2, 7), dtype=torch.int32, device=DEV))])


def test_repeat_runs_are_bitwise_identical(sbl):
    o = _operands("gpu/repeat", 1000, 896, 896)
    args = (dev(o["xq"]), dev(o["beta"]), dev(o["packed"]), dev(o["g"]))
    y1, a1 = sbl.sparse_bitlinear_gemm(*args, want_acc=True)
    y2, a2 = sbl.sparse_bitlinear_gemm(*args, want_acc=True)
    assert torch.equal(y1, y2) and torch.equal(a1, a2)


def test_repeat_runs_of_the_large_tile_kernels_are_bitwise_identical(sbl):
    """Two calls of the dense and the 2:4 large-tile products (at least one
    256 x 256 tile per CU) give the same y and int32 accumulators bit for bit."""
    T, K, N = 16384, 896, 1024
    o = _operands("gpu/repeat_big", T, K, N, n=2, m=4)
    xq, beta, packed, g = dev(o["xq"]), dev(o["beta"]), dev(o["packed"]), dev(o["g"])
    img = sbl.sparse24_compress(packed)
    runs = [(sbl.sparse_bitlinear_gemm(xq, beta, packed, g, want_acc=True),
             sbl.sparse_bitlinear_gemm_sparse24(xq, beta, img, N, g, want_acc=True)) for _ in range(2)]
    (yd1, ad1), (ys1, as1) = runs[0]
    (yd2, ad2), (ys2, as2) = runs[1]
    assert torch.equal(yd1, yd2) and torch.equal(ad1, ad2)
    assert torch.equal(ys1, ys2) and torch.equal(as1, as2)
    assert torch.equal(yd1, ys1) and torch.equal(ad1, as1)


@pytest.mark.parametrize("T,N", [(300, 260), (1, 70), (4, 70), (16, 33)])
def test_widest_rows_the_boundary_accepts(sbl, T, N):
    """K = 65536, the widest rows the boundary accepts: the fused mask +
    quantise + pack, the activation quantiser and the product (the prefill
    kernel for 300 tokens, the decode product for 1 to 16) against the
    oracle, with accumulators up to 127 * 65536 in magnitude."""
    K = 65536
    W = synth.latent_weight(f"gpu/maxk/{T}x{N}/W", N, K)
    x = synth.activations_bf16(f"gpu/maxk/{T}x{N}/x", T, K)
    mask_d, packed_d, scale_d, sb_d = sbl.nm_mask_quant_pack(dev(W), 3, 4)
    xq_d, beta_d = sbl.act_quant_i8(dev(x))
    mask = oracle.nm_mask(W, 3, 4)
    assert np.array_equal(host(mask_d), mask)
    _check_quant(W, mask, 0, packed_d, scale_d, sb_d)
    xq, beta = oracle.act_quant(x)
    assert np.array_equal(host(xq_d), xq) and np.array_equal(host(beta_d), beta)
    codes = oracle.ternary_codes(W, mask, oracle.row_scale(W)[0])
    if T > 16:
        y, acc = sbl.sparse_bitlinear_gemm(xq_d, beta_d, packed_d, scale_d, want_acc=True)
    else:
        y, acc = sbl.sparse_bitlinear_gemv(xq_d, beta_d, packed_d, scale_d, want_acc=True)
    acc_ref = oracle.gemm_acc(xq, codes)
    assert np.array_equal(host(acc), acc_ref)
    assert_y_close(host(y), oracle.dequant(acc_ref, beta, oracle.row_scale(W)[0]))
    # the same codes against all-127 activations: the largest sums
    big = np.full((T, K), 127, np.int8)
    yb, accb = (sbl.sparse_bitlinear_gemm if T > 16 else sbl.sparse_bitlinear_gemv)(
        dev(big), dev(np.ones(T, np.float32)), packed_d, scale_d, want_acc=True)
    assert np.array_equal(host(accb), oracle.gemm_acc(big, codes))


def test_widest_rows_sparse24_and_ste(sbl):
    """K = 65536 on the 2:4 path (compressor and smfmac product, acc equal to
    the oracle's and y to the dense product's) and in the straight-through
    backward (every entry within its bound)."""
    T, N, K = 300, 260, 65536
    o = _operands("gpu/maxk/sp24", T, K, N, n=2, m=4)
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    sp = sbl.sparse24_compress(dev(o["packed"]), bad)
    y, acc = sbl.sparse_bitlinear_gemm_sparse24(dev(o["xq"]), dev(o["beta"]), sp, N, dev(o["g"]),
                                                want_acc=True)
    yd = sbl.sparse_bitlinear_gemm(dev(o["xq"]), dev(o["beta"]), dev(o["packed"]), dev(o["g"]))[0]
    assert int(bad.item()) == 0
    assert np.array_equal(host(acc), oracle.gemm_acc(o["xq"], o["codes"]))
    assert torch.equal(y, yd)
    # backward: 64 tokens, 32 outputs, K = 65536 inputs
    Ts, Ns = 64, 32
    dy = synth.grad_output("gpu/maxk/ste/dy", Ts, Ns)
    xq, beta, codes, g = o["xq"][:Ts], o["beta"][:Ts], o["codes"][:Ns], o["g"][:Ns]
    dx, dw = sbl.sparse_bitlinear_ste_backward(dev(dy), dev(xq), dev(beta),
                                               dev(oracle.pack_codes(codes)), dev(g))
    dx_ref, dw_ref = oracle.ste_backward(dy, xq, beta, codes, g)
    a = np.abs((dy * g[None, :]).astype(np.float32)).astype(np.float64)
    s = (beta / np.float32(127)).astype(np.float32)
    b = np.abs((dy * s[:, None]).astype(np.float32)).astype(np.float64)
    u = 2.0 ** -24
    bdx = (3 * Ns / 16 + 36) * u * (a @ np.abs(codes).astype(np.float64)) + 1e-37
    bdw = (3 * Ts / 16 + 36) * u * (b.T @ np.abs(xq).astype(np.float64)) * g[:, None].astype(np.float64) + 1e-37
    assert (np.abs(host(dx).astype(np.float64) - dx_ref) <= bdx).all()
    assert (np.abs(host(dw).astype(np.float64) - dw_ref) <= bdw).all()
