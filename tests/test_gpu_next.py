"""GPU parity of the operators around the forward path: RMSNorm fused into
the int8 activation quantisation, mask change/verify counts, and the
per-tensor absmean scale.  Through the C ABI, against the CPU oracle on the
same seeded inputs; bit-exact everywhere (codes, scales, x~, beta, counts).
"""
import numpy as np
import pytest

import oracle
from brute import unpack_bits

from sparse_linear_layers_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def sbl():
    import sparse_linear_layers_amd as m
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.load()
    return m


def dev(a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    return t.cpu().numpy()


# ------------------------------------------------------ RMSNorm -> int8
@pytest.mark.parametrize("T,K", [(1, 64), (3, 256), (128, 896), (77, 4864), (5, 8192),
                                 (4, 9216), (2, 65536)])
@pytest.mark.parametrize("eps", [1e-6, 0.0, 1.1920928955078125e-07])
def test_rmsnorm_act_quant(sbl, T, K, eps):
    x = synth.activations_bf16(f"gpu/rms/{T}x{K}", T, K)
    w = synth.norm_weight(f"gpu/rms/{K}/w", K)
    xq_ref, beta_ref, _ = oracle.rmsnorm_act_quant(x, w, eps)
    xq, beta = sbl.rmsnorm_act_quant_i8(dev(x), dev(w), eps)
    assert np.array_equal(host(beta), beta_ref)
    assert np.array_equal(host(xq), xq_ref)


def test_rmsnorm_act_quant_edge_tokens(sbl):
    K = 896
    x = synth.activations_bf16("gpu/rms/edge", 6, K)
    x[0] = 0                                                    # zero token
    x[1] = synth.float_to_bf16_bits(np.full(K, -2.5, np.float32))  # constant token
    x[2] = synth.float_to_bf16_bits(synth.rng("gpu/rms/edge/big").standard_normal(K).astype(np.float32) * np.float32(1e30))
    x[3] = synth.float_to_bf16_bits(synth.rng("gpu/rms/edge/small").standard_normal(K).astype(np.float32) * np.float32(1e-18))
    x[4, :] = 0
    x[4, 17] = synth.float_to_bf16_bits(np.array([3.0], np.float32))[0]  # one spike
    w = synth.norm_weight("gpu/rms/edge/w", K)
    w[5] = 0.0
    for eps in (1e-6, 0.0):
        xq_ref, beta_ref, _ = oracle.rmsnorm_act_quant(x, w, eps)
        xq, beta = sbl.rmsnorm_act_quant_i8(dev(x), dev(w), eps)
        assert np.array_equal(host(beta), beta_ref)
        assert np.array_equal(host(xq), xq_ref)


@pytest.mark.parametrize("K", [896, 4864])
def test_rmsnorm_act_quant_full_size(sbl, K):
    """The 0.5B skeleton's prefill activations (32768 tokens), compared in
    full."""
    T = synth.QWEN05B_PREFILL_TOKENS
    x = synth.activations_bf16(f"gpu/rms/full/{K}", T, K)
    w = synth.norm_weight(f"gpu/rms/full/{K}/w", K)
    xq_ref, beta_ref, _ = oracle.rmsnorm_act_quant(x, w, 1e-6)
    xq, beta = sbl.rmsnorm_act_quant_i8(dev(x), dev(w), 1e-6)
    assert np.array_equal(host(beta), beta_ref)
    assert np.array_equal(host(xq), xq_ref)


# --------------------------------------------------------- mask monitor
@pytest.mark.parametrize("rows,cols,n,m", [(3, 64, 3, 4), (37, 256, 2, 4), (512, 896, 3, 4),
                                           (64, 4864, 6, 8), (9, 1024, 4, 8), (1, 65536, 1, 4)])
@pytest.mark.parametrize("frac", [0.0, 0.003, 0.5])
def test_mask_stats(sbl, rows, cols, n, m, frac):
    W = synth.latent_weight(f"gpu/ms/{rows}x{cols}", rows, cols)
    new = host(sbl.nm_mask_create(dev(W), n, m))
    assert np.array_equal(new, oracle.nm_mask(W, n, m))
    old = synth.mask_flip(f"gpu/ms/{rows}x{cols}/{frac}", new, frac)
    bad = synth.mask_flip(f"gpu/ms/{rows}x{cols}/{frac}/bad", new, frac / 3)
    for o, nw in ((old, new), (new, old), (None, new), (None, bad), (old, bad)):
        got = host(sbl.nm_mask_stats(None if o is None else dev(o), dev(nw), rows, cols, n, m))
        assert tuple(int(v) for v in got) == oracle.mask_stats(o, nw, rows, cols, n, m)


def test_mask_stats_full_layer(sbl):
    """Every mask of one 0.5B-skeleton layer refreshed against a perturbed
    copy of the latent weights: the change counts of the seven matrices."""
    for name, N, K in synth.QWEN05B_LINEARS:
        W = synth.latent_weight(f"gpu/ms/layer/{name}", N, K)
        W2 = W + synth.latent_weight(f"gpu/ms/layer/{name}/step", N, K, std=1e-4)
        a = sbl.nm_mask_create(dev(W), 3, 4)
        b = sbl.nm_mask_create(dev(W2), 3, 4)
        got = host(sbl.nm_mask_stats(a, b, N, K, 3, 4))
        ref = oracle.mask_stats(oracle.nm_mask(W, 3, 4), oracle.nm_mask(W2, 3, 4), N, K, 3, 4)
        assert tuple(int(v) for v in got) == ref and ref[1] == 0 and ref[0] > 0


def test_mask_stats_empty(sbl):
    st = sbl.nm_mask_stats(None, torch.zeros(0, dtype=torch.uint8, device=DEV), 0, 64, 3, 4)
    assert host(st).tolist() == [0, 0]


# ----------------------------------------------------- per-tensor gamma
def _per_tensor_ref(W, mask, from_masked):
    g = oracle.tensor_scale(W, mask, from_masked)
    rows = W.shape[0]
    gam = np.full(rows, g, dtype=np.float32)
    codes = oracle.ternary_codes(W, mask, gam)
    return g, oracle.pack_codes(codes)


@pytest.mark.parametrize("rows,cols", [(1, 64), (37, 896), (512, 4864), (2048, 2048), (7, 9216)])
@pytest.mark.parametrize("mode", ["dense", "mask", "mask_from_masked"])
def test_ternary_quant_pack_per_tensor(sbl, rows, cols, mode):
    W = synth.latent_weight(f"gpu/pt/{rows}x{cols}", rows, cols)
    mask = oracle.nm_mask(W, 3, 4) if mode != "dense" else None
    fm = mode == "mask_from_masked"
    g, packed_ref = _per_tensor_ref(W, mask, fm)
    flags = sbl.SCALE_PER_TENSOR | (sbl.SCALE_FROM_MASKED if fm else 0)
    packed, scale, sb = sbl.ternary_quant_pack(dev(W), dev(mask) if mask is not None else None, flags)
    assert (host(scale) == g).all()
    assert (host(sb).view(np.uint16) == oracle.bf16_rne(float(g))).all()
    assert np.array_equal(host(packed), packed_ref)


@pytest.mark.parametrize("n,m", [(3, 4), (2, 4), (6, 8)])
@pytest.mark.parametrize("rows,cols", [(21, 896), (16, 4864), (4, 9216)])
@pytest.mark.parametrize("fm", [False, True])
def test_nm_mask_quant_pack_per_tensor(sbl, n, m, rows, cols, fm):
    W = synth.latent_weight(f"gpu/ptf/{rows}x{cols}/{n}{m}", rows, cols)
    mask_ref = oracle.nm_mask(W, n, m)
    g, packed_ref = _per_tensor_ref(W, mask_ref, fm)
    flags = sbl.SCALE_PER_TENSOR | (sbl.SCALE_FROM_MASKED if fm else 0)
    mask, packed, scale, sb = sbl.nm_mask_quant_pack(dev(W), n, m, flags)
    assert np.array_equal(host(mask), mask_ref)
    assert (host(scale) == g).all()
    assert np.array_equal(host(packed), packed_ref)


def test_per_tensor_full_size_matrix(sbl):
    """The 0.5B skeleton's gate matrix (4864 x 896) with one scale."""
    W = synth.latent_weight("gpu/pt/gate", 4864, 896)
    g, packed_ref = _per_tensor_ref(W, oracle.nm_mask(W, 3, 4), False)
    _, packed, scale, _ = sbl.nm_mask_quant_pack(dev(W), 3, 4, sbl.SCALE_PER_TENSOR)
    assert (host(scale) == g).all()
    assert np.array_equal(host(packed), packed_ref)
    # the products take the replicated scale unchanged
    x = synth.activations_bf16("gpu/pt/gate/x", 96, 896)
    xq, beta = oracle.act_quant(x)
    y, acc = sbl.sparse_bitlinear_gemm(dev(xq), dev(beta), packed, scale, want_acc=True)
    codes = oracle.unpack_codes(packed_ref, 896)
    assert np.array_equal(host(acc), oracle.gemm_acc(xq, codes))


# ------------------------------------------------------ STE backward
def _ste_operands(tag, T, K, N):
    W = synth.latent_weight(f"{tag}/W", N, K)
    x = synth.activations_bf16(f"{tag}/x", T, K)
    mask = oracle.nm_mask(W, 3, 4)
    g, _ = oracle.row_scale(W)
    codes = oracle.ternary_codes(W, mask, g)
    xq, beta = oracle.act_quant(x)
    dy = synth.grad_output(f"{tag}/dy", T, N)
    return dict(codes=codes, packed=oracle.pack_codes(codes), g=g, xq=xq, beta=beta, dy=dy)


def _ste_bounds(o, rows=None, cols=None):
    """Per-entry error bounds of dx[rows] and dw[:, cols]: float
    accumulation of R exact products in 16-term matrix-core steps, three
    per 16 terms (one per bf16 piece), at most 32 partial sums and the
    final product with gamma: (3R/16 + 36) * 2^-24 * sum|terms|."""
    dy, g = o["dy"], o["g"]
    T, N = dy.shape
    dyr = dy if rows is None else dy[rows]
    a = np.abs((dyr * g[None, :]).astype(np.float32)).astype(np.float64)
    s = (o["beta"] / np.float32(127)).astype(np.float32)
    b = np.abs((dy * s[:, None]).astype(np.float32)).astype(np.float64)
    xq = o["xq"] if cols is None else o["xq"][:, cols]
    sdx = a @ np.abs(o["codes"]).astype(np.float64)
    sdw = (b.T @ np.abs(xq).astype(np.float64)) * g[:, None].astype(np.float64)
    u = 2.0 ** -24
    return (3 * N / 16 + 36) * u * sdx + 1e-37, (3 * T / 16 + 36) * u * sdw + 1e-37


@pytest.mark.parametrize("T,K,N", [(128, 256, 512), (300, 896, 200), (33, 64, 4), (1, 64, 1),
                                   (129, 4864, 260), (1000, 192, 130), (2048, 896, 128),
                                   (4100, 320, 96)])
def test_ste_backward(sbl, T, K, N):
    o = _ste_operands(f"gpu/ste/{T}x{K}x{N}", T, K, N)
    dx_ref, dw_ref = oracle.ste_backward(o["dy"], o["xq"], o["beta"], o["codes"], o["g"])
    args = [dev(o[k]) for k in ("dy", "xq", "beta", "packed", "g")]
    dx, dw = sbl.sparse_bitlinear_ste_backward(*args)
    bdx, bdw = _ste_bounds(o)
    assert (np.abs(host(dx).astype(np.float64) - dx_ref) <= bdx).all()
    assert (np.abs(host(dw).astype(np.float64) - dw_ref) <= bdw).all()
    # each output alone, and a caller workspace full of stale values: the
    # same bits (the reduction order is fixed)
    dx2, none = sbl.sparse_bitlinear_ste_backward(*args, want_dw=False)
    need = sbl.sparse_bitlinear_ste_workspace_bytes(T, K, N)
    ws = torch.full((max(need, 16),), 0x7f, dtype=torch.uint8, device=DEV)
    none2, dw2 = sbl.sparse_bitlinear_ste_backward(*args, want_dx=False, workspace=ws)
    assert none is None and none2 is None
    assert torch.equal(dx, dx2) and torch.equal(dw, dw2)


def test_ste_backward_empty_reductions(sbl):
    """No tokens: dw is a sum over nothing (zeros); no output rows: dx is."""
    K, N = 192, 40
    o = _ste_operands("gpu/ste/empty", 8, K, N)
    e = lambda *s: torch.empty(s, dtype=torch.float32, device=DEV)
    got = sbl.sparse_bitlinear_ste_backward(e(0, N), torch.empty((0, K), dtype=torch.int8, device=DEV),
                                            e(0), dev(o["packed"]), dev(o["g"]))
    assert got[0].shape == (0, K) and (host(got[1]) == 0).all()
    got = sbl.sparse_bitlinear_ste_backward(e(8, 0), dev(o["xq"]), dev(o["beta"]),
                                            torch.empty((0, K // 4), dtype=torch.uint8, device=DEV),
                                            e(0))
    assert (host(got[0]) == 0).all() and got[1].shape == (0, K)


@pytest.mark.parametrize("name,N,K", [("gate", 4864, 896), ("down", 896, 4864)])
def test_ste_backward_full_size_sampled(sbl, name, N, K):
    """The 0.5B skeleton's gate and down linears at 32768 tokens: dx on
    sampled token rows, dw on sampled input columns (each depends only on
    its own slice), against the oracle."""
    T = synth.QWEN05B_PREFILL_TOKENS
    o = _ste_operands(f"gpu/ste/full/{name}", T, K, N)
    dx, dw = sbl.sparse_bitlinear_ste_backward(dev(o["dy"]), dev(o["xq"]), dev(o["beta"]),
                                               dev(o["packed"]), dev(o["g"]))
    pick = synth.rng(f"gpu/ste/full/pick/{name}")
    rows = np.unique(np.concatenate([[0, T - 1], pick.choice(T, 62, replace=False)]))
    cols = np.unique(np.concatenate([[0, K - 1], pick.choice(K, 30, replace=False)]))
    dx_ref, _ = oracle.ste_backward(o["dy"][rows], o["xq"][rows], o["beta"][rows], o["codes"],
                                    o["g"], want_dw=False)
    _, dw_ref = oracle.ste_backward(o["dy"], o["xq"][:, cols], o["beta"], o["codes"][:, cols],
                                    o["g"], want_dx=False)
    bdx, bdw = _ste_bounds(o, rows=rows, cols=cols)
    assert (np.abs(host(dx)[rows].astype(np.float64) - dx_ref) <= bdx).all()
    assert (np.abs(host(dw)[:, cols].astype(np.float64) - dw_ref) <= bdw).all()


def test_ste_backward_single_term_reductions_are_exact(sbl):
    """Reductions with one nonzero term at full length: codes with one +-1
    per input column (dx sums 4864 output features), x~ with one +-1 per
    input column (dw sums 32768 tokens).  Each result is then one exact
    product (a float times +-1: the three bf16 pieces add back to it exactly
    and every other term is zero), so dx and dw must equal the oracle's bit
    for bit: a lost or mis-scaled bf16 piece, which the accumulation bound
    at these lengths would not catch, changes the low bits."""
    # dx: 1024 tokens, 4864 -> 896 (the gate linear's backward to its input)
    T, N, K = 1024, 4864, 896
    W = synth.latent_weight("gpu/ste1/W", N, K)
    g, _ = oracle.row_scale(W)
    codes = np.zeros((N, K), np.int8)
    k = np.arange(K)
    codes[(37 * k + 11) % N, k] = np.where(k % 3 == 0, -1, 1).astype(np.int8)
    xq, beta = oracle.act_quant(synth.activations_bf16("gpu/ste1/x", T, K))
    dy = synth.grad_output("gpu/ste1/dy", T, N)
    dx, _ = sbl.sparse_bitlinear_ste_backward(dev(dy), dev(xq), dev(beta), dev(oracle.pack_codes(codes)),
                                              dev(g), want_dw=False)
    dx_ref, _ = oracle.ste_backward(dy, xq, beta, codes, g, want_dw=False)
    assert np.array_equal(host(dx), dx_ref)
    # dw: 32768 tokens, 64 output features, 896 input columns
    T, N, K = synth.QWEN05B_PREFILL_TOKENS, 64, 896
    W = synth.latent_weight("gpu/ste1w/W", N, K)
    g, _ = oracle.row_scale(W)
    codes = oracle.ternary_codes(W, oracle.nm_mask(W, 3, 4), g)
    _, beta = oracle.act_quant(synth.activations_bf16("gpu/ste1w/x", T, K))
    xq = np.zeros((T, K), np.int8)
    k = np.arange(K)
    xq[(7919 * k + 5) % T, k] = np.where(k % 2 == 0, 1, -1).astype(np.int8)
    dy = synth.grad_output("gpu/ste1w/dy", T, N)
    _, dw = sbl.sparse_bitlinear_ste_backward(dev(dy), dev(xq), dev(beta), dev(oracle.pack_codes(codes)),
                                              dev(g), want_dx=False)
    _, dw_ref = oracle.ste_backward(dy, xq, beta, codes, g, want_dx=False)
    assert np.array_equal(host(dw), dw_ref)
    # the pieces below the top bf16 one carry weight here: dropping them
    # would move most results
    top = (dw_ref.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    assert (top != dw_ref).mean() > 0.9


def test_mask_stats_wide_gate_stack_as_benchmarked(sbl):
    """The mask monitor at the size the benchmark times: the 16 gate masks of
    the 2048/7168 stack stacked row-wise (114688 x 2048, 235M weights), the
    masks of the latent weights against those after a small update; counts
    equal to the oracle's over the same masks, the GPU masks equal to the
    oracle's, and the packed-code validator clean on the stack's codes."""
    rows, cols = 16 * 7168, 2048
    W = synth.latent_weight("gpu/ms/wide/W", rows, cols)
    W2 = W + synth.latent_weight("gpu/ms/wide/step", rows, cols, std=1e-4)
    a = sbl.nm_mask_create(dev(W), 3, 4)
    b = sbl.nm_mask_create(dev(W2), 3, 4)
    ma, mb = oracle.nm_mask(W, 3, 4), oracle.nm_mask(W2, 3, 4)
    assert np.array_equal(host(a), ma) and np.array_equal(host(b), mb)
    got = host(sbl.nm_mask_stats(a, b, rows, cols, 3, 4))
    ref = oracle.mask_stats(ma, mb, rows, cols, 3, 4)
    assert tuple(int(v) for v in got) == ref and ref[1] == 0 and ref[0] > 0
    _, packed, _, _ = sbl.nm_mask_quant_pack(dev(W), 3, 4, want_mask=False)
    assert host(sbl.packed_codes_check(packed, 3, 4)).tolist() == [0, 0]
