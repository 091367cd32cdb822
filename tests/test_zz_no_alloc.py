"""The allocation-free backward entry point against the one that takes a
caller workspace: identical dx and dw, bit for bit, over two calls in a row
(the second with a smaller problem, so the library's scratch holds the
first call's partial sums when the second starts), and the error for a
problem whose workspace exceeds the scratch."""
import numpy as np
import pytest

import oracle
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


def _problem(tag, T, K, N):
    W = synth.latent_weight(f"{tag}/W", N, K)
    g, _ = oracle.row_scale(W)
    packed = oracle.pack_codes(oracle.ternary_codes(W, oracle.nm_mask(W, 3, 4), g))
    xq, beta = oracle.act_quant(synth.activations_bf16(f"{tag}/x", T, K))
    dy = synth.grad_output(f"{tag}/dy", T, N)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return to(dy), to(xq), to(beta), to(packed), to(g)


def test_noalloc_matches_workspace_entry_point(sbl):
    # 8192 tokens of the 0.5B gate shape split the token sum of dw (partial
    # sums in the scratch); the second, smaller call splits it differently
    for T, K, N in [(8192, 896, 4864), (1000, 256, 300)]:
        print(f"[no-alloc] T={T} K={K} N={N}", flush=True)
        dy, xq, beta, packed, g = _problem(f"gpu/noalloc/{T}x{K}x{N}", T, K, N)
        assert sbl.sparse_bitlinear_ste_workspace_bytes(T, K, N) <= sbl.STE_SCRATCH_BYTES
        dx0, dw0 = sbl.sparse_bitlinear_ste_backward(dy, xq, beta, packed, g)
        dx1 = torch.full((T, K), float("nan"), device=DEV)
        dw1 = torch.full((N, K), float("nan"), device=DEV)
        sbl.sparse_bitlinear_ste_backward_noalloc(dy, xq, beta, packed, g, dx=dx1, dw=dw1)
        torch.cuda.synchronize()
        assert torch.equal(dx0, dx1)
        assert torch.equal(dw0, dw1)
        # dw alone, through the scratch again
        dw2 = torch.full((N, K), float("nan"), device=DEV)
        sbl.sparse_bitlinear_ste_backward_noalloc(dy, xq, beta, packed, g, dw=dw2)
        torch.cuda.synchronize()
        assert torch.equal(dw0, dw2)


def test_noalloc_refuses_problems_beyond_its_scratch(sbl):
    T, K, N = 1 << 25, 128, 64      # beta/127 alone needs 128 MiB
    assert sbl.sparse_bitlinear_ste_workspace_bytes(T, K, N) > sbl.STE_SCRATCH_BYTES
    lib = sbl.load()
    P = 0x10000                      # never dereferenced: the call fails first
    st = lib.sparse_bitlinear_ste_backward_noalloc(P, P, P, P, P, T, K, N, None, P,
                                                   sbl._stream(torch.device(DEV)))
    assert st == -6
