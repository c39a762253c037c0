"""GPU test of sherry_gemm_noalloc, the product for callers that cannot
allocate device memory: its split-K cells live in the library's static
per-GPU array instead of a caller's workspace.

Through the C ABI, it must return exactly what sherry_gemm returns (and the
oracle), on two calls in a row, the second with a smaller input, so the
array's contents left by the first call cannot leak into the second.
"""

import numpy as np
import pytest
import torch

import bit_weight_amd as bw
from bit_weight_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _case(orc, M, N, K, seed):
    W = synth.weights(N, K, 0.02, False, seed=seed)
    T, alpha = orc.quantize(W.numpy())
    packed, galpha = bw.quantize_pack(W.cuda())
    x = synth.activations(M, K, seed=seed + 1)
    gq, gs = bw.quantize_act(x.cuda())
    torch.cuda.synchronize()
    q, s = gq.cpu().numpy(), gs.cpu().numpy()
    _, y_ref = orc.gemm(q, s, T, alpha)
    return gq, gs, packed, galpha, y_ref


@pytest.mark.parametrize("shapes", [
    # (M, N, K): both split K (64-bit cells in the static array); the second is smaller
    [(8, 4096, 4096), (3, 1024, 2048)],
    # a chunked call (launches of 64 + 16 tokens sharing the cells), then a small one
    [(80, 2048, 16384), (1, 256, 1024)],
])
def test_noalloc_matches_gemm_two_calls(orc, shapes):
    for i, (M, N, K) in enumerate(shapes):
        print(f"noalloc call {i}: M={M} N={N} K={K} plan={bw.plan(M, N, K)}", flush=True)
        assert 0 < bw.workspace_bytes(M, N, K) <= bw.NOALLOC_SCRATCH_BYTES
        gq, gs, packed, galpha, y_ref = _case(orc, M, N, K, seed=9100 + 10 * i + M)
        y_na = bw.gemm_noalloc(gq, gs, packed, galpha, N, K)
        y_ws = bw.gemm(gq, gs, packed, galpha, N, K)
        torch.cuda.synchronize()
        a, b = y_na.cpu().numpy(), y_ws.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"call {i} differs from sherry_gemm"
        assert np.array_equal(a.view(np.uint32), y_ref.view(np.uint32)), f"call {i} differs from the oracle"


def test_noalloc_without_split_and_repeated(orc):
    """A shape with no K-split (no scratch used) and the same split shape
    called several times back to back: every call leaves the cells zero."""
    gq, gs, packed, galpha, y_ref = _case(orc, 8, 8192, 1024, seed=9300)
    assert bw.workspace_bytes(8, 8192, 1024) == 0
    y = bw.gemm_noalloc(gq, gs, packed, galpha, 8192, 1024)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32))
    gq, gs, packed, galpha, y_ref = _case(orc, 4, 4096, 4096, seed=9400)
    for _ in range(4):
        y = bw.gemm_noalloc(gq, gs, packed, galpha, 4096, 4096)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y_ref.view(np.uint32))
