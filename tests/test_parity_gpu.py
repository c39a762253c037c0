"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: packed codes, alpha, q, s_x and the int32 accumulators bit-exact; fp32
outputs within 1e-5 relative error (the epilogue order is pinned on both
sides, so they are expected to be bit-identical too).  Each side quantizes
and packs the same seeded fp32 inputs independently.
"""

import numpy as np
import pytest
import torch

import bit_weight_amd as bw
from bit_weight_amd import synth

pytestmark = pytest.mark.gpu

RTOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _say(*a):
    print(*a, flush=True)


def gpu_pack(W: torch.Tensor):
    packed, alpha = bw.quantize_pack(W.cuda())
    torch.cuda.synchronize()
    return packed, alpha


def assert_y_close(y_gpu: np.ndarray, y_ref: np.ndarray):
    denom = np.maximum(np.abs(y_ref), np.finfo(np.float32).tiny)
    rel = np.abs(y_gpu.astype(np.float64) - y_ref.astype(np.float64)) / denom
    # exact zeros must stay exact
    assert np.all((y_ref == 0) <= (y_gpu == 0))
    assert rel.max() <= RTOL, f"max rel err {rel.max():.3e}"


# ---------------------------------------------------------------- packer
@pytest.mark.parametrize("N,K,std,spikes", [(64, 128, 0.02, False), (256, 256, 0.02, False),
                                            (192, 384, 0.1, True), (320, 1152, 0.02, False),
                                            (68, 144, 0.02, False), (4, 16, 0.1, True),
                                            (196, 1040, 0.1, True)])
def test_pack_parity(orc, N, K, std, spikes):
    _say(f"pack N={N} K={K}")
    W = synth.weights(N, K, std, spikes, seed=100 + N + K)
    T, alpha = orc.quantize(W.numpy())
    packed, galpha = gpu_pack(W)
    assert np.array_equal(packed.cpu().numpy(), orc.pack(T))
    assert np.array_equal(galpha.cpu().numpy().view(np.uint32), alpha.view(np.uint32))


def test_pack_ties_zeros_and_signed_zero(orc):
    N, K = 128, 256
    W = synth.weights(N, K, 1.0, False, seed=7)
    W = torch.round(W * 2) / 2                 # many equal magnitudes
    W[0] = 0.0
    W[1] = -0.0
    W[2, :4] = torch.tensor([5.0, -5.0, 5.0, -5.0])
    W[3, 4:8] = torch.tensor([-0.0, 0.0, -1.0, -0.0])
    W[4] = 5.0 * torch.sign(torch.randn(K, generator=torch.Generator().manual_seed(3)))
    T, alpha = orc.quantize(W.numpy())
    packed, galpha = gpu_pack(W)
    assert np.array_equal(packed.cpu().numpy(), orc.pack(T))
    assert np.array_equal(galpha.cpu().numpy().view(np.uint32), alpha.view(np.uint32))


# ----------------------------------------------------- activation quantizer
@pytest.mark.parametrize("M,K,outl", [(1, 256, False), (16, 4096, False), (3, 11008, False),
                                      (512, 4096, True), (2, 4, False)])
def test_act_quant_parity(orc, M, K, outl):
    _say(f"act_quant M={M} K={K}")
    x = synth.activations(M, K, seed=300 + M, outlier_channels=outl)
    if M >= 3:
        x[1] = 0.0
    q, s = orc.act_quant(x.numpy())
    gq, gs = bw.quantize_act(x.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(gq.cpu().numpy(), q)
    assert np.array_equal(gs.cpu().numpy().view(np.uint32), s.view(np.uint32))


def test_act_quant_ties_golden(orc):
    x = torch.tensor([[127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5, 126.5, -127.0, 0.0, 0.0]])
    gq, gs = bw.quantize_act(x.cuda())
    q, s = orc.act_quant(x.numpy())
    assert gq.cpu().numpy().tolist() == q.tolist()
    assert gq.cpu().numpy()[0, :10].tolist() == [127, 2, 4, -2, -4, 0, 2, 0, 126, -127]
    assert float(gs[0]) == 1.0


def _golden_helpers():
    import os
    import sys
    gdir = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    if gdir not in sys.path:
        sys.path.insert(0, gdir)
    import exact_fp32
    return gdir, exact_fp32


def test_act_quant_scaled_golden(orc):
    """Scales other than 1 (golden from exact rational arithmetic): the GPU
    quantizer, and sherry_linear's fused quantizer through its product, follow
    one fp32 division x/s and round-half-even of that quotient."""
    import os
    gdir, ex = _golden_helpers()
    rows, cur = [], {}
    with open(os.path.join(gdir, "act_quant_scaled.txt")) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            key, val = line.split(":", 1)
            cur[key.strip()] = val.split()
            if key.strip() == "q":
                rows.append(([ex.from_hex(v) for v in cur["x"]], ex.from_hex(cur["s"][0]),
                             [int(v) for v in cur["q"]]))
                cur = {}
    x = torch.tensor(np.array([r[0] for r in rows], np.float32))
    gq, gs = bw.quantize_act(x.cuda())
    torch.cuda.synchronize()
    for m, (_, s_ref, q_ref) in enumerate(rows):
        assert gq[m].cpu().numpy().tolist() == q_ref, f"token {m}"
        assert gs[m].cpu().numpy().view(np.uint32) == np.float32(s_ref).view(np.uint32)
    # fused form (M = 3 <= 4 tokens): y must equal the oracle's product of the golden q
    M, K = x.shape
    N = 64
    W = synth.weights(N, K, 0.02, False, seed=4242)
    T, alpha = orc.quantize(W.numpy())
    packed, galpha = gpu_pack(W)
    assert bw.linear_plan(M, N, K)["fused"]
    q_ref = np.array([r[2] for r in rows], np.int8)
    s_ref = np.array([r[1] for r in rows], np.float32)
    _, y_ref = orc.gemm(q_ref, s_ref, T, alpha)
    gy = bw.linear(x.cuda(), packed, galpha, N, K).cpu().numpy()
    assert np.array_equal(gy.view(np.uint32), y_ref.view(np.uint32))


def test_epilogue_order_golden_every_path(orc):
    """y[i,i] = ((float)acc * s_x[i]) * alpha[i] for crafted accumulators that
    take the golden's values (exact rational arithmetic; each case one where
    the other two multiplication orders round differently), on every path."""
    import os
    gdir, ex = _golden_helpers()
    cases = []
    with open(os.path.join(gdir, "epilogue_order.txt")) as f:
        for line in f:
            if line.startswith("case:"):
                a, s_, al, y_ = line.split(":", 1)[1].split()
                cases.append((int(a), ex.from_hex(s_), ex.from_hex(al), ex.from_hex(y_)))
    C = len(cases)
    # every weight row is the block (+1,+1,+1,0) repeated, so acc[m,n] is the
    # sum of each block's first three q of token m, whatever n
    K = 88 * 128                                # 2816 blocks x 381 >= max |acc|
    W = torch.tensor([1.0, 1.0, 1.0, 0.0]).repeat(C, K // 4)
    T, alpha = orc.quantize(W.numpy())
    packed, _ = gpu_pack(W)
    q = np.zeros((C, K), np.int8)
    for m, (target, _, _, _) in enumerate(cases):
        rem = target
        for b in range(K // 4):
            for j in range(3):
                v = max(-127, min(127, rem))
                q[m, 4 * b + j] = v
                rem -= v
        assert rem == 0
    s_x = np.array([c[1] for c in cases], np.float32)
    al = np.array([c[2] for c in cases], np.float32)
    y_ref = np.array([c[3] for c in cases], np.float32)
    acc, y_orc = orc.gemm(q, s_x, T, al)
    assert np.array_equal(np.diag(acc), [c[0] for c in cases])
    gq, gs, gal = torch.tensor(q).cuda(), torch.tensor(s_x).cuda(), torch.tensor(al).cuda()
    for path, m0, m1 in [(None, 0, C), ("decode_mfma", 0, C), ("lut_gemv", 0, 16),
                         ("decode_mfma_gemv", 16, 32), ("decode_mfma_gemv", 40, 41)]:
        try:
            bw.plan_override(path)
            gy = bw.gemm(gq[m0:m1].contiguous(), gs[m0:m1].contiguous(), packed, gal, C, K).cpu().numpy()
        finally:
            bw.plan_override()
        d = np.array([gy[i, m0 + i] for i in range(m1 - m0)], np.float32)
        assert np.array_equal(d.view(np.uint32), y_ref[m0:m1].view(np.uint32)), path
        assert np.array_equal(gy.view(np.uint32), y_orc[m0:m1].view(np.uint32)), path


# ----------------------------------------------------- product, edge shapes
SHAPES = [(64, 128), (192, 384), (320, 1152)]
MS = [1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 33, 64, 65, 100, 128, 129, 130]


@pytest.fixture(scope="module")
def packed_cases(orc):
    out = {}
    for (N, K) in SHAPES:
        W = synth.weights(N, K, 0.02, False, seed=500 + N)
        T, alpha = orc.quantize(W.numpy())
        packed, galpha = gpu_pack(W)
        out[(N, K)] = (T, alpha, packed, galpha)
    return out


@pytest.mark.parametrize("M", MS)
@pytest.mark.parametrize("N,K", SHAPES)
def test_gemm_edges(orc, packed_cases, M, N, K):
    _say(f"gemm M={M} N={N} K={K} plan={bw.plan(M, N, K)}")
    T, alpha, packed, galpha = packed_cases[(N, K)]
    q = synth.int8_uniform(M, K, seed=700 + M + K)          # includes -128 and 127
    s_x = (torch.rand(M, generator=torch.Generator().manual_seed(M)) * 0.05 + 0.001).float()
    acc, y = orc.gemm(q.numpy(), s_x.numpy(), T, alpha)
    gacc = bw.gemm_i32(q.cuda(), packed, N, K)
    gy = bw.gemm(q.cuda(), s_x.cuda(), packed, galpha, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(gacc.cpu().numpy(), acc)
    assert_y_close(gy.cpu().numpy(), y)


PLANS = [(4, 1, 0), (4, 2, 3), (2, 2, 0), (2, 4, 2), (1, 1, 0), (1, 2, 5), (1, 8, 1), (4, 8, 1),
         (2, 1, 7), (8, 0, 0), (8, 2, 3), (8, 4, 2), (8, 0, 9)]   # 8: 4 row tiles x 2 waves


@pytest.mark.parametrize("rw,ch,splits", PLANS)
@pytest.mark.parametrize("M", [1, 2, 5, 8, 16])
def test_gemm_lut_plans(orc, packed_cases, rw, ch, splits, M):
    """Every LUT-GEMV launch shape (row tiles per workgroup, table stage size,
    K-splits incl. ragged ones) gives the same exact result."""
    N, K = 320, 1152                       # 5 row tiles, 9 k-tiles
    T, alpha, packed, galpha = packed_cases[(N, K)]
    q = synth.int8_uniform(M, K, seed=900 + M)
    acc = orc.gemm_i32(q.numpy(), T)
    try:
        bw.plan_override("lut_gemv", rw, ch, splits)
        _say(f"plan override lut rw={rw} ch={ch} splits={splits} M={M}: {bw.plan(M, N, K)}")
        gacc = bw.gemm_i32(q.cuda(), packed, N, K)
        torch.cuda.synchronize()
    finally:
        bw.plan_override()
    assert np.array_equal(gacc.cpu().numpy(), acc)


GEMV_PLANS = [(4, 0), (4, 1), (4, 2), (4, 3), (4, 9), (8, 0), (8, 1), (8, 2), (16, 0), (16, 1),
              (16, 5)]


@pytest.mark.parametrize("rw,splits", GEMV_PLANS)
@pytest.mark.parametrize("M", [1, 2, 5, 8, 13, 16, 17, 31, 32, 33, 50, 64, 65, 97, 128])
@pytest.mark.parametrize("N,K", [(320, 1152), (64, 128)])
def test_gemm_mfma_gemv_plans(orc, packed_cases, rw, splits, M, N, K):
    """Every launch shape of the small-M matrix-core GEMV (waves per row tile
    incl. idle ones, K-splits incl. ragged ones, one to four token blocks of
    16 with a ragged last block, launches of 64 tokens above M = 64 that
    share the split-K workspace) gives the same exact result, and the fp32
    output matches the oracle."""
    T, alpha, packed, galpha = packed_cases[(N, K)]
    q = synth.int8_uniform(M, K, seed=1900 + M + K)
    s_x = (torch.rand(M, generator=torch.Generator().manual_seed(M + 7)) * 0.05 + 0.001).float()
    acc, y = orc.gemm(q.numpy(), s_x.numpy(), T, alpha)
    try:
        bw.plan_override("decode_mfma_gemv", rw, 0, splits)
        _say(f"plan override gemv rw={rw} splits={splits} M={M} N={N} K={K}: {bw.plan(M, N, K)}")
        gacc = bw.gemm_i32(q.cuda(), packed, N, K)
        gy = bw.gemm(q.cuda(), s_x.cuda(), packed, galpha, N, K)
        torch.cuda.synchronize()
    finally:
        bw.plan_override()
    assert np.array_equal(gacc.cpu().numpy(), acc)
    assert_y_close(gy.cpu().numpy(), y)


# (waves per row tile, K): 4 to 8 k-tiles per wave with no K-split, which the
# GEMV runs as straight-line steps; ragged k-tile counts leave the waves
# uneven, and K = 1584 and 7248 end in a ragged k-tile
STRAIGHT_LINE = [(4, 13 * 128), (4, 1584), (4, 32 * 128), (8, 57 * 128), (8, 7248), (16, 128 * 128)]


@pytest.mark.parametrize("rw,K", STRAIGHT_LINE)
@pytest.mark.parametrize("M", [1, 3, 8, 16])
def test_gemm_gemv_straight_line_steps(orc, rw, K, M):
    """The GEMV's straight-line form (no K-split, 4 to 8 k-tiles per wave),
    with one token staged in LDS or loaded per step, on both code formats."""
    N = 192
    W = synth.weights(N, K, 0.02, M % 2 == 1, seed=7100 + K + rw)
    T, alpha = orc.quantize(W.numpy())
    packed, galpha = gpu_pack(W)
    p2, a2 = bw.quantize_pack2(W.cuda())
    q = synth.int8_uniform(M, K, seed=7200 + M + K)
    s_x = (torch.rand(M, generator=torch.Generator().manual_seed(M + 11)) * 0.05 + 0.001).float()
    acc, y = orc.gemm(q.numpy(), s_x.numpy(), T, alpha)
    try:
        bw.plan_override("decode_mfma_gemv", rw, 0, 1)
        p = bw.plan(M, N, K)
        _say(f"straight-line gemv rw={rw} M={M} N={N} K={K}: {p}")
        assert p["splits"] == 1 and 4 <= -(-((K + 127) // 128) // rw) <= 8
        gacc = bw.gemm_i32(q.cuda(), packed, N, K)
        gy = bw.gemm(q.cuda(), s_x.cuda(), packed, galpha, N, K)
        gy2 = bw.gemm2(q.cuda(), s_x.cuda(), p2, a2, N, K)
        torch.cuda.synchronize()
    finally:
        bw.plan_override()
    assert np.array_equal(gacc.cpu().numpy(), acc)
    assert_y_close(gy.cpu().numpy(), y)
    assert np.array_equal(gy2.cpu().numpy().view(np.uint32), gy.cpu().numpy().view(np.uint32))


# (the fused form holds at most 32 k-tiles: 8 waves reach 4 k-tiles from 25 on)
@pytest.mark.parametrize("rw,K,M", [(4, 13 * 128, 4), (4, 1584, 3), (4, 32 * 128, 1), (4, 32 * 128, 4),
                                    (8, 29 * 128, 2), (8, 3952, 1)])
def test_linear_fused_unsplit_long_waves(orc, rw, K, M):
    """sherry_linear's fused form (quantization inside the product) with no
    K-split and 4 to 8 k-tiles per wave, the range where the unfused product
    takes straight-line steps (the fused kernel keeps its loop): y matches
    the oracle and is bit-identical to sherry_quantize_act + sherry_gemm."""
    N = 192
    W = synth.weights(N, K, 0.02, True, seed=7300 + K + rw)
    x = synth.activations(M, K, seed=7400 + M + K, outlier_channels=True)
    T, alpha = orc.quantize(W.numpy())
    q, s = orc.act_quant(x.numpy())
    _, y = orc.gemm(q, s, T, alpha)
    packed, galpha = gpu_pack(W)
    try:
        bw.plan_override("decode_mfma_gemv", rw, 0, 1)
        lp = bw.linear_plan(M, N, K)
        _say(f"fused unsplit rw={rw} M={M} N={N} K={K}: {lp}")
        assert lp["fused"] and lp["splits"] == 1
        gl = bw.linear(x.cuda(), packed, galpha, N, K)
        gq, gs = bw.quantize_act(x.cuda())
        gy = bw.gemm(gq, gs, packed, galpha, N, K)
        torch.cuda.synchronize()
    finally:
        bw.plan_override()
    assert np.array_equal(gl.cpu().numpy().view(np.uint32), gy.cpu().numpy().view(np.uint32))
    assert_y_close(gl.cpu().numpy(), y)


@pytest.mark.parametrize("bm,kp", [(1, 2), (1, 4), (2, 2), (2, 4)])  # 64- / 128-token tiles, 2 / 4 k-phases
@pytest.mark.parametrize("M", [1, 7, 16, 17, 40, 64, 65, 100, 128, 129, 200, 300])
def test_gemm_prefill_kernel_at_small_m(orc, packed_cases, M, bm, kp):
    """The prefill kernel forced onto small and mid M with either tile height
    and 2 or 4 k-phases (rows past M clamped, a ragged last token tile,
    N = 320 ragged against 128- and 256-row tiles, 9 k-tiles: a short last
    step with 2 and with 4 phases)."""
    N, K = 320, 1152
    T, alpha, packed, galpha = packed_cases[(N, K)]
    q = synth.int8_uniform(M, K, seed=2900 + M)
    acc = orc.gemm_i32(q.numpy(), T)
    try:
        bw.plan_override("decode_mfma", bm, kp)
        p = bw.plan(M, N, K)
        assert p["path"] == "decode_mfma"
        assert p["grid"] == 8 * 1 * -(-M // (64 * bm))   # 2 or 3 n tiles -> one per XCD slot
        gacc = bw.gemm_i32(q.cuda(), packed, N, K)
        torch.cuda.synchronize()
    finally:
        bw.plan_override()
    assert np.array_equal(gacc.cpu().numpy(), acc)


def test_gemm_extreme_activations(orc, packed_cases):
    N, K = 192, 384
    T, alpha, packed, galpha = packed_cases[(N, K)]
    for M in (1, 4, 16, 40):
        for fill in (127, -128, 0):
            q = torch.full((M, K), fill, dtype=torch.int8)
            acc = orc.gemm_i32(q.numpy(), T)
            gacc = bw.gemm_i32(q.cuda(), packed, N, K)
            torch.cuda.synchronize()
            assert np.array_equal(gacc.cpu().numpy(), acc), (M, fill)


def test_gemm_deterministic_and_workspace_reuse(orc, packed_cases):
    outs = []
    for (N, K) in SHAPES + SHAPES:
        T, alpha, packed, galpha = packed_cases[(N, K)]
        q = synth.int8_uniform(1, K, seed=11)
        outs.append(bw.gemm_i32(q.cuda(), packed, N, K).cpu().numpy())
    for a, b in zip(outs[:3], outs[3:]):
        assert np.array_equal(a, b)


# ------------------------------------------------- the workloads, full size
def _workload_check(orc, name, sample_rows=None):
    w = synth.WORKLOADS[name]
    _say(f"workload {w.description}")
    W = synth.workload_weights(w)
    x = synth.workload_activations(w)
    T, alpha = orc.quantize(W.numpy())
    q, s = orc.act_quant(x.numpy())
    packed, galpha = gpu_pack(W)
    assert np.array_equal(packed.cpu().numpy(), orc.pack(T)), "packed codes"
    assert np.array_equal(galpha.cpu().numpy().view(np.uint32), alpha.view(np.uint32)), "alpha"
    del W
    gq, gs = bw.quantize_act(x.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(gq.cpu().numpy(), q), "q"
    assert np.array_equal(gs.cpu().numpy().view(np.uint32), s.view(np.uint32)), "s_x"
    if sample_rows is None:
        acc, y = orc.gemm(q, s, T, alpha)
        # every small-M path on the same inputs
        paths = ["lut_gemv", "decode_mfma_gemv"] if w.M <= 16 else [None]
        for path in paths:
            try:
                bw.plan_override(path)
                _say(f"  path {path}: {bw.plan(w.M, w.N, w.K)}")
                gacc = bw.gemm_i32(gq, packed, w.N, w.K).cpu().numpy()
                gy = bw.gemm(gq, gs, packed, galpha, w.N, w.K).cpu().numpy()
            finally:
                bw.plan_override()
            assert np.array_equal(gacc, acc), f"acc ({path})"
            assert_y_close(gy, y)
    else:
        gacc = bw.gemm_i32(gq, packed, w.N, w.K).cpu().numpy()
        gy = bw.gemm(gq, gs, packed, galpha, w.N, w.K).cpu().numpy()
        rows = sample_rows
        acc = orc.gemm_i32(q, np.ascontiguousarray(T[rows]))
        y = orc.epilogue(acc, s, np.ascontiguousarray(alpha[rows]))
        assert np.array_equal(gacc[:, rows], acc), "acc (sampled)"
        assert_y_close(np.ascontiguousarray(gy[:, rows]), y)


@pytest.mark.parametrize("name", ["1", "2a", "2b", "2c", "3a", "3b", "4"])
def test_workload_parity(orc, name):
    _workload_check(orc, name)


@pytest.fixture(scope="module")
def workload_5_ref(orc):
    """Workload 5 (M=512, K=4096, N=14336) and its full oracle product (the
    same oracle source built with OpenMP over the host cores; identical sums)."""
    w = synth.WORKLOADS["5"]
    W = synth.workload_weights(w)
    x = synth.workload_activations(w)
    T, alpha = orc.quantize(W.numpy())
    q, s = orc.act_quant(x.numpy())
    _say(f"workload 5: full oracle product on {orc.threads(parallel=True)} threads")
    acc, y = orc.gemm(q, s, T, alpha, parallel=True)
    packed, galpha = gpu_pack(W)
    assert np.array_equal(packed.cpu().numpy(), orc.pack(T)), "packed codes"
    assert np.array_equal(galpha.cpu().numpy().view(np.uint32), alpha.view(np.uint32)), "alpha"
    gq, gs = bw.quantize_act(x.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(gq.cpu().numpy(), q), "q"
    assert np.array_equal(gs.cpu().numpy().view(np.uint32), s.view(np.uint32)), "s_x"
    return w, acc, y, packed, galpha, gq, gs


@pytest.mark.parametrize("bm,kp", [(0, 0), (1, 2), (1, 4), (2, 2), (2, 4)])  # built-in, or forced tiles / k-phases
def test_workload_5_prefill_full(workload_5_ref, bm, kp):
    """Every one of the 7.3 M outputs of workload 5: int32 bit-exact, fp32
    within 1e-5 (bit-identical in practice)."""
    w, acc, y, packed, galpha, gq, gs = workload_5_ref
    try:
        bw.plan_override("decode_mfma" if bm else None, bm, kp)
        _say(f"workload 5 full: {bw.plan(w.M, w.N, w.K)}")
        gacc = bw.gemm_i32(gq, packed, w.N, w.K).cpu().numpy()
        gy = bw.gemm(gq, gs, packed, galpha, w.N, w.K).cpu().numpy()
    finally:
        bw.plan_override()
    assert np.array_equal(gacc, acc), "acc"
    assert_y_close(gy, y)


# ------------------------------------------------------ random shape sweep
def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 129)), int(rng.integers(129, 201))]))
        N = 4 * int(rng.integers(1, 257))          # 4 .. 1024, any multiple of 4
        K = 16 * int(rng.integers(1, 129))         # 16 .. 2048, any multiple of 16
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", _random_shapes(60, 9090))
def test_random_shapes_every_path(orc, M, N, K):
    """Seeded random shapes over the whole shape rule: the int32 product on
    every path that takes the shape, sherry_linear and (M <= 16) the 2-bit
    product, against the oracle."""
    W = synth.weights(N, K, 0.02, M % 3 == 0, seed=9100 + N + K)
    x = synth.activations(M, K, seed=9200 + M + K, outlier_channels=(M % 2 == 0))
    T, alpha = orc.quantize(W.numpy())
    q, s = orc.act_quant(x.numpy())
    acc, y = orc.gemm(q, s, T, alpha)
    packed, galpha = gpu_pack(W)
    assert np.array_equal(packed.cpu().numpy(), orc.pack(T)), "packed codes"
    gq, gs = bw.quantize_act(x.cuda())
    paths = [(None, 0, 0), ("decode_mfma", 1, 2), ("decode_mfma", 1, 4), ("decode_mfma", 2, 2),
             ("decode_mfma", 2, 4)]
    if M <= 16:
        paths += [("lut_gemv", 0, 0), ("decode_mfma_gemv", 0, 0)]
    elif M <= 128:
        paths += [("decode_mfma_gemv", 0, 0)]
    for path, rw, ch in paths:
        try:
            bw.plan_override(path, rw, ch)
            _say(f"random M={M} N={N} K={K} path {path}/{rw}/{ch}: {bw.plan(M, N, K)}")
            gacc = bw.gemm_i32(gq, packed, N, K).cpu().numpy()
        finally:
            bw.plan_override()
        assert np.array_equal(gacc, acc), f"acc ({path}, {rw}, {ch})"
    gy = bw.linear(x.cuda(), packed, galpha, N, K)
    torch.cuda.synchronize()
    assert_y_close(gy.cpu().numpy(), y)
    if M <= 16:                                    # the 2-bit format takes decode shapes
        p2, a2 = bw.quantize_pack2(W.cuda())
        gy2 = bw.gemm2(gq, gs, p2, a2, N, K)
        gy5 = bw.gemm(gq, gs, packed, galpha, N, K)
        torch.cuda.synchronize()
        assert np.array_equal(p2.cpu().numpy(), orc.pack2(T)), "2-bit codes"
        assert np.array_equal(gy2.cpu().numpy().view(np.uint32), gy5.cpu().numpy().view(np.uint32))
        assert_y_close(gy2.cpu().numpy(), y)


@pytest.mark.parametrize("M,N,K", [(1, 8192, 28672), (8, 8192, 28672), (16, 8192, 28672),
                                   (9, 4096, 4096), (16, 4096, 11008), (64, 4096, 4096),
                                   (88, 4096, 14336), (128, 4096, 14336), (64, 4096, 14336),
                                   (40, 5504, 8192)])
def test_gemm_gemv_plan_rule_shapes(orc, M, N, K):
    """The GEMV plans the built-in rule picks at these shapes: K split at
    wide N and long K for one token block (a wave keeps at most 8 or 16
    k-tiles), and 8 waves per row tile with few splits above 8 tokens at
    narrow N (one split at K=4096; no more workgroups than CUs: 4 splits at
    N=4096, K=14336, 2 at N=5504, K=8192; launches of 64 + 24 and 64 + 64
    tokens at M=88 and 128, K=14336, where the prefill's grid is small and
    its waves' K long): y and the int32 sums against the oracle."""
    W = synth.weights(N, K, 0.02, False, seed=9300 + N + K)
    x = synth.activations(M, K, seed=9400 + M + K)
    T, alpha = orc.quantize(W.numpy())
    q, s = orc.act_quant(x.numpy())
    acc, y = orc.gemm(q, s, T, alpha, parallel=True)
    packed, galpha = gpu_pack(W)
    gq, gs = bw.quantize_act(x.cuda())
    p = bw.plan(M, N, K)
    _say(f"plan rule M={M} N={N} K={K}: {p}")
    assert p["path"] == "decode_mfma_gemv"
    KT, RT = -(-K // 128), -(-N // 64)
    if RT >= 128 and M <= 16:
        per_wave = -(-(-(-KT // p["splits"])) // (p["block"] // 64))
        assert p["splits"] > 1 and per_wave <= (16 if M > 8 else 8), p
    if RT < 128 and M > 8:
        assert p["block"] == 512 and p["grid"] <= 256, p
    ws = torch.zeros(max(bw.workspace_bytes(M, N, K), 256), dtype=torch.uint8, device="cuda")
    gy = bw.gemm(gq, gs, packed, galpha, N, K, workspace=ws)
    gacc = bw.gemm_i32(gq, packed, N, K, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(gacc.cpu().numpy(), acc)
    assert_y_close(gy.cpu().numpy(), y)
    assert int(ws.count_nonzero()) == 0          # every split's cells left zero


# ------------------------------------------------------- HIP graph capture
@pytest.mark.parametrize("path,M,N,K", [(None, 1, 4096, 4096),        # fused step, K-split cells
                                        (None, 8, 1024, 2048),        # quantizer + GEMV
                                        ("lut_gemv", 3, 512, 1152),   # fused lookup tables
                                        (None, 200, 512, 640)])       # quantizer + prefill
def test_graph_replays_match_eager(orc, path, M, N, K):
    """sherry_linear and sherry_gemm captured into one HIP graph: every replay
    (with eager calls and synchronizations between replays, and inputs
    rewritten in place) is bit-identical to eager calls on the same inputs,
    and the K-split workspace stays zero throughout."""
    W = synth.weights(N, K, 0.02, False, seed=8100 + N)
    packed, galpha = gpu_pack(W)
    xs = [synth.activations(M, K, seed=8200 + i).cuda() for i in range(3)]
    try:
        bw.plan_override(path)
        _say(f"graph: path {path} M={M} N={N} K={K} linear plan {bw.linear_plan(M, N, K)}")
        ws = torch.zeros(max(bw.workspace_bytes(M, N, K), 256), dtype=torch.uint8, device="cuda")
        sc = torch.empty(max(bw.linear_scratch_bytes(M, N, K), 256), dtype=torch.uint8, device="cuda")
        x = xs[0].clone()
        q, s = bw.quantize_act(x)
        y1 = torch.empty((M, N), dtype=torch.float32, device="cuda")
        y2 = torch.empty((M, N), dtype=torch.float32, device="cuda")

        def calls():
            bw.linear(x, packed, galpha, N, K, out=y1, workspace=ws, scratch=sc)
            bw.gemm(q, s, packed, galpha, N, K, out=y2, workspace=ws)

        def eager(xv):
            qv, sv = bw.quantize_act(xv)
            e1 = bw.linear(xv, packed, galpha, N, K, workspace=ws,
                           scratch=torch.empty_like(sc))
            e2 = bw.gemm(qv, sv, packed, galpha, N, K, workspace=ws)
            torch.cuda.synchronize()
            return e1.clone(), e2.clone()

        calls()                           # warm up outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                calls()
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
        for r in range(6):
            xv = xs[r % 3]
            x.copy_(xv)
            qv, sv = bw.quantize_act(xv)
            q.copy_(qv)
            s.copy_(sv)
            torch.cuda.synchronize()
            e1, e2 = eager(xv)            # eager work between replays
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y1, e1), f"linear, replay {r}"
            assert torch.equal(y2, e2), f"gemm, replay {r}"
            assert int(ws.count_nonzero()) == 0, f"workspace left non-zero, replay {r}"
        # and the eager results are the oracle's
        T, alpha = orc.quantize(W.numpy())
        qo, so = orc.act_quant(xs[2].cpu().numpy())
        _, yo = orc.gemm(qo, so, T, alpha)
        assert_y_close(y1.cpu().numpy(), yo)
    finally:
        bw.plan_override()


# ----------------------------------------------- the shape rule's maxima
def test_max_k(orc):
    """K = 2^20 (8192 k-tiles per row; the GEMV's K-split plan, the lookup
    tables and the unfused sherry_linear), against the whole oracle product."""
    M, N, K = 1, 64, 1 << 20
    W = synth.weights(N, K, 0.02, False, seed=7001)
    x = synth.activations(M, K, seed=7002)
    T, alpha = orc.quantize(W.numpy())
    q, s = orc.act_quant(x.numpy())
    acc, y = orc.gemm(q, s, T, alpha)
    packed, galpha = gpu_pack(W)
    del W
    assert np.array_equal(packed.cpu().numpy(), orc.pack(T)), "packed codes"
    gq, gs = bw.quantize_act(x.cuda())
    for path in (None, "lut_gemv"):
        try:
            bw.plan_override(path)
            _say(f"max K: M={M} N={N} K={K} path {path}: {bw.plan(M, N, K)}")
            gacc = bw.gemm_i32(gq, packed, N, K).cpu().numpy()
            gy = bw.gemm(gq, gs, packed, galpha, N, K).cpu().numpy()
        finally:
            bw.plan_override()
        assert np.array_equal(gacc, acc), f"acc ({path})"
        assert_y_close(gy, y)
    _say(f"max K: linear, scratch {bw.linear_scratch_bytes(M, N, K)}")
    gy = bw.linear(x.cuda(), packed, galpha, N, K).cpu().numpy()
    assert_y_close(gy, y)


def test_max_n(orc):
    """N = 2^20 (16384 row tiles, one ragged k-tile of K = 16), every small-M
    path, against the whole oracle product."""
    M, N, K = 3, 1 << 20, 16
    W = synth.weights(N, K, 0.02, False, seed=7011)
    x = synth.activations(M, K, seed=7012)
    T, alpha = orc.quantize(W.numpy())
    q, s = orc.act_quant(x.numpy())
    acc, y = orc.gemm(q, s, T, alpha)
    packed, galpha = gpu_pack(W)
    del W
    assert np.array_equal(packed.cpu().numpy(), orc.pack(T)), "packed codes"
    gq, gs = bw.quantize_act(x.cuda())
    for path in (None, "lut_gemv", "decode_mfma"):
        try:
            bw.plan_override(path)
            _say(f"max N: M={M} N={N} K={K} path {path}: {bw.plan(M, N, K)}")
            gacc = bw.gemm_i32(gq, packed, N, K).cpu().numpy()
            gy = bw.gemm(gq, gs, packed, galpha, N, K).cpu().numpy()
        finally:
            bw.plan_override()
        assert np.array_equal(gacc, acc), f"acc ({path})"
        assert_y_close(gy, y)
    _say("max N: linear (fused)")
    gy = bw.linear(x.cuda(), packed, galpha, N, K).cpu().numpy()
    assert_y_close(gy, y)


def test_max_m(orc):
    """M = 2^20 tokens with N = 4096, so that m*N passes 2^31 (64-bit output
    offsets), on the prefill kernel and sherry_linear; sampled tokens, among
    them the first and the last, against the oracle."""
    M, N, K = 1 << 20, 4096, 16
    W = synth.weights(N, K, 0.02, False, seed=7021)
    x = synth.activations(M, K, seed=7022)
    T, alpha = orc.quantize(W.numpy())
    q, s = orc.act_quant(x.numpy())
    packed, galpha = gpu_pack(W)
    del W
    rng = np.random.default_rng(7023)
    toks = np.unique(np.concatenate([[0, 1, 127, 128, (1 << 19) - 1, 1 << 19, (1 << 19) + 1, M - 2, M - 1],
                                     rng.choice(M, 55, replace=False)]))
    assert (toks.astype(np.int64) * N).max() > 2 ** 31
    acc = orc.gemm_i32(np.ascontiguousarray(q[toks]), T)
    y = orc.epilogue(acc, np.ascontiguousarray(s[toks]), alpha)
    xg = x.cuda()
    gq, gs = bw.quantize_act(xg)
    assert np.array_equal(gq[torch.from_numpy(toks).cuda()].cpu().numpy(), q[toks]), "q (sampled)"
    ti = torch.from_numpy(toks).cuda()
    _say(f"max M: M={M} N={N} K={K}: {bw.plan(M, N, K)}")
    gacc = bw.gemm_i32(gq, packed, N, K)
    assert np.array_equal(gacc[ti].cpu().numpy(), acc), "acc (sampled)"
    del gacc
    gy = bw.gemm(gq, gs, packed, galpha, N, K)
    assert_y_close(gy[ti].cpu().numpy(), y)
    del gy
    _say("max M: linear")
    gy = bw.linear(xg, packed, galpha, N, K)
    assert_y_close(gy[ti].cpu().numpy(), y)
    del gy
    torch.cuda.empty_cache()


# ------------------------------------------- fused quantization + product
def _linear_check(orc, x, packed, T, alpha, galpha, N, K, what):
    q, s = orc.act_quant(x.numpy())
    acc, y = orc.gemm(q, s, T, alpha)
    xg = x.cuda()
    gy = bw.linear(xg, packed, galpha, N, K)
    gq, gs = bw.quantize_act(xg)
    gy2 = bw.gemm(gq, gs, packed, galpha, N, K)
    torch.cuda.synchronize()
    # identical to quantize + product on the GPU, and to the oracle
    assert np.array_equal(gy.cpu().numpy().view(np.uint32), gy2.cpu().numpy().view(np.uint32)), what
    assert_y_close(gy.cpu().numpy(), y)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 16, 100])
@pytest.mark.parametrize("N,K", SHAPES)
def test_linear_edges(orc, packed_cases, M, N, K):
    T, alpha, packed, galpha = packed_cases[(N, K)]
    x = synth.activations(M, K, seed=3100 + M + K, outlier_channels=(M % 2 == 1))
    if M >= 3:
        x[1] = 0.0                                   # an all-zero token
    _say(f"linear M={M} N={N} K={K} scratch={bw.linear_scratch_bytes(M, N, K)} plan={bw.plan(M, N, K)}")
    _linear_check(orc, x, packed, T, alpha, galpha, N, K, f"M={M}")


@pytest.mark.parametrize("path,rw,splits", [("decode_mfma_gemv", 4, 1), ("decode_mfma_gemv", 4, 3),
                                            ("decode_mfma_gemv", 16, 2), ("decode_mfma_gemv", 8, 9),
                                            ("lut_gemv", 0, 0), ("lut_gemv", 1, 3), ("lut_gemv", 2, 1),
                                            ("lut_gemv", 4, 9), ("lut_gemv", 8, 3), ("decode_mfma", 0, 0)])
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_linear_plans(orc, packed_cases, path, rw, splits, M):
    """Fused (both GEMVs) and unfused (prefill kernel) forms agree with the
    oracle and with quantize + product, at every launch shape."""
    N, K = 320, 1152
    T, alpha, packed, galpha = packed_cases[(N, K)]
    x = synth.activations(M, K, seed=4100 + M, outlier_channels=True)
    try:
        bw.plan_override(path, rw, 0, splits)
        _say(f"linear plan {path} rw={rw} splits={splits} M={M}: {bw.plan(M, N, K)}")
        _linear_check(orc, x, packed, T, alpha, galpha, N, K, f"{path} {rw} {splits}")
    finally:
        bw.plan_override()


@pytest.mark.parametrize("name", ["1", "2a", "2b", "2c", "3a", "3b", "4"])
def test_linear_workloads(orc, name):
    w = synth.WORKLOADS[name]
    W = synth.workload_weights(w)
    x = synth.workload_activations(w)
    T, alpha = orc.quantize(W.numpy())
    packed, galpha = gpu_pack(W)
    del W
    _say(f"linear workload {w.description} scratch={bw.linear_scratch_bytes(w.M, w.N, w.K)}")
    _linear_check(orc, x, packed, T, alpha, galpha, w.N, w.K, name)


@pytest.mark.parametrize("name", ["1", "2a", "2b", "3a", "3b"])
def test_linear_workloads_lut_fused(orc, name):
    """The lookup-table GEMV with the quantization fused in, at full size."""
    w = synth.WORKLOADS[name]
    W = synth.workload_weights(w)
    x = synth.workload_activations(w)
    T, alpha = orc.quantize(W.numpy())
    packed, galpha = gpu_pack(W)
    del W
    try:
        bw.plan_override("lut_gemv")
        assert bw.linear_scratch_bytes(w.M, w.N, w.K) == 0          # fused
        _say(f"linear workload {w.description} on the LUT path: {bw.plan(w.M, w.N, w.K)}")
        _linear_check(orc, x, packed, T, alpha, galpha, w.N, w.K, name)
    finally:
        bw.plan_override()


def test_grouped_projections_one_call(orc):
    """q/k/v-style group: one sherry_linear over the stacked packed weights
    equals the members' separate calls bit for bit, and the oracle."""
    K = 1152
    Ns = [320, 64, 192]
    Ws = [synth.weights(n, K, 0.02, False, seed=5100 + n) for n in Ns]
    parts = [gpu_pack(W) for W in Ws]
    packed, galpha = bw.concat_packed(parts, Ns, K)
    gstk, astk = gpu_pack(torch.cat(Ws))
    assert torch.equal(packed, gstk) and torch.equal(galpha, astk)
    T, alpha = orc.quantize(torch.cat(Ws).numpy())
    for M in (1, 3, 8):
        x = synth.activations(M, K, seed=5200 + M)
        gy = bw.linear(x.cuda(), packed, galpha, sum(Ns), K)
        sep = torch.cat([bw.linear(x.cuda(), p, a, n, K) for (p, a), n in zip(parts, Ns)], dim=1)
        torch.cuda.synchronize()
        assert np.array_equal(gy.cpu().numpy().view(np.uint32), sep.cpu().numpy().view(np.uint32))
        q, s = orc.act_quant(x.numpy())
        _, y = orc.gemm(q, s, T, alpha)
        assert_y_close(gy.cpu().numpy(), y)


def test_grouped_gate_up_llama7b(orc):
    """gate/up of the LLaMA-7B MLP (2 x [11008, 4096]) stacked into one
    [22016, 4096] matrix: one sherry_linear gives both projections from one
    x, bit-identical to two calls, and the oracle's."""
    K, Ns = 4096, [11008, 11008]
    Ws = [synth.weights(n, K, 0.02, False, seed=5300 + i) for i, n in enumerate(Ns)]
    parts = [gpu_pack(W) for W in Ws]
    packed, galpha = bw.concat_packed(parts, Ns, K)
    T, alpha = orc.quantize(torch.cat(Ws).numpy())
    assert np.array_equal(packed.cpu().numpy(), orc.pack(T)), "stacked codes"
    del Ws
    for M in (1, 4):
        x = synth.activations(M, K, seed=5400 + M)
        _say(f"gate/up M={M}: linear plan {bw.linear_plan(M, sum(Ns), K)}")
        gy = bw.linear(x.cuda(), packed, galpha, sum(Ns), K)
        sep = torch.cat([bw.linear(x.cuda(), p, a, n, K) for (p, a), n in zip(parts, Ns)], dim=1)
        torch.cuda.synchronize()
        assert np.array_equal(gy.cpu().numpy().view(np.uint32), sep.cpu().numpy().view(np.uint32))
        q, s = orc.act_quant(x.numpy())
        _, y = orc.gemm(q, s, T, alpha)
        assert_y_close(gy.cpu().numpy(), y)


# --------------------------------------------------- 2-bit baseline format
@pytest.mark.parametrize("N,K", SHAPES)
def test_pack2_parity(orc, N, K):
    """The 2-bit packer writes the oracle's 2-bit encoding of the same T, and
    the same alpha as the 5-bit packer."""
    W = synth.weights(N, K, 0.1, True, seed=6100 + N)
    T, alpha = orc.quantize(W.numpy())
    p2, a2 = bw.quantize_pack2(W.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(p2.cpu().numpy(), orc.pack2(T))
    assert np.array_equal(a2.cpu().numpy().view(np.uint32), alpha.view(np.uint32))


@pytest.mark.parametrize("rw,splits", [(4, 0), (4, 3), (8, 1), (16, 2)])
@pytest.mark.parametrize("M", [1, 3, 8, 16])
@pytest.mark.parametrize("N,K", [(320, 1152), (64, 128)])
def test_gemm2_parity(orc, rw, splits, M, N, K):
    """The 2-bit product equals the oracle and is bit-identical to the 5-bit
    product of the same weights."""
    W = synth.weights(N, K, 0.02, False, seed=6200 + N + K)
    T, alpha = orc.quantize(W.numpy())
    p5, a5 = gpu_pack(W)
    p2, a2 = bw.quantize_pack2(W.cuda())
    q = synth.int8_uniform(M, K, seed=6300 + M)
    s_x = (torch.rand(M, generator=torch.Generator().manual_seed(M + 3)) * 0.05 + 0.001).float()
    acc, y = orc.gemm(q.numpy(), s_x.numpy(), T, alpha)
    try:
        bw.plan_override("decode_mfma_gemv", rw, 0, splits)
        gy2 = bw.gemm2(q.cuda(), s_x.cuda(), p2, a2, N, K)
        gy5 = bw.gemm(q.cuda(), s_x.cuda(), p5, a5, N, K)
        torch.cuda.synchronize()
    finally:
        bw.plan_override()
    assert np.array_equal(gy2.cpu().numpy().view(np.uint32), gy5.cpu().numpy().view(np.uint32))
    assert_y_close(gy2.cpu().numpy(), y)


@pytest.mark.parametrize("name", ["2a", "3b", "4"])
def test_gemm2_workloads(orc, name):
    w = synth.WORKLOADS[name]
    W = synth.workload_weights(w)
    x = synth.workload_activations(w)
    T, alpha = orc.quantize(W.numpy())
    q, s = orc.act_quant(x.numpy())
    _, y = orc.gemm(q, s, T, alpha)
    p2, a2 = bw.quantize_pack2(W.cuda())
    del W
    gy = bw.gemm2(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda(), p2, a2, w.N, w.K)
    torch.cuda.synchronize()
    assert np.array_equal(p2.cpu().numpy(), orc.pack2(T))
    assert_y_close(gy.cpu().numpy(), y)


# ------------------------------------------- ragged shapes (padded tiles)
RAGGED = [(68, 144), (4, 16), (196, 1040), (452, 272)]


@pytest.fixture(scope="module")
def ragged_cases(orc):
    out = {}
    for (N, K) in RAGGED:
        W = synth.weights(N, K, 0.02, False, seed=8100 + N + K)
        T, alpha = orc.quantize(W.numpy())
        packed, galpha = gpu_pack(W)
        assert np.array_equal(packed.cpu().numpy(), orc.pack(T))
        out[(N, K)] = (T, alpha, packed, galpha)
    return out


RAGGED_PLANS = [(None, 0, 0), ("decode_mfma_gemv", 4, 3), ("decode_mfma_gemv", 16, 1),
                ("decode_mfma_gemv", 8, 2), ("lut_gemv", 0, 0), ("lut_gemv", 1, 3), ("lut_gemv", 8, 2),
                ("decode_mfma", 0, 0), ("decode_mfma", 1, 0), ("decode_mfma", 2, 0)]


@pytest.mark.parametrize("path,rw,splits,M", [
    (p, rw, sp, M) for (p, rw, sp) in RAGGED_PLANS for M in (1, 3, 9, 16, 40, 100, 129)
    if not (p == "lut_gemv" and M > 16)])        # the lookup-table path takes M <= 16
@pytest.mark.parametrize("N,K", RAGGED)
def test_gemm_ragged(orc, ragged_cases, path, rw, splits, M, N, K):
    """N not a multiple of 64 and K not a multiple of 128, on every path: the
    padding rows are not stored and the padding blocks add nothing."""
    T, alpha, packed, galpha = ragged_cases[(N, K)]
    q = synth.int8_uniform(M, K, seed=8300 + M + K)
    s_x = (torch.rand(M, generator=torch.Generator().manual_seed(M + 11)) * 0.05 + 0.001).float()
    acc, y = orc.gemm(q.numpy(), s_x.numpy(), T, alpha)
    try:
        bw.plan_override(path, rw, 0, splits)
        _say(f"ragged gemm {path} rw={rw} splits={splits} M={M} N={N} K={K}: {bw.plan(M, N, K)}")
        gacc = bw.gemm_i32(q.cuda(), packed, N, K)
        gy = bw.gemm(q.cuda(), s_x.cuda(), packed, galpha, N, K)
        torch.cuda.synchronize()
    finally:
        bw.plan_override()
    assert np.array_equal(gacc.cpu().numpy(), acc)
    assert_y_close(gy.cpu().numpy(), y)


@pytest.mark.parametrize("path", [None, "lut_gemv", "decode_mfma"])
@pytest.mark.parametrize("M", [1, 2, 4, 7])
@pytest.mark.parametrize("N,K", RAGGED)
def test_linear_ragged(orc, ragged_cases, path, M, N, K):
    T, alpha, packed, galpha = ragged_cases[(N, K)]
    x = synth.activations(M, K, seed=8500 + M + K, outlier_channels=True)
    try:
        bw.plan_override(path)
        _say(f"ragged linear {path} M={M} N={N} K={K}")
        _linear_check(orc, x, packed, T, alpha, galpha, N, K, f"{path} M={M}")
    finally:
        bw.plan_override()


@pytest.mark.parametrize("M", [1, 5, 16])
@pytest.mark.parametrize("N,K", RAGGED)
def test_gemm2_ragged(orc, M, N, K):
    """The 2-bit format padded the same way; its product equals the 5-bit one."""
    W = synth.weights(N, K, 0.02, False, seed=8700 + N + K)
    T, alpha = orc.quantize(W.numpy())
    p5, a5 = gpu_pack(W)
    p2, a2 = bw.quantize_pack2(W.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(p2.cpu().numpy(), orc.pack2(T))
    q = synth.int8_uniform(M, K, seed=8800 + M)
    s_x = (torch.rand(M, generator=torch.Generator().manual_seed(M + 5)) * 0.05 + 0.001).float()
    acc, y = orc.gemm(q.numpy(), s_x.numpy(), T, alpha)
    gy2 = bw.gemm2(q.cuda(), s_x.cuda(), p2, a2, N, K)
    gy5 = bw.gemm(q.cuda(), s_x.cuda(), p5, a5, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(gy2.cpu().numpy().view(np.uint32), gy5.cpu().numpy().view(np.uint32))
    assert_y_close(gy2.cpu().numpy(), y)
