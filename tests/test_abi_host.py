"""Host-only checks of the C ABI: the library loads, exports every function
include/sherry.h declares, and rejects bad arguments before any HIP call
(so these run without a GPU)."""

import ctypes
import os
import re

import numpy as np
import pytest

import bit_weight_amd as bw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sherry.h")

OK, NULL, SHAPE, ALIGN, WS = 0, -1, -2, -3, -4
FAKE = 0x10000        # 64 KiB-aligned dummy device address (never dereferenced)


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sherry_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    L = bw.lib()
    names = _declared()
    assert "sherry_gemm" in names and "sherry_quantize_pack" in names
    for name in names:
        assert hasattr(L, name), name


def test_status_strings():
    L = bw.lib()
    for code, name in bw.STATUS.items():
        assert L.sherry_status_string(code).decode().startswith(name)
    assert L.sherry_status_string(99).decode() == "SHERRY_ERR_UNKNOWN"
    # every status the header declares has a name in the binding
    declared = {int(v): k for k, v in re.findall(r"\b(SHERRY_\w+)\s*=\s*(-?\d+)", open(HEADER).read())}
    assert declared == bw.STATUS
    assert "workspace is left zero" in L.sherry_status_string(-7).decode()


def test_packed_bytes():
    assert bw.packed_bytes(4096, 4096) == 4096 * 4096 * 5 // 32 == 2_621_440
    assert bw.packed_bytes(28672, 8192) == 36_700_160
    assert bw.packed_bytes(14336, 4096) == 9_175_040
    assert bw.packed_bytes(4096, 11008) == 7_045_120
    assert bw.packed_bytes(256, 256) == 10_240
    assert bw.packed_bytes(64, 100) == 0          # K % 16 != 0
    assert bw.packed_bytes(66, 128) == 0          # N % 4 != 0
    # ragged shapes are padded to whole 64 x 128 tiles of 1280 bytes
    assert bw.packed_bytes(68, 144) == 2 * 2 * 1280
    assert bw.packed_bytes(4, 16) == 1280
    assert bw.lib().sherry_packed2_bytes(68, 144) == 2 * 2 * 2048


def test_sizes_at_the_int64_extremes_are_rejected():
    """Size queries and plans return 0 / SHERRY_ERR_SHAPE for sizes near the
    int64 limits and for negative ones, without overflowing on the way (the
    sanitizer build of this library runs this test too)."""
    L = bw.lib()
    extremes = [2 ** 31 - 1, 2 ** 31, 2 ** 32 + 128, 2 ** 40, 2 ** 62, 2 ** 63 - 1, -1, -(2 ** 63)]
    out = [ctypes.c_int() for _ in range(6)]
    refs = [ctypes.byref(v) for v in out]
    for a in extremes:
        for b in (64, 128, a):
            assert L.sherry_packed_bytes(a, b) == 0 and L.sherry_packed_bytes(b, a) == 0, (a, b)
            assert L.sherry_packed2_bytes(a, b) == 0 and L.sherry_packed2_bytes(b, a) == 0, (a, b)
            assert L.sherry_workspace_bytes(8, a, b) == 0 and L.sherry_workspace_bytes(a, 64, 128) == 0
            assert L.sherry_linear_scratch_bytes(a, b, 128) == 0, (a, b)
            assert L.sherry_gemm_plan(a, 64, 128, *refs[:5]) == SHAPE, (a, b)
            assert L.sherry_gemm_plan(8, a, b, *refs[:5]) == SHAPE, (a, b)
            assert L.sherry_linear_plan(a, b, 128, *refs) == SHAPE, (a, b)
            assert _gemm(M=a, N=b, K=128) == SHAPE and _gemm(M=1, N=64, K=a) == SHAPE, (a, b)


def test_plan_dispatch_rule():
    for M in (1, 2, 3, 8, 15, 16):
        assert bw.plan(M, 4096, 4096)["path"] in ("lut_gemv", "decode_mfma_gemv")
    for M in (17, 31, 64):
        p = bw.plan(M, 4096, 4096)
        assert p["path"] == "decode_mfma_gemv" and p["block"] <= 512   # at most 8 waves
    for M in (65, 100, 128):   # the prefill's 64-token tiles with 4 k-phases
        assert bw.plan(M, 4096, 4096)["path"] == "decode_mfma"
        assert bw.workspace_bytes(M, 4096, 4096) == 0
    for M in (65, 88):         # small grid, long K: launches of 64 tokens on the GEMV
        assert bw.plan(M, 4096, 14336)["path"] == "decode_mfma_gemv"
        assert bw.workspace_bytes(M, 4096, 14336) in (0, 64 * 4096 * 8)
    for M in (129, 130, 512):
        assert bw.plan(M, 4096, 4096)["path"] == "decode_mfma"
    p = bw.plan(1, 4096, 4096)
    assert p["block"] in (256, 512, 1024) and p["grid"] >= 64
    # the workspace holds one 64-bit accumulator per output when split
    if p["splits"] > 1:
        assert bw.workspace_bytes(1, 4096, 4096) == 4096 * 8
    assert bw.workspace_bytes(512, 14336, 4096) == 0


def test_prefill_tile_height_rule():
    """The prefill GEMM takes the first tile shape whose grid fits the GPU in
    one round (<= 256 tiles): 64 tokens x 128 weight rows (4 k-phases), then
    128 x 128 (4 k-phases), then 64 x 256 (2 k-phases), else 128 x 256
    (2 k-phases).  Between 65 and 128 tokens it is the default, except on a
    prefill grid of at most 64 workgroups whose waves take more than 12
    k-tiles (up to M = 80), 18 (up to 96) or 24 (up to 128): there the
    64-token GEMV launches stay."""
    # LDS per workgroup of the four kernels, by (tokens, weight rows)
    lds = {(64, 256): 78080, (64, 128): 139520, (128, 256): 107016, (128, 128): 139792}
    def tiles(M, N, bm, bn):
        return -(-M // bm) * -(-N // bn)
    for M, N in [(129, 14336), (200, 14336), (256, 14336), (257, 14336), (512, 14336),
                 (128, 4096), (136, 4096), (300, 4096), (1000, 4096), (1100, 4096), (129, 65536),
                 (129, 28672), (384, 8192)]:
        p = bw.plan(M, N, 4096)
        assert p["path"] == "decode_mfma"
        bm, bn = next((s for s in ((64, 128), (128, 128), (64, 256)) if tiles(M, N, *s) <= 256),
                      (128, 256))
        assert p["lds_bytes"] == lds[(bm, bn)], (M, N)
        assert p["grid"] == 8 * -(-(-(-N // bn)) // 8) * -(-M // bm), (M, N)
    # 64 < M <= 128: the prefill, but the GEMV launches on a small grid with long K
    for M, N, K, want in [(65, 14336, 4096, "decode_mfma"), (96, 14336, 4096, "decode_mfma"),
                          (128, 14336, 4096, "decode_mfma"), (65, 4096, 4096, "decode_mfma"),
                          (100, 4096, 4096, "decode_mfma"), (65, 28672, 8192, "decode_mfma"),
                          (80, 4096, 14336, "decode_mfma_gemv"), (88, 4096, 14336, "decode_mfma_gemv"),
                          (128, 4096, 14336, "decode_mfma_gemv"), (96, 4096, 11008, "decode_mfma_gemv"),
                          (97, 4096, 11008, "decode_mfma"), (80, 4096, 8192, "decode_mfma_gemv"),
                          (81, 4096, 8192, "decode_mfma"), (65, 4096, 6144, "decode_mfma"),
                          (65, 4096, 6272, "decode_mfma_gemv"), (65, 5504, 8192, "decode_mfma"),
                          (65, 1024, 8192, "decode_mfma_gemv"), (88, 1024, 8192, "decode_mfma")]:
        assert bw.plan(M, N, K)["path"] == want, (M, N, K)


def test_plan_override_changes_plan_and_workspace():
    try:
        base = bw.plan(1, 4096, 4096)
        bw.plan_override("lut_gemv", rw=2, ch=2, splits=8)
        p = bw.plan(1, 4096, 4096)
        assert p["path"] == "lut_gemv"
        assert p["splits"] == 8 and p["grid"] == 32 * 8
        assert bw.workspace_bytes(1, 4096, 4096) == 4096 * 8
        bw.plan_override("lut_gemv", splits=1)
        assert bw.workspace_bytes(1, 4096, 4096) == 0
        bw.plan_override("lut_gemv", rw=8, splits=4)       # 4 row tiles x 2 waves
        p = bw.plan(16, 4096, 4096)
        assert p["block"] == 512 and p["grid"] == 16 * 4 and p["lds_bytes"] == 2 * 32 * 8 * 32 * 4
        bw.plan_override("lut_gemv", rw=8, splits=32)      # 1-k-tile splits: 4 waves instead
        p = bw.plan(16, 4096, 4096)
        assert p["block"] == 256 and p["grid"] == 16 * 32
        bw.plan_override("decode_mfma_gemv", rw=4, splits=4)
        p = bw.plan(3, 4096, 4096)
        assert p["path"] == "decode_mfma_gemv" and p["grid"] == 64 * 4 and p["block"] == 256
        bw.plan_override("decode_mfma_gemv", rw=16, splits=2)
        p = bw.plan(3, 4096, 4096)
        assert p["grid"] == 64 * 2 and p["block"] == 1024
        assert bw.workspace_bytes(3, 4096, 4096) == 3 * 4096 * 8
        bw.plan_override("decode_mfma")
        assert bw.plan(2, 4096, 4096)["path"] == "decode_mfma"
        assert bw.workspace_bytes(2, 4096, 4096) == 0
        assert bw.plan(40, 4096, 4096)["path"] == "decode_mfma"   # forced on 16 < M <= 64 too
        assert bw.plan(100, 4096, 4096)["path"] == "decode_mfma"
        assert bw.plan(200, 4096, 4096)["path"] == "decode_mfma"
        bw.plan_override("lut_gemv")
        assert bw.plan(40, 4096, 4096)["path"] == "decode_mfma_gemv"   # no table path above 16
        bw.plan_override("decode_mfma_gemv", rw=16)
        assert bw.plan(40, 4096, 4096)["block"] == 512
        assert bw.plan(100, 4096, 4096)["path"] == "decode_mfma_gemv"
        assert bw.plan(129, 4096, 4096)["path"] == "decode_mfma"
        with pytest.raises(bw.SherryError):
            bw.plan_override("lut_gemv", rw=3)
        assert bw.lib().sherry_gemm_plan_override(3, 0, 0, 0) == SHAPE
        assert bw.lib().sherry_gemm_plan_override(-2, 0, 0, 0) == SHAPE
    finally:
        bw.plan_override()
    assert bw.plan(1, 4096, 4096) == base


def _gemm(**kw):
    a = dict(x=FAKE, s=FAKE, p=FAKE, al=FAKE, y=FAKE, M=1, N=64, K=128, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return bw.lib().sherry_gemm(a["x"], a["s"], a["p"], a["al"], a["y"], a["M"], a["N"], a["K"],
                                a["ws"], a["wsb"], None)


def test_gemm_null_pointers():
    for k in ("x", "s", "p", "al", "y"):
        assert _gemm(**{k: None}) == NULL, k
    assert bw.lib().sherry_gemm_i32(FAKE, FAKE, None, 1, 64, 128, FAKE, 1 << 30, None) == NULL


@pytest.mark.parametrize("M,N,K", [(0, 64, 128), (1, 0, 128), (1, 64, 0), (1, 64, 100),
                                   (1, 64, 132), (1, 65, 128), (1, 98, 128), (-1, 64, 128),
                                   (1, 64, (1 << 20) + 128), (1 << 21, 64, 128)])
def test_gemm_bad_shapes(M, N, K):
    assert _gemm(M=M, N=N, K=K) == SHAPE


def test_gemm_misaligned():
    assert _gemm(x=FAKE + 4) == ALIGN
    assert _gemm(p=FAKE + 8) == ALIGN
    assert _gemm(y=FAKE + 2) == ALIGN
    # outputs are 16-byte aligned (the prefill GEMM stores 16 bytes per lane)
    assert _gemm(y=FAKE + 4) == ALIGN
    assert _gemm(y=FAKE + 8) == ALIGN
    assert _gemm(s=FAKE + 1) == ALIGN
    assert _gemm(al=FAKE + 2) == ALIGN


def test_gemm_workspace_checks():
    M, N, K = 1, 4096, 4096
    need = bw.workspace_bytes(M, N, K)
    assert need > 0
    assert _gemm(M=M, N=N, K=K, ws=None) == WS
    assert _gemm(M=M, N=N, K=K, wsb=need - 1) == WS
    assert _gemm(M=M, N=N, K=K, ws=FAKE + 64) == ALIGN


def test_quantize_pack_and_act_validation():
    L = bw.lib()
    assert L.sherry_quantize_pack(None, 64, 128, FAKE, FAKE, None) == NULL
    assert L.sherry_quantize_pack(FAKE, 64, 100, FAKE, FAKE, None) == SHAPE
    assert L.sherry_quantize_pack(FAKE + 4, 64, 128, FAKE, FAKE, None) == ALIGN
    assert L.sherry_quantize_pack(FAKE, 64, 128, FAKE + 4, FAKE, None) == ALIGN
    assert L.sherry_quantize_act(FAKE, 1, 128, None, FAKE, None) == NULL
    assert L.sherry_quantize_act(FAKE, 0, 128, FAKE, FAKE, None) == SHAPE
    assert L.sherry_quantize_act(FAKE, 1, 6, FAKE, FAKE, None) == SHAPE
    assert L.sherry_quantize_act(FAKE + 8, 1, 128, FAKE, FAKE, None) == ALIGN


def test_python_wrapper_rejects_cpu_and_noncontiguous():
    import torch
    with pytest.raises(RuntimeError):
        bw.quantize_pack(torch.zeros(64, 128))
    with pytest.raises(RuntimeError):
        bw.quantize_act(torch.zeros(1, 128))


def test_linear_plan():
    """sherry_linear's plan: the product's, except that the fused form on the
    matrix-core GEMV with a K-split takes twice the waves per row tile and,
    from 8 K-splits on, half the splits; it keeps a K-split, so it needs the
    product's workspace."""
    for M, N, K in [(1, 4096, 4096), (4, 4096, 4096), (1, 4096, 11008), (1, 11008, 4096),
                    (1, 256, 256), (16, 4096, 4096), (512, 14336, 4096), (2, 4096, 11008)]:
        g, lp = bw.plan(M, N, K), bw.linear_plan(M, N, K)
        assert lp["fused"] == (bw.linear_scratch_bytes(M, N, K) == 0)
        if not lp["fused"] or g["path"] != "decode_mfma_gemv" or g["splits"] == 1:
            assert {k: v for k, v in lp.items() if k != "fused"} == g, (M, N, K)
            continue
        assert lp["path"] == g["path"] and lp["splits"] > 1
        assert lp["block"] == min(1024, 2 * g["block"])
        want = g["splits"] // 2 if g["splits"] >= 8 else g["splits"]
        KT = (K + 127) // 128
        assert lp["splits"] == -(-KT // -(-KT // want))            # as the product rounds splits
        assert lp["grid"] == (N + 63) // 64 * lp["splits"]
        # fusable: at most 32 k-tiles per split held in LDS as int8
        assert -(-KT // lp["splits"]) <= 32
    # LLaMA-7B down projection (K=11008): 8 splits of 4 waves -> 4 splits of 8 waves
    g, lp = bw.plan(1, 4096, 11008), bw.linear_plan(1, 4096, 11008)
    assert (g["splits"], g["block"]) == (8, 256) and (lp["splits"], lp["block"]) == (4, 512)
    # an override of waves or splits keeps the product's plan for the fused form
    try:
        bw.plan_override("decode_mfma_gemv", rw=4, splits=4)
        lp = bw.linear_plan(1, 4096, 4096)
        assert (lp["block"], lp["splits"], lp["fused"]) == (256, 4, True)
    finally:
        bw.plan_override()
    assert bw.lib().sherry_linear_plan(1, 98, 128, None, None, None, None, None, None) == SHAPE


def test_linear_scratch_and_validation():
    L = bw.lib()
    # fused (M <= 4, M*K <= 16384): no scratch
    assert bw.linear_scratch_bytes(1, 4096, 4096) == 0
    try:   # the lookup-table path fuses the quantization under the same limits
        bw.plan_override("lut_gemv")
        assert bw.linear_scratch_bytes(1, 4096, 4096) == 0
        assert bw.linear_scratch_bytes(4, 4096, 4096) == 0
        assert bw.linear_scratch_bytes(5, 4096, 4096) == 5 * 4096 + 256
        assert bw.linear_scratch_bytes(2, 4096, 11008) == 2 * 11008 + 256   # M*K > 16384
    finally:
        bw.plan_override()
    # not fused: q [M,K] + s_x [M], each rounded up to 256 bytes
    assert bw.linear_scratch_bytes(16, 4096, 4096) == 16 * 4096 + 256
    assert bw.linear_scratch_bytes(512, 14336, 4096) == 512 * 4096 + 2048
    assert bw.linear_scratch_bytes(1, 64, 100) == 0
    base = dict(x=FAKE, p=FAKE, al=FAKE, y=FAKE, M=1, N=64, K=128, ws=FAKE, wsb=1 << 30,
                sc=FAKE, scb=1 << 30, st=None)
    args = lambda **kw: [kw.get(k, v) for k, v in base.items()]
    for k in ("x", "p", "al", "y"):
        assert L.sherry_linear(*args(**{k: None})) == NULL, k
    assert L.sherry_linear(*args(K=100)) == SHAPE
    assert L.sherry_linear(*args(N=98)) == SHAPE
    assert L.sherry_linear(*args(x=FAKE + 4)) == ALIGN
    assert L.sherry_linear(*args(p=FAKE + 8)) == ALIGN
    M, N, K = 8, 4096, 4096            # unfused (M > 4) and split along K
    need_ws, need_sc = bw.workspace_bytes(M, N, K), bw.linear_scratch_bytes(M, N, K)
    assert need_ws > 0 and need_sc > 0
    assert L.sherry_linear(*args(M=M, N=N, K=K, ws=None)) == WS
    assert L.sherry_linear(*args(M=M, N=N, K=K, wsb=need_ws - 1)) == WS
    assert L.sherry_linear(*args(M=M, N=N, K=K, sc=None)) == WS
    assert L.sherry_linear(*args(M=M, N=N, K=K, scb=need_sc - 1)) == WS
    assert L.sherry_linear(*args(M=M, N=N, K=K, sc=FAKE + 64)) == ALIGN


def test_two_bit_baseline_sizes_and_validation():
    L = bw.lib()
    assert L.sherry_packed2_bytes(4096, 4096) == 4096 * 4096 // 4
    assert L.sherry_packed2_bytes(64, 100) == 0
    assert L.sherry_gemm2_workspace_bytes(17, 4096, 4096) == 0          # decode shapes only
    assert L.sherry_quantize_pack2(None, 64, 128, FAKE, FAKE, None) == NULL
    assert L.sherry_quantize_pack2(FAKE, 64, 100, FAKE, FAKE, None) == SHAPE
    assert L.sherry_quantize_pack2(FAKE, 64, 128, FAKE + 4, FAKE, None) == ALIGN
    g2 = lambda **kw: L.sherry_gemm2(*[kw.get(k, v) for k, v in dict(
        x=FAKE, s=FAKE, p=FAKE, al=FAKE, y=FAKE, M=1, N=64, K=128, ws=FAKE, wsb=1 << 30,
        st=None).items()])
    for k in ("x", "s", "p", "al", "y"):
        assert g2(**{k: None}) == NULL, k
    assert g2(M=17) == SHAPE
    assert g2(K=100) == SHAPE
    assert g2(p=FAKE + 8) == ALIGN
    need = L.sherry_gemm2_workspace_bytes(1, 4096, 4096)
    assert need > 0
    assert g2(N=4096, K=4096, ws=None) == WS
    assert g2(N=4096, K=4096, wsb=need - 1) == WS


def _random_shape_rule_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice([rng.integers(1, 17), rng.integers(17, 129), rng.integers(129, 4097),
                            rng.integers(1, 1 << 20)]))
        N = 4 * int(rng.choice([rng.integers(1, 1025), rng.integers(1, 1 << 18)]))
        K = 16 * int(rng.choice([rng.integers(1, 1025), rng.integers(1, 1 << 16)]))
        out.append((M, N, K))
    return out


def test_plan_invariants_over_random_shapes():
    """Host planning over 2000 seeded shapes of the whole shape rule: the path
    rule, launch sizes that fit the hardware, K-splits that are all non-empty,
    a workspace that holds one 64-bit cell per output of a launch whenever K
    is split, and a fused sherry_linear only within its limits."""
    for M, N, K in _random_shape_rule_shapes(2000, 4242):
        p, lp = bw.plan(M, N, K), bw.linear_plan(M, N, K)
        KT, RT = -(-K // 128), -(-N // 64)
        assert p["block"] in (256, 512, 1024) and 1 <= p["grid"] < 2 ** 31, (M, N, K, p)
        assert 0 < p["lds_bytes"] <= 160 * 1024, (M, N, K, p)
        if M <= 16:
            assert p["path"] in ("lut_gemv", "decode_mfma_gemv"), (M, N, K, p)
        elif M <= 64:
            assert p["path"] == "decode_mfma_gemv", (M, N, K, p)
        elif M > 128 or -(-N // 128) > 32:   # past M = 128, or a prefill grid over 64
            assert p["path"] == "decode_mfma", (M, N, K, p)
        ws = bw.workspace_bytes(M, N, K)
        if p["path"] == "decode_mfma":
            assert p["splits"] == 1 and ws == 0
            # 64- or 128-token tiles of 256 or 128 weight rows (2 or 4 k-phases)
            bm, bn = {78080: (64, 256), 139520: (64, 128), 107016: (128, 256),
                      139792: (128, 128)}[p["lds_bytes"]]
            assert p["grid"] == 8 * -(-(-(-N // bn)) // 8) * -(-M // bm), (M, N, K, p)
            # 4 k-phases only when the real tiles (the grid less its XCD padding) fit one round
            assert -(-M // bm) * -(-N // bn) <= 256 or bn == 256, (M, N, K, p)
            continue
        s = p["splits"]
        assert 1 <= s <= KT and -(-KT // -(-KT // s)) == s, (M, N, K, p)   # no empty split
        if p["path"] == "lut_gemv":
            assert p["grid"] % s == 0 and p["grid"] // s <= RT
        else:
            assert p["grid"] == RT * s, (M, N, K, p)
        assert ws == (min(M, 64) * N * 8 if s > 1 else 0), (M, N, K, p, ws)
        fused = lp["fused"]
        assert fused == (bw.linear_scratch_bytes(M, N, K) == 0)
        if fused:
            assert M <= 4 and M * K <= 16384, (M, N, K, lp)
            assert -(-KT // lp["splits"]) <= 32 and lp["block"] <= 1024
            assert bw.workspace_bytes(M, N, K) >= (M * N * 8 if lp["splits"] > 1 else 0)


# ------------------------------------------------ sherry_gemm_noalloc (host)
def _noalloc(**kw):
    a = dict(x=FAKE, s=FAKE, p=FAKE, al=FAKE, y=FAKE, M=1, N=64, K=128)
    a.update(kw)
    return bw.lib().sherry_gemm_noalloc(a["x"], a["s"], a["p"], a["al"], a["y"], a["M"], a["N"], a["K"],
                                        None)


def test_noalloc_argument_errors():
    for k in ("x", "s", "p", "al", "y"):
        assert _noalloc(**{k: None}) == NULL, k
    assert _noalloc(M=0) == SHAPE and _noalloc(K=100) == SHAPE and _noalloc(N=65) == SHAPE
    assert _noalloc(x=FAKE + 4) == ALIGN and _noalloc(y=FAKE + 4) == ALIGN and _noalloc(p=FAKE + 8) == ALIGN


def test_noalloc_rejects_shapes_beyond_its_static_scratch():
    """The static split-K scratch holds 8 MiB per GPU: a plan whose cells
    need more is refused on the host, before anything is enqueued."""
    assert bw.NOALLOC_SCRATCH_BYTES == 8 << 20
    try:
        # force a K-split on a wide shape: 32 x 65536 cells of 8 bytes = 16 MiB
        bw.plan_override("decode_mfma_gemv", 4, 0, 2)
        assert bw.workspace_bytes(32, 65536, 256) == 16 << 20
        assert _noalloc(M=32, N=65536, K=256) == WS
        # 16 x 65536 cells are exactly 8 MiB: accepted by the size check (the
        # call then needs the device, which this host has not)
        assert bw.workspace_bytes(16, 65536, 256) == 8 << 20
        assert _noalloc(M=16, N=65536, K=256) not in (WS, SHAPE, ALIGN, NULL)
    finally:
        bw.plan_override()


# ------------------------------------------------ diagnostics (host checks)
def test_probe_argument_errors():
    """The benchmark's probes reject bad arguments before any HIP call."""
    L = bw.lib()
    assert L.sherry_probe_read(None, 1024, FAKE, 256, 256, 4, None) == NULL
    assert L.sherry_probe_read(FAKE, 1024, None, 256, 256, 4, None) == NULL
    for nbytes, grid, block, unroll in ((0, 256, 256, 4), (1000, 256, 256, 4), (1024, 0, 256, 4),
                                        (1024, 256, 100, 4), (1024, 256, 2048, 4), (1024, 256, 256, 3)):
        assert L.sherry_probe_read(FAKE, nbytes, FAKE, grid, block, unroll, None) == SHAPE
    assert L.sherry_probe_read(FAKE + 4, 1024, FAKE, 256, 256, 4, None) == ALIGN
    assert L.sherry_probe_decode(16, None, 256, 256, None) == NULL
    for iters, grid, block in ((0, 256, 256), ((1 << 20) + 1, 256, 256), (16, 0, 256), (16, 256, 96),
                               (16, 256, 2048)):
        assert L.sherry_probe_decode(iters, FAKE, grid, block, None) == SHAPE
    assert L.sherry_probe_decode(16, FAKE + 2, 256, 256, None) == ALIGN
    # 16 groups of 4 codes per thread and trip
    assert L.sherry_probe_decode_codes(256, 256, 1024) == 256 * 256 * 1024 * 16 * 4
    assert L.sherry_probe_decode_codes(0, 256, 1024) == 0
