"""Pins for the CPU oracle against what the Sherry page and mathematics fix.

Each test checks the oracle against something other than itself: brute force
over all candidates, exhaustive joint search, a numeric line search, the
page's worked block, hand-derived golden bytes, exact library arithmetic
(torch float64 matmul is exact on these integers), invariants stated on the
page (values in {-1,0,1}; exactly 3 nonzeros per block), or closed forms.
"""

import itertools
import os

import numpy as np
import pytest
import torch

from bit_weight_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# All 32 blocks with exactly three nonzeros in {-1,+1}, enumerated here
# independently of the oracle's pattern table.
ALL32 = np.array([v for v in itertools.product((-1, 0, 1), repeat=4)
                  if sum(1 for e in v if e != 0) == 3], dtype=np.int8)


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            out.setdefault(key.strip(), []).append(val.split())
    return out


def test_all32_has_32():
    assert ALL32.shape == (32, 4)


def test_patterns_are_canonical(orc):
    seen = set()
    for p in range(16):
        v = orc.pattern(p)
        nz = v[v != 0]
        assert nz.size == 3 and set(v.tolist()) <= {-1, 0, 1}
        assert nz[0] == 1, "canonical pattern: first nonzero is +1"
        seen.add(tuple(v.tolist()))
    assert len(seen) == 16


def test_codes_are_a_bijection_onto_all32(orc):
    dec = np.stack([orc.decode_code(c) for c in range(32)])
    assert {tuple(r) for r in dec.tolist()} == {tuple(r) for r in ALL32.tolist()}
    for c in range(32):
        assert orc.encode_block(dec[c]) == c
        # sign bit is the lowest bit: code 2p+1 is the negation of code 2p
        if c % 2 == 0:
            assert np.array_equal(dec[c + 1], -dec[c])
            assert np.array_equal(dec[c], orc.pattern(c // 2))


def test_encode_rejects_non_34_blocks(orc):
    for bad in ([0, 0, 1, 1], [1, 1, 1, 1], [2, 0, 1, 1], [0, 1, -1, 3], [0, 0, 0, 0]):
        assert orc.encode_block(bad) == -1


def test_worked_block_from_page(orc):
    g = _golden("worked_block.txt")
    block = np.array([float(v) for v in g["block"][0]], np.float32)
    W = np.tile(block, 32)[None, :]          # one row, K = 128
    T, alpha = orc.quantize(W)
    assert np.array_equal(T[0, :4], block.astype(np.int8))
    assert alpha[0] == np.float32(float(g["alpha"][0][0]))
    c = orc.encode_block(block.astype(np.int8))
    assert c == int(g["code"][0][0])
    assert c == 2 * int(g["p"][0][0]) + int(g["s"][0][0])


def _random_blocks(n, seed):
    rng = np.random.default_rng(seed)
    w = rng.normal(0, 1, size=(n, 4)).astype(np.float32)
    # ties and special values: repeated magnitudes, zeros, spikes
    w[: n // 10] = np.round(w[: n // 10])
    w[n // 10: n // 5] = rng.choice([-5.0, 5.0, 0.0, 0.1, -0.1], size=(n // 10, 4))
    return w


def test_quantizer_attains_bruteforce_optimum_per_block(orc):
    w = _random_blocks(20000, 1)
    T, _ = orc.quantize(w.reshape(-1, 4))            # each block its own row
    assert np.all((T != 0).sum(1) == 3)
    w64 = w.astype(np.float64)
    best = (w64 @ ALL32.T.astype(np.float64)).max(1)
    got = (w64 * T).sum(1)
    np.testing.assert_allclose(got, best, rtol=0, atol=1e-12)


def test_quantizer_tie_rule_drops_lowest_index_minimum(orc):
    w = _random_blocks(5000, 2)
    T, _ = orc.quantize(w)
    a = np.abs(w)
    zero_pos = np.argmax(T == 0, axis=1)
    first_min = np.argmax(a == a.min(1, keepdims=True), axis=1)
    assert np.array_equal(zero_pos, first_min)


def test_equal_spikes_and_signed_zero(orc):
    T, alpha = orc.quantize(np.array([[5.0, -5.0, 5.0, -5.0]], np.float32))
    assert T.tolist() == [[0, -1, 1, -1]] and alpha[0] == 5.0
    T, alpha = orc.quantize(np.array([[0.0, -0.0, -0.0, -0.0]], np.float32))
    assert T.tolist() == [[0, 1, 1, 1]] and alpha[0] == 0.0


@pytest.mark.parametrize("B,rows", [(2, 40), (3, 4)])
def test_joint_exhaustive_search_tiny_rows(orc, B, rows):
    """Per-row alpha: the closed form attains the minimum of ||W - aT||^2 over
    every combination of exactly-3-nonzero blocks, each with its best a."""
    rng = np.random.default_rng(10 + B)
    combos = np.array([np.concatenate(c) for c in itertools.product(ALL32, repeat=B)],
                      dtype=np.float64)                     # [32^B, 4B]
    tt = (combos * combos).sum(1)                           # = 3B
    for _ in range(rows):
        W = rng.normal(0, 1, size=(1, 4 * B)).astype(np.float32)
        T, alpha = orc.quantize(W)
        w = W[0].astype(np.float64)
        wt = combos @ w
        err_min = (w @ w - wt * wt / tt).min()
        err_or = ((w - float(alpha[0]) * T[0]) ** 2).sum()
        assert err_or <= err_min + 1e-6 * (w @ w)


def test_alpha_matches_numeric_line_search(orc):
    rng = np.random.default_rng(3)
    W = rng.normal(0, 0.02, size=(8, 256)).astype(np.float32)
    T, alpha = orc.quantize(W)
    for n in range(8):
        w, t = W[n].astype(np.float64), T[n].astype(np.float64)
        f = lambda a: ((w - a * t) ** 2).sum()
        lo, hi = 0.0, float(np.abs(w).max())
        gr = (np.sqrt(5) - 1) / 2
        for _ in range(200):
            a1, a2 = hi - gr * (hi - lo), lo + gr * (hi - lo)
            if f(a1) < f(a2):
                hi = a2
            else:
                lo = a1
        assert abs(alpha[n] - (lo + hi) / 2) <= 1e-6 * alpha[n]


def test_pack_roundtrip_and_size(orc):
    rng = np.random.default_rng(4)
    for N, K in [(64, 128), (128, 384), (192, 256)]:
        codes = rng.integers(0, 32, size=(N, K // 4))
        T = ALL32[codes].reshape(N, K)
        P = orc.pack(T)
        assert P.size == N * K * 5 // 32
        assert np.array_equal(orc.unpack(P, N, K), T)


def test_pack_golden_layout(orc):
    g = _golden("packed_layout_64x128.txt")
    T = np.tile(np.array([0, 1, 1, 1], np.int8), (64, 32))
    for row, blk in ([int(a) for a in v] for v in g["special"]):
        T[row, 4 * blk: 4 * blk + 4] = [-1, 0, 1, -1]
    want = np.zeros(64 * 128 * 5 // 32, np.uint8)
    for off, val in g["byte"]:
        want[int(off)] = int(val, 16)
    assert np.array_equal(orc.pack(T), want)


def test_lut_equals_direct_dot_and_negation_symmetry(orc):
    q = synth.int8_uniform(3, 64, seed=5).numpy()
    L = orc.lut(q)
    for m in range(3):
        for seg in range(16):
            x = q[m, 4 * seg: 4 * seg + 4].astype(np.int64)
            for v in ALL32:
                c = orc.encode_block(v)
                p, s = c >> 1, c & 1
                val = -L[m, seg, p] if s else L[m, seg, p]
                assert val == int((v.astype(np.int64) * x).sum())


def test_gemm_int32_equals_exact_float64_matmul(orc):
    rng = np.random.default_rng(6)
    q = synth.int8_uniform(7, 512, seed=6).numpy()
    T = ALL32[rng.integers(0, 32, size=(96, 128))].reshape(96, 512)
    acc = orc.gemm_i32(q, T)
    ref = torch.from_numpy(q).double() @ torch.from_numpy(T).double().T
    assert np.array_equal(acc, ref.numpy().astype(np.int64))


def test_gemm_one_hot_and_constant_rows(orc):
    rng = np.random.default_rng(7)
    K = 256
    T = ALL32[rng.integers(0, 32, size=(64, K // 4))].reshape(64, K)
    for k in (0, 1, 131, K - 1):
        e = np.zeros((1, K), np.int8)
        e[0, k] = 1
        assert np.array_equal(orc.gemm_i32(e, T)[0], T[:, k].astype(np.int32))
    c = np.full((1, K), 127, np.int8)
    assert np.array_equal(orc.gemm_i32(c, T)[0], 127 * T.astype(np.int32).sum(1))
    c = np.full((1, K), -128, np.int8)
    assert np.array_equal(orc.gemm_i32(c, T)[0], -128 * T.astype(np.int32).sum(1))


def test_epilogue_within_two_ulp_of_exact(orc):
    rng = np.random.default_rng(8)
    acc = rng.integers(-1_000_000, 1_000_000, size=(5, 300)).astype(np.int32)
    s = rng.uniform(0.001, 0.1, size=5).astype(np.float32)
    a = rng.uniform(0.001, 0.1, size=300).astype(np.float32)
    y = orc.epilogue(acc, s, a)
    exact = (acc.astype(np.float64) * s[:, None].astype(np.float64)
             * a[None, :].astype(np.float64)).astype(np.float32)
    ulp = np.spacing(np.abs(exact))
    assert np.all(np.abs(y.astype(np.float64) - exact) <= 2 * ulp)


def test_act_quant_golden_ties(orc):
    g = _golden("act_quant_ties.txt")
    x = np.array([[float(v) for v in g["x"][0]]], np.float32)
    q, s = orc.act_quant(x)
    assert s[0] == np.float32(float(g["s"][0][0]))
    assert q[0].tolist() == [int(v) for v in g["q"][0]]


def test_act_quant_properties(orc):
    x = synth.activations(6, 1000, seed=9, outlier_channels=True).numpy()
    x[5] = 0.0
    q, s = orc.act_quant(x)
    assert s[5] == 1.0 and not q[5].any()
    for m in range(5):
        amax = np.abs(x[m]).max()
        assert s[m] == np.float32(amax / np.float32(127.0))
        assert q[m].min() >= -127 and q[m].max() <= 127
        assert abs(int(q[m][np.argmax(np.abs(x[m]))])) == 127
        err = np.abs(x[m].astype(np.float64) - q[m] * np.float64(s[m]))
        assert np.all(err <= 0.5 * s[m] * (1 + 1e-5))


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_every_block_has_three_nonzeros_on_workload_data(orc, name):
    w = synth.WORKLOADS[name]
    W = synth.weights(64, w.K, w.w_std, w.w_spikes, w.seed_w).numpy()
    T, alpha = orc.quantize(W)
    # the page's diagnostic: histogram over bins [-1.5,-0.5,0.5,1.5] holds all
    hist, _ = np.histogram(T, bins=[-1.5, -0.5, 0.5, 1.5])
    assert hist.sum() == T.size
    assert np.all((T.reshape(64, -1, 4) != 0).sum(-1) == 3)
    assert np.all(alpha > 0)


def test_packed_layout_stacks_along_n(orc):
    """Weights stacked along N give stacked packed bytes (row groups are
    stored one after another), which is what grouping projections relies on."""
    rng = np.random.default_rng(31)
    T1 = orc.quantize(rng.normal(0, 0.02, (192, 384)).astype(np.float32))[0]
    T2 = orc.quantize(rng.normal(0, 0.02, (64, 384)).astype(np.float32))[0]
    both = orc.pack(np.concatenate([T1, T2]))
    assert np.array_equal(both, np.concatenate([orc.pack(T1), orc.pack(T2)]))


# ------------------------------------------------ 2-bit baseline format
def test_pack2_golden_layout(orc):
    """The 2-bit baseline layout against hand-derived bytes."""
    T = np.zeros((64, 128), np.int8)
    expect = {}
    for line in open(os.path.join(GOLDEN, "packed2_layout_64x128.txt")):
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        if f[0] == "set":
            T[int(f[1]), int(f[2])] = int(f[3])
        elif f[0] == "expect":
            expect[int(f[1])] = int(f[2], 16)
    got = orc.pack2(T)
    want = np.zeros(2048, np.uint8)
    for b, v in expect.items():
        want[b] = v
    assert np.array_equal(got, want)


def test_pack2_roundtrip_any_ternary(orc):
    """Unstructured ternary (any mix of -1/0/+1) survives pack2/unpack2, and
    the Sherry ternarization does too; a 5-bit and a 2-bit packing of the
    same T describe the same matrix."""
    rng = np.random.default_rng(8)
    T = rng.integers(-1, 2, size=(192, 384)).astype(np.int8)
    assert np.array_equal(orc.unpack2(orc.pack2(T), 192, 384), T)
    T3, _ = orc.quantize(rng.normal(0, 0.02, (128, 256)).astype(np.float32))
    assert np.array_equal(orc.unpack2(orc.pack2(T3), 128, 256),
                          orc.unpack(orc.pack(T3), 128, 256))
    assert orc.pack2(T3).size * 5 == orc.pack(T3).size * 8   # 2 vs 1.25 bit per weight


@pytest.mark.parametrize("N,K", [(70, 144), (1, 4), (64, 132), (100, 128), (65, 260)])
def test_padded_layout_is_code_zero_padding(orc, N, K):
    """A matrix whose N is not a multiple of 64 or whose K is not a multiple of
    128 is stored as the padded matrix (N up to 64, K up to 128) whose extra
    blocks are code 0, i.e. the block [0, +1, +1, +1]: its bytes equal those
    of packing that padded matrix through the unpadded layout, and the
    padding bytes are zero."""
    rng = np.random.default_rng(N * 1000 + K)
    T, _ = orc.quantize(rng.standard_normal((N, K)).astype(np.float32))
    Np, Kp = -(-N // 64) * 64, -(-K // 128) * 128
    assert orc.packed_bytes(N, K) == Np * Kp * 5 // 32
    assert orc.packed2_bytes(N, K) == Np * Kp // 4
    assert orc.encode_block(np.array([0, 1, 1, 1], np.int8)) == 0
    full = np.tile(np.array([0, 1, 1, 1], np.int8), (Np, Kp // 4))
    full[:N, :K] = T
    P = orc.pack(T)
    assert np.array_equal(P, orc.pack(full))
    assert np.array_equal(orc.unpack(P, N, K), T)
    # the same for the 2-bit format, whose padding is 00 (zero weights)
    full2 = np.zeros((Np, Kp), np.int8)
    full2[:N, :K] = T
    assert np.array_equal(orc.pack2(T), orc.pack2(full2))
    assert np.array_equal(orc.unpack2(orc.pack2(T), N, K), T)


# ------------------------------------------- scaled act quant, epilogue order
# Golden values written by tests/golden/make_*.py with exact rational
# arithmetic (fractions.Fraction): no oracle and no GPU took part.
import sys as _sys  # noqa: E402

_sys.path.insert(0, GOLDEN)
import exact_fp32  # noqa: E402
import make_act_quant_scaled  # noqa: E402
import make_epilogue_order  # noqa: E402


def _act_quant_scaled_rows():
    rows, cur = [], {}
    with open(os.path.join(GOLDEN, "act_quant_scaled.txt")) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            key, val = line.split(":", 1)
            cur[key.strip()] = val.split()
            if key.strip() == "q":
                rows.append((np.array([exact_fp32.from_hex(v) for v in cur["x"]], np.float32),
                             exact_fp32.from_hex(cur["s"][0]),
                             np.array([int(v) for v in cur["q"]], np.int8)))
                cur = {}
    return rows


def test_golden_files_are_what_their_scripts_write():
    for name, mod in (("act_quant_scaled.txt", make_act_quant_scaled),
                      ("epilogue_order.txt", make_epilogue_order)):
        with open(os.path.join(GOLDEN, name)) as f:
            assert f.read() == mod.render(), f"{name} differs from its writer's output"


def test_exact_fp32_rounding_agrees_with_ieee_on_known_values():
    # the helpers themselves: 1/3 and 2/3 in binary32, a tie, and a power of two
    F = exact_fp32.Fraction
    assert float(exact_fp32.fp32_round(F(1, 3))) == float(np.float32(1) / np.float32(3))
    assert float(exact_fp32.fp32_round(F(2, 3))) == float(np.float32(2) / np.float32(3))
    # 1 + 2^-24 lies halfway between 1 and 1 + 2^-23: ties to the even significand (1)
    assert exact_fp32.fp32_round(1 + F(1, 2 ** 24)) == 1
    assert exact_fp32.fp32_round(1 + F(3, 2 ** 24)) == 1 + F(2, 2 ** 23)
    assert exact_fp32.fp32_round(F(2) ** -100) == F(2) ** -100
    assert [exact_fp32.round_half_even(F(v, 2)) for v in (-5, -3, -1, 1, 3, 5)] == [-2, -2, 0, 0, 2, 2]


def test_act_quant_golden_scaled(orc):
    """Scales other than 1: q follows one correctly rounded fp32 division x/s
    and a round-half-even of that fp32 quotient (the workloads' rule s =
    max|x|/127, symmetric; reading of the quantizer)."""
    rows = _act_quant_scaled_rows()
    assert len(rows) == 3
    X = np.stack([r[0] for r in rows])
    q, s = orc.act_quant(X)
    for m, (x, s_ref, q_ref) in enumerate(rows):
        assert s[m].view(np.uint32) == np.float32(s_ref).view(np.uint32)
        assert np.array_equal(q[m], q_ref), f"token {m}"
        # the golden separates the reading from its two near alternatives
        rcp = np.clip(np.rint(x * (np.float32(1) / np.float32(s_ref))), -127, 127)
        exact = np.clip(np.rint(x.astype(np.float64) / np.float64(s_ref)), -127, 127)
        assert (rcp != q_ref).any() and (exact != q_ref).any()


def _epilogue_cases():
    out = []
    with open(os.path.join(GOLDEN, "epilogue_order.txt")) as f:
        for line in f:
            if line.startswith("case:"):
                a, s, al, y = line.split(":", 1)[1].split()
                out.append((int(a), exact_fp32.from_hex(s), exact_fp32.from_hex(al),
                            exact_fp32.from_hex(y)))
    return out


def test_epilogue_order_golden(orc):
    """y = ((float)acc * s_x) * alpha, each product rounded to fp32 in that
    order (the page's single float rescale after the integer add tree; reading
    of the epilogue).  Every case is one where the other two orders differ."""
    cases = _epilogue_cases()
    assert len(cases) == 48
    for acc, s, al, y_ref in cases:
        y = orc.epilogue(np.array([[acc]], np.int32), np.array([s], np.float32),
                         np.array([al], np.float32))[0, 0]
        assert y.view(np.uint32) == y_ref.view(np.uint32), (acc, s, al)
        assert (np.float32(acc) * al) * s != y_ref and np.float32(acc) * (s * al) != y_ref


def test_parallel_oracle_build_gives_identical_products(orc):
    rng = np.random.default_rng(12)
    q = rng.integers(-128, 128, (5, 640)).astype(np.int8)
    T = orc.quantize(rng.normal(0, 0.02, (300, 640)).astype(np.float32))[0]
    assert np.array_equal(orc.gemm_i32(q, T), orc.gemm_i32(q, T, parallel=True))
    assert orc.threads(parallel=False) == 1
