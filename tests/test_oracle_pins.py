"""Pins for the CPU oracle (runs without a GPU).

The pages print no worked numeric example of a norm, product or argmax, so the
oracle is pinned by what mathematics fixes independently of its own code:
exact rational brute force (BF16 values are dyadic rationals), 50-digit decimal
evaluation of the transcendental steps, closed forms, invariants, and
independent library conversions (numpy's float16 cast, torch's bfloat16 cast).
Each test names the mistake it is meant to catch.
"""
import math
import struct
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as O

getcontext().prec = 60
RNG = np.random.default_rng(12345)


# ----------------------------------------------------------- independent helpers
def rne_bf16_bits(fr: Fraction) -> int:
    """Round an exact rational to BF16 (nearest, ties to even) with integer math only."""
    if fr == 0:
        return 0
    sign = 0x8000 if fr < 0 else 0
    a = abs(fr)
    # e = floor(log2 a)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 7)
    q = a / ulp
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r > Fraction(255) * Fraction(2) ** 120:
        return sign | 0x7F80
    if r == 0:
        return sign
    bits = struct.unpack("<I", struct.pack("<f", float(r)))[0]
    assert float(r) == r  # exactly representable
    return sign | (bits >> 16)


def bf16_val(h: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", (h & 0xFFFF) << 16))[0])


def rand_bf16(shape, std=1.0, mean=0.0):
    t = torch.from_numpy((RNG.standard_normal(shape) * std + mean).astype(np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def dec(fr: Fraction) -> Decimal:
    return Decimal(fr.numerator) / Decimal(fr.denominator)


def dec_to_frac(d: Decimal) -> Fraction:
    return Fraction(d)


def dtanh(x: Decimal) -> Decimal:
    e2 = (2 * x).exp()
    return (e2 - 1) / (e2 + 1)


def dgelu_tanh(z: Decimal) -> Decimal:
    c = (Decimal(2) / dpi()).sqrt()
    return Decimal("0.5") * z * (1 + dtanh(c * (z + Decimal("0.044715") * z ** 3)))


def dpi() -> Decimal:
    # Machin's formula, 60 digits
    def arctan_inv(n):
        x = Decimal(1) / n
        x2 = x * x
        s, t, k = Decimal(0), x, 1
        while True:
            term = t / k
            if abs(term) < Decimal(10) ** -65:
                break
            s += term if (k // 2) % 2 == 0 else -term
            t *= x2
            k += 2
        return s
    return 4 * (4 * arctan_inv(5) - arctan_inv(239))


def dsilu(z: Decimal) -> Decimal:
    return z / (1 + (-z).exp())


# ------------------------------------------------------------------- encodings
def test_bf16_roundtrip_every_pattern():
    """Catches a decode/encode mismatch anywhere in the BF16 range (incl. subnormals, +-0, inf)."""
    for h in range(0, 1 << 16):
        if (h & 0x7F80) == 0x7F80 and (h & 0x7F):
            continue  # NaN payloads
        assert O.f64_to_bf16(O.bf16_to_f64(h)) == h, hex(h)


def test_bf16_rounding_matches_torch_cast():
    """float32 inputs: the oracle's direct binary64 -> BF16 rounding must equal torch's
    independent float32 -> bfloat16 cast (round to nearest even), ties included."""
    vals = list(RNG.standard_normal(3000).astype(np.float32) * np.float32(3.0))
    # exact ties: a BF16 value plus half an ulp, both parities
    for h in (0x3F80, 0x3F81, 0xBF80, 0xBF81, 0x0001, 0x0002, 0x7F7F, 0x4000):
        lo = np.uint32(h) << np.uint32(16)
        vals.append(np.array([lo | np.uint32(0x8000)], dtype=np.uint32).view(np.float32)[0])
    vals = np.array(vals, dtype=np.float32)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([O.f64_to_bf16(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(ref, got)


def test_bf16_rounding_matches_exact_rationals():
    """binary64 inputs that are not float32 values: compare with integer-only RNE."""
    for v in list(RNG.standard_normal(2000) * 10.0) + [1.0 + 2.0 ** -8 + 2.0 ** -40, 2.0 ** -130 * 1.37]:
        assert O.f64_to_bf16(v) == rne_bf16_bits(Fraction(v)), v


def test_f16_rounding_matches_numpy_cast():
    """numpy's float64 -> float16 cast is an independent round-to-nearest-even."""
    vals = np.concatenate([RNG.standard_normal(3000) * 8.0, RNG.standard_normal(200) * 1e-5,
                           np.array([65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25,
                                     1.5 * 2.0 ** -24, 2.0 ** -14, -0.0, 1e6])])
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([O.f64_to_f16(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(ref, got)


def test_f16_roundtrip_every_pattern():
    for h in range(0, 1 << 16):
        if (h & 0x7C00) == 0x7C00 and (h & 0x3FF):
            continue
        assert O.f64_to_f16(O.f16_to_f64(h)) == h, hex(h)
        assert O.f16_to_f64(h) == float(np.array([h], dtype=np.uint16).view(np.float16)[0]) or \
            (h & 0x7FFF) == 0


# -------------------------------------------------------------------- product
def test_matvec_identity_is_exact():
    """Identity weights: one non-zero term per row, so the product is x-hat bit for bit."""
    K = 96
    W = np.zeros((K, K), dtype=np.uint16)
    W[np.arange(K), np.arange(K)] = 0x3F80
    xh = rand_bf16(K)
    acc = O.matvec(W, xh)
    assert np.array_equal(acc, O.bf16_array_to_f64(xh))


def test_matvec_reads_rows_not_columns():
    """A single off-diagonal entry W[0][1] = 1 catches a transposed operand."""
    K = 16
    W = np.zeros((K, K), dtype=np.uint16)
    W[0, 1] = 0x3F80
    xh = rand_bf16(K)
    acc = O.matvec(W, xh)
    want = np.zeros(K)
    want[0] = O.bf16_array_to_f64(xh)[1]
    assert np.array_equal(acc, want)


def test_matvec_rank_one_dyadic_exact():
    """W = u v^T with small dyadic entries: every product and sum is exact, y = u (v . x)."""
    N, K = 24, 40
    u = RNG.integers(-8, 9, N) / 8.0
    v = RNG.integers(-8, 9, K) / 8.0
    Wf = np.outer(u, v).astype(np.float32)
    W = torch.from_numpy(Wf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_array_to_f64(W), np.outer(u, v))  # representable
    xh = rand_bf16(K)
    xs = [bf16_val(int(h)) for h in xh]
    dot = sum(Fraction(vk) * xk for vk, xk in zip(v, xs))
    acc = O.matvec(W, xh)
    for n in range(N):
        assert Fraction(acc[n]) == Fraction(u[n]) * dot


def test_stage_brute_force_8x8_rational():
    """8x8 product + BF16 output vs exact rational arithmetic (no norm, no epilogue)."""
    for trial in range(20):
        W = rand_bf16((8, 8))
        x = rand_bf16((1, 8))
        y = O.stage(x, W)
        for n in range(8):
            exact = sum(bf16_val(int(W[n, k])) * bf16_val(int(x[0, k])) for k in range(8))
            assert int(y[0, n]) == rne_bf16_bits(exact), (trial, n)


def test_matvec_threads_bit_identical_and_close_to_numpy():
    W = rand_bf16((2048, 384), std=0.02)
    xh = rand_bf16(384)
    O.set_threads(1)
    a1 = O.matvec(W, xh)
    O.set_threads(8)
    a8 = O.matvec(W, xh)
    O.set_threads(1)
    assert np.array_equal(a1, a8)
    ref = O.bf16_array_to_f64(W) @ O.bf16_array_to_f64(xh)
    assert np.max(np.abs(a1 - ref)) <= 1e-13 * np.max(np.abs(ref)) + 1e-300


def test_matvec_rows_matches_matvec():
    W = rand_bf16((300, 64))
    xh = rand_bf16(64)
    rows = np.array([0, 7, 299, 150], dtype=np.int64)
    assert np.array_equal(O.matvec_rows(W, rows, xh), O.matvec(W, xh)[rows])


# ---------------------------------------------------------------------- norms
def test_rmsnorm_unit_gain_rms_closed_form():
    """Unit gain: mean of squares of the (un-rounded) output equals m / (m + eps)."""
    for eps in (1e-6, 0.5):
        x = rand_bf16(1536)
        out = O.norm_f64(O.NORM_RMS, x, None, None, eps)
        xv = O.bf16_array_to_f64(x)
        m = np.mean(xv * xv)
        assert abs(np.mean(out * out) - m / (m + eps)) <= 1e-13


def test_rmsnorm_gain_and_scale_invariance():
    x = rand_bf16(256)
    g = rand_bf16(256, std=0.1, mean=1.0)
    a = O.norm_bf16(O.NORM_RMS, x, g, None, 0.0)
    x4 = O.bf16_array_to_f64(x) * 4.0
    x4b = np.array([O.f64_to_bf16(v) for v in x4], dtype=np.uint16)
    b = O.norm_bf16(O.NORM_RMS, x4b, g, None, 0.0)
    assert np.array_equal(a, b)  # power-of-two scale, eps = 0: exact invariance
    two = np.full(256, 0x4000, dtype=np.uint16)  # gain 2 doubles the un-rounded output
    assert np.array_equal(O.norm_f64(O.NORM_RMS, x, two, None, 1e-6),
                          2.0 * O.norm_f64(O.NORM_RMS, x, None, None, 1e-6))


def test_rmsnorm_one_hot():
    K = 64
    x = np.zeros(K, dtype=np.uint16)
    x[5] = O.f64_to_bf16(-3.0)
    g = rand_bf16(K, std=0.1, mean=1.0)
    eps = 1e-6
    got = O.norm_bf16(O.NORM_RMS, x, g, None, eps)
    val = dec(Fraction(-3)) / ((dec(Fraction(9, K)) + dec(Fraction(eps))).sqrt()) * dec(bf16_val(int(g[5])))
    assert int(got[5]) == rne_bf16_bits(dec_to_frac(val))
    assert np.all(np.delete(got, 5) & 0x7FFF == 0)


def _dec_rmsnorm_bits(x, g, eps):
    xs = [bf16_val(int(h)) for h in x]
    m = sum(v * v for v in xs) / len(xs)
    r = 1 / (dec(m) + dec(Fraction(eps))).sqrt()
    return [rne_bf16_bits(dec_to_frac(dec(v) * r * dec(bf16_val(int(gk))))) for v, gk in zip(xs, g)]


def test_rmsnorm_decimal_brute_force_and_eps_placement():
    """50-digit evaluation; the small-magnitude case makes eps comparable to the
    mean square, so eps outside the root or added to the rms would fail."""
    for std in (1.0, 1e-3):
        x = rand_bf16(128, std=std)
        g = rand_bf16(128, std=0.1, mean=1.0)
        got = O.norm_bf16(O.NORM_RMS, x, g, None, 1e-6)
        want = _dec_rmsnorm_bits(x, g, 1e-6)
        assert [int(v) for v in got] == want


def test_layernorm_closed_forms_and_invariances():
    x = rand_bf16(768, std=2.0, mean=0.5)
    eps = 1e-5
    out = O.norm_f64(O.NORM_LAYER, x, None, None, eps)
    xv = O.bf16_array_to_f64(x)
    v = np.var(xv)
    assert abs(np.mean(out)) <= 1e-13
    assert abs(np.mean(out * out) - v / (v + eps)) <= 1e-12
    # beta shifts the output; gamma scales it
    beta = np.full(768, O.f64_to_bf16(0.25), dtype=np.uint16)
    gam = np.full(768, 0x4000, dtype=np.uint16)
    sh = O.norm_f64(O.NORM_LAYER, x, gam, beta, eps)
    assert np.max(np.abs(sh - (2.0 * out + 0.25))) <= 1e-13
    # shift invariance on integer-valued inputs (exact in BF16)
    xi = RNG.integers(-60, 61, 768).astype(np.float64)
    xb = np.array([O.f64_to_bf16(t) for t in xi], dtype=np.uint16)
    xb8 = np.array([O.f64_to_bf16(t + 8.0) for t in xi], dtype=np.uint16)
    a = O.norm_f64(O.NORM_LAYER, xb, None, None, eps)
    b = O.norm_f64(O.NORM_LAYER, xb8, None, None, eps)
    assert np.max(np.abs(a - b)) <= 1e-12


def test_layernorm_decimal_brute_force():
    x = rand_bf16(96, std=1.5, mean=-0.3)
    g = rand_bf16(96, std=0.1, mean=1.0)
    b = rand_bf16(96, std=0.02)
    eps = 1e-5
    got = O.norm_bf16(O.NORM_LAYER, x, g, b, eps)
    xs = [bf16_val(int(h)) for h in x]
    mu = sum(xs) / len(xs)
    var = sum((t - mu) ** 2 for t in xs) / len(xs)
    r = 1 / (dec(var) + dec(Fraction(eps))).sqrt()
    want = [rne_bf16_bits(dec_to_frac(dec(t - mu) * r * dec(bf16_val(int(gk))) + dec(bf16_val(int(bk)))))
            for t, gk, bk in zip(xs, g, b)]
    assert [int(v) for v in got] == want


# ------------------------------------------------------------------ epilogues
@pytest.mark.parametrize("z", [-6.0, -2.5, -1.0, -0.3, 0.0, 0.1, 0.7, 1.0, 2.0, 5.5])
def test_gelu_tanh_and_silu_decimal(z):
    gd = float(dgelu_tanh(Decimal(z)))
    sd = float(dsilu(Decimal(z)))
    assert abs(O.gelu_tanh(z) - gd) <= 4e-16 * max(1.0, abs(gd))
    assert abs(O.silu(z) - sd) <= 4e-16 * max(1.0, abs(sd))


def test_gelu_silu_odd_part_identity_and_tanh_form():
    """f(z) - f(-z) = z holds for both (tanh is odd, sigmoid(z)+sigmoid(-z)=1);
    the tanh form differs from the erf form by ~1e-4 near z=1 (catches the wrong form)."""
    for z in np.linspace(-7, 7, 57):
        assert abs(O.gelu_tanh(z) - O.gelu_tanh(-z) - z) <= 1e-14 * max(1, abs(z))
        assert abs(O.silu(z) - O.silu(-z) - z) <= 1e-14 * max(1, abs(z))
    erf_form = 0.5 * (1 + math.erf(1 / math.sqrt(2)))
    assert abs(O.gelu_tanh(1.0) - erf_form) > 1e-5
    assert O.gelu_tanh(0.0) == 0.0 and O.silu(0.0) == 0.0
    assert abs(O.gelu_tanh(12.0) - 12.0) < 1e-12 and abs(O.gelu_tanh(-12.0)) < 1e-12


def test_stage_epilogues_against_rationals():
    """bias + GELU, SwiGLU with up == gate and up == 0, residual with zero weights."""
    N, K = 12, 16
    W = rand_bf16((N, K), std=0.3)
    x = rand_bf16((2, K))
    bias = rand_bf16(N, std=0.1)
    res = rand_bf16((2, N))
    exact = [[sum(bf16_val(int(W[n, k])) * bf16_val(int(x[b, k])) for k in range(K)) for n in range(N)]
             for b in range(2)]
    y = O.stage(x, W, epi=O.EPI_GELU_TANH, bias=bias)
    for b in range(2):
        for n in range(N):
            z = exact[b][n] + bf16_val(int(bias[n]))
            assert int(y[b, n]) == rne_bf16_bits(dec_to_frac(dgelu_tanh(dec(z))))
    ys = O.stage(x, W, epi=O.EPI_SWIGLU, W_up=W)
    for b in range(2):
        for n in range(N):
            z = exact[b][n]
            assert int(ys[b, n]) == rne_bf16_bits(dec_to_frac(dsilu(dec(z)) * dec(z)))
    y0 = O.stage(x, W, epi=O.EPI_SWIGLU, W_up=np.zeros_like(W))
    assert np.all((y0 & 0x7FFF) == 0)
    yr = O.stage(x, np.zeros_like(W), residual=res)
    assert np.array_equal(yr, res)
    yr2 = O.stage(x, W, residual=res)
    for b in range(2):
        for n in range(N):
            assert int(yr2[b, n]) == rne_bf16_bits(exact[b][n] + bf16_val(int(res[b, n])))


def test_stage_rounds_xhat_before_the_product():
    """The contract rounds x-hat to BF16 before the product: the stage's acc equals
    the product of the rounded x-hat, not of the un-rounded normalised values."""
    x = rand_bf16((1, 64))
    g = rand_bf16(64, std=0.1, mean=1.0)
    W = rand_bf16((8, 64))
    y, xh, acc = O.stage(x, W, norm=O.NORM_RMS, gamma=g, want_xh=True, want_acc=True)
    assert np.array_equal(xh[0], O.norm_bf16(O.NORM_RMS, x[0], g, None, 1e-6))
    assert np.array_equal(acc[0], O.matvec(W, xh[0]))


# -------------------------------------------------------------------- LM head
def test_lmhead_planted_row_and_ties():
    V, K = 500, 64
    h = rand_bf16((1, K))
    g = rand_bf16(K, std=0.1, mean=1.0)
    W = rand_bf16((V, K), std=0.02)
    xh = O.norm_bf16(O.NORM_RMS, h[0], g, None, 1e-6)
    planted = np.array([O.f64_to_bf16(4.0 * v) for v in O.bf16_array_to_f64(xh)], dtype=np.uint16)
    W[321] = planted
    idx, mx, logits = O.lmhead_argmax(h, g, W, want_logits=True)
    assert idx[0] == 321
    assert mx[0] == logits[0, 321] == np.max(logits[0])
    assert np.array_equal(logits[0], O.matvec(W, xh))
    W[77] = planted  # duplicated maximum -> lowest index
    idx2, _ = O.lmhead_argmax(h, g, W)
    assert idx2[0] == 77
    idx3, _ = O.lmhead_argmax(h, g, np.tile(W[5], (V, 1)))  # all equal -> 0
    assert idx3[0] == 0


# ------------------------------------------------------------- FP16 norm rows
def test_rmsnorm_rows_f16_vs_numpy():
    R, K = 6, 1536
    x = (RNG.standard_normal((R, K))).astype(np.float16)
    g = (1 + 0.1 * RNG.standard_normal(K)).astype(np.float16)
    eps = 1e-6
    got = O.rmsnorm_rows_f16(x.view(np.uint16), g.view(np.uint16), eps)
    xv = x.astype(np.float64)
    ref = xv / np.sqrt(np.mean(xv * xv, axis=1, keepdims=True) + eps) * g.astype(np.float64)
    want = ref.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_swiglu_operand_order_asymmetric():
    """SwiGLU reads the first matrix as the gate: s = R(silu(W x) * (W_up x))
    ("One Token, Kernel by Kernel", section "The setup": SwiGLU MLP).  Gate and up
    are different, both non-zero, so the swapped reading silu(W_up x) * (W x)
    gives other bits; the cases are checked against exact rational sums and
    60-digit decimal SiLU, and the swap is shown to fail the same check."""
    N, K = 16, 32
    x = rand_bf16((2, K))
    W = rand_bf16((N, K), std=0.3)
    cases = [rand_bf16((N, K), std=0.5)]  # an unrelated up matrix
    onehot = np.zeros((N, K), dtype=np.uint16)
    for n in range(N):
        onehot[n, (5 * n + 3) % K] = 0x4000  # 2.0 at one column: up = 2 x_k exactly
    cases.append(onehot)
    for W_up in cases:
        ys = O.stage(x, W, epi=O.EPI_SWIGLU, W_up=W_up)
        swapped_differs = False
        for b in range(2):
            for n in range(N):
                ag = sum(bf16_val(int(W[n, k])) * bf16_val(int(x[b, k])) for k in range(K))
                au = sum(bf16_val(int(W_up[n, k])) * bf16_val(int(x[b, k])) for k in range(K))
                want = rne_bf16_bits(dec_to_frac(dsilu(dec(ag)) * dec(au)))
                swap = rne_bf16_bits(dec_to_frac(dsilu(dec(au)) * dec(ag)))
                assert int(ys[b, n]) == want, (b, n)
                swapped_differs |= swap != want
        assert swapped_differs, "the case must tell the gate from the up matrix"


def rne_f16_bits(fr: Fraction) -> int:
    """Round an exact rational to IEEE binary16 (nearest, ties to even), integer math only."""
    if fr == 0:
        return 0
    sign = 0x8000 if fr < 0 else 0
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -14)  # subnormals share the smallest normal exponent's ulp
    ulp = Fraction(2) ** (e - 10)
    q = a / ulp
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r >= 65520:  # rounds past the largest finite value
        return sign | 0x7C00
    bits = int(np.array([float(r)], dtype=np.float16).view(np.uint16)[0])
    assert Fraction(float(np.float16(float(r)))) == r  # exactly representable
    return sign | bits


def test_rmsnorm_rows_f16_eps_placement():
    """The FP16 rows norm puts eps inside the root, y = R16(x (mean x^2 + eps)^-1/2 g)
    ("GPU Kernel Optimization" README, section "Architecture": mean square, rsqrt,
    weight multiply).  Rows of std 1e-3 make the mean square comparable to
    eps = 1e-6, so eps outside the root, eps dropped or eps added after the
    mean's division all give other bits; checked against exact FP16 inputs,
    60-digit decimal arithmetic and integer-only rounding to FP16."""
    R, K = 3, 96
    x = (RNG.standard_normal((R, K)) * 1e-3).astype(np.float16)
    g = (1 + 0.1 * RNG.standard_normal(K)).astype(np.float16)
    eps32 = float(np.float32(1e-6))
    got = O.rmsnorm_rows_f16(x.view(np.uint16), g.view(np.uint16), eps32)
    xs = [[Fraction(float(v)) for v in row] for row in x]
    gs = [Fraction(float(v)) for v in g]
    deps = dec(Fraction(eps32))
    alt_differs = {"outside": False, "dropped": False}
    for r in range(R):
        ms = dec(sum(v * v for v in xs[r]) / K)
        assert abs(ms - deps) < 2 * deps, "mean square must be comparable to eps"
        inv = 1 / (ms + deps).sqrt()
        inv_out = 1 / (ms.sqrt() + deps)
        inv_drop = 1 / ms.sqrt()
        for k in range(K):
            xk, gk = dec(xs[r][k]), dec(gs[k])
            want = rne_f16_bits(dec_to_frac(xk * inv * gk))
            assert int(got[r, k]) == want, (r, k)
            alt_differs["outside"] |= rne_f16_bits(dec_to_frac(xk * inv_out * gk)) != want
            alt_differs["dropped"] |= rne_f16_bits(dec_to_frac(xk * inv_drop * gk)) != want
    assert all(alt_differs.values()), alt_differs
