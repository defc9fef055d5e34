"""Pins of the oracle's decode attention (CPU only).

The attention of one new token over a static cache ("Making small PyTorch ops
faster on a laptop GPU", section "A full decode step is a different story";
"One Token, Kernel by Kernel", section "The fix: Part 10's split-KV kernel")
is pinned here by results that do not come from the oracle's own formula:

* a cache with one valid position returns that position's value exactly;
* equal keys give equal weights, so the output is the exact rational mean of
  the values, rounded once (integer rounding below);
* a planted key whose score exceeds all others by hundreds selects its value
  exactly, and only in the query heads of its own key/value group;
* two positions with scores 0 and c give the closed-form logistic weight,
  which fixes the score scale;
* 60-digit decimal brute force on tiny random inputs;
* slots after the new token never reach the output (NaN there is harmless),
  and slots other than the new one are never written.
"""
from __future__ import annotations

import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O
from tests.test_oracle_pins import bf16_val as _bf16_val, dec, rand_bf16, rne_bf16_bits

BF16_NAN = 0x7FC0


def bf16_val(h) -> Fraction:
    return _bf16_val(int(h))


D = 128


def _zeros(*shape):
    return np.zeros(shape, dtype=np.uint16)


def _bits(x: float) -> int:
    return rne_bf16_bits(Fraction(x))


def test_single_position_returns_the_new_value():
    B, Hq, Hkv, S = 2, 12, 2, 9
    q = rand_bf16((B, Hq, D))
    kn, vn = rand_bf16((B, Hkv, D)), rand_bf16((B, Hkv, D))
    kc = np.full((B, Hkv, S, D), BF16_NAN, dtype=np.uint16)
    vc = np.full((B, Hkv, S, D), BF16_NAN, dtype=np.uint16)
    out, kc2, vc2 = O.decode_attention(q, kn, vn, kc, vc, np.zeros(B, np.int32))
    for h in range(Hq):
        np.testing.assert_array_equal(out[:, h], vn[:, h // 6])
    np.testing.assert_array_equal(kc2[:, :, 0], kn)
    np.testing.assert_array_equal(vc2[:, :, 0], vn)
    # every other slot keeps its old bits
    np.testing.assert_array_equal(kc2[:, :, 1:], kc[:, :, 1:])
    np.testing.assert_array_equal(vc2[:, :, 1:], vc[:, :, 1:])


def test_equal_keys_give_the_exact_mean():
    B, Hq, Hkv, S, pos = 1, 4, 1, 40, 36
    q = rand_bf16((B, Hq, D))
    key = rand_bf16((D,))
    kc = np.broadcast_to(key, (B, Hkv, S, D)).copy()
    vc = rand_bf16((B, Hkv, S, D))
    kn = key.reshape(1, 1, D).copy()
    vn = rand_bf16((B, Hkv, D))
    out, _, _ = O.decode_attention(q, kn, vn, kc, vc, np.array([pos], np.int32))
    vals = [[bf16_val(vc[0, 0, t, j]) for j in range(D)] for t in range(pos)]
    vals.append([bf16_val(vn[0, 0, j]) for j in range(D)])
    for j in range(D):
        mean = sum(v[j] for v in vals) / (pos + 1)
        want = rne_bf16_bits(mean)
        for h in range(Hq):
            assert out[0, h, j] == want, (h, j)


def test_planted_key_selects_its_value_in_its_own_group_only():
    B, Hq, Hkv, S, pos = 1, 12, 2, 64, 50
    u = rand_bf16((D,))
    q = np.broadcast_to(u, (B, Hq, D)).copy()
    kc = _zeros(B, Hkv, S, D)              # group 0: all keys zero -> equal weights
    kc[0, 1, :pos] = rand_bf16((pos, D), std=0.05)
    t_star = 17
    # 64 u in BF16 is exact (a power-of-two scale); its score is 64 |u|^2 / sqrt(D)
    kc[0, 1, t_star] = (u.astype(np.uint32) + (6 << 7)).astype(np.uint16) * (u != 0)
    vc = rand_bf16((B, Hkv, S, D))
    kn = _zeros(B, Hkv, D)
    kn[0, 1] = rand_bf16((D,), std=0.05)
    vn = rand_bf16((B, Hkv, D))
    out, _, _ = O.decode_attention(q, kn, vn, kc, vc, np.array([pos], np.int32))
    assert all(bf16_val(kc[0, 1, t_star, j]) == 64 * bf16_val(u[j]) for j in range(D))
    for h in range(6, 12):
        np.testing.assert_array_equal(out[0, h], vc[0, 1, t_star])
    vals = [[bf16_val(vc[0, 0, t, j]) for j in range(D)] for t in range(pos)]
    vals.append([bf16_val(vn[0, 0, j]) for j in range(D)])
    want = [rne_bf16_bits(sum(v[j] for v in vals) / (pos + 1)) for j in range(D)]
    for h in range(6):
        assert list(out[0, h]) == want


@pytest.mark.parametrize("c", [1.0, 2.0, -3.0, 16.0])
def test_two_positions_logistic_weight_fixes_the_scale(c):
    q = _zeros(1, 1, D)
    q[0, 0, 0] = _bits(1.0)
    kc, vc = _zeros(1, 1, 4, D), _zeros(1, 1, 4, D)
    kn, vn = _zeros(1, 1, D), _zeros(1, 1, D)
    kn[0, 0, 0] = _bits(c)         # the new key at slot 1 scores c / sqrt(D); slot 0 scores 0
    vn[0, 0, :] = _bits(1.0)       # value 1 at slot 1, value 0 at slot 0
    out, _, _, of = O.decode_attention(q, kn, vn, kc, vc, np.array([1], np.int32), want_f64=True)
    w = 1.0 / (1.0 + math.exp(-c / math.sqrt(D)))
    assert np.allclose(of[0, 0], w, rtol=1e-14, atol=0)
    assert out[0, 0, 0] == rne_bf16_bits(Fraction(w))


def _dexp(x: Decimal) -> Decimal:
    return x.exp()


def test_decimal_brute_force_tiny():
    getcontext().prec = 60
    B, Hq, Hkv, S, d = 2, 4, 2, 6, 8
    q = rand_bf16((B, Hq, d))
    kc, vc = rand_bf16((B, Hkv, S, d)), rand_bf16((B, Hkv, S, d))
    kn, vn = rand_bf16((B, Hkv, d)), rand_bf16((B, Hkv, d))
    pos = np.array([3, 5], np.int32)
    scale = Fraction(1, 2)
    out, kc2, vc2, of = O.decode_attention(q, kn, vn, kc, vc, pos, scale=0.5, want_f64=True)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            keys = [kc[b, g, t] for t in range(pos[b])] + [kn[b, g]]
            vals = [vc[b, g, t] for t in range(pos[b])] + [vn[b, g]]
            s = [scale * sum(bf16_val(q[b, h, j]) * bf16_val(k[j]) for j in range(d)) for k in keys]
            e = [_dexp(dec(x)) for x in s]
            tot = sum(e)
            for j in range(d):
                v = sum(ei * dec(bf16_val(vv[j])) for ei, vv in zip(e, vals)) / tot
                assert abs(Decimal(of[b, h, j]) - v) <= abs(v) * Decimal("1e-13") + Decimal("1e-300"), (b, h, j)
            # the oracle reads the appended cache back: those slots now hold the new key/value
            np.testing.assert_array_equal(kc2[b, :, pos[b]], kn[b])
            np.testing.assert_array_equal(vc2[b, :, pos[b]], vn[b])


def test_slots_after_the_new_token_are_never_read():
    B, Hq, Hkv, S = 2, 12, 2, 300
    pos = np.array([130, 7], np.int32)
    q = rand_bf16((B, Hq, D))
    kn, vn = rand_bf16((B, Hkv, D)), rand_bf16((B, Hkv, D))
    kc, vc = rand_bf16((B, Hkv, S, D)), rand_bf16((B, Hkv, S, D))
    kz, vz = kc.copy(), vc.copy()
    for b in range(B):
        kc[b, :, pos[b] + 1:] = BF16_NAN
        vc[b, :, pos[b] + 1:] = BF16_NAN
        kz[b, :, pos[b] + 1:] = 0
        vz[b, :, pos[b] + 1:] = 0
    out, kc2, _ = O.decode_attention(q, kn, vn, kc, vc, pos)
    ref, _, _ = O.decode_attention(q, kn, vn, kz, vz, pos)
    np.testing.assert_array_equal(out, ref)
    assert not np.any((out & 0x7F80) == 0x7F80)
    for b in range(B):
        np.testing.assert_array_equal(kc2[b, :, :pos[b]], kc[b, :, :pos[b]])
        np.testing.assert_array_equal(kc2[b, :, pos[b] + 1:], kc[b, :, pos[b] + 1:])


def test_out_of_range_position_appends_nothing_and_outputs_zero():
    B, Hq, Hkv, S = 3, 12, 2, 16
    q = rand_bf16((B, Hq, D))
    kn, vn = rand_bf16((B, Hkv, D)), rand_bf16((B, Hkv, D))
    kc, vc = rand_bf16((B, Hkv, S, D)), rand_bf16((B, Hkv, S, D))
    pos = np.array([-1, 16, 3], np.int32)
    out, kc2, vc2 = O.decode_attention(q, kn, vn, kc, vc, pos)
    assert not out[:2].any()
    np.testing.assert_array_equal(kc2[:2], kc[:2])
    np.testing.assert_array_equal(vc2[:2], vc[:2])
    assert out[2].any()


def test_threads_bit_identical():
    B, Hq, Hkv, S = 2, 12, 2, 257
    q = rand_bf16((B, Hq, D))
    kn, vn = rand_bf16((B, Hkv, D)), rand_bf16((B, Hkv, D))
    kc, vc = rand_bf16((B, Hkv, S, D)), rand_bf16((B, Hkv, S, D))
    pos = np.array([256, 100], np.int32)
    O.set_threads(1)
    a = O.decode_attention(q, kn, vn, kc, vc, pos, want_f64=True)
    O.set_threads(max(2, O.max_threads()))
    b = O.decode_attention(q, kn, vn, kc, vc, pos, want_f64=True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
