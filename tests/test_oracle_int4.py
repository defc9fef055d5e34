"""Pins of the oracle's 4-bit weight product (CPU only).

"One Token, Kernel by Kernel", section "4-bit weights": 4-bit integer weights
in groups of 128.  The layout is this library's reading (low nibble = even k;
a BF16 scale s and zero z per row and group; w = s q + z).  Pinned by:
* a single non-zero code picks out one input, which fixes the nibble order;
* scale 0 leaves the zero times the group's input sum, exactly;
* codes all c with unit scale give c times the input sum, exactly;
* exact rational brute force over random codes, scales and zeros;
* thread-count bit-identity.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O
from tests.test_oracle_pins import bf16_val as _bf16_val, rand_bf16, rne_bf16_bits

ONE = 0x3F80


def bf16_val(h) -> Fraction:
    return _bf16_val(int(h))


def pack(q: np.ndarray) -> np.ndarray:
    """Codes [N][K] in 0..15 -> bytes [N][K/2] (even k in the low nibble)."""
    q = q.astype(np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


@pytest.mark.parametrize("k", [0, 1, 2, 127, 128, 255])
def test_one_code_selects_one_input(k):
    N, K = 2, 256
    q = np.zeros((N, K), np.uint8)
    q[1, k] = 1
    sc = np.full((N, K // 128), ONE, np.uint16)
    zr = np.zeros((N, K // 128), np.uint16)
    x = rand_bf16((1, K))
    y = O.matvec_int4(pack(q), sc, zr, x)
    assert y[0, 0] == 0
    assert y[0, 1] == x[0, k]


def test_zero_scale_leaves_zero_times_group_sum():
    N, K = 3, 384
    q = np.random.default_rng(1).integers(0, 16, (N, K)).astype(np.uint8)
    sc = np.zeros((N, K // 128), np.uint16)
    zr = rand_bf16((N, K // 128))
    x = rand_bf16((2, K))
    y, acc = O.matvec_int4(pack(q), sc, zr, x, want_acc=True)
    for b in range(2):
        for n in range(N):
            want = sum(bf16_val(zr[n, g]) * sum(bf16_val(x[b, k]) for k in range(128 * g, 128 * g + 128))
                       for g in range(K // 128))
            assert y[b, n] == rne_bf16_bits(want)


@pytest.mark.parametrize("c", [0, 1, 7, 15])
def test_constant_codes_unit_scale(c):
    N, K = 2, 256
    q = np.full((N, K), c, np.uint8)
    sc = np.full((N, K // 128), ONE, np.uint16)
    zr = np.zeros((N, K // 128), np.uint16)
    x = rand_bf16((1, K))
    y = O.matvec_int4(pack(q), sc, zr, x)
    want = c * sum(bf16_val(v) for v in x[0])
    assert y[0, 0] == y[0, 1] == rne_bf16_bits(want)


def test_rational_brute_force():
    rng = np.random.default_rng(5)
    N, K, B = 4, 256, 3
    q = rng.integers(0, 16, (N, K)).astype(np.uint8)
    sc = rand_bf16((N, K // 128), std=0.01)
    zr = rand_bf16((N, K // 128), std=0.05)
    x = rand_bf16((B, K))
    y = O.matvec_int4(pack(q), sc, zr, x)
    for b in range(B):
        for n in range(N):
            tot = sum((bf16_val(sc[n, k // 128]) * int(q[n, k]) + bf16_val(zr[n, k // 128])) * bf16_val(x[b, k])
                      for k in range(K))
            assert y[b, n] == rne_bf16_bits(tot), (b, n)


def test_threads_bit_identical():
    rng = np.random.default_rng(9)
    N, K = 300, 1536
    W4 = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sc, zr, x = rand_bf16((N, K // 128), std=0.01), rand_bf16((N, K // 128), std=0.05), rand_bf16((2, K))
    O.set_threads(1)
    a = O.matvec_int4(W4, sc, zr, x, want_acc=True)
    O.set_threads(max(2, O.max_threads()))
    b = O.matvec_int4(W4, sc, zr, x, want_acc=True)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
