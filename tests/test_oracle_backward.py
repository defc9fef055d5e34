"""Pins for the oracle's backward pass (runs without a GPU).

The pages give no numbers for a gradient, so the backward definitions are
pinned by what fixes a derivative independently of the oracle's code:
float64 autograd of the same forward (a library routine that shares nothing
with the oracle), central finite differences, the invariances of LayerNorm
(its output does not change when a constant is added to the input, nor, at
eps = 0, when the input is scaled), and exact rational sums where the
rounding points decide the bits.  Each test names the mistake it is meant to
catch.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import oracle as O

RNG = np.random.default_rng(4242)


def rand_bf16(shape, std=1.0, mean=0.0):
    t = torch.from_numpy((RNG.standard_normal(shape) * std + mean).astype(np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f64(bits):
    return O.bf16_array_to_f64(bits)


def block_params(N, K, bias=True, gamma=True, beta=True):
    p = {"W": rand_bf16((N, K), std=1.0 / np.sqrt(K))}
    if bias:
        p["bias"] = rand_bf16((N,), std=0.1)
    if gamma:
        p["gamma"] = rand_bf16((K,), std=0.2, mean=1.0)
    if beta:
        p["beta"] = rand_bf16((K,), std=0.1)
    return p


def autograd_block(x, p, gy, eps):
    """float64 autograd of LayerNorm -> Linear -> GELU-tanh, loss = sum(gy * y)."""
    xt = torch.tensor(f64(x), requires_grad=True)
    W = torch.tensor(f64(p["W"]), requires_grad=True)
    K = xt.shape[1]
    g = torch.tensor(f64(p["gamma"]), requires_grad=True) if "gamma" in p else None
    be = torch.tensor(f64(p["beta"]), requires_grad=True) if "beta" in p else None
    b = torch.tensor(f64(p["bias"]), requires_grad=True) if "bias" in p else None
    xh = F.layer_norm(xt, (K,), g, be, eps)
    z = xh @ W.T
    if b is not None:
        z = z + b
    y = F.gelu(z, approximate="tanh")
    (y * torch.tensor(gy)).sum().backward()
    out = {"gx": xt.grad.numpy(), "gW": W.grad.numpy()}
    if b is not None:
        out["gb"] = b.grad.numpy()
    if g is not None:
        out["ggamma"] = g.grad.numpy()
    if be is not None:
        out["gbeta"] = be.grad.numpy()
    return out


def rel_err(a, ref):
    scale = max(float(np.sqrt(np.mean(ref * ref))), 1e-300)
    return float(np.max(np.abs(a - ref))) / scale


# ------------------------------------------------------------------ GELU'
def test_gelu_grad_closed_values():
    """GELU'(0) = 1/2 exactly (t = 0); the slope tends to 1 and 0 far out.  A
    wrong constant term (0.5 dropped or doubled) fails the first line."""
    assert O.gelu_tanh_grad(0.0) == 0.5
    assert abs(O.gelu_tanh_grad(12.0) - 1.0) < 1e-15
    assert abs(O.gelu_tanh_grad(-12.0)) < 1e-15


def test_gelu_grad_matches_finite_differences_and_autograd():
    """Central differences of the oracle's own GELU (error ~1e-10) and torch's
    float64 autograd of gelu(approximate='tanh').  A dropped chain-rule factor
    (the 3 * 0.044715 z^2 term, or the c) fails by far more than 1e-7."""
    zs = np.concatenate([np.linspace(-8.0, 8.0, 161), RNG.standard_normal(64) * 3.0])
    h = 1e-5
    zt = torch.tensor(zs, requires_grad=True)
    F.gelu(zt, approximate="tanh").sum().backward()
    auto = zt.grad.numpy()
    for z, a in zip(zs, auto):
        fd = (O.gelu_tanh(z + h) - O.gelu_tanh(z - h)) / (2 * h)
        g = O.gelu_tanh_grad(z)
        assert abs(g - fd) <= 1e-7 * max(1.0, abs(fd)), (z, g, fd)
        assert abs(g - a) <= 1e-14 * max(1.0, abs(a)), (z, g, a)


# ----------------------------------------------------------- block backward
@pytest.mark.parametrize("B,N,K,bias,gamma,beta", [
    (1, 8, 8, True, True, True),
    (3, 37, 24, True, True, True),     # ragged rows, odd batch
    (4, 64, 96, False, True, True),    # no bias
    (2, 16, 40, True, False, False),   # unit gain, zero shift
    (16, 48, 32, True, True, False),   # batch 16, gain without shift
    (5, 24, 64, True, True, True),     # N < K
])
def test_block_backward_exact_matches_float64_autograd(B, N, K, bias, gamma, beta):
    """rnd = 0 is the exact derivative of the unrounded block: it must equal
    float64 autograd to rounding noise.  A dropped LayerNorm term (the mean or
    the u * mean(gu u) projection), a transposed W in gxh, the gain applied on
    the wrong side, or a missing bias/gain/shift gradient all fail by O(1)."""
    eps = float(np.float32(1e-5))
    x = rand_bf16((B, K), mean=0.3)
    p = block_params(N, K, bias, gamma, beta)
    gy = RNG.standard_normal((B, N))
    ref = autograd_block(x, p, gy, eps)
    got = O.block_backward(x, p["W"], gy, gamma=p.get("gamma"), beta=p.get("beta"), eps=eps,
                           bias=p.get("bias"), rnd=False)
    assert set(ref) <= set(got)
    for k in ref:
        assert got[k].shape == ref[k].shape, k
        assert rel_err(got[k], ref[k]) < 1e-11, (k, rel_err(got[k], ref[k]))


def test_layernorm_backward_invariances():
    """LayerNorm(x + c) = LayerNorm(x), so sum_k gx = 0 for every row; at
    eps = 0 also LayerNorm(a x) = LayerNorm(x), so sum_k gx x = 0.  A dropped
    mean term breaks the first, a dropped projection term the second."""
    B, N, K = 4, 32, 48
    x = rand_bf16((B, K), std=2.0, mean=1.0)
    p = block_params(N, K)
    gy = RNG.standard_normal((B, N))
    got = O.block_backward(x, p["W"], gy, gamma=p["gamma"], beta=p["beta"], eps=0.0,
                           bias=p["bias"], rnd=False)
    gx = got["gx"]
    scale = float(np.abs(gx).max())
    assert np.all(np.abs(gx.sum(axis=1)) < 1e-12 * scale * K)
    assert np.all(np.abs((gx * f64(x)).sum(axis=1)) < 1e-12 * scale * K * 4)


def test_block_backward_rounded_outputs_are_bf16_and_near_exact():
    """rnd = 1: every output is a BF16 value and sits within BF16 rounding
    (plus the propagated rounding of gz and xh) of the exact derivative."""
    B, N, K = 8, 40, 56
    eps = float(np.float32(1e-5))
    x = rand_bf16((B, K), mean=0.2)
    p = block_params(N, K)
    gy = rand_bf16((B, N), std=1e-3)
    r = O.block_backward(x, p["W"], gy, gamma=p["gamma"], beta=p["beta"], eps=eps, bias=p["bias"])
    e = O.block_backward(x, p["W"], gy, gamma=p["gamma"], beta=p["beta"], eps=eps, bias=p["bias"],
                         rnd=False)
    for k in ("gx", "gW", "gb", "ggamma", "gbeta", "gz"):
        O.to_bf16_bits(r[k])  # raises unless BF16 values
        tol = 2.0 ** -7 * np.abs(e[k]) + 2e-2 * np.sqrt(np.mean(e[k] ** 2))
        assert np.all(np.abs(r[k] - e[k]) <= tol), k


def test_block_backward_rounding_points_exact_rationals():
    """W = 0 and bias = 0 make z = 0, GELU'(0) = 1/2 and gz = gy / 2 exactly.
    Then gb = R(sum_b gy/2) and gW[n][k] = R(sum_b gy[b][n]/2 * xh[b][k]) with
    xh the ROUNDED LayerNorm output (the pinned forward norm), all exact
    rationals rounded once; gx, ggamma and gbeta are exactly zero.  Using the
    unrounded xh, or rounding inside the batch sum, fails."""
    from test_oracle_pins import rne_bf16_bits, bf16_val  # the forward pins' independent rounding

    B, N, K = 6, 5, 16
    eps = float(np.float32(1e-5))
    x = rand_bf16((B, K), mean=0.1)
    gamma = rand_bf16((K,), std=0.3, mean=1.0)
    beta = rand_bf16((K,), std=0.2)
    W = np.zeros((N, K), dtype=np.uint16)
    bias = np.zeros(N, dtype=np.uint16)
    gy = rand_bf16((B, N), std=0.7)
    r = O.block_backward(x, W, gy, gamma=gamma, beta=beta, eps=eps, bias=bias)
    xh = np.stack([O.norm_bf16(O.NORM_LAYER, x[b], gamma, beta, eps) for b in range(B)])
    for n in range(N):
        s = sum((bf16_val(int(gy[b, n])) / 2 for b in range(B)), Fraction(0))
        assert O.to_bf16_bits(r["gb"][n:n + 1])[0] == rne_bf16_bits(s)
        for k in range(K):
            s = sum((bf16_val(int(gy[b, n])) / 2 * bf16_val(int(xh[b, k])) for b in range(B)), Fraction(0))
            assert O.to_bf16_bits(r["gW"][n, k:k + 1])[0] == rne_bf16_bits(s), (n, k)
    assert np.all(r["gx"] == 0) and np.all(r["ggamma"] == 0) and np.all(r["gbeta"] == 0)
    assert np.array_equal(r["gz"], f64(gy) / 2)


def test_mean_square_grad():
    """g = R(2 y / (B N)): exact scaling when B N is a power of two (compared
    with float64 autograd of mean(y^2)); otherwise one correct rounding of the
    exact rational."""
    from test_oracle_pins import rne_bf16_bits, bf16_val

    y = rand_bf16((4, 16))
    yt = torch.tensor(f64(y), requires_grad=True)
    yt.square().mean().backward()
    assert np.array_equal(f64(O.mean_square_grad(y)), yt.grad.numpy())
    y = rand_bf16((3, 7))
    g = O.mean_square_grad(y)
    for b in range(3):
        for n in range(7):
            assert g[b, n] == rne_bf16_bits(2 * bf16_val(int(y[b, n])) / 21)


def test_chain_backward_matches_autograd_with_rounded_activations():
    """Three blocks, last-block-first: with rnd = 0 the chain equals float64
    autograd of the chain whose forward values are the BF16 block outputs
    (rounding passed straight through in the backward).  Visiting the blocks
    in the wrong order, or handing a block its own input gradient instead of
    the next block's, fails."""
    B, D, L = 3, 24, 3
    eps = float(np.float32(1e-5))
    layers = [block_params(D, D) for _ in range(L)]
    xs = [rand_bf16((B, D))]
    for p in layers:
        xs.append(O.stage(xs[-1], p["W"], norm=O.NORM_LAYER, epi=O.EPI_GELU_TANH, gamma=p["gamma"],
                          beta=p["beta"], bias=p["bias"], eps=eps))
    per, gx = O.chain_backward(xs, layers, eps=eps, rnd=False)

    params = []
    h = torch.tensor(f64(xs[0]), requires_grad=True)
    cur = h
    for i, p in enumerate(layers):
        t = {k: torch.tensor(f64(v), requires_grad=True) for k, v in p.items()}
        params.append(t)
        z = F.layer_norm(cur, (D,), t["gamma"], t["beta"], eps) @ t["W"].T + t["bias"]
        y = F.gelu(z, approximate="tanh")
        # forward value = the stored BF16 output; gradient passes straight through
        cur = y + (torch.tensor(f64(xs[i + 1])) - y).detach()
    gy = torch.tensor(f64(O.mean_square_grad(xs[-1])))
    (cur * gy).sum().backward()
    assert rel_err(gx, h.grad.numpy()) < 1e-11
    for i in range(L):
        for k, kk in (("W", "gW"), ("bias", "gb"), ("gamma", "ggamma"), ("beta", "gbeta")):
            assert rel_err(per[i][kk], params[i][k].grad.numpy()) < 1e-11, (i, k)


def test_given_gz_replaces_only_the_rounding_decision():
    """gz_in = the oracle's own gz reproduces every output bit for bit; a
    different gz_in changes the products (gW, gb, gx) as the definition says:
    gb becomes R(sum_b gz_in) exactly."""
    from test_oracle_pins import rne_bf16_bits, bf16_val

    B, N, K = 4, 24, 32
    eps = float(np.float32(1e-5))
    x = rand_bf16((B, K))
    p = block_params(N, K)
    gy = rand_bf16((B, N), std=0.1)
    r = O.block_backward(x, p["W"], gy, gamma=p["gamma"], beta=p["beta"], eps=eps, bias=p["bias"])
    r2 = O.block_backward(x, p["W"], gy, gamma=p["gamma"], beta=p["beta"], eps=eps, bias=p["bias"],
                          gz_in=O.to_bf16_bits(r["gz"]))
    for k in r:
        assert np.array_equal(r[k], r2[k]), k
    alt = rand_bf16((B, N), std=0.05)
    r3 = O.block_backward(x, p["W"], gy, gamma=p["gamma"], beta=p["beta"], eps=eps, bias=p["bias"],
                          gz_in=alt)
    assert np.array_equal(r3["gz"], r["gz"])
    for n in range(N):
        s = sum((bf16_val(int(alt[b, n])) for b in range(B)), Fraction(0))
        assert O.to_bf16_bits(r3["gb"][n:n + 1])[0] == rne_bf16_bits(s)
