"""CPU oracle for the decode-step weight stream -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  The product library (``weight_gemv_norm_amd``)
never imports, links or calls it, and it never imports the product library.

The arithmetic lives in ``wgn_oracle.c`` (plain C, binary64, sequential sums);
this module compiles it with gcc, loads it with ctypes and marshals numpy arrays.
BF16 and FP16 tensors are passed as ``uint16`` bit patterns.

Every function below follows the definition stated in ``wgn_oracle.c``'s header,
which cites the page passage each step comes from.  Parity status: the norm,
product, epilogue, argmax, decode-attention, 4-bit product and block-backward definitions are pinned by the ``-m "not gpu"``
tests in ``tests/test_oracle_pins.py``, ``tests/test_oracle_attention.py``, ``tests/test_oracle_int4.py`` and
``tests/test_oracle_backward.py`` (closed forms, invariants, exact rational brute force, FP64 autograd
and finite differences); the values for random inputs are "parity unpinned"
beyond the oracle itself, because the pages print no worked numeric example.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wgn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

NORM_NONE, NORM_RMS, NORM_LAYER = 0, 1, 2
EPI_NONE, EPI_GELU_TANH, EPI_SWIGLU = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc -O2 (no fast-math), OpenMP over rows."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", "-std=c11", "-D_GNU_SOURCE", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        D = ctypes.c_double
        I = ctypes.c_int
        lib.wgo_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.wgo_bf16_to_f64.restype = D
        lib.wgo_f64_to_bf16.argtypes = [D]
        lib.wgo_f64_to_bf16.restype = ctypes.c_uint16
        lib.wgo_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.wgo_f16_to_f64.restype = D
        lib.wgo_f64_to_f16.argtypes = [D]
        lib.wgo_f64_to_f16.restype = ctypes.c_uint16
        lib.wgo_gelu_tanh.argtypes = [D]
        lib.wgo_gelu_tanh.restype = D
        lib.wgo_silu.argtypes = [D]
        lib.wgo_silu.restype = D
        lib.wgo_norm_bf16.argtypes = [I, P, P, P, I64, D, P]
        lib.wgo_norm_bf16.restype = None
        lib.wgo_norm_f64.argtypes = [I, P, P, P, I64, D, P]
        lib.wgo_norm_f64.restype = None
        lib.wgo_set_threads.argtypes = [I]
        lib.wgo_set_threads.restype = None
        lib.wgo_max_threads.argtypes = []
        lib.wgo_max_threads.restype = I
        lib.wgo_matvec.argtypes = [P, I64, I64, P, P]
        lib.wgo_matvec.restype = None
        lib.wgo_matvec_rows.argtypes = [P, I64, P, I64, P, P]
        lib.wgo_matvec_rows.restype = None
        lib.wgo_stage.argtypes = [I, I, I64, I64, I64, P, I64, P, P, D, P, P, P, P, I64,
                                  P, I64, P, P]
        lib.wgo_stage.restype = None
        lib.wgo_lmhead_argmax.argtypes = [I, P, I64, P, D, P, I64, I64, I64, P, P, P]
        lib.wgo_lmhead_argmax.restype = None
        lib.wgo_rmsnorm_rows_f16.argtypes = [P, I64, P, D, P, I64, I64, I64]
        lib.wgo_rmsnorm_rows_f16.restype = None
        lib.wgo_decode_attention.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, D, P, P]
        lib.wgo_decode_attention.restype = None
        lib.wgo_matvec_int4.argtypes = [P, P, P, I64, I64, P, I64, I64, P, P]
        lib.wgo_matvec_int4.restype = None
        lib.wgo_gelu_tanh_grad.argtypes = [D]
        lib.wgo_gelu_tanh_grad.restype = D
        lib.wgo_mean_square_grad.argtypes = [P, I64, I64, I64, P, I64]
        lib.wgo_mean_square_grad.restype = None
        lib.wgo_block_backward.argtypes = [I64, I64, I64, P, I64, P, P, D, P, P, P, I64, P, I,
                                           P, P, P, P, P, P]
        lib.wgo_block_backward.restype = None
        _lib = lib
        return lib


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def set_threads(n: int) -> None:
    _load().wgo_set_threads(int(n))


def max_threads() -> int:
    return int(_load().wgo_max_threads())


# ------------------------------------------------------------------ scalars
def bf16_to_f64(h: int) -> float:
    return _load().wgo_bf16_to_f64(int(h))


def f64_to_bf16(v: float) -> int:
    return int(_load().wgo_f64_to_bf16(float(v)))


def f16_to_f64(h: int) -> float:
    return _load().wgo_f16_to_f64(int(h))


def f64_to_f16(v: float) -> int:
    return int(_load().wgo_f64_to_f16(float(v)))


def gelu_tanh(z: float) -> float:
    return _load().wgo_gelu_tanh(float(z))


def silu(z: float) -> float:
    return _load().wgo_silu(float(z))


def bf16_array_to_f64(a) -> np.ndarray:
    """Exact decode of a uint16 BF16 array (vectorised, independent of the C path)."""
    a = np.asarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------- vectors
def norm_bf16(norm: int, x, gamma=None, beta=None, eps: float = 1e-6):
    x = _u16(x)
    K = x.shape[-1]
    out = np.empty(K, dtype=np.uint16)
    g = None if gamma is None else _u16(gamma)
    b = None if beta is None else _u16(beta)
    _load().wgo_norm_bf16(norm, _ptr(x), _ptr(g), _ptr(b), K, float(eps), _ptr(out))
    return out


def norm_f64(norm: int, x, gamma=None, beta=None, eps: float = 1e-6):
    x = _u16(x)
    K = x.shape[-1]
    out = np.empty(K, dtype=np.float64)
    g = None if gamma is None else _u16(gamma)
    b = None if beta is None else _u16(beta)
    _load().wgo_norm_f64(norm, _ptr(x), _ptr(g), _ptr(b), K, float(eps), _ptr(out))
    return out


def matvec(W, xh):
    W = _u16(W)
    xh = _u16(xh)
    N, K = W.shape
    assert xh.shape == (K,)
    acc = np.empty(N, dtype=np.float64)
    _load().wgo_matvec(_ptr(W), N, K, _ptr(xh), _ptr(acc))
    return acc


def matvec_rows(W, rows, xh):
    """Rows of the product for selected row indices (W may be a large array)."""
    W = _u16(W)
    N, K = W.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < N)
    acc = np.empty(rows.size, dtype=np.float64)
    _load().wgo_matvec_rows(_ptr(W), K, _ptr(rows), rows.size, _ptr(_u16(xh)), _ptr(acc))
    return acc


def stage(x, W, *, norm=NORM_NONE, epi=EPI_NONE, gamma=None, beta=None, eps=1e-6,
          W_up=None, bias=None, residual=None, want_xh=False, want_acc=False):
    """One norm-fused product stage.  x: [B][K] uint16 BF16; returns y [B][N] uint16."""
    x = _u16(np.atleast_2d(x))
    W = _u16(W)
    B, K = x.shape
    N, K2 = W.shape
    assert K == K2
    if epi == EPI_SWIGLU:
        assert W_up is not None and W_up.shape == W.shape
        W_up = _u16(W_up)
    res = None
    if residual is not None:
        res = _u16(np.atleast_2d(residual))
        assert res.shape == (B, N)
    y = np.empty((B, N), dtype=np.uint16)
    xh = np.empty((B, K), dtype=np.uint16) if want_xh else None
    acc = np.empty((B, N), dtype=np.float64) if want_acc else None
    _load().wgo_stage(norm, epi, N, K, B, _ptr(x), K,
                      _ptr(None if gamma is None else _u16(gamma)),
                      _ptr(None if beta is None else _u16(beta)), float(eps),
                      _ptr(W), _ptr(W_up), _ptr(None if bias is None else _u16(bias)),
                      _ptr(res), N, _ptr(y), N, _ptr(xh), _ptr(acc))
    out = [y]
    if want_xh:
        out.append(xh)
    if want_acc:
        out.append(acc)
    return out[0] if len(out) == 1 else tuple(out)


def lmhead_argmax(h, g, W, *, eps=1e-6, norm=NORM_RMS, want_logits=False):
    """Final norm + LM head + argmax.  h: [B][K] uint16; returns (idx int32[B], max f64[B][, logits])."""
    h = _u16(np.atleast_2d(h))
    W = _u16(W)
    B, K = h.shape
    V, K2 = W.shape
    assert K == K2
    idx = np.empty(B, dtype=np.int32)
    mx = np.empty(B, dtype=np.float64)
    logits = np.empty((B, V), dtype=np.float64) if want_logits else None
    _load().wgo_lmhead_argmax(norm, _ptr(h), K, _ptr(None if g is None else _u16(g)), float(eps),
                              _ptr(W), V, K, B, _ptr(idx), _ptr(mx), _ptr(logits))
    if want_logits:
        return idx, mx, logits
    return idx, mx


def rmsnorm_rows_f16(x, g, eps=1e-6):
    """Standalone RMSNorm over FP16 rows (uint16 bit patterns)."""
    x = _u16(np.atleast_2d(x))
    R, K = x.shape
    y = np.empty((R, K), dtype=np.uint16)
    _load().wgo_rmsnorm_rows_f16(_ptr(x), K, _ptr(_u16(g)), float(eps), _ptr(y), K, R, K)
    return y


def decode_attention(q, k_new, v_new, k_cache, v_cache, pos, scale=None, want_f64=False):
    """One new token of grouped-query attention over a static cache.

    q [B][Hq][D], k_new/v_new [B][Hkv][D], caches [B][Hkv][S][D] (uint16 BF16
    bits), pos int32 [B].  The caches are not modified: updated copies are
    returned.  scale defaults to 1/sqrt(D).  Returns (out, k_cache', v_cache')
    and, with want_f64, the un-rounded outputs as a fourth item.
    """
    q, k_new, v_new = _u16(q), _u16(k_new), _u16(v_new)
    kc, vc = _u16(k_cache).copy(), _u16(v_cache).copy()
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    B, Hq, D = q.shape
    B2, Hkv, S, D2 = kc.shape
    assert B2 == B and D2 == D and vc.shape == kc.shape and Hq % Hkv == 0
    assert k_new.shape == (B, Hkv, D) and v_new.shape == (B, Hkv, D) and pos.shape == (B,)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, Hq, D), dtype=np.uint16)
    of = np.empty((B, Hq, D), dtype=np.float64) if want_f64 else None
    _load().wgo_decode_attention(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(kc), _ptr(vc), _ptr(pos),
                                 B, Hq, Hkv, S, D, float(scale), _ptr(out), _ptr(of))
    if want_f64:
        return out, kc, vc, of
    return out, kc, vc


def matvec_int4(W4, scales, zeros, x, want_acc=False):
    """4-bit product: W4 uint8 [N][K/2] (low nibble = even k), scales/zeros
    uint16 BF16 bits [N][K/128], x uint16 [B][K].  Returns y uint16 [B][N]
    (and the binary64 sums with want_acc)."""
    W4 = np.ascontiguousarray(W4, dtype=np.uint8)
    x = _u16(np.atleast_2d(x))
    N, K2 = W4.shape
    B, K = x.shape
    assert K2 * 2 == K and K % 128 == 0
    sc, zr = _u16(scales), _u16(zeros)
    assert sc.shape == (N, K // 128) and zr.shape == (N, K // 128)
    y = np.empty((B, N), dtype=np.uint16)
    acc = np.empty((B, N), dtype=np.float64) if want_acc else None
    _load().wgo_matvec_int4(_ptr(W4), _ptr(sc), _ptr(zr), N, K, _ptr(x), K, B, _ptr(y), _ptr(acc))
    return (y, acc) if want_acc else y


# ------------------------------------------------------------------ backward
def gelu_tanh_grad(z: float) -> float:
    return _load().wgo_gelu_tanh_grad(float(z))


def mean_square_grad(y):
    """Gradient of mean(y^2) over a [B][N] BF16 output: R(2 y / (B N)), uint16 bits."""
    y = _u16(np.atleast_2d(y))
    B, N = y.shape
    g = np.empty((B, N), dtype=np.uint16)
    _load().wgo_mean_square_grad(_ptr(y), N, N, B, _ptr(g), N)
    return g


def block_backward(x, W, gy, *, gamma=None, beta=None, eps=1e-5, bias=None, rnd=True, gz_in=None):
    """Backward of one LayerNorm -> Linear(+bias) -> GELU-tanh block.

    x [B][K], W [N][K]: uint16 BF16; gy [B][N]: uint16 BF16 or float64 values.
    Returns a dict of binary64
    arrays: gx [B][K], gW [N][K], gb [N] (bias given), ggamma and gbeta [K]
    (gamma / beta given), gz [B][N].  With rnd=True every one of them holds
    BF16 values (convert with ``to_bf16_bits``).  gz_in ([B][N], uint16 BF16
    or float64): a rounding decision taken elsewhere; the products and the
    norm backward then start from it (the returned gz is still the oracle's)."""
    x = _u16(np.atleast_2d(x))
    W = _u16(W)
    gy = np.atleast_2d(gy)
    gy = bf16_array_to_f64(gy) if gy.dtype == np.uint16 else np.ascontiguousarray(gy, dtype=np.float64)
    B, K = x.shape
    N, K2 = W.shape
    assert K == K2 and gy.shape == (B, N)
    out = {"gx": np.empty((B, K)), "gW": np.empty((N, K)), "gz": np.empty((B, N))}
    out["gb"] = np.empty(N) if bias is not None else None
    out["ggamma"] = np.empty(K) if gamma is not None else None
    out["gbeta"] = np.empty(K) if beta is not None else None
    if gz_in is not None:
        gz_in = np.atleast_2d(gz_in)
        gz_in = bf16_array_to_f64(gz_in) if gz_in.dtype == np.uint16 else np.ascontiguousarray(gz_in, np.float64)
        assert gz_in.shape == (B, N)
    _load().wgo_block_backward(N, K, B, _ptr(x), K,
                               _ptr(None if gamma is None else _u16(gamma)),
                               _ptr(None if beta is None else _u16(beta)), float(eps),
                               _ptr(W), _ptr(None if bias is None else _u16(bias)),
                               _ptr(gy), N, _ptr(gz_in), 1 if rnd else 0,
                               _ptr(out["gx"]), _ptr(out["gW"]), _ptr(out["gb"]),
                               _ptr(out["ggamma"]), _ptr(out["gbeta"]), _ptr(out["gz"]))
    return {k: v for k, v in out.items() if v is not None}


def to_bf16_bits(a) -> np.ndarray:
    """BF16 bit patterns of binary64 values that are BF16 values (exact)."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    f = a.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), a, equal_nan=True), "not BF16 values"
    u = f.view(np.uint32)
    assert not np.any(u & 0xFFFF), "not BF16 values"
    return (u >> 16).astype(np.uint16)


def chain_backward(xs, layers, gy_last=None, *, eps=1e-5, rnd=True):
    """Backward of a chain of LayerNorm -> Linear -> GELU-tanh blocks, last block first.

    xs[i]: [B][K_i] uint16 input of block i (the forward's saved activations);
    xs[len(layers)]: the chain output, used for the mean-square loss when
    gy_last is None.  layers[i]: dict with W, and optionally bias, gamma, beta
    (uint16).  Returns (per-block list of block_backward dicts, gx of the chain
    input).  Between blocks the input gradient is BF16 (rnd=True) or binary64."""
    gy = mean_square_grad(xs[-1]) if gy_last is None else gy_last
    out = [None] * len(layers)
    for i in range(len(layers) - 1, -1, -1):
        L = layers[i]
        r = block_backward(xs[i], L["W"], gy, gamma=L.get("gamma"), beta=L.get("beta"), eps=eps,
                           bias=L.get("bias"), rnd=rnd)
        out[i] = r
        gy = to_bf16_bits(r["gx"]) if rnd else r["gx"]
    return out, out[0]["gx"]
