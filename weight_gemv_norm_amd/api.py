"""Thin Python binding of libwgn.so with the C-ABI's names.

torch tensors are used only as device memory and streams: every step of the
computation runs in the library's HIP kernels.  There is no fallback path: if
the library is missing or a call fails, these functions raise.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence

import torch

from . import _lib as L
from ._lib import (EPI_ARGMAX, EPI_GELU_TANH, EPI_NONE, EPI_SWIGLU, NORM_LAYER,  # noqa: F401
                   NORM_NONE, NORM_RMS, BF16, FP16, AttnStage, ChainOpts, Grad, Plan, Stage, WgnError)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _row_stride(t: torch.Tensor) -> int:
    if t.dim() == 1:
        return t.shape[0]
    assert t.dim() == 2 and t.stride(1) == 1, "activations must be [batch][stride] with unit inner stride"
    return t.stride(0)


def _need(cond: bool, msg: str) -> None:
    """Argument check before any call into the library (the C ABI cannot see
    tensor sizes, so a mismatch would read or write out of bounds)."""
    if not cond:
        raise ValueError(msg)


def _same_device(*ts: torch.Tensor) -> None:
    dev = ts[0].device
    _need(dev.type == "cuda", "tensors must be on the GPU")
    _need(all(t.device == dev for t in ts), "tensors must be on one device")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def make_stage(W: torch.Tensor, x: torch.Tensor, y: torch.Tensor, *, norm: int = NORM_NONE,
               eps: float = 1e-6, gamma: Optional[torch.Tensor] = None,
               beta: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
               epi: int = EPI_NONE, W_up: Optional[torch.Tensor] = None,
               residual: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
               maxval: Optional[torch.Tensor] = None, pre: Optional[torch.Tensor] = None) -> Stage:
    """Describe y = R(residual + epi(W . norm(x) + bias)) over device tensors.

    pre: FP32 [batch][N] that a GELU stage fills with its pre-activation (the
    wgn_stage `logits` field of a GELU stage), for the backward pass."""
    assert logits is None or pre is None, "logits (argmax) and pre (GELU) are one field"
    if pre is not None:
        logits = pre
    assert W.dim() == 2 and W.is_contiguous()
    N, K = W.shape
    s = Stage()
    s.N, s.K = N, K
    s.W = _ptr(W)
    s.W_up = _ptr(W_up)
    s.bias = _ptr(bias)
    s.norm = norm
    s.eps = eps
    s.gamma = _ptr(gamma)
    s.beta = _ptr(beta)
    s.epi = epi
    s.x = _ptr(x)
    s.x_stride = _row_stride(x)
    s.residual = _ptr(residual)
    s.res_stride = _row_stride(residual) if residual is not None else 0
    s.y = _ptr(y)
    s.y_stride = _row_stride(y) if epi != EPI_ARGMAX else 0
    s.logits = _ptr(logits)
    s.maxval = _ptr(maxval)
    return s


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Zero-filled device workspace (256-byte aligned)."""
    t = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


def device_cu_count() -> int:
    return int(L.lib().wgn_device_cu_count())


def gemv_norm_workspace_bytes(stage: Stage, batch: int) -> int:
    return int(L.lib().wgn_gemv_norm_workspace_bytes(ctypes.byref(stage), batch))


def gemv_norm(stage: Stage, batch: int, ws: Optional[torch.Tensor] = None, stream=None) -> None:
    st = L.lib().wgn_gemv_norm(ctypes.byref(stage), batch, _ptr(ws),
                               0 if ws is None else ws.numel(), _stream(stream))
    L.check(st, "wgn_gemv_norm")


def gemm_norm_workspace_bytes(stage: Stage, batch: int) -> int:
    return int(L.lib().wgn_gemm_norm_workspace_bytes(ctypes.byref(stage), batch))


def gemm_norm(stage: Stage, batch: int, ws: Optional[torch.Tensor] = None, stream=None, device="cuda") -> None:
    """wgn_gemm_norm: one stage at batch 1-128 on the matrix cores (tiled product; RMSNorm as a pass of its own)."""
    if ws is None:
        ws = workspace(gemm_norm_workspace_bytes(stage, batch), device)
    st = L.lib().wgn_gemm_norm(ctypes.byref(stage), batch, _ptr(ws), ws.numel(), _stream(stream))
    L.check(st, "wgn_gemm_norm")


def lmhead_argmax_workspace_bytes(batch: int) -> int:
    return int(L.lib().wgn_lmhead_argmax_workspace_bytes(batch))


def lmhead_argmax(h: torch.Tensor, gamma: Optional[torch.Tensor], eps: float, W_lm: torch.Tensor,
                  idx_out: torch.Tensor, max_out: Optional[torch.Tensor] = None,
                  logits_out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                  stream=None) -> None:
    h2 = h if h.dim() == 2 else h.view(1, -1)
    B, K = h2.shape
    V = W_lm.shape[0]
    if ws is None:
        ws = workspace(lmhead_argmax_workspace_bytes(B), h.device)
    st = L.lib().wgn_lmhead_argmax(_ptr(h2), _row_stride(h2), B, K, _ptr(gamma), eps, _ptr(W_lm), V,
                                   _ptr(idx_out), _ptr(max_out), _ptr(logits_out), _ptr(ws), ws.numel(),
                                   _stream(stream))
    L.check(st, "wgn_lmhead_argmax")


def lmhead_argmax_static(h: torch.Tensor, gamma: Optional[torch.Tensor], eps: float, W_lm: torch.Tensor,
                         idx_out: torch.Tensor, max_out: Optional[torch.Tensor] = None,
                         logits_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """wgn_lmhead_argmax_static: the LM head + argmax with the library's fixed
    scratch; allocates nothing (no workspace tensor either)."""
    h2 = h if h.dim() == 2 else h.view(1, -1)
    B, K = h2.shape
    V = W_lm.shape[0]
    st = L.lib().wgn_lmhead_argmax_static(_ptr(h2), _row_stride(h2), B, K, _ptr(gamma), eps, _ptr(W_lm), V,
                                          _ptr(idx_out), _ptr(max_out), _ptr(logits_out), _stream(stream))
    L.check(st, "wgn_lmhead_argmax_static")


def rmsnorm_rows(x: torch.Tensor, gamma: torch.Tensor, eps: float, y: torch.Tensor, stream=None) -> None:
    assert x.dim() == 2 and x.dtype in (torch.float16, torch.bfloat16) and y.dtype == x.dtype
    dtype = FP16 if x.dtype == torch.float16 else BF16
    st = L.lib().wgn_rmsnorm_rows(_ptr(x), _row_stride(x), _ptr(gamma), eps, _ptr(y), _row_stride(y),
                                  x.shape[0], x.shape[1], dtype, _stream(stream))
    L.check(st, "wgn_rmsnorm_rows")


def gemv_int4(x: torch.Tensor, W4: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor, y: torch.Tensor,
              stream=None) -> None:
    """wgn_gemv_int4: x [B][K] BF16, W4 [N][K/2] uint8 (low nibble = even k),
    scales/zeros [N][K/128] BF16, y [B][N] BF16."""
    x2 = x if x.dim() == 2 else x.view(1, -1)
    y2 = y if y.dim() == 2 else y.view(1, -1)
    B, K = x2.shape
    _need(W4.dim() == 2 and W4.dtype == torch.uint8 and W4.is_contiguous(), "W4 must be a contiguous uint8 [N][K/2]")
    N = W4.shape[0]
    _need(W4.shape[1] * 2 == K, "W4 holds %d codes per row, x has K = %d" % (W4.shape[1] * 2, K))
    _need(K % 128 == 0, "K must be a multiple of 128")
    for name, t in (("scales", scales), ("zeros", zeros)):
        _need(t.dtype == torch.bfloat16 and t.is_contiguous() and tuple(t.shape) == (N, K // 128),
              "%s must be a contiguous BF16 [N][K/128] = [%d][%d], got %s %s" % (name, N, K // 128,
                                                                         tuple(t.shape), t.dtype))
    _need(x2.dtype == torch.bfloat16 and y2.dtype == torch.bfloat16, "x and y must be BF16")
    _need(y2.shape[0] == B and y2.shape[1] >= N, "y must be [batch][>= N]")
    _same_device(x2, W4, scales, zeros, y2)
    st = L.lib().wgn_gemv_int4(_ptr(x2), _row_stride(x2), B, K, _ptr(W4), _ptr(scales), _ptr(zeros), N, _ptr(y2),
                               _row_stride(y2), _stream(stream))
    L.check(st, "wgn_gemv_int4")


def stream_read(src: torch.Tensor, grid: int, threads: int = 256, depth: int = 8,
                sink: Optional[torch.Tensor] = None, stream=None) -> None:
    """wgn_stream_read: one plain streaming read of src's bytes (the measured
    read ceiling); sink is a device int32 tensor the kernel may write."""
    assert src.is_contiguous()
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=src.device)
    nbytes = src.numel() * src.element_size()
    st = L.lib().wgn_stream_read(_ptr(src), nbytes, grid, threads, depth, _ptr(sink), _stream(stream))
    L.check(st, "wgn_stream_read")


def decode_attention_workspace_bytes(batch: int, q_heads: int, kv_heads: int, slots: int,
                                     head_dim: int = 128) -> int:
    return int(L.lib().wgn_decode_attention_workspace_bytes(batch, q_heads, kv_heads, slots, head_dim))


def decode_attention(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                     v_cache: torch.Tensor, pos: torch.Tensor, out: torch.Tensor, scale: Optional[float] = None,
                     ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """wgn_decode_attention over contiguous device tensors: q/out [B][Hq][D],
    k_new/v_new [B][Hkv][D], caches [B][Hkv][S][D] (all BF16), pos int32 [B]."""
    _need(q.dim() == 3 and k_cache.dim() == 4, "q must be [B][Hq][D] and k_cache [B][Hkv][S][D]")
    B, Hq, D = q.shape
    _, Hkv, S, _ = k_cache.shape
    _need(tuple(k_cache.shape) == (B, Hkv, S, D), "k_cache must be [%d][Hkv][S][%d]" % (B, D))
    _need(tuple(v_cache.shape) == tuple(k_cache.shape), "v_cache must have k_cache's shape")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(tuple(t.shape) == (B, Hkv, D), "%s must be [%d][%d][%d], got %s" % (name, B, Hkv, D, tuple(t.shape)))
    _need(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    _need(tuple(pos.shape) == (B,) and pos.dtype == torch.int32, "pos must be int32 [batch]")
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("out", out)):
        _need(t.dtype == torch.bfloat16, "%s must be BF16" % name)
    for t in (q, k_new, v_new, k_cache, v_cache, pos, out):
        _need(t.is_contiguous(), "every tensor must be contiguous")
    _same_device(q, k_new, v_new, k_cache, v_cache, pos, out)
    if scale is None:
        scale = D ** -0.5
    if ws is None:
        ws = workspace(decode_attention_workspace_bytes(B, Hq, Hkv, S, D), q.device)
    st = L.lib().wgn_decode_attention(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(pos),
                                      B, Hq, Hkv, S, D, scale, _ptr(out), _ptr(ws), ws.numel(), _stream(stream))
    L.check(st, "wgn_decode_attention")


def make_attn_stage(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                    v_cache: torch.Tensor, pos: torch.Tensor, out: torch.Tensor,
                    scale: Optional[float] = None) -> AttnStage:
    """A wgn_attn_stage (attention inside a chain) over device tensors: q/out
    [B][Hq*D] (or [B][Hq][D]), k_new/v_new [B][Hkv*D], caches [B][Hkv][S][D]
    (all BF16, rows may be strided), pos int32 [B]."""
    _need(k_cache.dim() == 4, "k_cache must be [B][Hkv][S][D]")
    B, Hkv, S, D = k_cache.shape
    _need(tuple(v_cache.shape) == tuple(k_cache.shape), "v_cache must have k_cache's shape")
    q2, o2, k2, v2 = (t.reshape(t.shape[0], -1) if t.dim() == 3 else t for t in (q, out, k_new, v_new))
    _need(q2.shape[0] == B and q2.shape[1] % D == 0, "q must be [%d][Hq*%d]" % (B, D))
    _need(tuple(o2.shape) == tuple(q2.shape), "out must have q's shape")
    for name, t in (("k_new", k2), ("v_new", v2)):
        _need(tuple(t.shape) == (B, Hkv * D), "%s must be [%d][%d]" % (name, B, Hkv * D))
    _need(tuple(pos.shape) == (B,) and pos.dtype == torch.int32, "pos must be int32 [batch]")
    for name, t in (("q", q2), ("k_new", k2), ("v_new", v2), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("out", o2)):
        _need(t.dtype == torch.bfloat16, "%s must be BF16" % name)
        _need(t.stride(-1) == 1, "%s must have unit stride along its rows" % name)
    for t in (k_cache, v_cache, pos):
        _need(t.is_contiguous(), "caches and pos must be contiguous")
    _same_device(q2, k2, v2, k_cache, v_cache, pos, o2)
    a = AttnStage()
    a.q, a.q_stride = _ptr(q2), _row_stride(q2)
    a.k_new, a.k_stride = _ptr(k2), _row_stride(k2)
    a.v_new, a.v_stride = _ptr(v2), _row_stride(v2)
    a.k_cache, a.v_cache, a.pos = _ptr(k_cache), _ptr(v_cache), _ptr(pos)
    a.out, a.out_stride = _ptr(o2), _row_stride(o2)
    a.q_heads, a.kv_heads, a.slots, a.head_dim = q2.shape[1] // D, Hkv, S, D
    a.scale = D ** -0.5 if scale is None else scale
    return a


PATH_AUTO, PATH_VECTOR, PATH_MATRIX, PATH_TILED = 0, 1, 2, 3


def _opts(mode: int, grid: int, trace: bool = False, path: int = PATH_AUTO, fuse: bool = True,
          ring: int = 0) -> ChainOpts:
    o = ChainOpts()
    o.mode = mode
    o.grid = grid
    o.trace = 1 if trace else 0
    o.path = path
    o.no_fuse = 0 if fuse else 1
    o.ring = ring
    return o


def chain_workspace_bytes(stages: Sequence[Stage], batch: int, mode: int = 0, grid: int = 0,
                          path: int = PATH_AUTO) -> int:
    arr = L.stage_array(stages)
    o = _opts(mode, grid, path=path)
    return int(L.lib().wgn_chain_workspace_bytes(arr, len(stages), batch, ctypes.byref(o)))


class Chain:
    """A planned chain (wgn_chain_create); run() enqueues one pass."""

    def __init__(self, stages: Sequence[Stage], batch: int, mode: int = 0, grid: int = 0,
                 ws: Optional[torch.Tensor] = None, stream=None, device="cuda", trace: bool = False,
                 path: int = PATH_AUTO, fuse: bool = True, ring: int = 0,
                 attn: Optional[Sequence] = None):
        """ring: 0 chooses the streaming waves' block-buffer ring by the chain's
        shape; 1..3 force ring 0..2 (wgn_chain_opts.ring).  attn: (before,
        AttnStage) pairs, attention items run before stage `before`
        (wgn_chain_create_attn)."""
        self._arr = L.stage_array(stages)
        self.n_stages = len(stages)
        self.batch = batch
        o = _opts(mode, grid, trace, path, fuse, ring)
        attn = list(attn or [])
        self._att = (L.AttnStage * max(1, len(attn)))()
        self._before = (ctypes.c_int32 * max(1, len(attn)))()
        for i, (before, a) in enumerate(attn):
            self._before[i] = before
            self._att[i] = a
        na = len(attn)
        need = L.lib().wgn_chain_attn_workspace_bytes(self._arr, len(stages), self._att, self._before, na, batch,
                                                      ctypes.byref(o))
        if need == 0:
            # planning failed: let create report the precise status
            need = 256
        self.ws = ws if ws is not None else workspace(need, device)
        h = ctypes.c_void_p()
        st = L.lib().wgn_chain_create_attn(self._arr, len(stages), self._att, self._before, na, batch,
                                           ctypes.byref(o), _ptr(self.ws), self.ws.numel(), _stream(stream),
                                           ctypes.byref(h))
        L.check(st, "wgn_chain_create_attn" if na else "wgn_chain_create")
        self._h = h

    def run(self, stream=None, plan: Optional[Plan] = None, side=None) -> None:
        """One pass; with a prefetch plan (mode-1 chains), touch passes run on `side`."""
        if plan is None:
            L.check(L.lib().wgn_chain_run(self._h, _stream(stream)), "wgn_chain_run")
        else:
            L.check(L.lib().wgn_chain_run_plan(self._h, ctypes.byref(plan), _stream(stream),
                                               _stream(side) if side is not None else None),
                    "wgn_chain_run_plan")

    def tune_plan(self, side, reps: int = 15, stream=None) -> Plan:
        """wgn_chain_plan_tune: measure prefetch candidates against plain runs."""
        out = Plan()
        L.check(L.lib().wgn_chain_plan_tune(self._h, _stream(stream), _stream(side), reps, ctypes.byref(out)),
                "wgn_chain_plan_tune")
        return out

    def check(self, stream=None) -> None:
        L.check(L.lib().wgn_chain_check(self._h, _stream(stream)), "wgn_chain_check")

    def set_wait_us(self, us: int) -> None:
        """wgn_chain_set_wait_us: bound of the in-kernel waits of later runs (-1 = default)."""
        L.check(L.lib().wgn_chain_set_wait_us(self._h, int(us)), "wgn_chain_set_wait_us")

    @property
    def num_phases(self) -> int:
        return int(L.lib().wgn_chain_num_phases(self._h))

    @property
    def grid(self) -> int:
        return int(L.lib().wgn_chain_grid(self._h))

    @property
    def ring(self) -> int:
        return int(L.lib().wgn_chain_ring(self._h))

    def trace(self, stream=None):
        """Timestamps of the last run, shape [phases][grid][TRACE_POINTS], in 10 ns ticks."""
        import numpy as np
        n = self.num_phases * self.grid * L.TRACE_POINTS
        out = np.zeros(n, dtype=np.uint64)
        st = L.lib().wgn_chain_trace(self._h, _stream(stream),
                                     out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), n)
        L.check(st, "wgn_chain_trace")
        return out.reshape(self.num_phases, self.grid, L.TRACE_POINTS)

    def stage_phases(self) -> List[int]:
        out = (ctypes.c_int32 * self.n_stages)()
        L.check(L.lib().wgn_chain_stage_phases(self._h, out), "wgn_chain_stage_phases")
        return list(out)

    def close(self) -> None:
        if getattr(self, "_h", None):
            L.lib().wgn_chain_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def layer_chain(stages: Sequence[Stage], batch: int, mode: int = 0, grid: int = 0,
                ws: Optional[torch.Tensor] = None, stream=None, device="cuda", path: int = PATH_AUTO,
                plan: Optional[Plan] = None, side=None) -> None:
    """wgn_layer_chain: plan, run and release a chain in one call (a prefetch
    plan needs mode 1 and a side stream)."""
    arr = L.stage_array(stages)
    o = _opts(mode, grid, path=path)
    if ws is None:
        nbytes = (L.lib().wgn_workspace_bytes(arr, len(stages), batch, 0) if (batch > 16 or path == PATH_TILED) else
                  L.lib().wgn_chain_workspace_bytes(arr, len(stages), batch, ctypes.byref(o)))
        ws = workspace(nbytes, device)
    st = L.lib().wgn_layer_chain(arr, len(stages), batch, ctypes.byref(o),
                                 ctypes.byref(plan) if plan is not None else None, _ptr(ws), ws.numel(),
                                 _stream(stream), _stream(side) if side is not None else None)
    L.check(st, "wgn_layer_chain")


def workspace_bytes(stages: Sequence[Stage], batch: int, V: int = 0) -> int:
    """wgn_workspace_bytes: one size serving every call on these stages (and an LM head of V rows)."""
    arr = L.stage_array(stages)
    return int(L.lib().wgn_workspace_bytes(arr, len(stages), batch, int(V)))


def plan_tune(stages: Sequence[Stage], batch: int, side, ws: Optional[torch.Tensor] = None, stream=None,
              device="cuda") -> Plan:
    """wgn_plan_tune: tune a prefetch plan for a stage list (one-launch-per-phase chain)."""
    arr = L.stage_array(stages)
    if ws is None:
        ws = workspace(workspace_bytes(stages, batch), device)
    out = Plan()
    st = L.lib().wgn_plan_tune(arr, len(stages), batch, ctypes.byref(out), _ptr(ws), ws.numel(), _stream(stream),
                               _stream(side))
    L.check(st, "wgn_plan_tune")
    return out


def partition_selftest(stages: Sequence[Stage], batch: int, grid: int, path: int = PATH_AUTO,
                       fuse: bool = True) -> int:
    arr = L.stage_array(stages)
    o = _opts(0, grid, path=path, fuse=fuse)
    return int(L.lib().wgn_partition_selftest(arr, len(stages), batch, ctypes.byref(o)))


def plan_phases(stages: Sequence[Stage], batch: int, grid: int = 0, path: int = PATH_AUTO, fuse: bool = True):
    """Host-only planning: (number of phases, phase of each stage's output)."""
    arr = L.stage_array(stages)
    o = _opts(0, grid, path=path, fuse=fuse)
    out = (ctypes.c_int32 * len(stages))()
    n = int(L.lib().wgn_plan_phases(arr, len(stages), batch, ctypes.byref(o), out))
    if n < 0:
        raise WgnError(n, "wgn_plan_phases")
    return n, list(out)


def first_wave_of_unit(u: int, units: int, waves: int) -> int:
    return int(L.lib().wgn_first_wave_of_unit(u, units, waves))


# ------------------------------------------------------------------ backward
def make_grad(gW: torch.Tensor, gbias: Optional[torch.Tensor] = None, ggamma: Optional[torch.Tensor] = None,
              gbeta: Optional[torch.Tensor] = None, gy: Optional[torch.Tensor] = None,
              gz: Optional[torch.Tensor] = None) -> Grad:
    """Describe one block's gradient outputs (wgn_grad)."""
    g = Grad()
    g.gW, g.gbias, g.ggamma, g.gbeta, g.gy, g.gz = (_ptr(gW), _ptr(gbias), _ptr(ggamma), _ptr(gbeta), _ptr(gy),
                                                    _ptr(gz))
    return g


def backward_workspace_bytes(stages: Sequence[Stage], batch: int) -> int:
    return int(L.lib().wgn_backward_workspace_bytes(L.stage_array(stages), len(stages), batch))


class Backward:
    """A planned backward pass (wgn_backward_create); run() enqueues one pass."""

    def __init__(self, stages: Sequence[Stage], batch: int, grads: Sequence[Grad],
                 g_out: Optional[torch.Tensor] = None, g_in: Optional[torch.Tensor] = None,
                 ws: Optional[torch.Tensor] = None, stream=None, device="cuda"):
        assert len(grads) == len(stages)
        self._arr = L.stage_array(stages)
        self._grads = (Grad * len(grads))(*grads)
        need = L.lib().wgn_backward_workspace_bytes(self._arr, len(stages), batch)
        self.ws = ws if ws is not None else workspace(max(int(need), 256), device)
        h = ctypes.c_void_p()
        st = L.lib().wgn_backward_create(self._arr, len(stages), batch, self._grads, _ptr(g_out),
                                         _row_stride(g_out) if g_out is not None else 0, _ptr(g_in),
                                         _row_stride(g_in) if g_in is not None else 0, _ptr(self.ws),
                                         self.ws.numel(), _stream(stream), ctypes.byref(h))
        L.check(st, "wgn_backward_create")
        self._h = h

    def run(self, prefetch: bool = True, stream=None) -> None:
        L.check(L.lib().wgn_backward_run(self._h, 1 if prefetch else 0, _stream(stream)), "wgn_backward_run")

    def check(self, stream=None) -> None:
        L.check(L.lib().wgn_backward_check(self._h, _stream(stream)), "wgn_backward_check")

    def set_wait_us(self, us: int) -> None:
        L.check(L.lib().wgn_backward_set_wait_us(self._h, int(us)), "wgn_backward_set_wait_us")

    @property
    def grid(self) -> int:
        return int(L.lib().wgn_backward_grid(self._h))

    def set_trace(self, buf: Optional[torch.Tensor]) -> None:
        """Record per-block timestamps of later runs into buf (int64 device
        tensor of n_stages x grid x 5 slots); None stops."""
        L.check(L.lib().wgn_backward_set_trace(self._h, _ptr(buf), 0 if buf is None else buf.numel()),
                "wgn_backward_set_trace")

    def close(self) -> None:
        if getattr(self, "_h", None):
            L.lib().wgn_backward_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def chain_backward(stages: Sequence[Stage], batch: int, grads: Sequence[Grad], g_out: Optional[torch.Tensor] = None,
                   g_in: Optional[torch.Tensor] = None, prefetch: bool = True, ws: Optional[torch.Tensor] = None,
                   stream=None, device="cuda") -> None:
    """wgn_chain_backward: create, run and release a backward pass in one call."""
    arr = L.stage_array(stages)
    gr = (Grad * len(grads))(*grads)
    if ws is None:
        ws = workspace(max(int(L.lib().wgn_backward_workspace_bytes(arr, len(stages), batch)), 256), device)
    st = L.lib().wgn_chain_backward(arr, len(stages), batch, gr, _ptr(g_out),
                                    _row_stride(g_out) if g_out is not None else 0, _ptr(g_in),
                                    _row_stride(g_in) if g_in is not None else 0, 1 if prefetch else 0,
                                    _ptr(ws), ws.numel(), _stream(stream))
    L.check(st, "wgn_chain_backward")
