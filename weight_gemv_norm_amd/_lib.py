"""ctypes view of libwgn.so (include/wgn.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build only: the product never loads another library.
LIB_PATH = os.path.join(HERE, "libwgn.so")

TRACE_POINTS = 12
OK, E_ARG, E_ALIGN, E_UNSUPPORTED, E_WORKSPACE, E_HIP, E_DEVICE, E_TIMEOUT = 0, -1, -2, -3, -4, -5, -6, -7
NORM_NONE, NORM_RMS, NORM_LAYER = 0, 1, 2
EPI_NONE, EPI_GELU_TANH, EPI_SWIGLU, EPI_ARGMAX = 0, 1, 2, 3
BF16, FP16, FP32 = 0, 1, 2

P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64
F32 = ctypes.c_float
SZ = ctypes.c_size_t


class Stage(ctypes.Structure):
    """Mirror of wgn_stage."""
    _fields_ = [
        ("N", I32), ("K", I32),
        ("W", P), ("W_up", P), ("bias", P),
        ("norm", I32), ("eps", F32),
        ("gamma", P), ("beta", P),
        ("epi", I32),
        ("x", P), ("x_stride", I64),
        ("residual", P), ("res_stride", I64),
        ("y", P), ("y_stride", I64),
        ("logits", P), ("maxval", P),
    ]


class AttnStage(ctypes.Structure):
    """Mirror of wgn_attn_stage."""
    _fields_ = [
        ("q", P), ("q_stride", I64),
        ("k_new", P), ("k_stride", I64),
        ("v_new", P), ("v_stride", I64),
        ("k_cache", P), ("v_cache", P), ("pos", P),
        ("out", P), ("out_stride", I64),
        ("q_heads", I32), ("kv_heads", I32), ("slots", I32), ("head_dim", I32),
        ("scale", F32),
    ]


class ChainOpts(ctypes.Structure):
    """Mirror of wgn_chain_opts."""
    _fields_ = [("mode", I32), ("grid", I32), ("trace", I32), ("path", I32), ("no_fuse", I32),
                ("ring", I32), ("reserved", I32 * 2)]


class Plan(ctypes.Structure):
    """Mirror of wgn_plan."""
    _fields_ = [("prefetch", I32), ("distance", I32), ("blocks", I32), ("frac_pct", I32),
                ("plain_us", F32), ("best_us", F32), ("speedup_lo", F32), ("candidates", I32)]


class Grad(ctypes.Structure):
    """Mirror of wgn_grad."""
    _fields_ = [("gW", P), ("gbias", P), ("ggamma", P), ("gbeta", P), ("gy", P), ("gz", P)]


class WgnError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = "%s failed: %s (%d)" % (what, status_string(status), status)
        if status == E_HIP:
            msg += " [%s]" % lib().wgn_last_hip_error().decode()
        super().__init__(msg)
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree libwgn.so; raise loudly if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libwgn.so is not built (run __graft_entry__.build() or "
                           "python weight_gemv_norm_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    SP = ctypes.POINTER(Stage)
    OP = ctypes.POINTER(ChainOpts)
    sig = {
        "wgn_status_string": ([I32], ctypes.c_char_p),
        "wgn_version": ([], I32),
        "wgn_last_hip_error": ([], ctypes.c_char_p),
        "wgn_device_cu_count": ([], I32),
        "wgn_gemv_norm_workspace_bytes": ([SP, I32], SZ),
        "wgn_gemv_norm": ([SP, I32, P, SZ, P], I32),
        "wgn_gemm_norm_workspace_bytes": ([SP, I32], SZ),
        "wgn_gemm_norm": ([SP, I32, P, SZ, P], I32),
        "wgn_lmhead_argmax_workspace_bytes": ([I32], SZ),
        "wgn_lmhead_argmax": ([P, I64, I32, I32, P, F32, P, I32, P, P, P, P, SZ, P], I32),
        "wgn_lmhead_argmax_static": ([P, I64, I32, I32, P, F32, P, I32, P, P, P, P], I32),
        "wgn_rmsnorm_rows": ([P, I64, P, F32, P, I64, I32, I32, I32, P], I32),
        "wgn_gemv_int4": ([P, I64, I32, I32, P, P, P, I32, P, I64, P], I32),
        "wgn_stream_read": ([P, SZ, I32, I32, I32, P, P], I32),
        "wgn_decode_attention_workspace_bytes": ([I32, I32, I32, I32, I32], ctypes.c_size_t),
        "wgn_decode_attention": ([P, P, P, P, P, P, I32, I32, I32, I32, I32, F32, P, P, ctypes.c_size_t, P], I32),
        "wgn_chain_workspace_bytes": ([SP, I32, I32, OP], SZ),
        "wgn_chain_create": ([SP, I32, I32, OP, P, SZ, P, ctypes.POINTER(P)], I32),
        "wgn_chain_attn_workspace_bytes": ([SP, I32, ctypes.POINTER(AttnStage), ctypes.POINTER(I32), I32, I32, OP],
                                           SZ),
        "wgn_chain_create_attn": ([SP, I32, ctypes.POINTER(AttnStage), ctypes.POINTER(I32), I32, I32, OP, P, SZ, P,
                                   ctypes.POINTER(P)], I32),
        "wgn_chain_run": ([P, P], I32),
        "wgn_chain_check": ([P, P], I32),
        "wgn_chain_set_wait_us": ([P, I64], I32),
        "wgn_chain_num_phases": ([P], I32),
        "wgn_chain_grid": ([P], I32),
        "wgn_chain_ring": ([P], I32),
        "wgn_chain_trace": ([P, P, ctypes.POINTER(ctypes.c_uint64), SZ], I32),
        "wgn_chain_stage_phases": ([P, ctypes.POINTER(I32)], I32),
        "wgn_chain_destroy": ([P], None),
        "wgn_layer_chain": ([SP, I32, I32, OP, ctypes.POINTER(Plan), P, SZ, P, P], I32),
        "wgn_workspace_bytes": ([SP, I32, I32, I32], SZ),
        "wgn_chain_run_plan": ([P, ctypes.POINTER(Plan), P, P], I32),
        "wgn_chain_plan_tune": ([P, P, P, I32, ctypes.POINTER(Plan)], I32),
        "wgn_plan_tune": ([SP, I32, I32, ctypes.POINTER(Plan), P, SZ, P, P], I32),
        "wgn_first_wave_of_unit": ([I32, I32, I32], I32),
        "wgn_partition_selftest": ([SP, I32, I32, OP], I32),
        "wgn_plan_phases": ([SP, I32, I32, OP, ctypes.POINTER(I32)], I32),
        "wgn_backward_workspace_bytes": ([SP, I32, I32], SZ),
        "wgn_backward_create": ([SP, I32, I32, ctypes.POINTER(Grad), P, I64, P, I64, P, SZ, P,
                                 ctypes.POINTER(P)], I32),
        "wgn_backward_run": ([P, I32, P], I32),
        "wgn_backward_check": ([P, P], I32),
        "wgn_backward_set_wait_us": ([P, I64], I32),
        "wgn_backward_grid": ([P], I32),
        "wgn_backward_set_trace": ([P, P, SZ], I32),
        "wgn_backward_destroy": ([P], None),
        "wgn_chain_backward": ([SP, I32, I32, ctypes.POINTER(Grad), P, I64, P, I64, I32, P, SZ, P], I32),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def status_string(s: int) -> str:
    return lib().wgn_status_string(int(s)).decode()


def check(status: int, what: str) -> None:
    if status != OK:
        raise WgnError(status, what)


def stage_array(stages):
    arr = (Stage * len(stages))()
    for i, s in enumerate(stages):
        arr[i] = s
    return arr
