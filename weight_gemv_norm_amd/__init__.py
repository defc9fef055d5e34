"""MI355X (gfx950) decode-step weight stream: norm-fused BF16 GEMV chains.

The computation lives in libwgn.so (hand-written HIP, C ABI in include/wgn.h);
this package only marshals arguments.  Importing it does not load the library;
the first call does, and raises if the library was not built.
"""
from .api import (Chain, gemv_norm, gemv_norm_workspace_bytes, layer_chain, lmhead_argmax,  # noqa: F401
                  lmhead_argmax_workspace_bytes, make_stage, rmsnorm_rows, chain_workspace_bytes,
                  partition_selftest, first_wave_of_unit, workspace, device_cu_count, plan_phases,
                  PATH_AUTO, PATH_VECTOR, PATH_MATRIX, PATH_TILED, Plan, WgnError, decode_attention,
                  decode_attention_workspace_bytes, gemv_int4, stream_read,
                  workspace_bytes, plan_tune, lmhead_argmax_static, gemm_norm,
                  gemm_norm_workspace_bytes, make_grad, backward_workspace_bytes, Backward,
                  chain_backward, make_attn_stage)
