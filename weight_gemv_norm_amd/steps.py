"""Stage lists for the pages' workloads, over caller-owned device tensors.

A Llama-class decoder block at batch B becomes six stages; every stage writes
its own buffer, so each intermediate can be checked:

  Q, K, V : RMSNorm(h; g1) -> W_q / W_k / W_v            -> q, k, v
  O       : W_o . a (attention output), + residual h       -> h1
  gate/up : RMSNorm(h1; g2) -> silu(W_g x) * (W_u x)       -> s
  down    : W_d . s, + residual h1                         -> h'

("One Token, Kernel by Kernel: A Decode Step on a Laptop GPU", sections "The
setup" (RMSNorm, grouped-query attention, SwiGLU MLP) and "What one block
launches" (seven weight products per block; the residual add is folded into a
neighbouring kernel)).  The attention itself is not on the weight stream: the
O projection reads a given attention-output vector.  The step ends with the
final RMSNorm, the LM head and the argmax ("The whole step").

The LayerNorm -> Linear -> GELU chain follows "Making small PyTorch ops faster
on a laptop GPU", section "Beyond language models".
"""
from __future__ import annotations

from typing import Dict, List

import torch

from .api import (EPI_ARGMAX, EPI_GELU_TANH, EPI_NONE, EPI_SWIGLU, NORM_LAYER, NORM_NONE, NORM_RMS,
                  make_stage)


def alloc(B: int, n: int, device, dtype=torch.bfloat16) -> torch.Tensor:
    return torch.empty((B, n), dtype=dtype, device=device)


def decoder_stages(inp: Dict, device, with_lmhead: bool = True, logits: bool = False):
    """Stages of one decode step over the tensors of synth.make_stage_tensors
    (decoder_block_1536 / decode_step_1536x28).  Returns (stages, buffers)."""
    B = inp["batch"]
    eps = inp["eps"]
    layers = inp["layers"]
    h = inp["h"]
    bufs = {"h": [h], "q": [], "k": [], "v": [], "h1": [], "s": []}
    stages = []
    for L in layers:
        Hd = L["wq"].shape[1]
        q = alloc(B, L["wq"].shape[0], device)
        k = alloc(B, L["wk"].shape[0], device)
        v = alloc(B, L["wv"].shape[0], device)
        h1 = alloc(B, Hd, device)
        s = alloc(B, L["wg"].shape[0], device)
        hn = alloc(B, Hd, device)
        stages.append(make_stage(L["wq"], h, q, norm=NORM_RMS, eps=eps, gamma=L["g1"]))
        stages.append(make_stage(L["wk"], h, k, norm=NORM_RMS, eps=eps, gamma=L["g1"]))
        stages.append(make_stage(L["wv"], h, v, norm=NORM_RMS, eps=eps, gamma=L["g1"]))
        stages.append(make_stage(L["wo"], L["a"], h1, norm=NORM_NONE, residual=h))
        stages.append(make_stage(L["wg"], h1, s, norm=NORM_RMS, eps=eps, gamma=L["g2"], epi=EPI_SWIGLU,
                                 W_up=L["wu"]))
        stages.append(make_stage(L["wd"], s, hn, norm=NORM_NONE, residual=h1))
        for name, t in (("q", q), ("k", k), ("v", v), ("h1", h1), ("s", s)):
            bufs[name].append(t)
        bufs["h"].append(hn)
        h = hn
    if with_lmhead and "W_lm" in inp:
        V = inp["W_lm"].shape[0]
        idx = torch.full((B,), -1, dtype=torch.int32, device=device)
        mx = torch.empty((B,), dtype=torch.float32, device=device)
        lg = torch.empty((B, V), dtype=torch.float32, device=device) if logits else None
        stages.append(make_stage(inp["W_lm"], h, idx, norm=NORM_RMS, eps=eps, gamma=inp["g_f"],
                                 epi=EPI_ARGMAX, maxval=mx, logits=lg))
        bufs["idx"], bufs["maxval"], bufs["logits"] = idx, mx, lg
    return stages, bufs


def ln_gelu_chain_stages(inp: Dict, device):
    """Stages of the LayerNorm -> Linear -> GELU-tanh chain.  Returns (stages, buffers)."""
    B = inp["batch"]
    eps = inp["eps"]
    x = inp["x"]
    outs = [x]
    stages = []
    for L in inp["layers"]:
        y = alloc(B, L["W"].shape[0], device)
        stages.append(make_stage(L["W"], x, y, norm=NORM_LAYER, eps=eps, gamma=L["gamma"], beta=L["beta"],
                                 bias=L["bias"], epi=EPI_GELU_TANH))
        outs.append(y)
        x = y
    return stages, {"x": outs}


def decode_step_bytes(inp: Dict) -> Dict[str, int]:
    """Algorithmic bytes of one decode step: every weight, norm gain and
    activation tensor counted once (weights dominate)."""
    B = inp["batch"]
    wbytes = gbytes = abytes = 0
    for L in inp["layers"]:
        for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
            wbytes += L[n].numel() * 2
        gbytes += (L["g1"].numel() + L["g2"].numel()) * 2
        Hd = L["wq"].shape[1]
        I_ = L["wg"].shape[0]
        # reads: h, a ; writes: q, k, v, h1, s, h'  (h1 and s re-read count once)
        abytes += B * 2 * (Hd + Hd + L["wq"].shape[0] + L["wk"].shape[0] + L["wv"].shape[0] + Hd + I_ + Hd)
    if "W_lm" in inp:
        wbytes += inp["W_lm"].numel() * 2
        gbytes += inp["g_f"].numel() * 2
        abytes += B * 4 * 2  # idx + max
    return {"weights": wbytes, "gains": gbytes, "activations": abytes,
            "total": wbytes + gbytes + abytes}
