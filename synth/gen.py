"""Seeded normal samples and the workload recipes (shapes + distributions).

Recipes follow the shapes the pages give for a Llama-class 1.5B decoder
("One Token, Kernel by Kernel: A Decode Step on a Laptop GPU", sections "The
setup", "The whole step", "The GEMVs, through Nsight Compute") and the
LayerNorm -> Linear -> GELU chain of "Making small PyTorch ops faster on a
laptop GPU", section "Beyond language models".  Weights are synthetic: the
pages' trained weights and real-text prefill are not used (only their shapes).

Distribution notation: a spread written as 1/K is a variance (std 1/sqrt(K));
a decimal spread (0.02, 0.1) is a standard deviation.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch


def seed_of(workload: int, layer: int, tensor: int) -> int:
    """Deterministic seed for (workload id, layer, tensor id)."""
    return ((workload * 1_000_003 + layer) * 1_009 + tensor) & 0x7FFF_FFFF_FFFF_FFFF


def normal(shape, std: float, seed: int, mean: float = 0.0, dtype=torch.bfloat16,
           device="cpu") -> torch.Tensor:
    """mean + std * N(0,1), drawn in float32 from a seeded generator, then rounded
    (round-to-nearest-even) to ``dtype``."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


def bf16_bits_to_numpy(t: torch.Tensor) -> np.ndarray:
    """BF16 tensor (any device) -> numpy uint16 bit patterns on the host."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f16_bits_to_numpy(t: torch.Tensor) -> np.ndarray:
    assert t.dtype == torch.float16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


# ------------------------------------------------------------------ workloads
H, I, V = 1536, 8960, 151936
NQ, NKV, HEAD_DIM = 12, 2, 128
N_LAYERS = 28


@dataclass
class Workload:
    name: str
    wid: int
    batch: int
    desc: str
    extra: Dict = field(default_factory=dict)


WORKLOADS = {
    "rmsnorm_gemv_256": Workload("rmsnorm_gemv_256", 1, 1,
                                 "RMSNorm(eps 1e-6, gain 1+N(0,0.1)) + 256x256 GEMV, W std 1/16, x N(0,1), batch 1"),
    "ln_gelu_chain_768x72": Workload("ln_gelu_chain_768x72", 2, 4,
                                     "72 x [LayerNorm(768) -> Linear 768x768 (W std 1/sqrt(768), bias std 0.02) -> GELU-tanh]"),
    "decoder_block_1536": Workload("decoder_block_1536", 3, 1,
                                   "one Llama-style block at hidden 1536 (Q/K/V/O, gate/up 8960 + SwiGLU, down), weights std 0.02"),
    "decode_step_1536x28": Workload("decode_step_1536x28", 4, 1,
                                    "28 blocks of decoder_block_1536 + final RMSNorm + LM head 151936x1536 + argmax"),
    "rmsnorm_rows_960x1536_f16": Workload("rmsnorm_rows_960x1536_f16", 5, 960,
                                          "standalone RMSNorm over 960 x 1536 FP16 rows (prefill shape)"),
}


def block_shapes(hidden: int = H, inter: int = I, n_q: int = NQ, n_kv: int = NKV):
    """Weight matrix shapes [N][K] of one decoder block, in stream order.
    The query projection spans the hidden size (n_q heads x head_dim); the key
    and value projections span n_kv heads of the same head_dim."""
    q = hidden
    kv = hidden * n_kv // n_q
    return [("wq", q, hidden), ("wk", kv, hidden), ("wv", kv, hidden), ("wo", hidden, q),
            ("wg", inter, hidden), ("wu", inter, hidden), ("wd", hidden, inter)]


def decode_step_weight_bytes(n_layers: int = N_LAYERS, hidden: int = H, inter: int = I,
                             vocab: int = V) -> int:
    """BF16 weight bytes read by one decode step (all block matrices + LM head)."""
    per_layer = sum(n * k for _, n, k in block_shapes(hidden, inter)) * 2
    return n_layers * per_layer + vocab * hidden * 2


def make_stage_tensors(workload: str, device="cpu", batch: Optional[int] = None,
                       n_layers: Optional[int] = None, vocab: Optional[int] = None,
                       hidden: Optional[int] = None, inter: Optional[int] = None,
                       seeded_ln_params: bool = False) -> Dict[str, object]:
    """Draw every input tensor of a workload.  Returns a dict of tensors.

    Optional overrides shrink a workload for quick tests while keeping its
    structure and distributions (never used for the benchmark's numbers).
    """
    w = WORKLOADS[workload]
    wid = w.wid
    B = batch if batch is not None else w.batch
    out: Dict[str, object] = {"workload": workload, "batch": B}
    if workload == "rmsnorm_gemv_256":
        K = hidden or 256
        out["x"] = normal((B, K), 1.0, seed_of(wid, 0, 0), device=device)
        out["g"] = normal((K,), 0.1, seed_of(wid, 0, 1), mean=1.0, device=device)
        out["W"] = normal((K, K), 1.0 / math.sqrt(K), seed_of(wid, 0, 2), device=device)
        out["eps"] = 1e-6
        return out
    if workload == "ln_gelu_chain_768x72":
        K = hidden or 768
        L = n_layers or 72
        out["x"] = normal((B, K), 1.0, seed_of(wid, 0, 0), device=device)
        layers = []
        for l in range(L):
            d = {
                "W": normal((K, K), 1.0 / math.sqrt(K), seed_of(wid, l + 1, 1), device=device),
                "bias": normal((K,), 0.02, seed_of(wid, l + 1, 2), device=device),
            }
            if seeded_ln_params:
                d["gamma"] = normal((K,), 0.1, seed_of(wid, l + 1, 3), mean=1.0, device=device)
                d["beta"] = normal((K,), 0.02, seed_of(wid, l + 1, 4), device=device)
            else:
                d["gamma"] = torch.ones(K, dtype=torch.bfloat16, device=device)
                d["beta"] = torch.zeros(K, dtype=torch.bfloat16, device=device)
            layers.append(d)
        out["layers"] = layers
        out["eps"] = 1e-5
        return out
    if workload in ("decoder_block_1536", "decode_step_1536x28"):
        Hd = hidden or H
        Id = inter or I
        L = 1 if workload == "decoder_block_1536" else (n_layers or N_LAYERS)
        out["h"] = normal((B, Hd), 1.0, seed_of(wid, 0, 0), device=device)
        layers = []
        for l in range(L):
            d = {"a": normal((B, Hd), 1.0, seed_of(wid, l + 1, 0), device=device),
                 "g1": normal((Hd,), 0.1, seed_of(wid, l + 1, 1), mean=1.0, device=device),
                 "g2": normal((Hd,), 0.1, seed_of(wid, l + 1, 2), mean=1.0, device=device)}
            for t, (name, n, k) in enumerate(block_shapes(Hd, Id)):
                d[name] = normal((n, k), 0.02, seed_of(wid, l + 1, 10 + t), device=device)
            layers.append(d)
        out["layers"] = layers
        out["eps"] = 1e-6
        if workload == "decode_step_1536x28":
            Vv = vocab or V
            out["g_f"] = normal((Hd,), 0.1, seed_of(wid, 0, 1), mean=1.0, device=device)
            out["W_lm"] = normal((Vv, Hd), 0.02, seed_of(wid, 0, 2), device=device)
        return out
    if workload == "rmsnorm_rows_960x1536_f16":
        R = batch or 960
        K = hidden or H
        out["x"] = normal((R, K), 1.0, seed_of(wid, 0, 0), dtype=torch.float16, device=device)
        out["g"] = normal((K,), 0.1, seed_of(wid, 0, 1), mean=1.0, dtype=torch.float16, device=device)
        out["eps"] = 1e-6
        return out
    raise KeyError(workload)


def layer_names() -> List[str]:
    return [n for n, _, _ in block_shapes()]


# ----------------------------------------------------------- decode attention
ATTN_WORKLOAD = 41


def make_attention_tensors(batch: int, slots: int, pos, q_heads: int = NQ, kv_heads: int = NKV,
                           head_dim: int = HEAD_DIM, seed: int = 0, layer: int = 0, nan_tail: bool = True,
                           device="cpu") -> Dict[str, torch.Tensor]:
    """One decode step's attention inputs: q [B][Hq][D], the new key/value
    [B][Hkv][D] and a static cache [B][Hkv][slots][D], all N(0,1) in BF16, with
    per-row positions pos (int32).  Slots after each row's position hold NaN
    when nan_tail is set (a cache that is not yet written), so that any use of
    them shows in the output.  The shapes follow the pages' model (12 query
    heads over 2 key/value heads of 128 dimensions); the random values stand
    in for a real prefill."""
    s = lambda t: seed_of(ATTN_WORKLOAD * 1000 + seed, layer, t)  # noqa: E731
    out = {
        "q": normal((batch, q_heads, head_dim), 1.0, s(1), device=device),
        "k_new": normal((batch, kv_heads, head_dim), 1.0, s(2), device=device),
        "v_new": normal((batch, kv_heads, head_dim), 1.0, s(3), device=device),
        "k_cache": normal((batch, kv_heads, slots, head_dim), 1.0, s(4), device=device),
        "v_cache": normal((batch, kv_heads, slots, head_dim), 1.0, s(5), device=device),
        "pos": torch.as_tensor(np.asarray(pos, dtype=np.int32).reshape(batch), device=device),
    }
    if nan_tail:
        for b, p in enumerate(np.asarray(pos).reshape(batch)):
            lo = max(int(p) + 1, 0)
            if lo < slots:
                out["k_cache"][b, :, lo:] = float("nan")
                out["v_cache"][b, :, lo:] = float("nan")
    return out


def make_kv_caches(batch: int, slots: int, pos, n_layers: int = N_LAYERS, kv_heads: int = NKV,
                   head_dim: int = HEAD_DIM, nan_tail: bool = True, device="cpu") -> List[Dict[str, torch.Tensor]]:
    """Per-layer static caches [B][Hkv][slots][D] ~ N(0,1) in BF16 (slots after
    each row's position NaN when nan_tail is set) and the positions, for a
    decode step whose keys, values and queries come from the step itself.
    The values stand in for a real prefill (the pages' model decodes after a
    960-token prompt)."""
    out = []
    for l in range(n_layers):
        t = make_attention_tensors(batch, slots, pos, q_heads=kv_heads, kv_heads=kv_heads, head_dim=head_dim,
                                   seed=7, layer=l, nan_tail=nan_tail, device=device)
        out.append({"k_cache": t["k_cache"], "v_cache": t["v_cache"], "pos": t["pos"]})
    return out


def make_int4_weights(N: int, K: int, seed: int = 0, device="cpu") -> Dict[str, torch.Tensor]:
    """Synthetic 4-bit weights in groups of 128, shaped like a quantised
    N(0, 0.02) matrix: codes uniform in 0..15 packed two per byte (low nibble
    = even k), per-group scales near 0.1/15 and zeros near -0.05 (BF16)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed_of(43, seed, 0)))
    W4 = torch.randint(0, 256, (N, K // 2), generator=g, dtype=torch.uint8)
    sc = (torch.randn((N, K // 128), generator=g) * 0.001 + 0.1 / 15).abs().to(torch.bfloat16)
    zr = (torch.randn((N, K // 128), generator=g) * 0.005 - 0.05).to(torch.bfloat16)
    return {"W4": W4.to(device), "scales": sc.to(device), "zeros": zr.to(device)}
