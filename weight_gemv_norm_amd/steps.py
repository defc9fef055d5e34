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

from typing import Dict, List, Optional

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


class DecodeStepWithAttention:
    """A decode step whose attention is computed, not seeded: per layer the
    Q/K/V products, wgn_decode_attention over that layer's static cache (the
    new key/value appended at each row's position), then O, the SwiGLU MLP
    and down ("One Token, Kernel by Kernel", sections "What one block
    launches" and "The fix: Part 10's split-KV kernel").

    fused=True: one chain, one persistent launch per step; each layer's
    attention runs inside it as two phases without weights
    (wgn_chain_create_attn), between {Q, K, V} and {O}.
    fused=None (default): the faster of the two as measured on MI355X with
    the pages' shapes -- one launch at batch 1-2 (1,386 / 1,525 us against
    1,538 / 1,539 with 1,024-slot caches) and for long caches (32,768 slots,
    batch 4: 1,900 against 2,139 us); attention launches from batch 3 with
    caches of at most 4,096 slots (1,024 slots: 1,603 / 1,739 against 1,693
    / 1,839 us; the 4,096-slot bound itself was not measured).
    fused=False: one chain {Q, K, V of layer 0}; then per layer one
    wgn_decode_attention launch and one chain {O, gate/up, down, and the next
    layer's Q, K, V} (the last chain ends with the final norm, LM head and
    argmax), every chain a persistent kernel of its own.
    Buffers: q/k/v/a/h1/s/h per layer as in decoder_stages, with a [B][Hq*D]
    the attention output that feeds O."""

    def __init__(self, inp: Dict, caches: List[Dict], device, mode: int = 0, fused: Optional[bool] = None,
                 ring: int = 0):
        from . import api as W
        B = inp["batch"]
        eps = inp["eps"]
        layers = inp["layers"]
        h = inp["h"]
        self.B, self.caches = B, caches
        bufs = {"h": [h], "q": [], "k": [], "v": [], "a": [], "h1": [], "s": []}
        qkv = []
        for L in layers:
            q = alloc(B, L["wq"].shape[0], device)
            k = alloc(B, L["wk"].shape[0], device)
            v = alloc(B, L["wv"].shape[0], device)
            qkv.append([make_stage(L["wq"], h, q, norm=NORM_RMS, eps=eps, gamma=L["g1"]),
                        make_stage(L["wk"], h, k, norm=NORM_RMS, eps=eps, gamma=L["g1"]),
                        make_stage(L["wv"], h, v, norm=NORM_RMS, eps=eps, gamma=L["g1"])])
            Hd = L["wq"].shape[1]
            a = alloc(B, L["wo"].shape[1], device)
            h1 = alloc(B, Hd, device)
            s = alloc(B, L["wg"].shape[0], device)
            hn = alloc(B, Hd, device)
            for name, t in (("q", q), ("k", k), ("v", v), ("a", a), ("h1", h1), ("s", s)):
                bufs[name].append(t)
            bufs["h"].append(hn)
            h = hn
        tail = []
        if "W_lm" in inp:
            idx = torch.full((B,), -1, dtype=torch.int32, device=device)
            mx = torch.empty((B,), dtype=torch.float32, device=device)
            tail = [make_stage(inp["W_lm"], h, idx, norm=NORM_RMS, eps=eps, gamma=inp["g_f"], epi=EPI_ARGMAX,
                               maxval=mx)]
            bufs["idx"], bufs["maxval"] = idx, mx
        self.bufs = bufs
        if fused is None:
            fused = B <= 2 or max(c["k_cache"].shape[2] for c in caches) > 4096
        self.fused = fused
        hd = 128  # head dimension of the attention kernel
        NQ, NKV = layers[0]["wq"].shape[0] // hd, layers[0]["wk"].shape[0] // hd
        if fused:
            stages, att = list(qkv[0]), []
            for l, L in enumerate(layers):
                h_in, h1, s, hn = bufs["h"][l], bufs["h1"][l], bufs["s"][l], bufs["h"][l + 1]
                c = caches[l]
                att.append((len(stages), W.make_attn_stage(bufs["q"][l], bufs["k"][l], bufs["v"][l], c["k_cache"],
                                                           c["v_cache"], c["pos"], bufs["a"][l])))
                stages += [make_stage(L["wo"], bufs["a"][l], h1, norm=NORM_NONE, residual=h_in),
                           make_stage(L["wg"], h1, s, norm=NORM_RMS, eps=eps, gamma=L["g2"], epi=EPI_SWIGLU,
                                      W_up=L["wu"]),
                           make_stage(L["wd"], s, hn, norm=NORM_NONE, residual=h1)]
                stages += qkv[l + 1] if l + 1 < len(layers) else tail
            self.chains = [W.Chain(stages, B, mode=mode, attn=att, ring=ring)]
            self.attn = []
            self.n_launches = 1 if mode == 0 else self.chains[0].num_phases
            return
        self.chains = [W.Chain(qkv[0], B, mode=mode, ring=ring)]
        self.attn = []
        for l, L in enumerate(layers):
            h_in, h1, s, hn = bufs["h"][l], bufs["h1"][l], bufs["s"][l], bufs["h"][l + 1]
            st = [make_stage(L["wo"], bufs["a"][l], h1, norm=NORM_NONE, residual=h_in),
                  make_stage(L["wg"], h1, s, norm=NORM_RMS, eps=eps, gamma=L["g2"], epi=EPI_SWIGLU, W_up=L["wu"]),
                  make_stage(L["wd"], s, hn, norm=NORM_NONE, residual=h1)]
            st += qkv[l + 1] if l + 1 < len(layers) else tail
            self.chains.append(W.Chain(st, B, mode=mode, ring=ring))
            c = caches[l]
            S = c["k_cache"].shape[2]
            self.attn.append(dict(
                q=bufs["q"][l].view(B, NQ, hd), k_new=bufs["k"][l].view(B, NKV, hd),
                v_new=bufs["v"][l].view(B, NKV, hd), k_cache=c["k_cache"], v_cache=c["v_cache"], pos=c["pos"],
                out=bufs["a"][l].view(B, NQ, hd),
                ws=W.workspace(W.decode_attention_workspace_bytes(B, NQ, NKV, S, hd), device)))
        self.n_launches = len(self.chains) + len(self.attn)

    def run(self, stream=None) -> None:
        from . import api as W
        self.chains[0].run(stream)
        for l, at in enumerate(self.attn):
            W.decode_attention(at["q"], at["k_new"], at["v_new"], at["k_cache"], at["v_cache"], at["pos"],
                               at["out"], ws=at["ws"], stream=stream)
            self.chains[l + 1].run(stream)

    def check(self, stream=None) -> None:
        for c in self.chains:
            c.check(stream)

    def capture(self) -> "torch.cuda.CUDAGraph":
        """The whole step captured once in a HIP graph ("One Token, Kernel by
        Kernel", section "Step 3: where the 14.8 ms go": the step is replayed
        as one graph): the 57 launches then cost one host call.  Every launch's arguments are fixed and no call enqueues a
        memset, so replays are equivalent to run()."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.run(stream=s)  # first use of every launch path outside capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            self.run(stream=s)
        torch.cuda.synchronize()
        return g


class BatchedStep:
    """A stage list at batch 1-128 (path 3; the only one above 16): wgn_layer_chain runs it stage by stage on
    the matrix cores (each stage a tiled product, RMSNorm as a pass of its
    own), with one workspace; capture() records a call in a HIP graph (the
    page's replayed step), so replays cost one host call."""

    def __init__(self, stages, batch: int, device):
        from .api import workspace, workspace_bytes
        self.stages, self.batch = list(stages), int(batch)
        self.ws = workspace(workspace_bytes(self.stages, self.batch), device)
        norms = sum(1 for st in self.stages if st.norm != 0)
        self.n_launches = 1 + len(self.stages) + norms  # counter clear, products, norm passes

    def run(self, stream=None) -> None:
        from .api import layer_chain, PATH_TILED
        layer_chain(self.stages, self.batch, ws=self.ws, stream=stream, path=PATH_TILED)

    def capture(self) -> "torch.cuda.CUDAGraph":
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.run(stream=s)  # first use of every launch path outside capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            self.run(stream=s)
        torch.cuda.synchronize()
        return g


def ln_gelu_chain_stages(inp: Dict, device, keep_pre: bool = False):
    """Stages of the LayerNorm -> Linear -> GELU-tanh chain.  Returns (stages,
    buffers); keep_pre: each stage also keeps its FP32 pre-activation (for
    the backward pass) in buffers["pre"]."""
    B = inp["batch"]
    eps = inp["eps"]
    x = inp["x"]
    outs = [x]
    pres = []
    stages = []
    for L in inp["layers"]:
        N = L["W"].shape[0]
        y = alloc(B, N, device)
        pre = alloc(B, N, device, torch.float32) if keep_pre else None
        stages.append(make_stage(L["W"], x, y, norm=NORM_LAYER, eps=eps, gamma=L.get("gamma"), beta=L.get("beta"),
                                 bias=L.get("bias"), epi=EPI_GELU_TANH, pre=pre))
        outs.append(y)
        pres.append(pre)
        x = y
    return stages, {"x": outs, "pre": pres}


class TrainStep:
    """One small-batch training step of the LayerNorm -> Linear -> GELU chain:
    the forward chain (keeping each block's pre-activation), then the backward
    pass from the gradient of the mean of the squared output, last block first
    ("Making small PyTorch ops faster on a laptop GPU", section "It works in
    training too": the example step's loss is the mean of the squared output,
    and the backward fetches the weights of block i-1 while block i runs).
    The parameter gradients land in self.grads[i] (gW, gb, ggamma, gbeta);
    keep=True also keeps each block's output gradient gy and pre-activation
    gradient gz, and the chain-input gradient g_in.  prefetch: the backward
    requests each block's weight tiles before waiting for the block after it
    (off by default: on this GPU it did not clear +1 % when measured; the
    bench's A/B pass measures it on every run)."""

    def __init__(self, inp: Dict, device, prefetch: bool = False, keep: bool = True, g_out=None):
        from .api import Backward, Chain, make_grad
        self.inp, self.B, self.prefetch = inp, inp["batch"], prefetch
        self.stages, self.bufs = ln_gelu_chain_stages(inp, device, keep_pre=True)
        self.fwd = Chain(self.stages, self.B)
        self.grads = []
        gstructs = []
        for L in inp["layers"]:
            N, K = L["W"].shape
            g = {"gW": torch.empty((N, K), dtype=torch.bfloat16, device=device)}
            if L.get("bias") is not None:
                g["gb"] = torch.empty(N, dtype=torch.bfloat16, device=device)
            if L.get("gamma") is not None:
                g["ggamma"] = torch.empty(K, dtype=torch.bfloat16, device=device)
            if L.get("beta") is not None:
                g["gbeta"] = torch.empty(K, dtype=torch.bfloat16, device=device)
            if keep:
                g["gy"] = alloc(self.B, N, device)
                g["gz"] = alloc(self.B, N, device)
            self.grads.append(g)
            gstructs.append(make_grad(g["gW"], g.get("gb"), g.get("ggamma"), g.get("gbeta"), g.get("gy"),
                                      g.get("gz")))
        K0 = inp["layers"][0]["W"].shape[1]
        self.g_in = alloc(self.B, K0, device) if keep else None
        self.bwd = Backward(self.stages, self.B, gstructs, g_out=g_out, g_in=self.g_in, device=device)

    def forward(self, stream=None) -> None:
        self.fwd.run(stream)

    def backward(self, stream=None) -> None:
        self.bwd.run(self.prefetch, stream)

    def run(self, stream=None) -> None:
        self.forward(stream)
        self.backward(stream)

    def check(self) -> None:
        self.fwd.check()
        self.bwd.check()

    def capture(self) -> "torch.cuda.CUDAGraph":
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.run(stream=s)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            self.run(stream=s)
        torch.cuda.synchronize()
        return g


def train_step_bytes(inp: Dict) -> Dict[str, int]:
    """Algorithmic bytes of one training step (forward + backward): every
    weight read twice (forward product, backward product) and every weight
    gradient written once dominate; activations, pre-activations and the
    small parameter tensors are counted once per pass that moves them."""
    B = inp["batch"]
    w = sum(L["W"].numel() * 2 for L in inp["layers"])
    small = act = 0
    for L in inp["layers"]:
        N, K = L["W"].shape
        small += 2 * (2 * K + N) * 2                  # gamma, beta, bias read; their gradients written
        act += B * (K * 2 + N * 2 + N * 4) * 2        # x and y (BF16) and z (FP32): forward writes, backward reads
    return {"weights_fwd": w, "weights_bwd": w, "weight_grads": w, "small": small, "activations": act,
            "total": 3 * w + small + act}


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
