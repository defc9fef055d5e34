"""GPU parity of wgn_decode_attention against the oracle.

Every case compares, on the same seeded inputs:
* the output, element by element, within |d| <= 1e-2 |ref| + 1e-3 rms(ref);
* both caches after the call, bit for bit (the append writes exactly the new
  token's slot, nothing else changes).
Slots after each row's position hold NaN, so a read that reaches the output
shows up as a non-finite value.  Sizes cover one slot, one chunk, ragged
chunk tails, one to four merge levels, and the full 32,768-slot cache
of the pages' longest context.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import gen
from tests.gpu_util import assert_close_bf16, bits, say

pytestmark = pytest.mark.gpu


def _run(t, ws=None, stream=None):
    import weight_gemv_norm_amd as W
    out = torch.empty_like(t["q"])
    W.decode_attention(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["pos"], out, ws=ws,
                       stream=stream)
    return out


def _oracle(t):
    return O.decode_attention(bits(t["q"]), bits(t["k_new"]), bits(t["v_new"]), bits(t["k_cache"]),
                              bits(t["v_cache"]), t["pos"].cpu().numpy())


def _check(t, what):
    ref_out, ref_k, ref_v = _oracle(t)
    out = _run(t)
    torch.cuda.synchronize()
    worst = assert_close_bf16(bits(out), ref_out, what)
    np.testing.assert_array_equal(bits(t["k_cache"]), ref_k, err_msg=what + ": key cache")
    np.testing.assert_array_equal(bits(t["v_cache"]), ref_v, err_msg=what + ": value cache")
    return worst


CASES = [
    (1, 1, [0]),                                  # one slot: no merge
    (1, 128, [127]),                              # one full chunk
    (2, 129, [128, 0]),                           # two chunks; the new token alone in the second
    (3, 1000, [999, 500, 127]),                   # ragged tails, one merge level
    (4, 4096, [4095, 129, 2048, 3000]),           # 32 chunks: two full merge levels
    (2, 4224, [4223, 4100]),                      # 33 chunks: three levels, ragged groups
    (1, 32768, [32767]),                          # the pages' longest context, full cache
    (4, 32768, [32767, 20000, 1023, 31000]),
    (1, 140000, [139999]),                        # 1,094 chunks: four merge levels
]


@pytest.mark.parametrize("batch,slots,pos", CASES)
def test_decode_attention_matches_oracle(batch, slots, pos):
    say("decode_attention batch %d slots %d pos %s" % (batch, slots, pos))
    t = gen.make_attention_tensors(batch, slots, pos, seed=slots, device="cuda")
    _check(t, "attention b%d s%d" % (batch, slots))


@pytest.mark.parametrize("hq,hkv", [(1, 1), (2, 1), (4, 2), (6, 1), (8, 1), (16, 2), (3, 3), (14, 2)])
def test_decode_attention_group_sizes(hq, hkv):
    say("decode_attention heads %d/%d" % (hq, hkv))
    t = gen.make_attention_tensors(2, 700, [699, 300], q_heads=hq, kv_heads=hkv, seed=hq * 10 + hkv,
                                   device="cuda")
    _check(t, "attention heads %d/%d" % (hq, hkv))


def test_decode_attention_out_of_range_rows():
    say("decode_attention positions out of range")
    t = gen.make_attention_tensors(3, 300, [5, 5, 200], seed=7, nan_tail=False, device="cuda")
    t["pos"] = torch.tensor([-1, 300, 200], dtype=torch.int32, device="cuda")
    k0, v0 = t["k_cache"].clone(), t["v_cache"].clone()
    _check(t, "attention out-of-range rows")
    out = _run(t)
    torch.cuda.synchronize()
    assert not bits(out)[:2].any()
    assert torch.equal(t["k_cache"][:2].view(torch.int16), k0[:2].view(torch.int16))
    assert torch.equal(t["v_cache"][:2].view(torch.int16), v0[:2].view(torch.int16))


def test_decode_attention_successive_tokens_reuse_the_workspace():
    """Three decode steps in a row on one cache and one workspace: each call
    appends its token and must leave the arrival counters at zero, or the
    next call's merge would start from a wrong count."""
    import weight_gemv_norm_amd as W
    say("decode_attention successive tokens")
    B, S = 2, 9000
    t = gen.make_attention_tensors(B, S, [5000, 8990], seed=11, device="cuda")
    ws = W.workspace(W.decode_attention_workspace_bytes(B, 12, 2, S))
    for step in range(3):
        ref_out, ref_k, ref_v = _oracle(t)
        out = _run(t, ws=ws)
        torch.cuda.synchronize()
        assert_close_bf16(bits(out), ref_out, "step %d" % step)
        np.testing.assert_array_equal(bits(t["k_cache"]), ref_k)
        np.testing.assert_array_equal(bits(t["v_cache"]), ref_v)
        nxt = gen.make_attention_tensors(B, 1, [0, 0], seed=100 + step, device="cuda")
        t["q"], t["k_new"], t["v_new"] = nxt["q"], nxt["k_new"], nxt["v_new"]
        t["pos"] += 1


def test_decode_attention_graph_replays():
    """Captured once, replayed with the position advanced by one on the device
    between replays (the valid length is read at run time); every replay
    matches the oracle and an eager call on the same inputs."""
    import weight_gemv_norm_amd as W
    say("decode_attention graph replays")
    B, S = 1, 32768
    t = gen.make_attention_tensors(B, S, [20000], seed=21, device="cuda")
    ws = W.workspace(W.decode_attention_workspace_bytes(B, 12, 2, S))
    out = torch.empty_like(t["q"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _ = _run(t, ws=ws, stream=s)  # warm the launch path outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    t = gen.make_attention_tensors(B, S, [20000], seed=21, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        W.decode_attention(t["q"], t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["pos"], out, ws=ws,
                           stream=s)
    for rep in range(3):
        ref_out, ref_k, ref_v = _oracle(t)
        g.replay()
        torch.cuda.synchronize()
        assert_close_bf16(bits(out), ref_out, "replay %d" % rep)
        np.testing.assert_array_equal(bits(t["k_cache"]), ref_k)
        np.testing.assert_array_equal(bits(t["v_cache"]), ref_v)
        eager = _run(t, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(eager.view(torch.int16), out.view(torch.int16)), rep
        t["pos"] += 1                 # the next slot: NaN until this replay's append
        t["k_new"].mul_(0.5)


@pytest.mark.parametrize("fused,batch,pos,slots,mode,ring", [
    (False, 1, [960], 1024, 0, 0), (False, 2, [960, 37], 1024, 0, 0),
    (True, 1, [960], 1024, 0, 0),                 # the pages' step: one launch, attention inside
    (True, 2, [960, 37], 1024, 0, 0),
    (True, 4, [1023, 0, 500, -1], 1024, 0, 0),    # full cache, first slot, a row with no valid slot
    (True, 1, [4223], 4224, 0, 0),                # several passes per chunk, ragged last chunk
    (True, 3, [4000, 17, 2047], 4224, 0, 0),
    (True, 2, [960, 37], 1024, 0, 2),             # the 5 x 8-unit ring
    (True, 5, [960, 37, 1023, 0, 640], 1024, 0, 0),  # matrix-core path
    (True, 2, [960, 37], 1024, 1, 0),             # one launch per phase
    (True, 2, [960, 32767], 32768, 0, 0),         # a short and a full row of a long cache
])
def test_decode_step_with_attention_teacher_forced(fused, batch, pos, slots, mode, ring):
    """Two decoder blocks whose attention is computed (Q/K/V -> decode
    attention over the cache -> O -> MLP), then the LM head: every stage is
    checked against the oracle on the GPU's own inputs to it, the caches bit
    for bit, and the argmax.  fused: attention as phases of the chain's one
    launch; else its own launches between chains."""
    from weight_gemv_norm_amd import steps
    from tests.gpu_util import check_argmax
    say("decode step with attention fused %s batch %d pos %s slots %d mode %d ring %d"
        % (fused, batch, pos, slots, mode, ring))
    dev = "cuda"
    inp = gen.make_stage_tensors("decode_step_1536x28", device=dev, batch=batch, n_layers=2, vocab=4096)
    caches = gen.make_kv_caches(batch, slots, pos, n_layers=2, device=dev)
    before = [(bits(c["k_cache"]), bits(c["v_cache"])) for c in caches]
    step = steps.DecodeStepWithAttention(inp, caches, dev, fused=fused, mode=mode, ring=ring)
    if fused and mode == 0:
        assert step.n_launches == 1
    step.run()
    torch.cuda.synchronize()
    step.check()
    b = step.bufs
    eps = float(np.float32(inp["eps"]))
    for l, L in enumerate(inp["layers"]):
        h = bits(b["h"][l])
        for name, w in (("q", "wq"), ("k", "wk"), ("v", "wv")):
            ref = O.stage(h, bits(L[w]), norm=O.NORM_RMS, eps=eps, gamma=bits(L["g1"]))
            assert_close_bf16(bits(b[name][l]), ref, "layer %d %s" % (l, name))
        q = bits(b["q"][l]).reshape(batch, 12, 128)
        kn = bits(b["k"][l]).reshape(batch, 2, 128)
        vn = bits(b["v"][l]).reshape(batch, 2, 128)
        ref_a, ref_k, ref_v = O.decode_attention(q, kn, vn, before[l][0], before[l][1],
                                                 caches[l]["pos"].cpu().numpy())
        assert_close_bf16(bits(b["a"][l]).reshape(batch, 12, 128), ref_a, "layer %d attention" % l)
        np.testing.assert_array_equal(bits(caches[l]["k_cache"]), ref_k)
        np.testing.assert_array_equal(bits(caches[l]["v_cache"]), ref_v)
        ref = O.stage(bits(b["a"][l]), bits(L["wo"]), residual=h)
        assert_close_bf16(bits(b["h1"][l]), ref, "layer %d O" % l)
        ref = O.stage(bits(b["h1"][l]), bits(L["wg"]), norm=O.NORM_RMS, eps=eps, gamma=bits(L["g2"]),
                      epi=O.EPI_SWIGLU, W_up=bits(L["wu"]))
        assert_close_bf16(bits(b["s"][l]), ref, "layer %d gate/up" % l)
        ref = O.stage(bits(b["s"][l]), bits(L["wd"]), residual=bits(b["h1"][l]))
        assert_close_bf16(bits(b["h"][l + 1]), ref, "layer %d down" % l)
    _, _, lg = O.lmhead_argmax(bits(b["h"][-1]), bits(inp["g_f"]), bits(inp["W_lm"]), eps=eps, want_logits=True)
    for r in range(batch):
        check_argmax(int(b["idx"][r]), lg[r], "argmax row %d" % r)


@pytest.mark.parametrize("fused", [True, False])
def test_decode_step_with_attention_graph_replays_match_eager(fused):
    """The composed step captured in one HIP graph: three replays, with eager
    work between them, each bit-identical to an eager run (every replay
    appends the same key/value at the same slot, so the outputs repeat)."""
    from weight_gemv_norm_amd import steps
    say("decode step with attention: graph replays, fused %s" % fused)
    dev = "cuda"
    inp = gen.make_stage_tensors("decode_step_1536x28", device=dev, batch=2, n_layers=2, vocab=4096)
    caches = gen.make_kv_caches(2, 1024, [960, 500], n_layers=2, device=dev)
    step = steps.DecodeStepWithAttention(inp, caches, dev, fused=fused)
    step.run()
    torch.cuda.synchronize()
    eager = {k: [t.clone() for t in step.bufs[k]] for k in ("a", "h")}
    idx = step.bufs["idx"].clone()
    g = step.capture()
    for rep in range(3):
        for k in ("a", "h"):
            for t in step.bufs[k][1:] if k == "h" else step.bufs[k]:
                t.zero_()
        step.bufs["idx"].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ("a", "h"):
            for x, y in zip(step.bufs[k], eager[k]):
                assert torch.equal(x.view(torch.int16), y.view(torch.int16)), (rep, k)
        assert torch.equal(step.bufs["idx"], idx), rep
        step.check()


@pytest.mark.parametrize("hq,hkv,batch,slots,pos", [
    (8, 1, 1, 200, [199]),          # 8 query heads per key/value head: two full sweeps of four
    (3, 3, 2, 300, [17, 299]),      # one query head per key/value head
    (9, 3, 3, 700, [650, 0, 64]),   # three per head, three key/value heads
    (14, 2, 2, 129, [128, 100]),    # seven per head (a partial second sweep)
])
def test_attention_phases_group_sizes(hq, hkv, batch, slots, pos):
    """Attention items inside a small chain {RMSNorm -> Q, K, V} -> attention
    -> {O + residual} for other query/key-value head ratios than the pages'
    model: q, k, v, the attention output (against the oracle on the GPU's own
    q, k, v), both caches bit for bit, and O."""
    import weight_gemv_norm_amd as W
    from weight_gemv_norm_amd.api import make_stage, NORM_RMS, NORM_NONE
    say("attention phases hq %d hkv %d batch %d slots %d pos %s" % (hq, hkv, batch, slots, pos))
    dev, H, D = "cuda", 256, 128
    s = lambda t: gen.seed_of(901, hq * 100 + hkv, t)  # noqa: E731
    h = gen.normal((batch, H), 1.0, s(1), device=dev)
    g1 = gen.normal((H,), 0.1, s(2), mean=1.0, device=dev)
    wq = gen.normal((hq * D, H), 0.05, s(3), device=dev)
    wk = gen.normal((hkv * D, H), 0.05, s(4), device=dev)
    wv = gen.normal((hkv * D, H), 0.05, s(5), device=dev)
    wo = gen.normal((H, hq * D), 0.02, s(6), device=dev)
    q = torch.empty((batch, hq * D), dtype=torch.bfloat16, device=dev)
    k = torch.empty((batch, hkv * D), dtype=torch.bfloat16, device=dev)
    v = torch.empty((batch, hkv * D), dtype=torch.bfloat16, device=dev)
    a = torch.full((batch, hq * D), float("nan"), dtype=torch.bfloat16, device=dev)
    h1 = torch.empty((batch, H), dtype=torch.bfloat16, device=dev)
    t = gen.make_attention_tensors(batch, slots, pos, q_heads=hq, kv_heads=hkv, seed=5, device=dev)
    kc0, vc0 = bits(t["k_cache"]), bits(t["v_cache"])
    stages = [make_stage(wq, h, q, norm=NORM_RMS, eps=1e-6, gamma=g1),
              make_stage(wk, h, k, norm=NORM_RMS, eps=1e-6, gamma=g1),
              make_stage(wv, h, v, norm=NORM_RMS, eps=1e-6, gamma=g1),
              make_stage(wo, a, h1, norm=NORM_NONE, residual=h)]
    att = W.make_attn_stage(q, k, v, t["k_cache"], t["v_cache"], t["pos"], a)
    ch = W.Chain(stages, batch, attn=[(3, att)])
    assert ch.num_phases == 4
    ch.run()
    torch.cuda.synchronize()
    ch.check()
    eps = float(np.float32(1e-6))
    for name, wt, out in (("q", wq, q), ("k", wk, k), ("v", wv, v)):
        ref = O.stage(bits(h), bits(wt), norm=O.NORM_RMS, eps=eps, gamma=bits(g1))
        assert_close_bf16(bits(out), ref, name)
    ref_a, ref_k, ref_v = O.decode_attention(bits(q).reshape(batch, hq, D), bits(k).reshape(batch, hkv, D),
                                             bits(v).reshape(batch, hkv, D), kc0, vc0, t["pos"].cpu().numpy())
    assert_close_bf16(bits(a).reshape(batch, hq, D), ref_a, "attention")
    np.testing.assert_array_equal(bits(t["k_cache"]), ref_k)
    np.testing.assert_array_equal(bits(t["v_cache"]), ref_v)
    assert_close_bf16(bits(h1), O.stage(bits(a), bits(wo), residual=bits(h)), "O")
