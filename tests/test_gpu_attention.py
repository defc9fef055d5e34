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
