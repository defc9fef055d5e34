"""GPU tests of the optional Infinity-Cache prefetch plan (touch passes on a
second stream, chains with one launch per phase): a plan changes no output
bit, the argument checks hold, and the tuner returns a plan that obeys its
acceptance rule ("Making small PyTorch ops faster on a laptop GPU", sections
"Prefetching the next layer while this one runs" and "Measuring instead of
predicting")."""
import pytest
import torch

from synth import gen
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import weight_gemv_norm_amd as W
    from weight_gemv_norm_amd import steps
    from weight_gemv_norm_amd import _lib as L

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()
    yield


def snapshot(bufs):
    out = []
    for v in bufs.values():
        for t in (v if isinstance(v, list) else [v]):
            if isinstance(t, torch.Tensor):
                out.append(t.detach().clone())
    return out


def same_bits(a, b):
    return len(a) == len(b) and all(torch.equal(x.view(torch.uint8) if x.dtype != torch.int32 else x,
                                                y.view(torch.uint8) if y.dtype != torch.int32 else y)
                                    for x, y in zip(a, b))


def plan(d, blocks, frac):
    p = W.Plan()
    p.prefetch, p.distance, p.blocks, p.frac_pct = 1, d, blocks, frac
    return p


@pytest.mark.parametrize("B", [1, 4, 16])
def test_plan_runs_are_bit_identical_decode(B):
    """Two decoder blocks + a 20000-row LM head: plain per-phase launches, the
    persistent kernel and per-phase launches with touch passes agree bit for
    bit (batch 16 includes K-windowed launches)."""
    say("prefetch plan decode_step 2 layers V=20000 B=%d" % B)
    inp = gen.make_stage_tensors("decode_step_1536x28", device=DEV, batch=B, n_layers=2, vocab=20000)
    stages, bufs = steps.decoder_stages(inp, DEV)
    ch0 = W.Chain(stages, B, mode=0)
    ch0.run()
    ch0.check()
    ref = snapshot(bufs)
    ch1 = W.Chain(stages, B, mode=1)
    side = torch.cuda.Stream()
    for p in (plan(1, 64, 100), plan(2, 16, 50), plan(4, 256, 1)):
        for t in bufs["h"][1:] + bufs["s"] + [bufs["idx"]]:
            t.zero_()
        ch1.run(plan=p, side=side)
        # later work on the main stream sees the whole run (joined back)
        got = snapshot(bufs)
        torch.cuda.synchronize()
        assert same_bits(ref, got), "plan d=%d blocks=%d frac=%d changed outputs" % (
            p.distance, p.blocks, p.frac_pct)


def test_plan_runs_are_bit_identical_ln_chain():
    say("prefetch plan ln_gelu_chain_768x72 B=4")
    inp = gen.make_stage_tensors("ln_gelu_chain_768x72", device=DEV, batch=4, seeded_ln_params=True)
    stages, bufs = steps.ln_gelu_chain_stages(inp, DEV)
    ch1 = W.Chain(stages, 4, mode=1)
    ch1.run()
    torch.cuda.synchronize()
    ref = snapshot(bufs)
    side = torch.cuda.Stream()
    for _ in range(3):
        ch1.run(plan=plan(1, 16, 100), side=side)
    torch.cuda.synchronize()
    assert same_bits(ref, snapshot(bufs))


def test_plan_argument_checks():
    say("prefetch plan argument checks")
    inp = gen.make_stage_tensors("ln_gelu_chain_768x72", device=DEV, batch=1, n_layers=3)
    stages, bufs = steps.ln_gelu_chain_stages(inp, DEV)
    ch0 = W.Chain(stages, 1, mode=0)
    ch1 = W.Chain(stages, 1, mode=1)
    side = torch.cuda.Stream()
    cur = torch.cuda.current_stream()
    with pytest.raises(W.WgnError) as e:
        ch0.run(plan=plan(1, 16, 100), side=side)
    assert e.value.status == L.E_UNSUPPORTED
    for bad in (plan(0, 16, 100), plan(5, 16, 100), plan(1, 0, 100), plan(1, 2048, 100), plan(1, 16, 0),
                plan(1, 16, 101)):
        with pytest.raises(W.WgnError) as e:
            ch1.run(plan=bad, side=side)
        assert e.value.status == L.E_ARG
    with pytest.raises(W.WgnError) as e:
        ch1.run(plan=plan(1, 16, 100), side=cur)
    assert e.value.status == L.E_ARG
    with pytest.raises(W.WgnError) as e:
        ch0.tune_plan(side, reps=3)
    assert e.value.status == L.E_UNSUPPORTED
    # a plain plan runs any chain
    ch0.run(plan=W.Plan(), side=None)
    ch0.check()


def test_plan_tune_follows_its_rule():
    """The tuner measures its candidates and keeps one only when the lower end
    of its 95 % interval clears +1 %; otherwise the plan is plain."""
    say("prefetch plan tune ln_gelu_chain_768x72 B=4 (24 layers)")
    inp = gen.make_stage_tensors("ln_gelu_chain_768x72", device=DEV, batch=4, n_layers=24)
    stages, bufs = steps.ln_gelu_chain_stages(inp, DEV)
    ch1 = W.Chain(stages, 4, mode=1)
    side = torch.cuda.Stream()
    p = ch1.tune_plan(side, reps=5)
    assert p.candidates == 12
    assert p.plain_us > 0 and p.best_us > 0
    if p.prefetch:
        assert p.speedup_lo > 1.01
    else:
        assert not p.speedup_lo > 1.01
    assert 1 <= p.distance <= 2 and p.blocks in (16, 64, 256) and p.frac_pct in (50, 100)
    ch1.run(plan=p, side=side)
    torch.cuda.synchronize()
