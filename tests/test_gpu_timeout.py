"""A persistent chain whose in-kernel wait gives up must not let a later run
proceed on the flags and tickets it left behind: every later run exits at once
and writes nothing until wgn_chain_check has reset the counters.  The time-out
is forced from the host with a zero wait bound (wgn_chain_set_wait_us), so
every kernel ends normally; no kernel is made to hang."""
import numpy as np
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


def _outputs(bufs):
    out = []
    for v in bufs.values():
        for t in (v if isinstance(v, list) else [v]):
            if t is not None:
                out.append(t)
    return out


def test_timed_out_run_blocks_later_runs_until_check():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say("timeout: 2-layer decode chain, batch 1, zero wait bound")
    inp = gen.make_stage_tensors("decode_step_1536x28", device=DEV, batch=1, n_layers=2, vocab=4096)
    stages, bufs = steps.decoder_stages(inp, DEV)
    outs = _outputs(bufs)[1:]  # every buffer a stage writes (bufs["h"][0] is the input)
    ch = W.Chain(stages, 1)
    ch.run()
    ch.check()
    ref = [t.clone() for t in outs]

    ch.set_wait_us(0)  # a wait gives up at its first poll that misses a flag
    ch.run()
    torch.cuda.synchronize()
    for t in outs:
        t.view(torch.uint8).fill_(0xA5)
    ch.set_wait_us(-1)
    ch.run()  # no check in between: this run must write nothing
    torch.cuda.synchronize()
    for t in outs:
        assert bool((t.view(torch.uint8) == 0xA5).all()), "a run after a time-out wrote its outputs"
    with pytest.raises(W.WgnError) as e:
        ch.check()
    assert e.value.status == L.E_TIMEOUT
    ch.check()  # the counters were reset by the call above
    ch.run()
    ch.check()
    for t, r in zip(outs, ref):
        assert torch.equal(t, r), "outputs after the reset differ from the first run"
