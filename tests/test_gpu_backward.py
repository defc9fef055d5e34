"""GPU parity of the training step: the forward chain's kept pre-activations
and the backward pass (wgn_backward_*) against the CPU oracle, block by block
and teacher-forced (each block's oracle backward runs on the forward
activations and the output gradient the GPU produced for that block, and
takes the GPU's BF16 rounding of gz, a quantisation decision, as given);
plus the invariants: prefetch on and off and repeated runs give the same
bits, graph replays match eager runs, and a forced time-out is reported."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import gen
from tests.gpu_util import assert_close, assert_close_bf16, bits, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import weight_gemv_norm_amd as W
    from weight_gemv_norm_amd import steps
    from weight_gemv_norm_amd import _lib as L

DEV = "cuda"
EPS = float(np.float32(1e-5))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()
    O.set_threads(min(16, O.max_threads()))
    yield


def f64(t):
    return O.bf16_array_to_f64(bits(t))


def chain_inputs(dims, B, seed, bias=True, gamma=True, beta=True):
    """A LayerNorm -> Linear -> GELU chain with widths dims[0] -> dims[1] -> ...
    (seeded N(0,1) input, W ~ N(0, 1/K), bias ~ N(0, 0.02), gain ~ 1 + N(0, 0.1),
    shift ~ N(0, 0.02): the LayerNorm-chain workload's distributions)."""
    inp = {"batch": B, "eps": 1e-5, "x": gen.normal((B, dims[0]), 1.0, seed, device=DEV), "layers": []}
    for i in range(len(dims) - 1):
        K, N = dims[i], dims[i + 1]
        s = seed + 10 * (i + 1)
        d = {"W": gen.normal((N, K), 1.0 / np.sqrt(K), s + 1, device=DEV)}
        if bias:
            d["bias"] = gen.normal((N,), 0.02, s + 2, device=DEV)
        if gamma:
            d["gamma"] = gen.normal((K,), 0.1, s + 3, mean=1.0, device=DEV)
        if beta:
            d["beta"] = gen.normal((K,), 0.02, s + 4, device=DEV)
        inp["layers"].append(d)
    return inp


def check_training_step(ts, what, g_out=None, layers=None):
    """Teacher-forced oracle comparison of every block (or the given ones)."""
    inp, B = ts.inp, ts.B
    xs = ts.bufs["x"]
    n = len(inp["layers"])
    last_gy = O.mean_square_grad(bits(xs[n])) if g_out is None else bits(g_out)
    assert_close_bf16(bits(ts.grads[n - 1]["gy"]), last_gy, what + ": gy of the last block")
    for i in (range(n) if layers is None else layers):
        Ld = inp["layers"][i]
        g = ts.grads[i]
        opt = {k: bits(Ld[k]) for k in ("gamma", "beta", "bias") if Ld.get(k) is not None}
        r = O.block_backward(bits(xs[i]), bits(Ld["W"]), bits(g["gy"]), eps=EPS, gz_in=bits(g["gz"]), **opt)
        tag = "%s block %d" % (what, i)
        # the comparison must not be between two vanishing gradients
        assert np.sqrt(np.mean(r["gW"] ** 2)) > 1e-30 and np.count_nonzero(bits(g["gW"])) > g["gW"].numel() // 2, tag
        assert_close(f64(g["gz"]), r["gz"], tag + " gz")
        assert_close_bf16(bits(g["gW"]), O.to_bf16_bits(r["gW"]), tag + " gW")
        if "bias" in opt:
            assert_close_bf16(bits(g["gb"]), O.to_bf16_bits(r["gb"]), tag + " gb")
        if "gamma" in opt:
            assert_close_bf16(bits(g["ggamma"]), O.to_bf16_bits(r["ggamma"]), tag + " ggamma")
        if "beta" in opt:
            assert_close_bf16(bits(g["gbeta"]), O.to_bf16_bits(r["gbeta"]), tag + " gbeta")
        gx = ts.g_in if i == 0 else ts.grads[i - 1]["gy"]
        assert_close(f64(gx), r["gx"], tag + " gx")


def snapshot(ts):
    out = [bits(ts.g_in)]
    for g in ts.grads:
        out += [bits(v) for v in g.values()]
    return out


@pytest.mark.parametrize("B", [1, 4, 16])
def test_forward_keeps_pre_activation(B):
    """A GELU stage with `pre` set writes z = acc + bias (FP32) and the same
    outputs as without it."""
    say("backward: forward pre-activation B=%d" % B)
    inp = chain_inputs([264, 200, 136], B, 7100)
    st, bufs = steps.ln_gelu_chain_stages(inp, DEV, keep_pre=True)
    W.Chain(st, B).run()
    st0, bufs0 = steps.ln_gelu_chain_stages(inp, DEV)
    W.Chain(st0, B).run()
    torch.cuda.synchronize()
    for i, Ld in enumerate(inp["layers"]):
        assert torch.equal(bufs["x"][i + 1], bufs0["x"][i + 1])
        _, acc = O.stage(bits(bufs["x"][i]), bits(Ld["W"]), norm=O.NORM_LAYER, eps=EPS, gamma=bits(Ld["gamma"]),
                         beta=bits(Ld["beta"]), bias=bits(Ld["bias"]), epi=O.EPI_GELU_TANH, want_acc=True)
        assert_close(bufs["pre"][i].double().cpu().numpy(), acc, "pre-activation of stage %d" % i)


def test_batched_path_keeps_pre_activation():
    """The same through the tiled matrix-core products (batch 32)."""
    say("backward: forward pre-activation, tiled path B=32")
    B = 32
    inp = chain_inputs([264, 200], B, 7200)
    st, bufs = steps.ln_gelu_chain_stages(inp, DEV, keep_pre=True)
    W.layer_chain(st, B, path=W.PATH_TILED)
    torch.cuda.synchronize()
    Ld = inp["layers"][0]
    _, acc = O.stage(bits(bufs["x"][0]), bits(Ld["W"]), norm=O.NORM_LAYER, eps=EPS, gamma=bits(Ld["gamma"]),
                     beta=bits(Ld["beta"]), bias=bits(Ld["bias"]), epi=O.EPI_GELU_TANH, want_acc=True)
    assert_close(bufs["pre"][0].double().cpu().numpy(), acc, "pre-activation, tiled path")


@pytest.mark.parametrize("B", [1, 3, 4, 16])
def test_backward_ragged_chain(B):
    """Widths 264 -> 200 -> 136 -> 72 -> 328: rows and columns that end inside
    a 32 x 64 tile, blocks that widen and narrow."""
    say("backward: ragged chain B=%d" % B)
    inp = chain_inputs([264, 200, 136, 72, 328], B, 7300 + B)
    ts = steps.TrainStep(inp, DEV)
    ts.run()
    ts.check()
    check_training_step(ts, "ragged B=%d" % B)


def test_backward_without_affine_or_bias():
    """Unit gain, zero shift and no bias (NULL pointers): no gain, shift or
    bias gradients are asked for."""
    say("backward: no gamma/beta/bias")
    inp = chain_inputs([192, 256, 128], 4, 7400, bias=False, gamma=False, beta=False)
    ts = steps.TrainStep(inp, DEV)
    ts.run()
    ts.check()
    check_training_step(ts, "no affine")


def test_backward_given_output_gradient():
    """g_out given instead of the mean-square loss."""
    say("backward: given output gradient")
    B = 4
    inp = chain_inputs([256, 256, 256], B, 7500)
    g_out = gen.normal((B, 256), 1e-3, 7599, device=DEV)
    ts = steps.TrainStep(inp, DEV, g_out=g_out)
    ts.run()
    ts.check()
    assert torch.equal(ts.grads[-1]["gy"], g_out)
    check_training_step(ts, "given g_out", g_out=g_out)


@pytest.mark.parametrize("B", [4, 16])
def test_backward_ln_gelu_chain_768x72(B):
    """The LayerNorm chain workload (72 blocks of 768) at batch 4 and 16, every
    block checked."""
    say("backward: ln_gelu_chain_768x72 B=%d" % B)
    inp = gen.make_stage_tensors("ln_gelu_chain_768x72", device=DEV, batch=B, seeded_ln_params=True)
    ts = steps.TrainStep(inp, DEV)
    ts.run()
    ts.check()
    check_training_step(ts, "768x72 B=%d" % B)


def test_prefetch_on_off_and_reruns_bit_identical():
    """The prefetch only moves when weight loads are issued: gradients are the
    same bits with it on and off, and on every rerun."""
    say("backward: prefetch on/off bit-identical")
    inp = gen.make_stage_tensors("ln_gelu_chain_768x72", device=DEV, batch=8, seeded_ln_params=True,
                                 n_layers=12)
    ts = steps.TrainStep(inp, DEV, prefetch=True)
    ts.run()
    ts.check()
    ref = snapshot(ts)
    for pf in (False, True, False):
        ts.prefetch = pf
        ts.backward()
        ts.check()
        for a, b in zip(ref, snapshot(ts)):
            assert np.array_equal(a, b), "prefetch=%s changed bits" % pf


def test_training_step_graph_replay():
    """Forward + backward captured in one HIP graph: every replay (with eager
    work between replays) gives the eager result's bits."""
    say("backward: graph replay")
    inp = gen.make_stage_tensors("ln_gelu_chain_768x72", device=DEV, batch=4, seeded_ln_params=True, n_layers=8)
    ts = steps.TrainStep(inp, DEV)
    ts.run()
    ts.check()
    ref = snapshot(ts)
    g = ts.capture()
    for rep in range(3):
        for t in ts.grads:
            t["gW"].zero_()
        ts.g_in.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ts.check()
        for a, b in zip(ref, snapshot(ts)):
            assert np.array_equal(a, b), "replay %d differs" % rep
        _ = torch.ones(1024, device=DEV).sum().item()  # eager work between replays


def test_forced_time_out_is_reported_and_cleared():
    """A wait bound of 0 makes the first unsuccessful poll give up: the kernel
    exits normally and check reports WGN_E_TIMEOUT; the next run (default
    bound) starts from cleared counters and gives the reference bits."""
    say("backward: forced time-out")
    inp = gen.make_stage_tensors("ln_gelu_chain_768x72", device=DEV, batch=4, seeded_ln_params=True, n_layers=6)
    ts = steps.TrainStep(inp, DEV)
    ts.run()
    ts.check()
    ref = snapshot(ts)
    ts.bwd.set_wait_us(0)
    ts.backward()
    with pytest.raises(W.WgnError) as e:
        ts.bwd.check()
    assert e.value.status == L.E_TIMEOUT
    ts.bwd.set_wait_us(-1)
    ts.backward()
    ts.bwd.check()
    for a, b in zip(ref, snapshot(ts)):
        assert np.array_equal(a, b)


def test_one_shot_call_matches_handle():
    """wgn_chain_backward (create + run + destroy) equals a handle's run."""
    say("backward: one-shot call")
    B = 2
    inp = chain_inputs([128, 192, 64], B, 7600)
    ts = steps.TrainStep(inp, DEV)
    ts.run()
    ts.check()
    ref = snapshot(ts)
    gs = [W.make_grad(g["gW"], g.get("gb"), g.get("ggamma"), g.get("gbeta"), g.get("gy"), g.get("gz"))
          for g in ts.grads]
    for t in ts.grads:
        t["gW"].zero_()
    W.chain_backward(ts.stages, B, gs, g_in=ts.g_in, prefetch=False)
    torch.cuda.synchronize()
    for a, b in zip(ref, snapshot(ts)):
        assert np.array_equal(a, b)
