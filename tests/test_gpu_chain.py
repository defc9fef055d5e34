"""GPU parity of whole chains (persistent kernel and one-launch-per-phase), per
stage and teacher-forced, against the CPU oracle; plus the invariants the
pages rely on: repeated runs and the two launch modes give the same bits."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import gen
from tests.gpu_util import assert_close_bf16, bits, check_argmax, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import weight_gemv_norm_amd as W
    from weight_gemv_norm_amd import steps
    from weight_gemv_norm_amd import _lib as L

DEV = "cuda"
EPS32 = float(np.float32(1e-6))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()
    yield


def rows_sample(N, k=48, seed=0):
    rng = np.random.default_rng(seed + N)
    r = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, k)]))
    return r


def check_stage_rows(what, W_, x, y, rows=None, **kw):
    """Oracle on the GPU's inputs; all rows, or the given row sample."""
    Wb = W_ if rows is None else W_[torch.as_tensor(rows, device=DEV)]
    up = kw.pop("W_up", None)
    if up is not None and rows is not None:
        up = up[torch.as_tensor(rows, device=DEV)]
    res = kw.pop("residual", None)
    if res is not None and rows is not None:
        res = res[:, torch.as_tensor(rows, device=DEV)].contiguous()
    g = kw.pop("gamma", None)
    ref = O.stage(bits(x.contiguous()), bits(Wb.contiguous()), gamma=None if g is None else bits(g),
                  W_up=None if up is None else bits(up.contiguous()),
                  residual=None if res is None else bits(res), **kw)
    yb = bits(y if rows is None else y[:, torch.as_tensor(rows, device=DEV)].contiguous())
    return assert_close_bf16(yb, ref, what)


def check_decoder(inp, bufs, layers_full, sample_other=True):
    """Per-stage teacher-forced check of a decode step's buffers."""
    worst = 0.0
    for l, Ld in enumerate(inp["layers"]):
        full = l in layers_full
        if not full and not sample_other:
            continue
        h, h1, s, hn = bufs["h"][l], bufs["h1"][l], bufs["s"][l], bufs["h"][l + 1]
        pick = (lambda N: None) if full else (lambda N: rows_sample(N, seed=l))
        for name, key in (("q", "wq"), ("k", "wk"), ("v", "wv")):
            worst = max(worst, check_stage_rows("L%d %s" % (l, name), Ld[key], h, bufs[name][l],
                                                rows=pick(Ld[key].shape[0]), norm=O.NORM_RMS, eps=EPS32,
                                                gamma=Ld["g1"]))
        worst = max(worst, check_stage_rows("L%d o" % l, Ld["wo"], Ld["a"], h1, rows=pick(Ld["wo"].shape[0]),
                                            norm=O.NORM_NONE, residual=h))
        worst = max(worst, check_stage_rows("L%d gate/up" % l, Ld["wg"], h1, s, rows=pick(Ld["wg"].shape[0]),
                                            norm=O.NORM_RMS, eps=EPS32, gamma=Ld["g2"], epi=O.EPI_SWIGLU,
                                            W_up=Ld["wu"]))
        worst = max(worst, check_stage_rows("L%d down" % l, Ld["wd"], s, hn, rows=pick(Ld["wd"].shape[0]),
                                            norm=O.NORM_NONE, residual=h1))
    if "W_lm" in inp:
        hL = bufs["h"][-1]
        ridx, rmx, rlog = O.lmhead_argmax(bits(hL), bits(inp["g_f"]), bits(inp["W_lm"]), eps=EPS32,
                                          want_logits=True)
        for b in range(hL.shape[0]):
            check_argmax(int(bufs["idx"][b]), rlog[b], "lm head b=%d" % b)
    return worst


def snapshot(bufs):
    out = []
    for k in sorted(bufs):
        v = bufs[k]
        for t in (v if isinstance(v, list) else [v]):
            if t is not None:
                out.append(t.detach().clone())
    return out


def same_bits(a, b):
    return all(torch.equal(x.view(torch.int8) if x.dtype != torch.int32 else x,
                           y.view(torch.int8) if y.dtype != torch.int32 else y) for x, y in zip(a, b))


# ---------------------------------------------------------------- workloads
def test_decoder_block_1536_batch1():
    """One Llama-style block at hidden 1536, batch 1: three phases."""
    say("chain decoder_block_1536 B=1")
    inp = gen.make_stage_tensors("decoder_block_1536", device=DEV)
    stages, bufs = steps.decoder_stages(inp, DEV)
    ch = W.Chain(stages, 1)
    assert ch.num_phases == 3
    assert ch.stage_phases() == [0, 0, 0, 0, 1, 2]
    ch.run()
    ch.check()
    check_decoder(inp, bufs, layers_full={0})


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 8, 16])
def test_small_decode_step_all_batches(B):
    """Two full-width blocks + an LM head of 20000 rows, both launch modes;
    batch > 4 runs on the matrix cores, batch 16 streams the down projection
    in K windows."""
    say("chain decode_step 2 layers V=20000 B=%d" % B)
    inp = gen.make_stage_tensors("decode_step_1536x28", device=DEV, batch=B, n_layers=2, vocab=20000)
    stages, bufs = steps.decoder_stages(inp, DEV)
    ch = W.Chain(stages, B, mode=0)
    # block 1's output projection is hoisted (its residual add runs in block 0's
    # down projection); batch 16 streams each down projection in two K windows
    assert ch.num_phases == (8 if B > 8 else 6)
    ch.run()
    ch.check()
    check_decoder(inp, bufs, layers_full={0, 1})
    first = snapshot(bufs)
    ch.run()
    ch.check()
    assert same_bits(first, snapshot(bufs)), "persistent rerun not bit-identical"
    ch1 = W.Chain(stages, B, mode=1)
    ch1.run()
    torch.cuda.synchronize()
    assert same_bits(first, snapshot(bufs)), "per-phase launches differ from the persistent kernel"
    # without the cross-stage rewrite: every stage in its own place, same checks
    ch2 = W.Chain(stages, B, fuse=False)
    assert ch2.num_phases == (9 if B > 8 else 7)
    ch2.run()
    ch2.check()
    check_decoder(inp, bufs, layers_full={1})


def zero_outputs(bufs):
    for k, v in bufs.items():
        if k in ("h", "x"):
            v = v[1:]  # the chain's input
        for t in (v if isinstance(v, list) else [v]):
            if t is not None:
                t.zero_()


@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_rings_agree_decode(B):
    """Every block-buffer ring of the vector path gives the same bits: the
    rings change when loads are issued, not the order of any arithmetic.  The
    oracle checks the first; persistent and per-phase launches both run."""
    say("rings decode_step 2 layers V=20000 B=%d" % B)
    inp = gen.make_stage_tensors("decode_step_1536x28", device=DEV, batch=B, n_layers=2, vocab=20000)
    stages, bufs = steps.decoder_stages(inp, DEV)
    assert W.Chain(stages, B).ring == (0 if B == 1 else 2)
    ref = None
    for ring in (1, 2, 3):
        for mode in (0, 1):
            ch = W.Chain(stages, B, mode=mode, ring=ring)
            assert ch.ring == ring - 1
            zero_outputs(bufs)
            ch.run()
            ch.check()
            snap = snapshot(bufs)
            if ref is None:
                check_decoder(inp, bufs, layers_full={0, 1})
                ref = snap
            else:
                assert same_bits(ref, snap), "ring %d mode %d differs" % (ring - 1, mode)


@pytest.mark.parametrize("B", [1, 4])
def test_rings_agree_ln_chain(B):
    """The LayerNorm chain (a fraction of a unit per wave and phase) chooses
    ring 1 by itself; every ring gives the same bits, checked by the oracle."""
    say("rings ln_gelu_chain_768x72 B=%d" % B)
    inp = gen.make_stage_tensors("ln_gelu_chain_768x72", device=DEV, batch=B, seeded_ln_params=True)
    stages, bufs = steps.ln_gelu_chain_stages(inp, DEV)
    assert W.Chain(stages, B).ring == 1
    ref = None
    for ring in (2, 1, 3):
        ch = W.Chain(stages, B, ring=ring)
        zero_outputs(bufs)
        ch.run()
        ch.check()
        snap = snapshot(bufs)
        if ref is None:
            xs = bufs["x"]
            for i, Ld in enumerate(inp["layers"]):
                r = O.stage(bits(xs[i]), bits(Ld["W"]), norm=O.NORM_LAYER, eps=float(np.float32(1e-5)),
                            gamma=bits(Ld["gamma"]), beta=bits(Ld["beta"]), bias=bits(Ld["bias"]),
                            epi=O.EPI_GELU_TANH)
                assert_close_bf16(bits(xs[i + 1]), r, "ln-gelu ring %d layer %d" % (ring - 1, i))
            ref = snap
        else:
            assert same_bits(ref, snap), "ring %d differs" % (ring - 1)


@pytest.mark.parametrize("B", [1, 4, 16])
def test_ln_gelu_chain_768x72(B):
    """72 x [LayerNorm(768) -> Linear -> GELU-tanh], seeded LN params, per stage."""
    say("chain ln_gelu_chain_768x72 B=%d" % B)
    inp = gen.make_stage_tensors("ln_gelu_chain_768x72", device=DEV, batch=B, seeded_ln_params=True)
    stages, bufs = steps.ln_gelu_chain_stages(inp, DEV)
    ch = W.Chain(stages, B)
    assert ch.num_phases == 72
    ch.run()
    ch.check()
    xs = bufs["x"]
    for i, Ld in enumerate(inp["layers"]):
        ref = O.stage(bits(xs[i]), bits(Ld["W"]), norm=O.NORM_LAYER, eps=float(np.float32(1e-5)),
                      gamma=bits(Ld["gamma"]), beta=bits(Ld["beta"]), bias=bits(Ld["bias"]),
                      epi=O.EPI_GELU_TANH)
        assert_close_bf16(bits(xs[i + 1]), ref, "ln-gelu layer %d" % i)


@pytest.mark.parametrize("B", [1, 2, 3, 4, 8])
def test_phase_with_several_normalised_sources(B):
    """Independent stages over different inputs share one phase: RMSNorm and
    LayerNorm sources of different lengths (one ragged, one with no gain) are
    normalised together, then each stage is checked against the oracle."""
    say("chain several sources B=%d" % B)
    specs = [  # (N, K, norm, gamma, beta, epi)
        (300, 1536, O.NORM_RMS, True, False, O.EPI_NONE),
        (129, 768, O.NORM_LAYER, True, True, O.EPI_GELU_TANH),
        (64, 264, O.NORM_LAYER, False, False, O.EPI_NONE),
        (200, 520, O.NORM_RMS, False, False, O.EPI_NONE),
    ]
    stages, checks = [], []
    for i, (N, K, norm, hg, hb, epi) in enumerate(specs):
        seed = 900 + 10 * i
        Wt = gen.normal((N, K), 0.05, seed + 1, device=DEV)
        x = gen.normal((B, K), 1.0, seed + 2, mean=0.3 if norm == O.NORM_LAYER else 0.0, device=DEV)
        g = gen.normal((K,), 0.1, seed + 3, mean=1.0, device=DEV) if hg else None
        be = gen.normal((K,), 0.02, seed + 4, device=DEV) if hb else None
        bias = gen.normal((N,), 0.02, seed + 5, device=DEV) if epi == O.EPI_GELU_TANH else None
        y = torch.empty((B, N), dtype=torch.bfloat16, device=DEV)
        eps = 1e-5 if norm == O.NORM_LAYER else 1e-6
        stages.append(W.make_stage(Wt, x, y, norm=norm, eps=eps, gamma=g, beta=be, bias=bias, epi=epi))
        checks.append((Wt, x, y, norm, eps, g, be, bias, epi))
    ch = W.Chain(stages, B)
    assert ch.num_phases == 1
    ch.run()
    ch.check()
    torch.cuda.synchronize()
    for i, (Wt, x, y, norm, eps, g, be, bias, epi) in enumerate(checks):
        ref = O.stage(bits(x), bits(Wt), norm=norm, eps=float(np.float32(eps)), epi=epi,
                      gamma=None if g is None else bits(g), beta=None if be is None else bits(be),
                      bias=None if bias is None else bits(bias))
        assert_close_bf16(bits(y), ref, "source %d" % i)


def test_ln_gelu_chain_default_params():
    """Default-initialised LayerNorm (gain 1, shift 0), batch 4, the benchmark's configuration."""
    say("chain ln_gelu_chain_768x72 default LN B=4")
    inp = gen.make_stage_tensors("ln_gelu_chain_768x72", device=DEV, batch=4)
    stages, bufs = steps.ln_gelu_chain_stages(inp, DEV)
    ch = W.Chain(stages, 4)
    ch.run()
    ch.check()
    xs = bufs["x"]
    for i in (0, 35, 71):
        Ld = inp["layers"][i]
        ref = O.stage(bits(xs[i]), bits(Ld["W"]), norm=O.NORM_LAYER, eps=float(np.float32(1e-5)),
                      gamma=bits(Ld["gamma"]), beta=bits(Ld["beta"]), bias=bits(Ld["bias"]),
                      epi=O.EPI_GELU_TANH)
        assert_close_bf16(bits(xs[i + 1]), ref, "ln-gelu layer %d" % i)


@pytest.mark.parametrize("B", [1, 4, 8, 16])
def test_full_decode_step(B):
    """The 28-layer, 151936-vocab decode step in the benchmark's launch
    configuration at batch 1, 4, 8, 16: layers 0, 13, 27 and the LM head
    checked in full, every other stage on sampled rows."""
    say("chain decode_step_1536x28 full B=%d" % B)
    inp = gen.make_stage_tensors("decode_step_1536x28", device=DEV, batch=B)
    stages, bufs = steps.decoder_stages(inp, DEV)
    ch = W.Chain(stages, B)
    # 2 dependent phases per block after the first (output projections hoisted);
    # at batch 16 the down projections take two K windows and a hoisted product
    # that would overflow LDS stays in place
    if B <= 8:
        assert ch.num_phases == 3 + 2 * 27 + 1
    assert (ch.num_phases, ch.stage_phases()) == W.plan_phases(stages, B, grid=ch.grid)
    ch.run()
    ch.check()
    first = snapshot(bufs)
    check_decoder(inp, bufs, layers_full={0, 13, 27} if B <= 4 else {0, 27})
    for _ in range(2):
        ch.run()
    ch.check()
    assert same_bits(first, snapshot(bufs)), "decode step rerun not bit-identical"
