"""GPU parity of the batched matrix-core path (wgn_gemm_norm, and wgn_layer_chain
at batch 17-128) against the CPU oracle, teacher-forced per stage, on seeded
synthetic inputs: ragged batches, row tiles and K tails, every epilogue, tiles
shared between workgroups and their fixed-order sum, the argmax merge and the
decode step."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import gen
from tests.gpu_util import assert_close, assert_close_bf16, bits, check_argmax, say

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
    L.lib()  # fails loudly if the library is missing
    assert W.device_cu_count() > 0
    yield


def rnd(shape, std, seed, mean=0.0):
    return gen.normal(shape, std, seed, mean=mean, device=DEV)


CASES = [
    # (N, K, B, norm, epi, bias, residual, gamma)
    (1, 8, 17, O.NORM_RMS, O.EPI_NONE, False, False, True),          # one row, one 8-wide K step
    (37, 264, 32, O.NORM_NONE, O.EPI_GELU_TANH, True, False, False),  # ragged rows, K tail inside a step
    (1000, 520, 33, O.NORM_NONE, O.EPI_NONE, False, True, False),    # batch 33: three 16-row groups
    (300, 1536, 64, O.NORM_RMS, O.EPI_SWIGLU, False, True, True),    # tiles shared by 6 workgroups, two accumulator sets
    (1536, 8960, 128, O.NORM_NONE, O.EPI_NONE, False, True, False),  # the down projection: 24 tiles over 256 workgroups
    (8960, 1536, 128, O.NORM_RMS, O.EPI_SWIGLU, False, False, True),  # gate/up at batch 128
    (2048, 1536, 100, O.NORM_RMS, O.EPI_NONE, False, False, True),   # Q/K/V-sized, batch 100
    (17, 4096, 48, O.NORM_RMS, O.EPI_NONE, True, True, False),       # RMSNorm with a unit gain
    (513, 1024, 128, O.NORM_NONE, O.EPI_GELU_TANH, True, True, False),
    (37, 264, 32, O.NORM_LAYER, O.EPI_GELU_TANH, True, False, True),  # LayerNorm (gain and shift)
    (768, 768, 64, O.NORM_LAYER, O.EPI_GELU_TANH, True, False, True),  # the LayerNorm chain's shape
    (513, 1024, 20, O.NORM_LAYER, O.EPI_NONE, True, True, False),     # LayerNorm, unit gain, zero shift
    # 7 tiles x 150 windows over 256 workgroups of 4 or 5 windows: ranges that
    # start and end inside tiles, workgroups whose range crosses a tile boundary
    (448, 9600, 24, O.NORM_RMS, O.EPI_NONE, False, True, True),
    # 1028 tiles, 4 or more per workgroup: one workgroup per tile, a ragged last tile
    (65760, 128, 17, O.NORM_NONE, O.EPI_GELU_TANH, True, False, False),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c[:5]) for c in CASES])
def test_gemm_norm_shapes(case):
    N, K, B, norm, epi, use_bias, use_res, use_gamma = case
    say("gemm_norm N=%d K=%d B=%d norm=%d epi=%d" % (N, K, B, norm, epi))
    seed = hash(case) & 0xFFFF
    Wt = rnd((N, K), 0.05, seed + 1)
    Wu = rnd((N, K), 0.05, seed + 2) if epi == O.EPI_SWIGLU else None
    # a strided activation buffer: rows padded to K + 16 elements
    xs = torch.empty((B, K + 16), dtype=torch.bfloat16, device=DEV)
    xs[:, :K] = rnd((B, K), 1.0, seed + 3, mean=0.3 if norm == O.NORM_LAYER else 0.0)
    x = xs[:, :K]
    gamma = rnd((K,), 0.1, seed + 4, mean=1.0) if (norm != O.NORM_NONE and use_gamma) else None
    beta = rnd((K,), 0.02, seed + 5) if (norm == O.NORM_LAYER and use_gamma) else None
    bias = rnd((N,), 0.02, seed + 6) if use_bias else None
    res = rnd((B, N), 1.0, seed + 7) if use_res else None
    y = torch.empty((B, N), dtype=torch.bfloat16, device=DEV)
    eps = 1e-5 if norm == O.NORM_LAYER else 1e-6
    st = W.make_stage(Wt, x, y, norm=norm, eps=eps, gamma=gamma, beta=beta, bias=bias, epi=epi, W_up=Wu,
                      residual=res)
    ws = W.workspace(W.gemm_norm_workspace_bytes(st, B))
    W.gemm_norm(st, B, ws=ws)
    torch.cuda.synchronize()
    ref = O.stage(bits(x.contiguous()), bits(Wt), norm=norm, epi=epi, eps=float(np.float32(eps)),
                  gamma=None if gamma is None else bits(gamma), beta=None if beta is None else bits(beta),
                  W_up=None if Wu is None else bits(Wu),
                  bias=None if bias is None else bits(bias), residual=None if res is None else bits(res))
    assert_close_bf16(bits(y), ref, "gemm_norm %r" % (case,))
    # reruns give the same bits (shared tiles are added in contributor order) and leave
    # the workspace's tickets at zero
    first = y.clone()
    for _ in range(2):
        W.gemm_norm(st, B, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), y.view(torch.int16)), "rerun not bit-identical"
    ntiles = (N + 63) // 64
    assert int(ws[: (ntiles + 1) * 4].view(torch.int32).abs().sum()) == 0, "tickets not left at zero"


def test_gemm_norm_agrees_with_the_persistent_path_at_16():
    """At batch 16 both the persistent kernel's matrix-core path and this path
    run; both meet the oracle, and they agree within two tolerances."""
    say("gemm_norm vs gemv_norm at batch 16")
    N, K, B = 300, 1536, 16
    Wt, Wu = rnd((N, K), 0.05, 71), rnd((N, K), 0.05, 72)
    x = rnd((B, K), 1.0, 73)
    g = rnd((K,), 0.1, 74, mean=1.0)
    y1 = torch.empty((B, N), dtype=torch.bfloat16, device=DEV)
    y2 = torch.empty_like(y1)
    W.gemv_norm(W.make_stage(Wt, x, y1, norm=O.NORM_RMS, gamma=g, epi=O.EPI_SWIGLU, W_up=Wu), B)
    W.gemm_norm(W.make_stage(Wt, x, y2, norm=O.NORM_RMS, gamma=g, epi=O.EPI_SWIGLU, W_up=Wu), B)
    torch.cuda.synchronize()
    ref = O.stage(bits(x), bits(Wt), norm=O.NORM_RMS, epi=O.EPI_SWIGLU, eps=EPS32, gamma=bits(g), W_up=bits(Wu))
    assert_close_bf16(bits(y1), ref, "persistent path")
    assert_close_bf16(bits(y2), ref, "batched path")


@pytest.mark.parametrize("B", [17, 40, 128])
def test_gemm_norm_argmax(B):
    """RMSNorm + LM head (V = 20000: a ragged last row tile) + argmax with
    logits and maxima; keys and tickets are left at zero for the next call."""
    say("gemm_norm argmax V=20000 B=%d" % B)
    V, K = 20000, 1536
    h = rnd((B, K), 1.0, 80 + B)
    g = rnd((K,), 0.1, 81, mean=1.0)
    Wl = rnd((V, K), 0.02, 82)
    idx = torch.empty((B,), dtype=torch.int32, device=DEV)
    mx = torch.empty((B,), dtype=torch.float32, device=DEV)
    lg = torch.empty((B, V), dtype=torch.float32, device=DEV)
    st = W.make_stage(Wl, h, idx, norm=O.NORM_RMS, gamma=g, epi=L.EPI_ARGMAX, logits=lg, maxval=mx)
    ws = W.workspace(W.gemm_norm_workspace_bytes(st, B))
    for rep in range(2):
        idx.fill_(-1)
        W.gemm_norm(st, B, ws=ws)
        torch.cuda.synchronize()
        ridx, rmx, rlog = O.lmhead_argmax(bits(h), bits(g), bits(Wl), eps=EPS32, want_logits=True)
        assert_close(lg.double().cpu().numpy(), rlog, "logits B=%d" % B)
        lgc = lg.cpu()
        for b in range(B):
            check_argmax(int(idx[b]), rlog[b], "argmax b=%d rep %d" % (b, rep))
            # the GPU's own maximum and its lowest index
            assert float(mx[b]) == float(lgc[b].max()), b
            assert int(idx[b]) == int(torch.nonzero(lgc[b] == lgc[b].max())[0]), b
    ntiles = (V + 63) // 64
    keys_off = ((ntiles + 1) * 4 + 255) // 256 * 256
    assert int(ws[: (ntiles + 1) * 4].view(torch.int32).abs().sum()) == 0, "tickets not left at zero"
    assert int(ws[keys_off: keys_off + B * 8].abs().sum()) == 0, "argmax keys not left at zero"


def test_gemm_norm_argmax_planted_and_ties():
    """A planted maximum row, and several identical maximal rows: the lowest index wins."""
    say("gemm_norm argmax planted/ties B=32")
    V, K, B = 4096, 512, 32
    Wl = rnd((V, K), 0.02, 90)
    h = rnd((B, K), 1.0, 91)
    g = torch.ones((K,), dtype=torch.bfloat16, device=DEV)
    xh = torch.from_numpy(np.stack([O.bf16_array_to_f64(O.norm_bf16(O.NORM_RMS, bits(h[b]), bits(g), eps=EPS32))
                                    for b in range(B)]).astype(np.float32)).to(DEV)
    # rows 777, 1500 and 3000 all equal 4 x-hat of batch row 5 (a clear maximum for it)
    plant = (4.0 * xh[5]).to(torch.bfloat16)
    for r in (3000, 777, 1500):
        Wl[r] = plant
    idx = torch.empty((B,), dtype=torch.int32, device=DEV)
    st = W.make_stage(Wl, h, idx, norm=O.NORM_RMS, gamma=g, epi=L.EPI_ARGMAX)
    W.gemm_norm(st, B)
    torch.cuda.synchronize()
    assert int(idx[5]) == 777


@pytest.mark.parametrize("B", [32, 128])
def test_small_decode_step_batched(B):
    """Two full-width blocks + an LM head of 20000 rows through wgn_layer_chain
    at batch 32 and 128 (stage by stage on this path), teacher-forced per stage;
    a second call on the same workspace gives the same bits."""
    from tests.test_gpu_chain import check_decoder, snapshot, same_bits
    say("layer_chain decode_step 2 layers V=20000 B=%d" % B)
    inp = gen.make_stage_tensors("decode_step_1536x28", device=DEV, batch=B, n_layers=2, vocab=20000)
    stages, bufs = steps.decoder_stages(inp, DEV)
    ws = W.workspace(W.workspace_bytes(stages, B))
    W.layer_chain(stages, B, ws=ws)
    torch.cuda.synchronize()
    check_decoder(inp, bufs, layers_full={0, 1})
    first = snapshot(bufs)
    W.layer_chain(stages, B, ws=ws)
    torch.cuda.synchronize()
    assert same_bits(first, snapshot(bufs)), "rerun not bit-identical"


def test_layer_chain_batched_after_a_persistent_chain():
    """A workspace that held a persistent chain (batch 16) serves the batched
    path next: its counters are cleared by the call."""
    say("layer_chain batch 16 then 24 on one workspace")
    inp16 = gen.make_stage_tensors("decode_step_1536x28", device=DEV, batch=16, n_layers=1, vocab=4096)
    st16, _ = steps.decoder_stages(inp16, DEV)
    inp24 = gen.make_stage_tensors("decode_step_1536x28", device=DEV, batch=24, n_layers=1, vocab=4096)
    st24, bufs24 = steps.decoder_stages(inp24, DEV)
    nbytes = max(W.workspace_bytes(st16, 16), W.workspace_bytes(st24, 24))
    ws = W.workspace(nbytes)
    W.layer_chain(st16, 16, ws=ws)
    torch.cuda.synchronize()
    W.layer_chain(st24, 24, ws=ws)
    torch.cuda.synchronize()
    from tests.test_gpu_chain import check_decoder
    check_decoder(inp24, bufs24, layers_full={0})


def test_gemm_norm_calls_share_a_workspace():
    """A call with few row tiles (its x-hat where a larger call keeps its
    tickets) and then one with many tiles on the same workspace: each call
    clears its own counters first."""
    say("gemm_norm: two calls on one workspace")
    B = 32
    x = rnd((B, 1536), 1.0, 60)
    g = rnd((1536,), 0.1, 61, mean=1.0)
    Wa = rnd((256, 1536), 0.05, 62)
    Wb, Wu = rnd((8960, 1536), 0.05, 63), rnd((8960, 1536), 0.05, 64)
    ya = torch.empty((B, 256), dtype=torch.bfloat16, device=DEV)
    yb = torch.empty((B, 8960), dtype=torch.bfloat16, device=DEV)
    sa = W.make_stage(Wa, x, ya, norm=O.NORM_RMS, gamma=g)
    sb = W.make_stage(Wb, x, yb, norm=O.NORM_RMS, gamma=g, epi=O.EPI_SWIGLU, W_up=Wu)
    ws = W.workspace(max(W.gemm_norm_workspace_bytes(sa, B), W.gemm_norm_workspace_bytes(sb, B)))
    ws.fill_(0xA5)  # any content
    W.gemm_norm(sa, B, ws=ws)
    W.gemm_norm(sb, B, ws=ws)
    torch.cuda.synchronize()
    ra = O.stage(bits(x), bits(Wa), norm=O.NORM_RMS, eps=EPS32, gamma=bits(g))
    rb = O.stage(bits(x), bits(Wb), norm=O.NORM_RMS, epi=O.EPI_SWIGLU, eps=EPS32, gamma=bits(g), W_up=bits(Wu))
    assert_close_bf16(bits(ya), ra, "first call")
    assert_close_bf16(bits(yb), rb, "second call")


@pytest.mark.parametrize("B", [1, 8])
def test_tiled_path_at_small_batch(B):
    """opts.path = 3 runs the batched path at any batch: the two-block decode
    step at batch 1 and 8, teacher-forced per stage (Q, K and V in one launch)."""
    from tests.test_gpu_chain import check_decoder
    say("layer_chain path 3 decode_step 2 layers V=20000 B=%d" % B)
    inp = gen.make_stage_tensors("decode_step_1536x28", device=DEV, batch=B, n_layers=2, vocab=20000)
    stages, bufs = steps.decoder_stages(inp, DEV)
    W.layer_chain(stages, B, path=W.PATH_TILED)
    torch.cuda.synchronize()
    check_decoder(inp, bufs, layers_full={0, 1})
