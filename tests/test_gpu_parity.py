"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by
element, teacher-forced per stage (each stage's oracle runs on the GPU's own
inputs to that stage), on seeded synthetic inputs."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import gen
from tests.gpu_util import (assert_close, assert_close_bf16, bits, check_argmax, f16_to_f64, say)

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
    L.lib()  # fails loudly if the library is missing
    assert W.device_cu_count() > 0
    yield


def rnd(shape, std, seed, mean=0.0):
    return gen.normal(shape, std, seed, mean=mean, device=DEV)


def oracle_stage_from_gpu(s_kind, W_, x, y, *, norm, eps=1e-6, gamma=None, beta=None, bias=None,
                          epi=O.EPI_NONE, W_up=None, residual=None):
    """Run the oracle on the GPU tensors' bits; return (gpu_bits, ref_bits)."""
    ref = O.stage(bits(x), bits(W_), norm=norm, epi=epi,
                  gamma=None if gamma is None else bits(gamma),
                  beta=None if beta is None else bits(beta), eps=float(np.float32(eps)),
                  W_up=None if W_up is None else bits(W_up),
                  bias=None if bias is None else bits(bias),
                  residual=None if residual is None else bits(residual))
    return bits(y), ref


# ------------------------------------------------------------------ one stage
def test_gemv_norm_rmsnorm_256():
    """RMSNorm(eps 1e-6, gain 1+N(0,0.1)) + 256x256 GEMV, batch 1, BF16 output."""
    say("gemv_norm rmsnorm_gemv_256")
    t = gen.make_stage_tensors("rmsnorm_gemv_256", device=DEV)
    y = torch.empty((1, 256), dtype=torch.bfloat16, device=DEV)
    st = W.make_stage(t["W"], t["x"], y, norm=W.api.NORM_RMS, eps=t["eps"], gamma=t["g"])
    W.gemv_norm(st, 1)
    torch.cuda.synchronize()
    g, r = oracle_stage_from_gpu(None, t["W"], t["x"], y, norm=O.NORM_RMS, eps=t["eps"], gamma=t["g"])
    assert_close_bf16(g, r, "rmsnorm_gemv_256")
    first = y.clone()
    for _ in range(3):
        W.gemv_norm(st, 1)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), y.view(torch.int16)), "rerun not bit-identical"


CASES = [
    # (N, K, B, norm, epi, bias, residual)
    (1, 8, 1, O.NORM_RMS, O.EPI_NONE, False, False),
    (37, 264, 2, O.NORM_LAYER, O.EPI_GELU_TANH, True, False),
    (1000, 520, 3, O.NORM_NONE, O.EPI_NONE, False, True),
    (300, 1536, 4, O.NORM_RMS, O.EPI_SWIGLU, False, True),
    (1536, 8960, 1, O.NORM_NONE, O.EPI_NONE, False, True),
    (513, 1024, 4, O.NORM_LAYER, O.EPI_NONE, True, True),
    (8960, 1536, 1, O.NORM_RMS, O.EPI_SWIGLU, False, False),
    # batch 1 LayerNorm (the control wave's own normalisation), ragged K
    (37, 264, 1, O.NORM_LAYER, O.EPI_GELU_TANH, True, False),
    (513, 1024, 1, O.NORM_LAYER, O.EPI_NONE, True, True),
    # matrix-core path (batch > 4): ragged tiles (N % 16), K tails, every epilogue
    (1, 8, 5, O.NORM_RMS, O.EPI_NONE, False, False),
    (37, 264, 8, O.NORM_LAYER, O.EPI_GELU_TANH, True, False),
    (1000, 520, 16, O.NORM_NONE, O.EPI_NONE, False, True),
    (300, 1536, 7, O.NORM_RMS, O.EPI_SWIGLU, False, True),
    (1536, 8960, 8, O.NORM_NONE, O.EPI_NONE, False, True),
    (513, 1024, 16, O.NORM_LAYER, O.EPI_NONE, True, True),
    (8960, 1536, 16, O.NORM_RMS, O.EPI_SWIGLU, False, False),
    (17, 4096, 12, O.NORM_RMS, O.EPI_NONE, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c[:5]) for c in CASES])
def test_gemv_norm_shapes(case):
    N, K, B, norm, epi, use_bias, use_res = case
    say("gemv_norm N=%d K=%d B=%d norm=%d epi=%d" % (N, K, B, norm, epi))
    seed = hash(case) & 0xFFFF
    Wt = rnd((N, K), 0.05, seed + 1)
    Wu = rnd((N, K), 0.05, seed + 2) if epi == O.EPI_SWIGLU else None
    # a strided activation buffer: rows padded to K + 16 elements
    xs = torch.empty((B, K + 16), dtype=torch.bfloat16, device=DEV)
    xs[:, :K] = rnd((B, K), 1.0, seed + 3, mean=0.3 if norm == O.NORM_LAYER else 0.0)
    x = xs[:, :K]
    gamma = rnd((K,), 0.1, seed + 4, mean=1.0) if norm != O.NORM_NONE else None
    beta = rnd((K,), 0.02, seed + 5) if norm == O.NORM_LAYER else None
    bias = rnd((N,), 0.02, seed + 6) if use_bias else None
    res = rnd((B, N), 1.0, seed + 7) if use_res else None
    y = torch.empty((B, N), dtype=torch.bfloat16, device=DEV)
    eps = 1e-5 if norm == O.NORM_LAYER else 1e-6
    st = W.make_stage(Wt, x, y, norm=norm, eps=eps, gamma=gamma, beta=beta, bias=bias, epi=epi, W_up=Wu,
                      residual=res)
    W.gemv_norm(st, B)
    torch.cuda.synchronize()
    g, r = oracle_stage_from_gpu(None, Wt, x.contiguous(), y, norm=norm, eps=eps, gamma=gamma, beta=beta,
                                 bias=bias, epi=epi, W_up=Wu, residual=res)
    assert_close_bf16(g, r, "gemv_norm %r" % (case,))


def test_gemv_norm_too_large_for_lds_needs_a_chain():
    """Batch 16 x K 8960 inputs do not fit in LDS: one launch refuses, a
    one-stage chain streams the stage in K windows."""
    say("gemv_norm 1536x8960 B=16 via K windows")
    N, K, B = 1536, 8960, 16
    Wt = rnd((N, K), 0.02, 901)
    x = rnd((B, K), 1.0, 902)
    res = rnd((B, N), 1.0, 903)
    y = torch.empty((B, N), dtype=torch.bfloat16, device=DEV)
    st = W.make_stage(Wt, x, y, residual=res)
    with pytest.raises(W.WgnError):
        W.gemv_norm(st, B)
    ch = W.Chain([st], B)
    assert ch.num_phases >= 2
    ch.run()
    ch.check()
    g, r = oracle_stage_from_gpu(None, Wt, x, y, norm=O.NORM_NONE, residual=res)
    assert_close_bf16(g, r, "down 1536x8960 B=16 K windows")


@pytest.mark.parametrize("B", [1, 3, 4])
def test_matrix_core_path_at_small_batch(B):
    """The matrix-core path is selectable at any batch; same tolerance."""
    say("chain path=matrix B=%d" % B)
    cases = [(300, 1536, O.NORM_RMS, O.EPI_SWIGLU), (37, 264, O.NORM_LAYER, O.EPI_GELU_TANH),
             (1536, 8960, O.NORM_NONE, O.EPI_NONE)]
    for N, K, norm, epi in cases:
        seed = N + K + B
        Wt = rnd((N, K), 0.05, seed + 1)
        Wu = rnd((N, K), 0.05, seed + 2) if epi == O.EPI_SWIGLU else None
        x = rnd((B, K), 1.0, seed + 3, mean=0.3 if norm == O.NORM_LAYER else 0.0)
        gamma = rnd((K,), 0.1, seed + 4, mean=1.0) if norm != O.NORM_NONE else None
        beta = rnd((K,), 0.02, seed + 5) if norm == O.NORM_LAYER else None
        bias = rnd((N,), 0.02, seed + 6) if epi == O.EPI_GELU_TANH else None
        res = rnd((B, N), 1.0, seed + 7) if epi == O.EPI_NONE else None
        y = torch.empty((B, N), dtype=torch.bfloat16, device=DEV)
        eps = 1e-5 if norm == O.NORM_LAYER else 1e-6
        st = W.make_stage(Wt, x, y, norm=norm, eps=eps, gamma=gamma, beta=beta, bias=bias, epi=epi, W_up=Wu,
                          residual=res)
        W.layer_chain([st], B, path=W.api.PATH_MATRIX)
        torch.cuda.synchronize()
        g, r = oracle_stage_from_gpu(None, Wt, x, y, norm=norm, eps=eps, gamma=gamma, beta=beta, bias=bias,
                                     epi=epi, W_up=Wu, residual=res)
        assert_close_bf16(g, r, "matrix path N=%d K=%d B=%d" % (N, K, B))


def test_gemv_norm_identity_and_zero_weights():
    """Identity weights return x-hat; zero weights return the residual bit for bit."""
    say("gemv_norm identity / zero weights")
    K = 1024
    I = torch.eye(K, dtype=torch.bfloat16, device=DEV)
    x = rnd((2, K), 1.0, 11)
    y = torch.empty((2, K), dtype=torch.bfloat16, device=DEV)
    W.gemv_norm(W.make_stage(I, x, y), 2)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), x.view(torch.int16))
    Z = torch.zeros((K, K), dtype=torch.bfloat16, device=DEV)
    res = rnd((2, K), 1.0, 12)
    W.gemv_norm(W.make_stage(Z, x, y, residual=res), 2)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), res.view(torch.int16))


# --------------------------------------------------------------------- LM head
def test_lmhead_argmax_full_vocab():
    """Final RMSNorm + LM head 151936 x 1536 + argmax at batch 1, 2 (vector
    path) and 8, 16 (matrix-core path), plus logits."""
    for B in (1, 2, 8, 16):
        say("lmhead_argmax V=151936 B=%d" % B)
        h = rnd((B, gen.H), 1.0, 100 + B)
        g = rnd((gen.H,), 0.1, 200, mean=1.0)
        Wl = rnd((gen.V, gen.H), 0.02, 300)
        idx = torch.full((B,), -1, dtype=torch.int32, device=DEV)
        mx = torch.empty((B,), dtype=torch.float32, device=DEV)
        lg = torch.empty((B, gen.V), dtype=torch.float32, device=DEV)
        W.lmhead_argmax(h, g, 1e-6, Wl, idx, mx, lg)
        torch.cuda.synchronize()
        ridx, rmx, rlog = O.lmhead_argmax(bits(h), bits(g), bits(Wl), eps=float(np.float32(1e-6)),
                                          want_logits=True)
        gl = lg.double().cpu().numpy()
        for b in range(B):
            assert_close(gl[b], rlog[b], "lm head logits b=%d" % b)
            check_argmax(int(idx[b]), rlog[b], "lm head b=%d" % b)
            assert float(mx[b]) == float(lg[b, int(idx[b])])


def test_lmhead_argmax_planted_and_ties():
    say("lmhead_argmax planted rows / ties")
    V, K = 50_000, 512
    h = rnd((1, K), 1.0, 7)
    Wl = rnd((V, K), 0.02, 8)
    idx = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    xh = torch.from_numpy(O.norm_bf16(O.NORM_NONE, bits(h[0]), None).view(np.int16)).to(DEV)
    planted = (xh.view(torch.bfloat16).float() * 4).to(torch.bfloat16)
    Wl[40_001] = planted
    W.lmhead_argmax(h, None, 1e-6, Wl, idx)
    torch.cuda.synchronize()
    assert int(idx[0]) == 40_001
    Wl[123] = planted  # duplicated maximum -> lowest index
    W.lmhead_argmax(h, None, 1e-6, Wl, idx)
    torch.cuda.synchronize()
    assert int(idx[0]) == 123
    Wl[:] = Wl[5]  # all rows equal -> index 0
    W.lmhead_argmax(h, None, 1e-6, Wl, idx)
    torch.cuda.synchronize()
    assert int(idx[0]) == 0


# --------------------------------------------------------------- norm rows
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_rmsnorm_rows_prefill_shape(dtype):
    say("rmsnorm_rows 960x1536 %s" % dtype)
    t = gen.make_stage_tensors("rmsnorm_rows_960x1536_f16", device=DEV)
    x = t["x"].to(dtype)
    g = t["g"].to(dtype)
    y = torch.empty_like(x)
    W.rmsnorm_rows(x, g, t["eps"], y)
    torch.cuda.synchronize()
    if dtype == torch.float16:
        ref = O.rmsnorm_rows_f16(bits(x), bits(g), float(np.float32(t["eps"])))
        assert_close(f16_to_f64(bits(y)), f16_to_f64(ref), "rmsnorm_rows f16")
    else:
        xb, gb = bits(x), bits(g)
        ref = np.stack([O.norm_bf16(O.NORM_RMS, xb[r], gb, None, float(np.float32(t["eps"])))
                        for r in range(x.shape[0])])
        assert_close_bf16(bits(y), ref, "rmsnorm_rows bf16")


def test_rmsnorm_rows_ragged_k():
    say("rmsnorm_rows ragged K=4104 / K=8")
    for R, K in ((5, 4104), (3, 8), (70, 1000)):
        x = gen.normal((R, K), 1.0, 77 + K, dtype=torch.float16, device=DEV)
        g = gen.normal((K,), 0.1, 78, mean=1.0, dtype=torch.float16, device=DEV)
        y = torch.empty_like(x)
        W.rmsnorm_rows(x, g, 1e-6, y)
        torch.cuda.synchronize()
        ref = O.rmsnorm_rows_f16(bits(x), bits(g), float(np.float32(1e-6)))
        assert_close(f16_to_f64(bits(y)), f16_to_f64(ref), "rmsnorm_rows K=%d" % K)
