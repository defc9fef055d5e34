"""wgn_lmhead_argmax_static (the allocation-free LM head + argmax) against the
workspace form wgn_lmhead_argmax, bit for bit, on two calls in a row -- the
second smaller (fewer rows, fewer batch rows) -- so the fixed scratch's ticket
left by the first call must be back at zero for the second."""
import numpy as np
import pytest
import torch

from synth import gen
from tests.gpu_util import bits, say

pytestmark = pytest.mark.gpu


def _inputs(B, V, K, seed):
    h = gen.normal((B, K), 1.0, gen.seed_of(61, seed, B), device="cuda")
    g = gen.normal((K,), 0.1, gen.seed_of(62, seed, 0), mean=1.0, device="cuda")
    Wlm = gen.normal((V, K), 0.02, gen.seed_of(63, seed, V), device="cuda")
    return h, g, Wlm


def _both(B, V, K, seed):
    import weight_gemv_norm_amd as W
    h, g, Wlm = _inputs(B, V, K, seed)
    out = []
    for static in (False, True):
        idx = torch.full((B,), -1, dtype=torch.int32, device="cuda")
        mx = torch.full((B,), float("nan"), dtype=torch.float32, device="cuda")
        lg = torch.full((B, V), float("nan"), dtype=torch.float32, device="cuda")
        if static:
            W.lmhead_argmax_static(h, g, 1e-6, Wlm, idx, mx, lg)
        else:
            W.lmhead_argmax(h, g, 1e-6, Wlm, idx, mx, lg)
        torch.cuda.synchronize()
        out.append((idx.cpu().numpy(), mx.cpu().numpy(), lg.cpu().numpy()))
    return out


def test_static_lmhead_matches_workspace_form_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    for (B, V, K, seed) in ((4, 151936, 1536, 1), (2, 50000, 1536, 2)):
        say("lmhead_argmax_static batch %d V %d K %d" % (B, V, K))
        (i0, m0, l0), (i1, m1, l1) = _both(B, V, K, seed)
        assert np.array_equal(i0, i1), (i0, i1)
        assert np.array_equal(m0.view(np.uint32), m1.view(np.uint32))
        assert np.array_equal(l0.view(np.uint32), l1.view(np.uint32))
        assert (i0 >= 0).all() and (i0 < V).all()
        # the index is the lowest attaining the maximum of the returned logits
        for b in range(B):
            assert l1[b, i1[b]] == m1[b] == l1[b].max()
            assert not (l1[b, :i1[b]] == m1[b]).any()


def test_static_lmhead_refuses_bad_arguments():
    import weight_gemv_norm_amd as W
    from weight_gemv_norm_amd import _lib as L
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    h, g, Wlm = _inputs(1, 1000, 1536, 3)
    idx = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = L.lib().wgn_lmhead_argmax_static(h.data_ptr(), 1536, 17, 1536, g.data_ptr(), 1e-6, Wlm.data_ptr(), 1000,
                                          idx.data_ptr(), None, None, None)
    assert st == L.E_ARG  # batch above 16
