"""GPU parity of wgn_gemv_int4 against the oracle ("One Token, Kernel by
Kernel", section "4-bit weights"), element by element within
|d| <= 1e-2 |ref| + 1e-3 rms(ref), over the decode step's matrix shapes
(several 1 KB slices per row, ragged row counts) and batches 1-8."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import gen
from tests.gpu_util import assert_close_bf16, bits, say

pytestmark = pytest.mark.gpu


def _run(N, K, B, seed):
    import weight_gemv_norm_amd as W
    t = gen.make_int4_weights(N, K, seed=seed, device="cuda")
    x = gen.normal((B, K), 1.0, gen.seed_of(44, seed, B), device="cuda")
    y = torch.empty((B, N), dtype=torch.bfloat16, device="cuda")
    W.gemv_int4(x, t["W4"], t["scales"], t["zeros"], y)
    torch.cuda.synchronize()
    ref = O.matvec_int4(t["W4"].cpu().numpy(), bits(t["scales"]), bits(t["zeros"]), bits(x))
    return bits(y), ref


@pytest.mark.parametrize("N,K,B", [(1, 128, 1), (17, 256, 1), (1536, 1536, 1), (256, 1536, 4), (8960, 1536, 1),
                                   (8960, 1536, 8), (1536, 8960, 1), (1536, 8960, 3), (1536, 8960, 4),
                                   (1536, 8960, 8), (4099, 1536, 2),
                                   (300, 2176, 5)])
def test_gemv_int4_matches_oracle(N, K, B):
    say("gemv_int4 N %d K %d batch %d" % (N, K, B))
    y, ref = _run(N, K, B, seed=N + K + B)
    assert_close_bf16(y, ref, "int4 %dx%d b%d" % (N, K, B))


@pytest.mark.parametrize("k", [0, 1, 30, 31, 32, 1023, 1024, 1535])
def test_gemv_int4_nibble_order(k):
    """One code of 1 at position k with unit scale and zero offset: the
    output is exactly x[k]."""
    import weight_gemv_norm_amd as W
    say("gemv_int4 nibble order k %d" % k)
    N, K = 16, 1536
    q = np.zeros((N, K), np.uint8)
    q[3, k] = 1
    W4 = torch.from_numpy((q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)).cuda()
    sc = torch.ones((N, K // 128), dtype=torch.bfloat16, device="cuda")
    zr = torch.zeros((N, K // 128), dtype=torch.bfloat16, device="cuda")
    x = gen.normal((1, K), 1.0, 99, device="cuda")
    y = torch.empty((1, N), dtype=torch.bfloat16, device="cuda")
    W.gemv_int4(x, W4, sc, zr, y)
    torch.cuda.synchronize()
    yb = bits(y)
    assert yb[0, 3] == bits(x)[0, k]
    assert not np.delete(yb[0], 3).any()
