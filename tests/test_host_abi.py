"""Host-side tests of libwgn.so (no GPU): the library loads, exports every
symbol include/wgn.h declares, validates arguments before touching the device,
and plans a work partition that covers every weight unit exactly once."""
import os
import re

import pytest

from weight_gemv_norm_amd import _lib as L
from weight_gemv_norm_amd.api import partition_selftest, first_wave_of_unit, plan_phases
from synth import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "wgn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(wgn_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    names = header_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in range(0, -8, -1):
        assert L.status_string(s) and L.status_string(s) != "unknown status"
    assert L.status_string(-99) == "unknown status"


def test_first_wave_formula_brute_force():
    for U in range(1, 80):
        for W in (1, 2, 3, 7, 8):
            owner = []
            for w in range(W):
                if U >= W:
                    lo, hi = (w * U) // W, ((w + 1) * U) // W
                    assert hi > lo  # no empty wave when there is enough work
                else:
                    lo, hi = min(w, U), min(w + 1, U)
                owner += [w] * (hi - lo)
            assert len(owner) == U
            for u in range(U):
                assert first_wave_of_unit(u, U, W) == owner[u]
    assert first_wave_of_unit(5, 5, 7) == -1


# ------------------------------------------------------------- fake stages
class Arena:
    """Hands out fake, 256-byte aligned, non-overlapping device addresses."""

    def __init__(self):
        self.next = 1 << 40

    def take(self, nbytes):
        p = self.next
        self.next += (nbytes + 4095) // 4096 * 4096 + 4096
        return p


def fake_stage(ar, N, K, B, norm=L.NORM_NONE, epi=L.EPI_NONE, x=None, residual=None, gamma=True,
               bias=False, beta=False):
    s = L.Stage()
    s.N, s.K = N, K
    s.W = ar.take(N * K * 2)
    s.W_up = ar.take(N * K * 2) if epi == L.EPI_SWIGLU else None
    s.bias = ar.take(N * 2) if bias else None
    s.norm = norm
    s.eps = 1e-6
    s.gamma = ar.take(K * 2) if (gamma and norm != L.NORM_NONE) else None
    s.beta = ar.take(K * 2) if (beta and norm == L.NORM_LAYER) else None
    s.epi = epi
    s.x = x if x is not None else ar.take(B * K * 2)
    s.x_stride = K
    s.residual = residual
    s.res_stride = N if residual else 0
    if epi == L.EPI_ARGMAX:
        s.y = ar.take(B * 4)
        s.y_stride = 0
    else:
        s.y = ar.take(B * N * 2)
        s.y_stride = N
    return s


def fake_decoder(ar, B, n_layers, H=1536, I=8960, V=None):
    stages = []
    h = ar.take(B * H * 2)
    for _ in range(n_layers):
        q = fake_stage(ar, H, H, B, L.NORM_RMS, x=h)
        k = fake_stage(ar, H // 6, H, B, L.NORM_RMS, x=h)
        v = fake_stage(ar, H // 6, H, B, L.NORM_RMS, x=h)
        k.gamma = v.gamma = q.gamma
        o = fake_stage(ar, H, H, B, L.NORM_NONE, residual=h)
        gu = fake_stage(ar, I, H, B, L.NORM_RMS, L.EPI_SWIGLU, x=o.y)
        d = fake_stage(ar, H, I, B, L.NORM_NONE, x=gu.y, residual=o.y)
        stages += [q, k, v, o, gu, d]
        h = d.y
    if V:
        stages.append(fake_stage(ar, V, H, B, L.NORM_RMS, L.EPI_ARGMAX, x=h))
    return stages


@pytest.mark.parametrize("B,path", [(1, 0), (4, 0), (1, 2), (4, 2), (5, 0), (8, 0), (16, 0)])
@pytest.mark.parametrize("grid", [256, 61, 32])
def test_partition_decoder_block(B, path, grid):
    ar = Arena()
    stages = fake_decoder(ar, B, 1)
    assert partition_selftest(stages, B, grid, path) == 0


@pytest.mark.parametrize("B", [1, 8, 16])
def test_partition_full_decode_step_shapes(B):
    ar = Arena()
    stages = fake_decoder(ar, B, 2, V=151936)
    assert partition_selftest(stages, B, 256) == 0


@pytest.mark.parametrize("path", [0, 2])
@pytest.mark.parametrize("K", [8, 24, 256, 520, 1536, 8960])
@pytest.mark.parametrize("N", [1, 5, 17, 97, 1000])
def test_partition_ragged_shapes(N, K, path):
    ar = Arena()
    st = [fake_stage(ar, N, K, 2, L.NORM_RMS),
          fake_stage(ar, max(1, N // 3), K, 2, L.NORM_NONE, L.EPI_SWIGLU)]
    for grid in (1, 3, 64, 256):
        r = partition_selftest(st, 2, grid, path)
        # a grid too small for the per-workgroup partial sums is refused, never mis-planned
        assert r == 0 or (r == L.E_UNSUPPORTED and grid <= 3), (grid, r)


def test_vector_path_refuses_large_batch():
    ar = Arena()
    st = [fake_stage(ar, 64, 64, 8, L.NORM_RMS)]
    assert partition_selftest(st, 8, 16, 1) == L.E_UNSUPPORTED
    assert partition_selftest(st, 8, 16, 0) == 0


@pytest.mark.parametrize("B", [9, 12, 16])
@pytest.mark.parametrize("grid", [256, 40])
def test_partition_k_windows(B, grid):
    """The 8960-long down-projection input does not fit in LDS at batch > 8:
    that phase is streamed in K windows with the row sums carried between
    them; the residual enters in the last window only."""
    ar = Arena()
    h = ar.take(B * 1536 * 2)
    s = ar.take(B * 8960 * 2)
    d = fake_stage(ar, 1536, 8960, B, L.NORM_NONE, x=s, residual=h)
    assert partition_selftest([d], B, grid) == 0
    n, where = plan_phases([d], B, grid)
    assert n >= 2 and where == [n - 1]
    if grid == 256:
        assert n == 2
    gu = fake_stage(ar, 8960, 1536, B, L.NORM_RMS, L.EPI_SWIGLU, x=h)
    gu.y = s
    assert partition_selftest([gu, d], B, grid) == 0
    assert plan_phases([gu, d], B, grid) == (n + 1, [0, n])
    # at batch 8 on the full grid the whole input fits: no windows
    d8 = fake_stage(ar, 1536, 8960, 8, L.NORM_NONE, x=s, residual=h)
    if grid == 256:
        assert plan_phases([d8], 8, grid) == (1, [0])


def test_hoisting_of_the_output_projection():
    """O's product depends on nothing and its residual is the previous block's
    output: it moves into the phase before that block's down projection, and
    its residual add runs in the down projection's epilogue."""
    ar = Arena()
    st = fake_decoder(ar, 1, 3, V=1000)
    assert plan_phases(st, 1, 64, fuse=False) == (10, [0, 0, 0, 0, 1, 2, 3, 3, 3, 3, 4, 5, 6, 6, 6, 6, 7, 8, 9])
    n, where = plan_phases(st, 1, 64)
    assert n == 8
    assert where == [0, 0, 0, 0, 1, 2,   # block 0: O's residual is the chain input, nothing to hoist
                     3, 3, 3, 2, 3, 4,   # block 1: O written in block 0's down phase
                     5, 5, 5, 4, 5, 6,   # block 2
                     7]
    for B, path in ((1, 0), (4, 0), (8, 0), (16, 0), (1, 2)):
        stb = fake_decoder(Arena(), B, 3, V=1000)
        assert partition_selftest(stb, B, 64, path) == 0
        assert partition_selftest(stb, B, 256, path) == 0


def test_hoisting_respects_hazards():
    ar = Arena()
    # the residual's producer is in the first phase: no earlier phase for the product
    h = ar.take(1536 * 2)
    a = fake_stage(ar, 1536, 1536, 1, x=h)
    o = fake_stage(ar, 1536, 1536, 1, residual=a.y)
    assert plan_phases([a, o], 1, 64) == (2, [0, 1])
    # an input that a stage of the chain writes is not hoisted
    ar = Arena()
    st = fake_decoder(ar, 1, 2)
    st[9].x = st[4].y  # layer-1 O reads the layer-0 SwiGLU output
    n, where = plan_phases(st, 1, 64)
    assert where[9] > where[5]  # O of layer 1 stays after layer 0's down projection
    assert partition_selftest(st, 1, 64) == 0
    # a stage between the residual's producer and O that reads O's output blocks the rewrite
    ar = Arena()
    st = fake_decoder(ar, 1, 2)
    spy = fake_stage(ar, 64, 1536, 1, x=st[9].y)  # reads h1 of layer 1 before O writes it
    chain = st[:6] + [spy] + st[6:]
    n2, where2 = plan_phases(chain, 1, 64)
    assert where2[10] > where2[5]
    assert partition_selftest(chain, 1, 64) == 0


def test_phase_split_at_stage_capacity():
    """Twelve independent stages on one input exceed a phase's run-list
    capacity (8 stages): the planner splits them over two phases."""
    ar = Arena()
    x = ar.take(1536 * 2)
    st = [fake_stage(ar, 64 + i, 1536, 1, L.NORM_RMS, x=x) for i in range(12)]
    for s in st[1:]:
        s.gamma = st[0].gamma  # one normalised source for all
    n, where = plan_phases(st, 1, 64)
    assert n == 2 and where == [0] * 8 + [1] * 4
    assert partition_selftest(st, 1, 64) == 0
    # with a gain each, they are four distinct normalised inputs per phase at most
    st2 = [fake_stage(ar, 64 + i, 1536, 1, L.NORM_RMS, x=x) for i in range(9)]
    assert plan_phases(st2, 1, 64) == (3, [0] * 4 + [1] * 4 + [2])


def test_normalised_input_too_large_is_refused():
    """A norm needs the whole input in LDS for its statistics, so a normalised
    input that does not fit cannot be windowed."""
    ar = Arena()
    st = fake_stage(ar, 64, 8960, 16, L.NORM_RMS)
    assert partition_selftest([st], 16, 64) == L.E_UNSUPPORTED


def test_partition_ln_chain():
    ar = Arena()
    x = ar.take(16 * 768 * 2)
    st = []
    for _ in range(5):
        s = fake_stage(ar, 768, 768, 4, L.NORM_LAYER, L.EPI_GELU_TANH, x=x, bias=True, beta=True)
        st.append(s)
        x = s.y
    assert partition_selftest(st, 4, 256) == 0


# -------------------------------------------------------- argument checks
def call_gemv(s, batch=1):
    import ctypes
    return L.lib().wgn_gemv_norm(ctypes.byref(s), batch, None, 0, None)


def test_invalid_arguments_rejected_before_device():
    ar = Arena()
    good = fake_stage(ar, 64, 64, 1, L.NORM_RMS)
    cases = []
    s = fake_stage(ar, 64, 60, 1, L.NORM_RMS); cases.append((s, 1, L.E_ARG))          # K % 8
    s = fake_stage(ar, 0, 64, 1); cases.append((s, 1, L.E_ARG))                        # N = 0
    s = fake_stage(ar, 64, 64, 1); s.W = None; cases.append((s, 1, L.E_ARG))           # null W
    s = fake_stage(ar, 64, 64, 1); s.W += 2; cases.append((s, 1, L.E_ALIGN))           # misaligned W
    s = fake_stage(ar, 64, 64, 1); s.x += 8; cases.append((s, 1, L.E_ALIGN))           # misaligned x
    s = fake_stage(ar, 64, 64, 2); s.x_stride = 68; cases.append((s, 2, L.E_ALIGN))    # stride % 8
    s = fake_stage(ar, 64, 64, 1); s.epi = 7; cases.append((s, 1, L.E_ARG))            # bad enum
    s = fake_stage(ar, 64, 64, 1, L.NORM_RMS, L.EPI_SWIGLU); s.W_up = None
    cases.append((s, 1, L.E_ARG))                                                      # SwiGLU w/o up
    s = fake_stage(ar, 64, 64, 1, L.NORM_NONE); s.gamma = ar.take(128)
    cases.append((s, 1, L.E_ARG))                                                      # gain w/o norm
    cases.append((good, 0, L.E_ARG))                                                   # batch 0
    cases.append((good, 17, L.E_ARG))                                                  # batch > 16
    s = fake_stage(ar, 64, 64, 1, L.NORM_RMS); s.eps = float("nan"); cases.append((s, 1, L.E_ARG))
    for st, b, want in cases:
        assert call_gemv(st, b) == want, (want,)


def test_chain_rejects_weights_written_by_a_stage():
    import ctypes
    ar = Arena()
    a = fake_stage(ar, 64, 64, 1)
    b = fake_stage(ar, 64, 64, 1, x=a.y)
    b.W = a.y  # a weight that an earlier stage writes
    arr = L.stage_array([a, b])
    assert L.lib().wgn_chain_workspace_bytes(arr, 2, 1, None) == 0
    assert partition_selftest([a, b], 1, 4) == L.E_ARG


def test_chain_phase_grouping_counts():
    """Q/K/V/O form one phase, gate/up one, down one: 3 phases per layer, +1 for the LM head."""
    import ctypes
    ar = Arena()
    st = fake_decoder(ar, 1, 3, V=1000)
    assert partition_selftest(st, 1, 16) == 0
    arr = L.stage_array(st)
    assert L.lib().wgn_chain_workspace_bytes(arr, len(st), 1, None) > 0


def test_chain_opts_ring_checked_before_device():
    """opts.ring takes 0 (auto) to 3; anything else is refused before the
    device is touched, as are non-zero reserved words."""
    import ctypes
    ar = Arena()
    st = fake_decoder(ar, 1, 1, V=1000)
    arr = L.stage_array(st)
    ws = ar.take(1 << 20)
    for ring, res in ((-1, 0), (4, 0), (0, 1), (2, 1)):
        o = L.ChainOpts()
        o.ring = ring
        o.reserved[1] = res
        h = ctypes.c_void_p()
        got = L.lib().wgn_chain_create(arr, len(st), 1, ctypes.byref(o), ws, 1 << 20, None, ctypes.byref(h))
        assert got == L.E_ARG, (ring, res, got)


def test_rmsnorm_rows_argument_checks():
    ar = Arena()
    x, g, y = ar.take(4096), ar.take(4096), ar.take(4096)
    f = L.lib().wgn_rmsnorm_rows
    assert f(x, 64, g, 1e-6, y, 64, 4, 60, L.FP16, None) == L.E_ARG
    assert f(x, 64, g, 1e-6, y, 64, 4, 64, 7, None) == L.E_ARG
    assert f(x + 2, 64, g, 1e-6, y, 64, 4, 64, L.FP16, None) == L.E_ALIGN
    assert f(x, 64, g, 1e-6, x + 64, 64, 4, 64, L.FP16, None) == L.E_ARG   # y overlaps x
    assert f(x, 64, g, 1e-6, y, 64, 0, 64, L.FP16, None) == L.OK           # empty: no-op


def test_workspace_size_scales_with_argmax():
    import ctypes
    ar = Arena()
    s = fake_stage(ar, 1000, 64, 2, L.NORM_RMS, L.EPI_ARGMAX)
    assert L.lib().wgn_gemv_norm_workspace_bytes(ctypes.byref(s), 2) > 0
    s2 = fake_stage(ar, 1000, 64, 2, L.NORM_RMS)
    assert L.lib().wgn_gemv_norm_workspace_bytes(ctypes.byref(s2), 2) == 0


def test_decode_step_weight_bytes_match_library_shapes():
    ar = Arena()
    st = fake_decoder(ar, 1, gen.N_LAYERS, V=gen.V)
    total = sum(s.N * s.K * 2 * (2 if s.epi == L.EPI_SWIGLU else 1) for s in st)
    assert total == gen.decode_step_weight_bytes() == 3_087_138_816


# ------------------------------------------------------------ decode attention
def _att_call(**kw):
    a = dict(q=0x10000, k_new=0x20000, v_new=0x30000, k_cache=0x1000000, v_cache=0x9000000, pos=0x40000,
             batch=1, q_heads=12, kv_heads=2, slots=300, head_dim=128, scale=0.088, out=0x50000,
             ws=0x100000000, ws_bytes=1 << 30)
    a.update(kw)
    return L.lib().wgn_decode_attention(a["q"], a["k_new"], a["v_new"], a["k_cache"], a["v_cache"], a["pos"],
                                        a["batch"], a["q_heads"], a["kv_heads"], a["slots"], a["head_dim"],
                                        a["scale"], a["out"], a["ws"], a["ws_bytes"], None)


def test_decode_attention_checks_arguments_before_the_device():
    assert _att_call(q=None) == L.E_ARG
    assert _att_call(pos=None) == L.E_ARG
    assert _att_call(q_heads=12, kv_heads=5) == L.E_ARG
    assert _att_call(slots=0) == L.E_ARG
    assert _att_call(batch=0) == L.E_ARG
    assert _att_call(scale=float("nan")) == L.E_ARG
    assert _att_call(head_dim=64) == L.E_UNSUPPORTED
    assert _att_call(q_heads=18, kv_heads=2) == L.E_UNSUPPORTED
    assert _att_call(slots=(1 << 24) + 1) == L.E_UNSUPPORTED
    assert _att_call(q=0x10008) == L.E_ALIGN
    assert _att_call(pos=0x40002) == L.E_ALIGN
    assert _att_call(out=0x1000000) == L.E_ARG                      # output inside the key cache
    assert _att_call(v_cache=0x1000000 + 4096) == L.E_ARG           # the caches overlap
    assert _att_call(ws=None) == L.E_WORKSPACE
    assert _att_call(ws=0x100000010) == L.E_WORKSPACE
    assert _att_call(ws_bytes=1000) == L.E_WORKSPACE


def _tree(slots, chunk=128, fan=8):
    counts = [-(-slots // chunk)]
    while counts[-1] > 1:
        counts.append(-(-counts[-1] // fan))
    return counts


@pytest.mark.parametrize("batch,hq,hkv,slots", [(1, 12, 2, 128), (1, 12, 2, 129), (1, 12, 2, 4096),
                                                (1, 12, 2, 32768), (4, 12, 2, 32768), (2, 8, 1, 40000),
                                                (3, 4, 4, 1 << 20)])
def test_decode_attention_workspace_layout(batch, hq, hkv, slots):
    """Partials for every level below the top (fan-in 8 over chunks of 128
    slots), then one arrival counter per merged item; each area 256-byte
    aligned."""
    counts = _tree(slots)
    G = hq // hkv
    entry = ((G * 130 + 3) // 4 * 4) * 4
    al = lambda v: (v + 255) // 256 * 256  # noqa: E731
    want = sum(al(batch * hkv * c * entry) for c in counts[:-1]) + sum(al(batch * hkv * c * 4) for c in counts[1:])
    got = L.lib().wgn_decode_attention_workspace_bytes(batch, hq, hkv, slots, 128)
    assert got == max(want, 256)


# ------------------------------------------------------------ 4-bit weights
def _i4_call(**kw):
    a = dict(x=0x10000, x_stride=1536, batch=1, K=1536, W4=0x1000000, scales=0x2000000, zeros=0x3000000,
             N=1536, y=0x4000000, y_stride=1536)
    a.update(kw)
    return L.lib().wgn_gemv_int4(a["x"], a["x_stride"], a["batch"], a["K"], a["W4"], a["scales"], a["zeros"],
                                 a["N"], a["y"], a["y_stride"], None)


def test_gemv_int4_checks_arguments_before_the_device():
    assert _i4_call(x=None) == L.E_ARG
    assert _i4_call(zeros=None) == L.E_ARG
    assert _i4_call(K=1500, x_stride=1500) == L.E_ARG          # not a multiple of 128
    assert _i4_call(batch=0) == L.E_ARG
    assert _i4_call(batch=9) == L.E_ARG
    assert _i4_call(N=0) == L.E_ARG
    assert _i4_call(batch=2, x_stride=1000) == L.E_ARG         # rows overlap
    assert _i4_call(x=0x10008) == L.E_ALIGN
    assert _i4_call(W4=0x1000004) == L.E_ALIGN
    assert _i4_call(batch=2, x_stride=1540, y_stride=1536) == L.E_ALIGN
    assert _i4_call(scales=0x2000001) == L.E_ALIGN
    assert _i4_call(batch=8, K=9728, x_stride=9728) == L.E_UNSUPPORTED   # x does not fit in 160 KB of LDS
    assert _i4_call(y=0x1000000) == L.E_ARG                    # output over the codes


def test_python_wrappers_check_tensor_shapes_before_the_library():
    """The C ABI cannot see tensor sizes: the wrappers refuse mismatched
    shapes and dtypes (CPU tensors here; the checks come before any call)."""
    import torch
    import weight_gemv_norm_amd as W
    bf = torch.bfloat16
    N, K = 64, 256
    x = torch.zeros(1, K, dtype=bf)
    W4 = torch.zeros(N, K // 2, dtype=torch.uint8)
    sc = torch.zeros(N, K // 128, dtype=bf)
    y = torch.zeros(1, N, dtype=bf)
    bad = [dict(scales=torch.zeros(N, K // 64, dtype=bf)),            # wrong group count
           dict(zeros=torch.zeros(N + 1, K // 128, dtype=bf)),        # wrong rows
           dict(scales=torch.zeros(N, K // 128, dtype=torch.float32)),
           dict(x=torch.zeros(1, K, dtype=torch.float16)),
           dict(W4=torch.zeros(N, K // 4, dtype=torch.uint8)),         # codes for another K
           dict(y=torch.zeros(1, N - 1, dtype=bf))]
    for b in bad:
        a = dict(x=x, W4=W4, scales=sc, zeros=sc.clone(), y=y)
        a.update(b)
        with pytest.raises(ValueError):
            W.gemv_int4(a["x"], a["W4"], a["scales"], a["zeros"], a["y"])
    with pytest.raises(ValueError):  # right shapes, but not on the GPU
        W.gemv_int4(x, W4, sc, sc.clone(), y)

    B, Hq, Hkv, S, D = 1, 12, 2, 256, 128
    q = torch.zeros(B, Hq, D, dtype=bf)
    kn = torch.zeros(B, Hkv, D, dtype=bf)
    kc = torch.zeros(B, Hkv, S, D, dtype=bf)
    pos = torch.zeros(B, dtype=torch.int32)
    bad = [dict(k_new=torch.zeros(B, Hkv + 1, D, dtype=bf)),
           dict(v_new=torch.zeros(B, Hkv, D, dtype=torch.float32)),
           dict(v_cache=torch.zeros(B, Hkv, S - 1, D, dtype=bf)),
           dict(pos=torch.zeros(B + 1, dtype=torch.int32)),
           dict(pos=torch.zeros(B, dtype=torch.int64)),
           dict(out=torch.zeros(B, Hq, D + 8, dtype=bf))]
    for b in bad:
        a = dict(q=q, k_new=kn, v_new=kn.clone(), k_cache=kc, v_cache=kc.clone(), pos=pos, out=q.clone())
        a.update(b)
        with pytest.raises(ValueError):
            W.decode_attention(a["q"], a["k_new"], a["v_new"], a["k_cache"], a["v_cache"], a["pos"], a["out"])


def test_stream_read_and_wait_bound_check_arguments():
    f = L.lib().wgn_stream_read
    assert f(None, 1024, 256, 256, 8, 0x1000, None) == L.E_ARG
    assert f(0x10000, 1000, 256, 256, 8, 0x1000, None) == L.E_ARG       # not a multiple of 16
    assert f(0x10000, 1024, 0, 256, 8, 0x1000, None) == L.E_ARG
    assert f(0x10000, 1024, 256, 100, 8, 0x1000, None) == L.E_ARG       # not whole waves
    assert f(0x10000, 1024, 256, 256, 3, 0x1000, None) == L.E_ARG       # depth not a power of two
    assert f(0x10008, 1024, 256, 256, 8, 0x1000, None) == L.E_ALIGN
    assert f(0x10000, 1024, 256, 256, 8, None, None) == L.E_ARG
    assert L.lib().wgn_chain_set_wait_us(None, 0) == L.E_ARG


def test_workspace_bytes_serves_every_call():
    """wgn_workspace_bytes covers the chain in both modes, each stage alone and
    the LM head; 0 when the stages cannot be planned."""
    import ctypes
    lib = L.lib()
    for B in (1, 4, 16):
        stages = fake_decoder(Arena(), B, 2, V=4096)
        arr = L.stage_array(stages)
        total = lib.wgn_workspace_bytes(arr, len(stages), B, 151936)
        assert total > 0
        for mode in (0, 1):
            o = L.ChainOpts()
            o.mode = mode
            assert total >= lib.wgn_chain_workspace_bytes(arr, len(stages), B, ctypes.byref(o))
        for st in stages:
            assert total >= lib.wgn_gemv_norm_workspace_bytes(ctypes.byref(st), B)
        assert total >= lib.wgn_lmhead_argmax_workspace_bytes(B)
    # batch 17-128: the batched matrix-core path, each stage through wgn_gemm_norm
    for B in (17, 64, 128):
        stages = fake_decoder(Arena(), B, 2, V=4096)
        arr = L.stage_array(stages)
        total = lib.wgn_workspace_bytes(arr, len(stages), B, 151936)
        assert total > 0
        for st in stages:
            need = lib.wgn_gemm_norm_workspace_bytes(ctypes.byref(st), B)
            assert 0 < need <= total
    assert lib.wgn_workspace_bytes(arr, len(stages), 129, 0) == 0   # batch out of range


def test_layer_chain_and_plan_tune_check_arguments_before_the_device():
    import ctypes
    stages = fake_decoder(Arena(), 1, 1, V=4096)
    arr = L.stage_array(stages)
    lib = L.lib()
    plan = L.Plan()
    plan.prefetch, plan.distance, plan.blocks, plan.frac_pct = 1, 1, 16, 50
    o = L.ChainOpts()  # mode 0: a persistent chain takes no prefetch plan
    assert lib.wgn_layer_chain(arr, len(stages), 1, ctypes.byref(o), ctypes.byref(plan), 0x100000, 1 << 30,
                               None, 0x1234) == L.E_UNSUPPORTED
    assert lib.wgn_plan_tune(arr, len(stages), 1, None, 0x100000, 1 << 30, None, 0x1234) == L.E_ARG


def call_gemm(st, b, ws=0x100000, ws_bytes=1 << 34):
    import ctypes
    return L.lib().wgn_gemm_norm(ctypes.byref(st), b, ws, ws_bytes, None)


def test_gemm_norm_workspace_layout():
    """Workspace of the batched path: tickets (one per 64-row tile + one),
    argmax keys, x-hat of a norm prologue, and the contributor slots of the
    tiles shared between workgroups (workgroups + tiles slots of 4 waves x
    accumulator sets x 16-row batch groups x 1 KB).  The launch's 256
    workgroups (one per compute unit; 256 when no device is visible) are
    spread evenly over the stage's 64-element windows, with at least 4
    windows each; a stage with 4 or more tiles per workgroup gives every tile
    its own workgroup."""
    import ctypes
    lib = L.lib()
    ar = Arena()
    al = lambda v: (v + 255) // 256 * 256  # noqa: E731
    # down projection at batch 128: 24 tiles x 140 windows over 256 workgroups
    d = fake_stage(ar, 1536, 8960, 128, L.NORM_NONE, residual=ar.take(128 * 1536 * 2))
    assert lib.wgn_gemm_norm_workspace_bytes(ctypes.byref(d), 128) == al(25 * 4) + (256 + 24) * 4 * 8 * 1024
    # gate/up at batch 32: 140 tiles x 24 windows; two accumulator sets; x-hat 32 x 1536
    gu = fake_stage(ar, 8960, 1536, 32, L.NORM_RMS, L.EPI_SWIGLU)
    assert lib.wgn_gemm_norm_workspace_bytes(ctypes.byref(gu), 32) == \
        al(141 * 4) + al(32 * 1536 * 2) + (256 + 140) * 4 * 2 * 2 * 1024
    # LM head at batch 17: 2374 tiles, one workgroup each (no slots), keys,
    # x-hat (gamma null: unit gain)
    lm = fake_stage(ar, 151936, 1536, 17, L.NORM_RMS, L.EPI_ARGMAX, gamma=False)
    assert lib.wgn_gemm_norm_workspace_bytes(ctypes.byref(lm), 17) == al(2375 * 4) + al(17 * 8) + al(17 * 1536 * 2)
    # LayerNorm prologue at batch 64: 12 tiles x 12 windows, 36 workgroups of 4 windows
    ln = fake_stage(ar, 768, 768, 64, L.NORM_LAYER, beta=True)
    assert lib.wgn_gemm_norm_workspace_bytes(ctypes.byref(ln), 64) == \
        al(13 * 4) + al(64 * 768 * 2) + (36 + 12) * 4 * 4 * 1024
    # one window per tile (K = 64): no tile is shared, no slots
    one = fake_stage(ar, 640, 64, 32, L.NORM_NONE)
    assert lib.wgn_gemm_norm_workspace_bytes(ctypes.byref(one), 32) == al(11 * 4)


def test_gemm_norm_checks_before_the_device():
    import ctypes
    lib = L.lib()
    ar = Arena()
    good = fake_stage(ar, 256, 512, 64, L.NORM_RMS)
    need = lib.wgn_gemm_norm_workspace_bytes(ctypes.byref(good), 64)
    assert need > 0
    assert call_gemm(good, 0) == L.E_ARG
    assert call_gemm(good, 129) == L.E_ARG
    assert lib.wgn_gemm_norm_workspace_bytes(ctypes.byref(good), 129) == 0
    am = fake_stage(ar, 256, 512, 64, L.NORM_RMS, L.EPI_ARGMAX, bias=True)
    assert call_gemm(am, 64) == L.E_UNSUPPORTED                    # argmax with a bias
    ov = fake_stage(ar, 256, 512, 64, L.NORM_RMS)
    ov.y = ov.x                                                     # output over the input
    assert call_gemm(ov, 64) == L.E_ARG
    assert call_gemm(good, 64, ws=0) == L.E_WORKSPACE
    assert call_gemm(good, 64, ws=0x100010) == L.E_WORKSPACE       # not 256-aligned
    assert call_gemm(good, 64, ws_bytes=need - 1) == L.E_WORKSPACE
    if L.lib().wgn_device_cu_count() == 0:
        assert call_gemm(good, 64, ws_bytes=need) == L.E_DEVICE    # every host check passed


def test_layer_chain_batched_checks_before_the_device():
    import ctypes
    lib = L.lib()
    stages = fake_decoder(Arena(), 32, 1, V=4096)
    arr = L.stage_array(stages)
    need = lib.wgn_workspace_bytes(arr, len(stages), 32, 0)
    assert need > 0
    plan = L.Plan()
    plan.prefetch, plan.distance, plan.blocks, plan.frac_pct = 1, 1, 16, 50
    o = L.ChainOpts()
    assert lib.wgn_layer_chain(arr, len(stages), 32, None, ctypes.byref(plan), 0x100000, need, None,
                               None) == L.E_UNSUPPORTED             # no prefetch plans on this path
    o.trace = 1
    assert lib.wgn_layer_chain(arr, len(stages), 32, ctypes.byref(o), None, 0x100000, need, None,
                               None) == L.E_UNSUPPORTED             # no trace
    assert lib.wgn_layer_chain(arr, len(stages), 32, None, None, 0x100000, need - 1, None,
                               None) == L.E_WORKSPACE
    if L.lib().wgn_device_cu_count() == 0:
        assert lib.wgn_layer_chain(arr, len(stages), 32, None, None, 0x100000, need, None, None) == L.E_DEVICE


# ----------------------------------------------------------- backward pass
def fake_train_chain(ar, B, n, D=768, K0=None):
    """n LayerNorm -> Linear -> GELU blocks with kept pre-activations, plus
    their gradient outputs (fake addresses)."""
    stages, grads = [], []
    x = None
    for i in range(n):
        K = K0 if (i == 0 and K0) else D
        s = fake_stage(ar, D, K, B, L.NORM_LAYER, L.EPI_GELU_TANH, x=x, bias=True, beta=True)
        s.eps = 1e-5
        s.logits = ar.take(B * D * 4)
        x = s.y
        stages.append(s)
        g = L.Grad()
        g.gW, g.gbias, g.ggamma, g.gbeta = ar.take(D * K * 2), ar.take(D * 2), ar.take(K * 2), ar.take(K * 2)
        g.gy, g.gz = ar.take(B * D * 2), ar.take(B * D * 2)
        grads.append(g)
    return stages, grads


def call_backward(stages, grads, B, ws=None, ws_bytes=None, g_in=None, gin_stride=0, g_out=None, g_stride=0):
    import ctypes
    arr = L.stage_array(stages)
    gr = (L.Grad * len(grads))(*grads)
    need = L.lib().wgn_backward_workspace_bytes(arr, len(stages), B)
    if ws is None:
        ws = 1 << 44
    h = ctypes.c_void_p()
    return L.lib().wgn_backward_create(arr, len(stages), B, gr, g_out, g_stride, g_in, gin_stride, ws,
                                       need if ws_bytes is None else ws_bytes, None, ctypes.byref(h))


def test_backward_workspace_layout():
    """The block table (136 bytes a block), then per block: statistics and
    x-hat; two partial buffers of the largest
    block (64-row blocks) and two buffers of per-tile shares (by block
    parity); one flag per tile of the largest block and the error word."""
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    for B in (1, 4, 16):
        ar = Arena()
        st, _ = fake_train_chain(ar, B, 72)
        need = L.lib().wgn_backward_workspace_bytes(L.stage_array(st), 72, B)
        tiles = 12 * 12
        want = (up(72 * 136) + 72 * (up(B * 8) + up(B * 768 * 2)) + 2 * (up(12 * B * 768 * 4) + up(tiles * B * 8))
                + up((tiles + 4) * 4))
        assert need == want, (B, need, want)
    ar = Arena()
    st, _ = fake_train_chain(ar, 17, 2)
    assert L.lib().wgn_backward_workspace_bytes(L.stage_array(st), 2, 17) == 0  # batch above 16
    st, _ = fake_train_chain(ar, 4, 2)
    st[1].epi = L.EPI_NONE
    st[1].logits = None
    assert L.lib().wgn_backward_workspace_bytes(L.stage_array(st), 2, 4) == 0  # not a GELU block


def test_backward_checks_before_the_device():
    """Every argument error is reported before the device is looked at (this
    host has none: a valid call ends in WGN_E_DEVICE)."""
    B = 4
    ar = Arena()
    st, gr = fake_train_chain(ar, B, 3)
    assert call_backward(st, gr, B) == L.E_DEVICE
    cases = []
    s2, g2 = fake_train_chain(ar, B, 3); s2[1].norm = L.NORM_RMS; s2[1].beta = None; g2[1].gbeta = None
    cases.append((s2, g2, L.E_UNSUPPORTED, "RMSNorm block"))
    s2, g2 = fake_train_chain(ar, B, 3); s2[2].logits = None
    cases.append((s2, g2, L.E_ARG, "no pre-activation"))
    s2, g2 = fake_train_chain(ar, B, 3); s2[0].residual = ar.take(B * 768 * 2); s2[0].res_stride = 768
    cases.append((s2, g2, L.E_UNSUPPORTED, "residual"))
    s2, g2 = fake_train_chain(ar, B, 3, K0=512); s2[1].K = 512
    cases.append((s2, g2, L.E_ARG, "shapes do not chain"))
    s2, g2 = fake_train_chain(ar, B, 3); g2[1].gbias = None
    cases.append((s2, g2, L.E_ARG, "bias without its gradient"))
    s2, g2 = fake_train_chain(ar, B, 3); s2[0].gamma = None
    cases.append((s2, g2, L.E_ARG, "gain gradient without a gain"))
    s2, g2 = fake_train_chain(ar, B, 3); g2[2].gW = None
    cases.append((s2, g2, L.E_ARG, "no weight gradient"))
    s2, g2 = fake_train_chain(ar, B, 3); g2[2].gW += 8
    cases.append((s2, g2, L.E_ALIGN, "weight gradient misaligned"))
    s2, g2 = fake_train_chain(ar, B, 3); g2[1].gz = g2[0].gW + 64
    cases.append((s2, g2, L.E_ARG, "two outputs overlap"))
    s2, g2 = fake_train_chain(ar, B, 3); g2[2].gW = s2[1].W
    cases.append((s2, g2, L.E_ARG, "an output overwrites a weight"))
    s2, g2 = fake_train_chain(ar, B, 3); g2[0].gy = s2[1].logits
    cases.append((s2, g2, L.E_ARG, "an output overwrites a pre-activation"))
    for s, g, want, what in cases:
        assert call_backward(s, g, B) == want, what
    assert call_backward(st, gr, 17) == L.E_ARG
    assert call_backward(st, gr, B, ws_bytes=1024) == L.E_WORKSPACE
    assert call_backward(st, gr, B, ws=(1 << 44) + 64) == L.E_WORKSPACE  # 256-byte alignment
    assert call_backward(st, gr, B, ws=st[0].W) == L.E_ARG  # workspace over a weight
    assert call_backward(st, gr, B, g_in=st[0].x, gin_stride=768) == L.E_ARG  # g_in over the input
    assert call_backward(st, gr, B, g_in=ar.take(B * 768 * 2), gin_stride=700) == L.E_ARG
    assert call_backward(st, gr, B, g_in=ar.take(B * 768 * 2) + 1, gin_stride=768) == L.E_ALIGN
    assert call_backward(st, gr, B, g_out=ar.take(B * 768 * 2), g_stride=768) == L.E_DEVICE
    import ctypes
    arr = L.stage_array(st)
    gra = (L.Grad * 3)(*gr)
    assert L.lib().wgn_chain_backward(arr, 3, B, gra, None, 0, None, 0, 2, 1 << 44, 1 << 30, None) == L.E_ARG
    assert L.lib().wgn_backward_run(None, 1, None) == L.E_ARG
    assert L.lib().wgn_backward_check(None, None) == L.E_ARG
    assert L.lib().wgn_backward_grid(None) == -1


# ------------------------------------------------- attention inside a chain
def fake_attn(ar, B, q_y, k_y, v_y, out, slots=1024, hq=12, hkv=2):
    a = L.AttnStage()
    a.q, a.q_stride = q_y, hq * 128
    a.k_new, a.k_stride = k_y, hkv * 128
    a.v_new, a.v_stride = v_y, hkv * 128
    a.k_cache = ar.take(B * hkv * slots * 256)
    a.v_cache = ar.take(B * hkv * slots * 256)
    a.pos = ar.take(B * 4)
    a.out, a.out_stride = out, hq * 128
    a.q_heads, a.kv_heads, a.slots, a.head_dim = hq, hkv, slots, 128
    a.scale = 128 ** -0.5
    return a


def attn_chain(ar, B, n_layers=2, slots=1024):
    """Stages and attention items of a decode step with computed attention:
    {Q, K, V} -> attention -> O -> gate/up -> down per layer."""
    stages, att = [], []
    h = ar.take(B * 1536 * 2)
    for _ in range(n_layers):
        q = fake_stage(ar, 1536, 1536, B, L.NORM_RMS, x=h)
        k = fake_stage(ar, 256, 1536, B, L.NORM_RMS, x=h)
        v = fake_stage(ar, 256, 1536, B, L.NORM_RMS, x=h)
        k.gamma = v.gamma = q.gamma  # one x-hat for the three
        a_out = ar.take(B * 1536 * 2)
        stages += [q, k, v]
        att.append((len(stages), fake_attn(ar, B, q.y, k.y, v.y, a_out, slots)))
        o = fake_stage(ar, 1536, 1536, B, L.NORM_NONE, x=a_out, residual=h)
        gu = fake_stage(ar, 8960, 1536, B, L.NORM_RMS, L.EPI_SWIGLU, x=o.y)
        d = fake_stage(ar, 1536, 8960, B, L.NORM_NONE, x=gu.y, residual=o.y)
        stages += [o, gu, d]
        h = d.y
    return stages, att


def attn_ws(stages, att, B, grid=256):
    arr = L.stage_array(stages)
    A = (L.AttnStage * max(1, len(att)))()
    before = (L.I32 * max(1, len(att)))()
    for i, (b, a) in enumerate(att):
        A[i], before[i] = a, b
    o = L.ChainOpts()
    o.grid = grid
    return L.lib().wgn_chain_attn_workspace_bytes(arr, len(stages), A, before, len(att), B, o)


@pytest.mark.parametrize("B", [1, 2, 4, 5, 16])
def test_attention_chain_plans(B):
    """A chain with attention items plans (workspace > 0) at every batch of
    both paths, and its workspace holds the partials: per (batch row,
    key/value head) one partial of 12/2 x 130 floats per chunk, about one
    chunk per workgroup and at most one per pass of cache slots."""
    ar = Arena()
    stages, att = attn_chain(ar, B)
    ws = attn_ws(stages, att, B)
    assert ws > 0
    # the same stages without attention (the attention output then an input
    # nobody writes) need less: no attention descriptors and no partials
    arr = L.stage_array(stages)
    o = L.ChainOpts()
    o.grid, o.no_fuse = 256, 1
    plain = L.lib().wgn_chain_workspace_bytes(arr, len(stages), B, o)
    assert 0 < plain < ws
    nchunk = min(max(1, 256 // (B * 2)), 1024 // (8 if B == 1 else 16))  # passes of 8 slots at batch 1
    part = B * 2 * nchunk * ((6 * 130 + 3) & ~3) * 4
    assert ws - plain >= part


def test_attention_chain_argument_checks():
    ar = Arena()
    stages, att = attn_chain(ar, 1)
    assert attn_ws(stages, att, 1) > 0
    bad = []
    for field, value in (("head_dim", 64), ("q_heads", 13), ("kv_heads", 0), ("slots", 0), ("scale", float("inf")),
                         ("pos", 0), ("q", None)):
        _, a0 = att[0]
        a = L.AttnStage.from_buffer_copy(a0)
        setattr(a, field, value)
        bad.append((field, [(att[0][0], a)] + att[1:]))
    _, a0 = att[0]
    a = L.AttnStage.from_buffer_copy(a0)
    a.q = a.q + 8  # not 16-byte aligned
    bad.append(("alignment", [(att[0][0], a)] + att[1:]))
    a = L.AttnStage.from_buffer_copy(a0)
    a.out = a.k_cache  # writes into its own cache
    bad.append(("overlap", [(att[0][0], a)] + att[1:]))
    bad.append(("order", [(att[1][0], att[0][1]), (att[0][0], att[1][1])]))
    bad.append(("position", [(len(stages) + 1, att[0][1])]))
    for what, items in bad:
        assert attn_ws(stages, items, 1) == 0, what
