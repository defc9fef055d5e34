"""Host model of the persistent kernel's in-workgroup schedule (no GPU).

The chain kernel runs one control wave and several weight-streaming waves per
workgroup; they meet only at workgroup barriers.  The LDS areas they share are
written by one side and read by the other between barriers:

* run lists (one LDS buffer per phase, DESC_BUFS buffers in a ring), written by
  the control wave DESC_AHEAD phases ahead (at the end of an iteration, after
  its flag store) and read by the streaming waves when they issue weight loads
  (up to two blocks beyond the one they consume);
* normalisation jobs, written at the end of the iteration before their phase;
* x-hat (written by the control wave, read by the streaming waves);
* partial sums (written by the streaming waves, read by the control wave's
  epilogue).

This file re-states the loops of both wave kinds as event lists and checks, for
random numbers of blocks per phase, that every read of an LDS area is separated
from the write that produced it and from the write that replaces it by at least
one barrier, and that both kinds of wave pass the same number of barriers.  The
two constants below mirror wgn_prog.h; the test reads them from the header so a
change there is modelled here.
"""
import os
import random
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_constant(name):
    src = open(os.path.join(ROOT, "weight_gemv_norm_amd", "csrc", "wgn_prog.h")).read()
    m = re.search(r"constexpr int %s = (\d+);" % name, src) or re.search(r"#define WGN_%s (\d+)" % name, src)
    assert m, name
    return int(m.group(1))


_PROG = open(os.path.join(ROOT, "weight_gemv_norm_amd", "csrc", "wgn_prog.h")).read()
# wgn_prog.h sizes the run-list ring per block-buffer ring; the model mirrors
# the two expressions (checked verbatim so that a change there fails here)
assert "constexpr int desc_bufs(int r) { return ring_slots(r) + 2 <= 4 ? 4 : 8; }" in _PROG
assert "constexpr int desc_ahead(int r) { return ring_slots(r) + 2; }" in _PROG


def desc_bufs_of(slots):
    return 4 if slots + 2 <= 4 else 8


def desc_ahead_of(slots):
    return slots + 2


DESC_BUFS = 4    # ring 0 (two block buffers)
DESC_AHEAD = 4
# 1 if the streaming waves refill only after the control wave has issued the
# epilogue's stores (a third barrier per phase)
EPI_BARRIER = header_constant("EPI_BARRIER")


def ring_table():
    """(slots, interleaved) of every ring, read from wgn_prog.h's ring_slots /
    ring_interleaved (nested conditionals on r)."""
    src = open(os.path.join(ROOT, "weight_gemv_norm_amd", "csrc", "wgn_prog.h")).read()
    n = header_constant("NUM_RINGS")

    def cond_fn(name):
        m = re.search(r"constexpr \w+ %s\(int r\) \{ return (.*?); \}" % name, src)
        assert m, name
        expr = m.group(1)

        def ev(e, r):
            e = e.strip()
            m2 = re.match(r"r == (\d+) \? (\w+) : (.*)$", e)
            if m2:
                return ev(m2.group(2), r) if r == int(m2.group(1)) else ev(m2.group(3), r)
            m3 = re.match(r"r == (\d+)$", e)
            if m3:
                return r == int(m3.group(1))
            return int(e) if e.isdigit() else {"true": True, "false": False}[e]
        return lambda r: ev(expr, r)
    slots, il = cond_fn("ring_slots"), cond_fn("ring_interleaved")
    return [(slots(r), bool(il(r))) for r in range(n)]


RINGS = ring_table()
SLOTS, INTERLEAVE = RINGS[0]


class Wave:
    def __init__(self):
        self.epoch = 0          # barriers passed so far
        self.events = []        # (epoch, kind, phase)

    def barrier(self):
        self.epoch += 1

    def ev(self, kind, phase):
        self.events.append((self.epoch, kind, phase))


def control_events(p0, p1, desc_ahead=DESC_AHEAD, norm=None, epi_barrier=EPI_BARRIER, share=False):
    """The control wave's loop: run-list builds, x-hat writes, partial reads.
    Phase q's run list is written at the end of iteration q - desc_ahead
    (after the flag store), and a phase's normalisation jobs at the end of the
    iteration before it; the first ones before the loop.  norm[p]: phase p has
    a normalised input, normalised by all waves between two extra barriers
    (inputs landed; partial statistics written)."""
    norm = norm or {}
    c = Wave()
    for q in range(p0, min(p1, p0 + desc_ahead)):
        c.ev("build", q)
    c.ev("write_job", p0)
    c.barrier()
    for p in range(p0, p1):
        c.ev("read_runs", p)       # header and run list of phase p (epilogue inputs)
        if share:
            c.barrier()            # flags seen: every wave copies its share of the inputs
        c.ev("write_xhat", p)      # raw inputs (and, without a norm, x-hat itself)
        if norm.get(p):
            c.barrier()            # inputs landed (the jobs were posted earlier)
            c.ev("read_job", p)
            c.ev("write_stats", p)
            c.barrier()            # partial statistics written
            c.ev("read_stats", p)
            c.ev("write_xhat", p)  # normalised slice
        c.barrier()                # x-hat ready
        c.barrier()                # partials complete
        c.ev("read_part", p)       # epilogue
        c.ev("read_runs", p)
        if epi_barrier:
            c.barrier()            # epilogue stores issued: streaming waves may refill
        # after the flag store: later lists and the next phase's jobs
        if p + desc_ahead < p1:
            c.ev("build", p + desc_ahead)
        if p + 1 < p1:
            c.ev("write_job", p + 1)
    return c


def stream_events(p0, p1, nblocks, norm=None, epi_barrier=EPI_BARRIER, slots=2, share=False):
    """One streaming wave's loop with a ring of `slots` block buffers.  nblocks[p] >= 1 is
    the number of blocks the wave walks in phase p (an empty share is one empty
    block)."""
    norm = norm or {}
    s = Wave()

    class St:
        pass

    S = St()
    S.p = p0
    S.k = 0            # blocks of phase S.p already loaded
    S.done = False

    def begin_phase(p):
        S.p, S.k = p, 0
        s.ev("read_runs", p)       # header copied into registers

    def load_block():
        if S.done:
            return ("empty", None, False)
        p = S.p
        s.ev("read_runs", p)       # lane-parallel unit descriptors
        S.k += 1
        last = S.k >= nblocks[p]
        if last:
            if p + 1 < p1:
                begin_phase(p + 1)
            else:
                S.done = True
        return ("blk", p, last)

    def phase_start(p):
        """Input copies (shared), norm steps (if any) and the x-hat barrier of phase p."""
        if share:
            s.barrier()            # flags seen
            s.ev("read_runs", p)   # the phase's x-hat offset and row stride
            s.ev("write_xhat", p)  # this wave's share of the input copies
        s.ev("read_runs", p)       # the phase's header: normalised input?
        if norm.get(p):
            s.barrier()            # inputs landed, jobs posted
            s.ev("read_job", p)
            s.ev("write_stats", p)
            s.barrier()
            s.ev("read_stats", p)
            s.ev("write_xhat", p)
        s.barrier()                # x-hat of phase p

    def consume(blk):
        kind, p, last = blk
        if kind == "blk":
            s.ev("read_xhat", p)
            s.ev("write_part", p)  # any block may end a row-part segment

    s.barrier()                    # run lists of the first phases are in LDS
    begin_phase(p0)
    ring = [load_block() for _ in range(slots)]
    phase_start(p0)
    p = p0
    ok = True
    while ok and p < p1:
        for i in range(slots):
            consume(ring[i])
            end = ring[i][2]
            if end:
                s.barrier()        # partials of phase p
                if share:
                    s.ev("read_runs", p)   # this wave's share of the epilogue rows
                    s.ev("read_part", p)
                if epi_barrier:
                    s.barrier()    # epilogue stores of phase p issued
            ring[i] = load_block()
            if end:
                p += 1
                if p < p1:
                    phase_start(p)
    return s


def check_schedule(p0, p1, nblocks, desc_bufs=DESC_BUFS, desc_ahead=DESC_AHEAD, norm=None,
                   slots=SLOTS, interleave=INTERLEAVE, share=False):
    """share: the matrix-core path's shared input copies and epilogue rows."""
    epi = 0 if interleave else EPI_BARRIER
    c = control_events(p0, p1, desc_ahead, norm, epi_barrier=epi, share=share)
    waves = [stream_events(p0, p1, nb, norm, epi_barrier=epi, slots=slots, share=share) for nb in nblocks]
    errors = []
    for s in waves:
        if s.epoch != c.epoch:
            errors.append("barrier count %d != %d" % (s.epoch, c.epoch))
    build_epoch = {q: e for e, k, q in c.events if k == "build"}
    xhat_epoch = {}
    for e, k, q in c.events + [ev for w in waves for ev in w.events]:
        if k == "write_xhat":
            xhat_epoch[q] = max(xhat_epoch.get(q, -1), e)
    xhat_first = {}
    for e, k, q in c.events:
        if k == "write_xhat":
            xhat_first.setdefault(q, e)
    job_w = {q: e for e, k, q in c.events if k == "write_job"}
    stats_w = {}
    for e, k, q in c.events + [ev for w in waves for ev in w.events]:
        if k == "write_stats":
            stats_w.setdefault(q, set()).add(e)
    for w in [c] + waves:
        for e, k, q in w.events:
            if k == "read_job" and not (e > job_w[q] and (q + 1 not in job_w or e < job_w[q + 1])):
                errors.append("norm job of %d read outside its lifetime" % q)
            if k == "read_stats" and not all(e > ws for ws in stats_w[q]):
                errors.append("statistics of %d read before all waves wrote them" % q)
    # statistics of phase q are overwritten only after every read of phase q-1's
    reads_stats = {}
    for w in [c] + waves:
        for e, k, q in w.events:
            if k == "read_stats":
                reads_stats.setdefault(q, []).append(e)
    prev = None
    for q in sorted(stats_w):
        if prev is not None and not all(min(stats_w[q]) > r for r in reads_stats[prev]):
            errors.append("statistics of %d overwritten while phase %d reads them" % (prev, q))
        prev = q
    part_first, part_last = {}, {}   # earliest and latest epilogue read of each phase's partials
    for w in [c] + waves:
        for e, k, q in w.events:
            if k == "read_part":
                part_first[q] = min(part_first.get(q, e), e)
                part_last[q] = max(part_last.get(q, e), e)
    for q in range(p0, p1):
        if q not in build_epoch:
            errors.append("phase %d never built" % q)
    # streaming-wave reads need a barrier after the build; the control wave
    # reads its own builds in program order, so only the overwrite matters there
    for s in waves:
        for e, k, q in s.events:
            if k != "read_runs":
                continue
            if not e > build_epoch[q]:
                errors.append("runs %d read in epoch %d, built in epoch %d" % (q, e, build_epoch[q]))
            nxt = q + desc_bufs
            if nxt in build_epoch and not e < build_epoch[nxt]:
                errors.append("runs %d read in epoch %d, overwritten by %d in epoch %d"
                              % (q, e, nxt, build_epoch[nxt]))
    build_pos = {q: i for i, (e, k, q) in enumerate(c.events) if k == "build"}
    for i, (e, k, q) in enumerate(c.events):
        if k == "read_runs":
            if not build_pos[q] < i or (q + desc_bufs in build_pos and not i < build_pos[q + desc_bufs]):
                errors.append("control wave reads runs %d out of order" % q)
    for s in waves:
        for e, k, q in s.events:
            if k == "read_xhat":
                if not e > xhat_epoch[q]:
                    errors.append("x-hat %d read before it is written" % q)
                if q + 1 in xhat_first and not e < xhat_first[q + 1]:
                    errors.append("x-hat %d read after phase %d overwrote it" % (q, q + 1))
            if k == "write_part":
                if not e < part_first[q]:
                    errors.append("partials of %d written after the epilogue read them" % q)
                if q - 1 in part_last and not e > part_last[q - 1]:
                    errors.append("partials of %d written before the epilogue of %d" % (q, q - 1))
    return errors


def test_schedule_random_block_counts():
    rng = random.Random(1234)
    for _ in range(3000):
        P = rng.randint(1, 12)
        W = rng.randint(1, 7)
        nb = [[rng.choice([1, 1, 1, 2, 3, 5]) for _ in range(P)] for _ in range(W)]
        errs = check_schedule(0, P, nb)
        assert not errs, (P, nb, errs[:3])


def test_schedule_exhaustive_small():
    import itertools
    for P in range(1, 7):
        for nb in itertools.product([1, 2, 3], repeat=P):
            errs = check_schedule(0, P, [list(nb), [1] * P])
            assert not errs, (nb, errs[:3])


def test_schedule_with_all_wave_norm():
    rng = random.Random(99)
    for _ in range(2000):
        P = rng.randint(1, 10)
        W = rng.randint(1, 7)
        nb = [[rng.choice([1, 1, 2, 3]) for _ in range(P)] for _ in range(W)]
        norm = {p: rng.random() < 0.6 for p in range(P)}
        errs = check_schedule(0, P, nb, norm=norm)
        assert not errs, (P, nb, norm, errs[:3])


@pytest.mark.parametrize("slots", [2, 3, 4, 5])
def test_schedule_slots_with_matching_ring(slots):
    """A ring of DESC_BUFS = slots + 2 run lists, written that many phases
    ahead, covers a wave with `slots` block buffers."""
    rng = random.Random(7 + slots)
    for _ in range(800):
        P = rng.randint(1, 12)
        W = rng.randint(1, 7)
        nb = [[rng.choice([1, 1, 1, 2, 3, 5]) for _ in range(P)] for _ in range(W)]
        norm = {p: rng.random() < 0.6 for p in range(P)}
        errs = check_schedule(0, P, nb, desc_bufs=slots + 2, desc_ahead=slots + 2, norm=norm, slots=slots,
                              interleave=0)
        assert not errs, (P, nb, norm, errs[:3])


@pytest.mark.parametrize("slots", [3, 4, 5])
def test_schedule_interleaved_refills(slots):
    rng = random.Random(11 + slots)
    for _ in range(800):
        P = rng.randint(1, 12)
        W = rng.randint(1, 7)
        nb = [[rng.choice([1, 1, 1, 2, 3, 5]) for _ in range(P)] for _ in range(W)]
        norm = {p: rng.random() < 0.6 for p in range(P)}
        errs = check_schedule(0, P, nb, desc_bufs=slots + 2, desc_ahead=slots + 2, norm=norm, slots=slots,
                              interleave=1)
        assert not errs, (P, nb, norm, errs[:3])


@pytest.mark.parametrize("ring", range(len(RINGS)))
def test_schedule_every_ring_with_the_header_constants(ring):
    """Each ring of the kernel, with the header's run-list ring size."""
    slots, il = RINGS[ring]
    bufs, ahead = desc_bufs_of(slots), desc_ahead_of(slots)
    rng = random.Random(31 + ring)
    for _ in range(1500):
        P = rng.randint(1, 14)
        W = rng.randint(1, 7)
        nb = [[rng.choice([1, 1, 1, 2, 3, 5]) for _ in range(P)] for _ in range(W)]
        norm = {p: rng.random() < 0.6 for p in range(P)}
        errs = check_schedule(0, P, nb, desc_bufs=bufs, desc_ahead=ahead, norm=norm, slots=slots,
                              interleave=int(il))
        assert not errs, (ring, P, nb, norm, errs[:3])


def test_ring_table_parsed():
    assert RINGS == [(2, False), (5, False), (4, True)]


def test_schedule_matrix_core_path_with_shared_inputs_and_epilogue():
    """The matrix-core path (ring 0, third barrier) with every wave copying
    inputs after an extra barrier and summing epilogue rows after the
    partials barrier."""
    rng = random.Random(77)
    for _ in range(2000):
        P = rng.randint(1, 12)
        W = rng.randint(1, 7)
        nb = [[rng.choice([1, 1, 1, 2, 3, 5]) for _ in range(P)] for _ in range(W)]
        norm = {p: rng.random() < 0.6 for p in range(P)}
        errs = check_schedule(0, P, nb, desc_bufs=4, desc_ahead=4, norm=norm, slots=2, interleave=0, share=True)
        assert not errs, (P, nb, norm, errs[:3])


def test_model_detects_short_ring_for_more_slots():
    errs = check_schedule(0, 10, [[1] * 10], desc_bufs=4, desc_ahead=4, slots=4)
    assert any("built in epoch" in e or "overwritten" in e for e in errs), errs


def test_schedule_launch_window():
    """A launch may cover phases [p0, p1) of a longer program."""
    for p0, p1 in [(3, 4), (2, 9), (5, 6)]:
        nb = [[1] * 9, [2] * 9]
        assert not check_schedule(p0, p1, nb)


def test_model_detects_building_too_late():
    """Lists written after the flag store need four phases of look-ahead:
    three is too little when a wave walks one-block phases, and the model
    must flag it."""
    errs = check_schedule(0, 8, [[1] * 8], desc_bufs=4, desc_ahead=3)
    assert any("built in epoch" in e for e in errs), errs


def test_model_detects_ring_too_small():
    errs = check_schedule(0, 8, [[1] * 8], desc_bufs=3, desc_ahead=4)
    assert any("overwritten" in e for e in errs), errs
