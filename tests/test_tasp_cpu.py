"""TASP schedule and step composition (host logic, no GPU).

TASP: Topology-aware Sequence Parallelism (abstract; method details):
the complete directed graph of n accelerators splits into n - 1 arc-disjoint
Hamiltonian cycles, and each ring iteration into as many concurrent
transfers.  These tests pin the decomposition to its definition, the closed
form of which slice a rank holds to an explicit simulation of the forwarding,
and the composed steps to the plain ring (same keys, same pair count)."""
import os

import numpy as np
import pytest

from ring_sequence_parallelism_amd import tasp
from ring_sequence_parallelism_amd import workloads as W


@pytest.mark.parametrize("n", [2, 3, 5, 7, 8, 9])
def test_decomposition_is_hamiltonian_and_arc_disjoint(n):
    cycles = tasp.hamiltonian_decomposition(n)
    assert len(cycles) == n - 1
    arcs = []
    for cyc in cycles:
        assert sorted(cyc) == list(range(n))          # visits every node once
        arcs += [(cyc[i], cyc[(i + 1) % n]) for i in range(n)]
    assert len(arcs) == len(set(arcs))                # no arc used twice
    assert set(arcs) == {(u, v) for u in range(n) for v in range(n) if u != v}   # every arc used


@pytest.mark.parametrize("n", [4, 6])
def test_no_decomposition_for_4_and_6(n):
    # the complete directed graphs on 4 and 6 nodes have none
    with pytest.raises(ValueError):
        tasp.hamiltonian_decomposition(n)


def _simulate(n, cycles, rank, iters):
    """Explicit forwarding: on every cycle each node passes on what it got one
    iteration earlier; returns, per iteration, the origin of each cycle's
    slice that `rank` receives."""
    succ = [{cyc[i]: cyc[(i + 1) % n] for i in range(n)} for cyc in cycles]
    held = [{v: v for v in range(n)} for _ in cycles]      # before iteration 1: own slice
    got = []
    for _ in range(iters):
        held = [{succ[c][v]: held[c][v] for v in range(n)} for c in range(len(cycles))]
        got.append([held[c][rank] for c in range(len(cycles))])
    return got


@pytest.mark.parametrize("n", [3, 5, 8])
def test_schedule_matches_simulated_forwarding(n):
    sch = tasp.TaspSchedule(n)
    for r in range(n):
        sim = _simulate(n, sch.cycles, r, n - 1)
        for it in range(1, n):
            assert [sch.source(r, it, c) for c in range(n - 1)] == sim[it - 1]


@pytest.mark.parametrize("n", [3, 5, 8])
def test_every_slice_arrives_once(n):
    sch = tasp.TaspSchedule(n)
    for r in range(n):
        for c in range(n - 1):
            srcs = [sch.source(r, it, c) for it in range(1, n)]
            assert sorted(srcs) == [x for x in range(n) if x != r]


@pytest.mark.parametrize("align", [1, 64])
@pytest.mark.parametrize("rows,k", [(4096, 7), (10, 7), (7, 7), (5, 7), (1, 3), (65536, 7), (4096, 15), (700, 7)])
def test_slice_bounds_partition(rows, k, align):
    b = tasp.slice_bounds(rows, k, align)
    assert len(b) == k and b[0][0] == 0 and b[-1][1] == rows
    assert all(b[i][1] == b[i + 1][0] for i in range(k - 1))
    assert all(x % align == 0 for x, _ in b if x < rows)          # boundaries on the alignment
    sizes = [y - x for x, y in b]
    full = [z for z in sizes[:-1]] + ([sizes[-1]] if rows % align == 0 else [])
    assert max(full) - min(full) <= align if full else True


@pytest.mark.parametrize("key,rank", [("c2", 3), ("c2", 0), ("c3", 5)])
def test_steps_cover_every_key_once(key, rank):
    w = W.WORKLOADS[key]
    sch = tasp.TaspSchedule(w.n_ranks) if w.n_ranks not in (4, 6) else None
    if sch is None:
        pytest.skip("no decomposition for this rank count")
    pos = []
    for it in range(w.n_ranks):
        sl = sch.step_slices(rank, it, w.chunk_len)
        segs = tasp.step_segments(w, sl)
        assert len(segs) <= 16
        pos.append(tasp.step_positions(w, sl))
    allpos = np.sort(np.concatenate(pos))
    assert np.array_equal(allpos, np.arange(w.seq))


def test_sixteen_ranks_decompose():
    sch = tasp.TaspSchedule(16)
    assert len(sch.cycles) == 15
    # 15 slices of a 4096-row contiguous chunk: one segment each
    w = W.WORKLOADS["c3"]
    for it in range(1, 16):
        segs = tasp.step_segments(w, sch.step_slices(5, it, w.chunk_len))
        assert len(segs) == 15


LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "ring_sequence_parallelism_amd", "librba.so")


@pytest.mark.skipif(not os.path.exists(LIB), reason="librba.so not built")
def test_tasp_pair_count_equals_plain_ring():
    # the host planner's exact counts over TASP's steps add up to the plain
    # ring's total for the 32K zigzag rank 3 (67,110,912 pairs per head)
    from ring_sequence_parallelism_amd import rba
    w = W.WORKLOADS["c2"]
    sch = tasp.TaspSchedule(w.n_ranks)
    a = rba.attn_params(w.hq, w.hkv, w.d, w.scale, rba.RBA_BF16, rba.RBA_MASK_CAUSAL)
    qs = rba.make_segs(w.rank_segments(w.rank))
    tot = 0
    for it in range(w.n_ranks):
        segs = tasp.step_segments(w, sch.step_slices(w.rank, it, w.chunk_len))
        _, p = rba.rba_plan_step(a, w.chunk_len, qs, w.chunk_len, rba.make_segs(segs))
        tot += p
    assert tot == 67_110_912
