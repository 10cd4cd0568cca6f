"""TASP step composition for one rank's ring, replayed on one GPU.

TASP: Topology-aware Sequence Parallelism (abstract; method details) splits
the all-to-all topology of n accelerators -- the complete directed graph on n
nodes -- into n - 1 arc-disjoint directed Hamiltonian cycles, and splits the
ring all-gather of KV chunks into the same number of concurrent ring
transfers.  The pages give no slicing rule; the reading used here is the
plainest one: every KV chunk is cut into n - 1 contiguous row slices (near
equal, with boundaries on the 64-row key tile), slice c travels along cycle
c, and at each iteration every node forwards to its successor on cycle c the
slice it received on that cycle one iteration earlier (at iteration 1, its
own slice c).

So at iteration s (1 <= s <= n - 1) rank r holds, for every cycle c, slice c
of the chunk that started s hops before r on cycle c.  Over the n - 1
iterations that is every slice of every other rank's chunk exactly once, and
iteration 0 is the rank's own chunk.  One ring step of the attention hot path
is then the rank's query chunk against the union of the slices it holds: up
to n - 1 slices from up to n - 1 source chunks, each slice one or two
position segments under the zigzag layout, which one rba_fwd_step takes as a
multi-segment KV chunk.

Everything here is host planning (integer bookkeeping).  Device memory for
the assembled KV of a step comes from torch; the attention arithmetic runs
in librba.so.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import workloads as W


def hamiltonian_decomposition(n: int) -> List[List[int]]:
    """n - 1 arc-disjoint directed Hamiltonian cycles covering every arc of the
    complete directed graph on nodes 0..n-1 (each cycle listed from node 0).

    Deterministic depth-first search over cycles in lexicographic order.  Such
    a decomposition exists for every n >= 2 except n = 4 and n = 6 (Tillson's
    theorem); for those the search is exhaustive and raises ValueError.
    """
    if n < 2:
        raise ValueError("need at least 2 nodes")
    used = set()
    cycles: List[List[int]] = []

    def cycles_from_0(path, visited):
        if len(path) == n:
            if (path[-1], path[0]) not in used:
                yield list(path)
            return
        u = path[-1]
        for v in range(n):
            if v in visited or (u, v) in used:
                continue
            path.append(v)
            visited.add(v)
            yield from cycles_from_0(path, visited)
            path.pop()
            visited.discard(v)

    def place(k):
        if k == n - 1:
            return True
        for cyc in cycles_from_0([0], {0}):
            arcs = [(cyc[i], cyc[(i + 1) % n]) for i in range(n)]
            used.update(arcs)
            cycles.append(cyc)
            if place(k + 1):
                return True
            cycles.pop()
            used.difference_update(arcs)
        return False

    if not place(0):
        raise ValueError(f"the complete directed graph on {n} nodes has no Hamiltonian decomposition")
    return cycles


def slice_bounds(rows: int, n_slices: int, align: int = 1) -> List[Tuple[int, int]]:
    """Contiguous row ranges [a, b) cutting `rows` rows into n_slices slices
    whose boundaries fall on multiples of `align` rows: the ceil(rows / align)
    units are shared out near-equally (the first ones get one unit more), so
    slice sizes differ by at most `align` rows; the last slice ends at `rows`.
    With fewer units than slices the trailing slices are empty."""
    units = -(-rows // align)
    base, extra = divmod(units, n_slices)
    out, u = [], 0
    for c in range(n_slices):
        v = u + base + (1 if c < extra else 0)
        out.append((min(u * align, rows), min(v * align, rows)))
        u = v
    return out


# Slice boundaries on multiples of the kernels' 64-row key tile, so that no
# key tile straddles two slices (a straddling tile holds rows of two source
# chunks and takes the per-element mask path).
SLICE_ALIGN = 64


@dataclasses.dataclass
class SliceRef:
    src: int               # source rank (owner of the chunk)
    cycle: int             # slice index = cycle index
    rows: Tuple[int, int]  # row range [a, b) inside the source chunk


class TaspSchedule:
    """Which slices a rank holds at each iteration of the decomposed ring."""

    def __init__(self, n: int, cycles: Optional[Sequence[Sequence[int]]] = None):
        self.n = n
        self.cycles = [list(c) for c in (cycles if cycles is not None else hamiltonian_decomposition(n))]
        # predecessor of each node on each cycle
        self.pred: List[Dict[int, int]] = []
        for cyc in self.cycles:
            p = {}
            for i, v in enumerate(cyc):
                p[v] = cyc[i - 1]
            self.pred.append(p)

    def source(self, rank: int, it: int, cycle: int) -> int:
        """Origin of the slice `cycle` that `rank` holds at iteration `it` (>= 1):
        the node `it` hops before it on that cycle."""
        v = rank
        for _ in range(it):
            v = self.pred[cycle][v]
        return v

    def step_slices(self, rank: int, it: int, chunk_len: int) -> List[SliceRef]:
        """The KV slices of iteration `it` (0: the rank's own chunk, whole)."""
        if it == 0:
            return [SliceRef(rank, -1, (0, chunk_len))]
        bounds = slice_bounds(chunk_len, len(self.cycles), SLICE_ALIGN)
        return [SliceRef(self.source(rank, it, c), c, bounds[c]) for c in range(len(self.cycles))
                if bounds[c][1] > bounds[c][0]]


def slice_segments(w: W.Workload, ref: SliceRef) -> List[Tuple[int, int, int]]:
    """Global position segments (start, length, stride) of a slice's rows, in
    row order."""
    out = []
    a, b = ref.rows
    for start, length, stride, row0 in _chunk_runs(w, ref.src):
        lo, hi = max(a, row0), min(b, row0 + length)
        if lo < hi:
            out.append((start + (lo - row0) * stride, hi - lo, stride))
    return out


def _chunk_runs(w: W.Workload, src: int):
    """(position start, length, stride, first row) of each position run of chunk `src`."""
    row0 = 0
    for start, length, stride in w.rank_runs(src):
        yield start, length, stride, row0
        row0 += length


def step_segments(w: W.Workload, slices: Sequence[SliceRef]) -> List[Tuple[int, int, int]]:
    """Position segments of a step's assembled KV (slices concatenated in order)."""
    segs: List[Tuple[int, int, int]] = []
    for ref in slices:
        segs.extend(slice_segments(w, ref))
    return segs


def step_positions(w: W.Workload, slices: Sequence[SliceRef]) -> np.ndarray:
    """Global positions of the assembled KV rows of a step, in row order."""
    return np.concatenate([s + d * np.arange(n) for s, n, d in step_segments(w, slices)])
