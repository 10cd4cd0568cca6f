"""Seeded synthetic inputs for the ring block-attention workloads.

This module generates inputs only: the five workload descriptions, the
bf16/fp32 Q, K, V and dO values, the packed-document lengths and the sampled
row lists.  It holds none of the attention arithmetic, so both the GPU path
and the CPU oracle can draw the identical values from it.

Every tensor is generated piecewise.  A sequence of ``S`` tokens is cut into
``n_pieces`` equal pieces, and piece ``p`` of tensor ``t`` comes from its own
stream ``SeedSequence(entropy=seed, spawn_key=(t, p))``.  Any holder of a piece
(a virtual rank, the oracle) can therefore regenerate exactly that piece
without materialising the whole sequence.

Values: ``standard_normal`` in float32, times the workload's value scale, then
rounded to nearest-even bf16 for the bf16 workloads.  bf16 tensors are handed
around as ``uint16`` bit patterns; :func:`bf16_bits_to_f32` widens them.

Layouts (which pieces a virtual rank holds) follow the workload text of the
ring-attention pages: a contiguous split gives rank ``r`` piece ``r``; the
zigzag split of Zigzag-Ring Attention gives rank ``r`` of ``n`` the pieces
``r`` and ``2n-1-r`` (TASP pages, experiment highlights: Zigzag-Ring
Attention is the load-balanced causal variant they compare against); the
striped split (Striped Attention, TASP citation map) gives rank ``r`` every
token at a position congruent to ``r`` modulo ``n``.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional, Sequence, Tuple

import numpy as np

# Stream ids used in the spawn key.
T_Q, T_K, T_V, T_DO, T_DOCS, T_ROWS = 0, 1, 2, 3, 4, 5

MASK_NONE, MASK_CAUSAL, MASK_DOC_CAUSAL = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, seed, value scale, split and mask."""

    name: str
    seed: int
    seq: int            # total tokens in the packed sequence
    n_ranks: int        # virtual ranks replayed on one GPU
    hq: int
    hkv: int
    d: int
    dtype: str          # "bf16" or "f32"
    value_scale: float  # inputs are N(0,1) * value_scale
    layout: str         # "contiguous", "zigzag" or "striped"
    mask: int           # MASK_* constant
    rank: int           # the rank whose replay is measured / checked
    backward: bool = False
    sampled_rows: Optional[int] = None   # oracle checks this many rows only
    doc_len_range: Optional[Tuple[int, int]] = None

    @property
    def n_pieces(self) -> int:
        return 2 * self.n_ranks if self.layout == "zigzag" else self.n_ranks

    @property
    def piece_len(self) -> int:
        return self.seq // self.n_pieces

    @property
    def chunk_len(self) -> int:
        return self.seq // self.n_ranks

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), as the fp32 value the kernels receive."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def rank_pieces(self, r: int) -> List[int]:
        if self.layout == "zigzag":
            return [r, 2 * self.n_ranks - 1 - r]
        return [r]

    def rank_segments(self, r: int) -> List[Tuple[int, int]]:
        """(start, length) of each contiguous run of global positions, in row
        order (contiguous and zigzag layouts)."""
        if self.layout == "striped":
            raise ValueError("a striped chunk is not a union of contiguous runs: use rank_runs")
        return [(p * self.piece_len, self.piece_len) for p in self.rank_pieces(r)]

    def rank_runs(self, r: int) -> List[Tuple[int, int, int]]:
        """(start, length, stride) of each run of global positions, in row
        order: the striped layout (token i on rank i mod n) is one run of
        stride n."""
        if self.layout == "striped":
            return [(r, self.chunk_len, self.n_ranks)]
        return [(s, n, 1) for s, n in self.rank_segments(r)]


# The five workloads.  Seeds: workload k uses seed k.
WORKLOADS = {
    "c1": Workload("c1_fp32_noncausal_2k", 1, 2048, 4, 2, 2, 64, "f32", 0.5,
                   "contiguous", MASK_NONE, 0),
    "c2": Workload("c2_bf16_causal_zigzag_32k", 2, 32768, 8, 32, 8, 128, "bf16", 1.0,
                   "zigzag", MASK_CAUSAL, 3),
    "c3": Workload("c3_bf16_packed_docs_64k", 3, 65536, 16, 32, 8, 128, "bf16", 1.0,
                   "contiguous", MASK_DOC_CAUSAL, 0, doc_len_range=(256, 16384)),
    "c4": Workload("c4_bf16_causal_zigzag_512k", 4, 524288, 8, 32, 8, 128, "bf16", 0.5,
                   "zigzag", MASK_CAUSAL, 0, sampled_rows=256),
    "c5": Workload("c5_bf16_backward_zigzag_32k", 5, 32768, 8, 32, 8, 128, "bf16", 1.0,
                   "zigzag", MASK_CAUSAL, 3, backward=True),
}


def scaled_workload(w: Workload, seq: int, hq: Optional[int] = None,
                    hkv: Optional[int] = None, d: Optional[int] = None,
                    n_ranks: Optional[int] = None, rank: Optional[int] = None,
                    seed: Optional[int] = None, name: Optional[str] = None) -> Workload:
    """A smaller copy of a workload (same split, mask and value distribution)."""
    return dataclasses.replace(
        w, name=name or f"{w.name}_s{seq}", seq=seq,
        hq=hq if hq is not None else w.hq, hkv=hkv if hkv is not None else w.hkv,
        d=d if d is not None else w.d,
        n_ranks=n_ranks if n_ranks is not None else w.n_ranks,
        rank=rank if rank is not None else w.rank,
        seed=seed if seed is not None else w.seed)


# ---------------------------------------------------------------------------
# bf16 bit handling (input preparation only)

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16, ties to even; returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# Piecewise tensor generation

def _rng(seed: int, tensor: int, piece: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=(tensor, piece)))


def gen_piece(w: Workload, tensor: int, piece: int) -> np.ndarray:
    """Piece ``piece`` of tensor ``tensor``: [piece_len, heads, d].

    Returns uint16 bf16 bits for bf16 workloads and float32 for f32 ones.
    Q and dO have ``hq`` heads, K and V ``hkv``.
    """
    heads = w.hq if tensor in (T_Q, T_DO) else w.hkv
    x = _rng(w.seed, tensor, piece).standard_normal((w.piece_len, heads, w.d), dtype=np.float32)
    if w.value_scale != 1.0:
        x *= np.float32(w.value_scale)
    if w.dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def gen_pieces(w: Workload, tensor: int, pieces: Sequence[int], threads: int = 8) -> np.ndarray:
    """Concatenation (along rows) of the given pieces, generated in parallel."""
    pieces = list(pieces)
    if not pieces:
        heads = w.hq if tensor in (T_Q, T_DO) else w.hkv
        return np.zeros((0, heads, w.d), dtype=np.uint16 if w.dtype == "bf16" else np.float32)
    with ThreadPoolExecutor(max(1, min(threads, len(pieces)))) as ex:
        parts = list(ex.map(lambda p: gen_piece(w, tensor, p), pieces))
    return np.concatenate(parts, axis=0) if len(parts) > 1 else parts[0]


def gen_rank_chunk(w: Workload, tensor: int, r: int, threads: int = 8) -> np.ndarray:
    """The rows virtual rank ``r`` holds of ``tensor`` (its chunk), in row order.
    A striped chunk takes every n-th row of the whole sequence (generated
    piecewise as for the contiguous split)."""
    if w.layout == "striped":
        return np.ascontiguousarray(gen_pieces(w, tensor, range(w.n_pieces), threads)[r::w.n_ranks])
    return gen_pieces(w, tensor, w.rank_pieces(r), threads)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Packed documents and sampled rows

def gen_doc_lengths(w: Workload) -> np.ndarray:
    """Document lengths of the packed buffer (log-uniform, last one truncated).

    u ~ U[ln lo, ln hi), L = clip(round(e^u), lo, hi); draw until the buffer
    is full, then cut the last document to fit.
    """
    lo, hi = w.doc_len_range
    rng = _rng(w.seed, T_DOCS, 0)
    lens: List[int] = []
    total = 0
    while total < w.seq:
        u = rng.uniform(math.log(lo), math.log(hi))
        L = int(min(max(round(math.exp(u)), lo), hi))
        L = min(L, w.seq - total)
        lens.append(L)
        total += L
    return np.asarray(lens, dtype=np.int64)


def gen_cu_seqlens(w: Workload) -> np.ndarray:
    """int32 [n_docs+1] cumulative document starts in packed (global) positions."""
    lens = gen_doc_lengths(w)
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    return cu.astype(np.int32)


def gen_sampled_rows(w: Workload, n: int, chunk_rows: int, piece_len: Optional[int] = None) -> np.ndarray:
    """Row indices (into the rank's chunk) that a sampled check looks at.

    The first and last row of each piece the chunk holds, then rows drawn
    uniformly without replacement until ``n`` distinct rows are chosen.
    Sorted ascending.
    """
    piece_len = piece_len or w.piece_len
    fixed = set()
    for p0 in range(0, chunk_rows, piece_len):
        fixed.add(p0)
        fixed.add(min(p0 + piece_len, chunk_rows) - 1)
    fixed = sorted(fixed)
    n = min(n, chunk_rows)
    rng = _rng(w.seed, T_ROWS, 0)
    rest = np.setdiff1d(np.arange(chunk_rows), np.asarray(fixed))
    extra = rng.choice(rest, size=max(0, n - len(fixed)), replace=False) if n > len(fixed) else []
    return np.sort(np.concatenate([np.asarray(fixed, dtype=np.int64), np.asarray(extra, dtype=np.int64)]))
