"""Helpers of the GPU parity tests: tolerances, comparison, oracle-side inputs.

Tolerances (stated for this method's outputs):
  bf16 class (outputs computed from bf16 inputs): max abs <= 2e-2 and
      mean abs <= 2e-3;
  fp32 class (fp32 inputs and outputs): max abs <= 1e-4;
  LSE: max abs <= 1e-3 on rows that have keys; rows without keys must be
      exactly -inf with an exactly zero output row.
"""
import numpy as np

import oracle
from ring_sequence_parallelism_amd import workloads as W

BF16_MAX, BF16_MEAN, F32_MAX, LSE_MAX = 2e-2, 2e-3, 1e-4, 1e-3


def assert_close(got, want, cls: str, what: str):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - want)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    if cls == "bf16":
        assert mx <= BF16_MAX and mean <= BF16_MEAN, f"{what}: max {mx:.3g} mean {mean:.3g}"
    else:
        assert mx <= F32_MAX, f"{what}: max {mx:.3g}"
    return mx, mean


def assert_lse(got, want, what: str):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape
    empty = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), empty), f"{what}: -inf pattern differs"
    assert not np.isnan(got).any(), f"{what}: NaN"
    if (~empty).any():
        mx = float(np.abs(got[~empty] - want[~empty]).max())
        assert mx <= LSE_MAX, f"{what}: LSE max {mx:.3g}"


def chunk_positions(w: W.Workload, r: int) -> np.ndarray:
    if w.layout == "zigzag":
        return oracle.zigzag_positions(w.seq, w.n_ranks, r)
    if w.layout == "striped":
        return oracle.striped_positions(w.seq, w.n_ranks, r)
    return oracle.contiguous_positions(w.seq, w.n_ranks, r)


def full_kv_f64(w: W.Workload, head=None):
    """K, V over the whole sequence in position order (pieces are contiguous runs)."""
    k = W.to_f64(W.gen_pieces(w, W.T_K, range(w.n_pieces)), w.dtype)
    v = W.to_f64(W.gen_pieces(w, W.T_V, range(w.n_pieces)), w.dtype)
    if head is not None:
        k, v = k[:, head:head + 1], v[:, head:head + 1]
    return k, v


def cu_or_none(w: W.Workload):
    return W.gen_cu_seqlens(w) if w.mask == W.MASK_DOC_CAUSAL else None
