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


# ---------------------------------------------------------------------------
# The oracle over many query rows, in parallel
#
# Query rows are independent in the forward, and in the backward dK / dV are
# sums over rows, so the oracle can be called on blocks of rows and the
# results concatenated (forward, dQ) or added (dK, dV).  Each block is also
# given only the keys its mask can allow (positions up to the block's last
# query; under the document mask, from the document start of its first
# query): a key outside that window is masked for every row of the block and
# contributes nothing, so the result is the same.  Blocks run in a thread
# pool (numpy releases the GIL in its array work) with one BLAS thread each.

def oracle_workers():
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _window(qpos_blk, mask, cu, nk):
    """[lo, hi) of key positions (keys are positions 0..nk-1) a block can see."""
    if mask == W.MASK_NONE:
        return 0, nk
    hi = int(qpos_blk.max()) + 1
    lo = 0
    if mask == W.MASK_DOC_CAUSAL:
        lo = int(cu[np.searchsorted(cu, int(qpos_blk.min()), side="right") - 1])
    return lo, min(hi, nk)


def _blocks(qpos, block):
    """Row blocks of consecutive rows (rows sorted by position inside each
    block keep windows tight for the layouts used here)."""
    return [np.arange(i, min(i + block, qpos.size)) for i in range(0, qpos.size, block)]


def oracle_attention_rows(q, k, v, qpos, mask, scale, cu=None, block=64):
    """oracle.attention of q (rows at positions qpos) against keys k, v at
    positions 0..len(k)-1, block by block on the keys each block can see."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    nq, hq = q.shape[0], q.shape[1]
    o = np.zeros((nq, hq, v.shape[2]))
    lse = np.full((hq, nq), -np.inf)
    nk = k.shape[0]

    def one(rows):
        lo, hi = _window(qpos[rows], mask, cu, nk)
        if hi <= lo:
            return rows, None, None
        ob, lb = oracle.attention(q[rows], k[lo:hi], v[lo:hi], qpos[rows], np.arange(lo, hi), mask, scale, cu,
                                  row_block=block)
        return rows, ob, lb

    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(oracle_workers()) as ex:
        for rows, ob, lb in ex.map(one, _blocks(qpos, block)):
            if ob is not None:
                o[rows] = ob
                lse[:, rows] = lb
    return o, lse


def oracle_backward_rows(q, k, v, do, qpos, mask, scale, cu=None, block=64):
    """oracle.attention_backward of q / dO (rows at positions qpos) against
    keys at positions 0..len(k)-1: dq per row, dk / dv summed over the row
    blocks, each block on the keys it can see.  Returns dq, dk, dv, O, LSE."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    nq, hq, d = q.shape
    nk = k.shape[0]
    dq = np.zeros_like(q, dtype=np.float64)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    o = np.zeros((nq, hq, v.shape[2]))
    lse = np.full((hq, nq), -np.inf)

    def one(rows):
        lo, hi = _window(qpos[rows], mask, cu, nk)
        if hi <= lo:
            return rows, lo, hi, None
        return rows, lo, hi, oracle.attention_backward(q[rows], k[lo:hi], v[lo:hi], do[rows], qpos[rows],
                                                       np.arange(lo, hi), mask, scale, cu, row_block=block)

    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(oracle_workers()) as ex:
        for rows, lo, hi, res in ex.map(one, _blocks(qpos, block)):
            if res is None:
                continue
            bdq, bdk, bdv, _, bo, blse = res
            dq[rows] = bdq
            dk[lo:hi] += bdk
            dv[lo:hi] += bdv
            o[rows] = bo
            lse[:, rows] = blse
    return dq, dk, dv, o, lse
