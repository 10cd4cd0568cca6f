"""The host's choice of the mask-free kernels (rba_step_full_tiles) is sound.

Whenever it reports a step full, an enumeration of the key tiles (forward,
dQ pass) and query blocks (dK/dV pass) that each workgroup of the launch
visits finds no pair the mask forbids and no tile or block reaching past its
chunk; a mask-free kernel run on such a step computes exactly what the
masked one does.  The enumeration follows the kernels' visiting rule: a
query-stationary workgroup visits the 64-row key tiles that hold a key at
or before its last query position (every tile without a mask); a dK/dV
workgroup of 128 keys visits the 32-row query blocks that hold a query at or
after its first key position.  The choice must also be taken where it
applies: the steps of a causal zigzag ring other than a rank's own chunk."""
import os

import numpy as np
import pytest

import oracle
from ring_sequence_parallelism_amd import rba

pytestmark = pytest.mark.skipif(not os.path.exists(rba.LIB_PATH), reason="librba.so not built")

BN, BQ, BK, WK = 64, 32, 128, 32     # key tile, query block, dK/dV keys per workgroup, keys per wave


def _pos(segs):
    return np.concatenate([s[0] + (s[2] if len(s) > 2 else 1) * np.arange(s[1]) for s in segs]).astype(np.int64)


def _seg_id(segs):
    return np.concatenate([np.full(s[1], i) for i, s in enumerate(segs)])


def _query_rows_per_wg(hq, hkv):
    g = hq // hkv
    hpw = 4 if g % 4 == 0 else (2 if g % 2 == 0 else 1)
    return (4 // hpw) * 32


def forward_tiles_full(mask, qpos, kpos, rows_per_wg):
    """Every tile each query-stationary workgroup visits is full for all its rows."""
    sq, sk = qpos.size, kpos.size
    for r0 in range(0, sq, rows_per_wg):
        q = qpos[r0:r0 + rows_per_wg]
        visit = np.ones(sk, bool) if mask == 0 else kpos <= q.max()
        for t in np.unique(np.nonzero(visit)[0] // BN):
            if (t + 1) * BN > sk:
                return False                                  # ragged tile
            k = kpos[t * BN:(t + 1) * BN]
            if mask == 1 and not (k[:, None] <= q[None, :]).all():
                return False
    return True


def dkdv_blocks_full(mask, qpos, kpos):
    """Every query block each dK/dV workgroup visits is allowed for all of its keys."""
    sq, sk = qpos.size, kpos.size
    for k0 in range(0, sk, BK):
        kt = kpos[k0:k0 + BK]
        visit = np.ones(sq, bool) if mask == 0 else qpos >= kt.min()
        for b in np.unique(np.nonzero(visit)[0] // BQ):
            if (b + 1) * BQ > sq:
                return False                                  # ragged block
            q = qpos[b * BQ:(b + 1) * BQ]
            for w0 in range(k0, min(k0 + BK, sk), WK):
                if w0 + WK > sk:
                    return False                              # ragged wave
                k = kpos[w0:w0 + WK]
                if mask == 1 and not (k[:, None] <= q[None, :]).all():
                    return False
    return True


def _random_layout(rng):
    """Q and KV segment lists on disjoint positions, often tile-aligned and
    often with every KV segment before the queries that see it."""
    nq, nk = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    unit_q = int(rng.choice([32, 32, 64, 7]))
    unit_k = int(rng.choice([64, 64, 32, 13]))
    qlens = [unit_q * int(rng.integers(1, 6)) for _ in range(nq)]
    klens = [unit_k * int(rng.integers(1, 5)) for _ in range(nk)]
    strides = lambda n: [int(rng.choice([1, 1, 1, 3])) for _ in range(n)]
    qst, kst = strides(nq), strides(nk)
    items = [("k", i) for i in range(nk)] + [("q", i) for i in range(nq)]
    if rng.random() < 0.5:
        rng.shuffle(items)
    p, qsegs, ksegs = int(rng.integers(0, 50)), [None] * nq, [None] * nk
    for kind, i in items:
        p += int(rng.integers(0, 40))
        ln, sd = (qlens[i], qst[i]) if kind == "q" else (klens[i], kst[i])
        seg = (p, ln, sd)
        if kind == "q":
            qsegs[i] = seg
        else:
            ksegs[i] = seg
        p += (ln - 1) * sd + 1
    # the chunks list their segments in any order
    return [qsegs[i] for i in rng.permutation(nq)], [ksegs[i] for i in rng.permutation(nk)]


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (8, 4), (6, 2), (2, 2)])
def test_full_tile_choice_is_sound(hq, hkv):
    rng = np.random.default_rng(hq * 31 + hkv)
    reported = 0
    for trial in range(300):
        mask = int(rng.choice([0, 1, 1]))
        qsegs, ksegs = _random_layout(rng)
        qpos, kpos = _pos(qsegs), _pos(ksegs)
        a = rba.attn_params(hq, hkv, 128, 0.088, rba.RBA_BF16, mask)
        ff, bf = rba.rba_step_full_tiles(a, qpos.size, rba.make_segs(qsegs), kpos.size, rba.make_segs(ksegs))
        rows = _query_rows_per_wg(hq, hkv)
        if ff:
            assert forward_tiles_full(mask, qpos, kpos, rows), (trial, qsegs, ksegs, mask)
        if bf:
            assert forward_tiles_full(mask, qpos, kpos, _query_rows_per_wg(hq, hkv)), (trial, qsegs, ksegs)
            assert dkdv_blocks_full(mask, qpos, kpos), (trial, qsegs, ksegs, mask)
        reported += ff + bf
    assert reported >= 60      # the choice is taken often enough for the check to mean something


def test_document_mask_never_full():
    cu = np.array([0, 512, 1024], dtype=np.int32)
    a = rba.attn_params(8, 2, 128, 0.088, rba.RBA_BF16, rba.RBA_MASK_DOC_CAUSAL, None, cu)
    a.cu_seqlens_dev = 0x10000   # planning never dereferences the device copy
    ff, bf = rba.rba_step_full_tiles(a, 256, rba.make_segs([(768, 256)]), 256, rba.make_segs([(512, 256)]))
    assert (ff, bf) == (0, 0)


def test_fp32_steps_never_full():
    a = rba.attn_params(4, 4, 64, 0.125, rba.RBA_F32, rba.RBA_MASK_CAUSAL)
    ff, bf = rba.rba_step_full_tiles(a, 128, rba.make_segs([(4096, 128)]), 128, rba.make_segs([(0, 128)]))
    assert (ff, bf) == (0, 0)
    a.dtype = rba.RBA_BF16   # the same step in bf16 takes the mask-free kernels
    assert rba.rba_step_full_tiles(a, 128, rba.make_segs([(4096, 128)]), 128, rba.make_segs([(0, 128)])) == (1, 1)


@pytest.mark.parametrize("rank", [0, 3, 7])
def test_zigzag_ring_steps_take_the_full_path(rank):
    """32K causal zigzag over 8 ranks: every step but the rank's own chunk is full."""
    seq, n = 32768, 8
    piece = seq // (2 * n)
    segs = lambda r: [(r * piece, piece), ((2 * n - 1 - r) * piece, piece)]
    assert np.array_equal(_pos(segs(rank)), oracle.zigzag_positions(seq, n, rank))
    a = rba.attn_params(32, 8, 128, 0.088, rba.RBA_BF16, rba.RBA_MASK_CAUSAL)
    for j in range(n):
        ff, bf = rba.rba_step_full_tiles(a, 2 * piece, rba.make_segs(segs(rank)), 2 * piece, rba.make_segs(segs(j)))
        assert (ff, bf) == ((0, 0) if j == rank else (1, 1)), j
