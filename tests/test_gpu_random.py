"""GPU parity on seeded random step geometries, against the fp64 oracle.

Each case draws its head counts, head dimension, mask, row counts, segment
layout (contiguous runs at random gaps, sometimes one strided run), document
cuts and score scale from its seed, then checks every element: the plain
forward step (O, LSE), the merging forward step against the oracle's merge
of a random earlier partial with this step's, the backward step's dQ, dK
and dV, and the forward step with a workspace on long key ranges (where
few row groups may split their key tiles over several workgroups).  Sizes
stay small enough for the oracle to finish in well under a second per case
while spanning several tiles and a ragged tail."""
import numpy as np
import pytest
import torch

import oracle
from ring_sequence_parallelism_amd import rba
from ring_sequence_parallelism_amd import workloads as W
from ring_sequence_parallelism_amd.ring import to_device

from _gpu_util import assert_close, assert_lse

pytestmark = pytest.mark.gpu
DEV = "cuda"

HEADS = [(4, 4), (8, 2), (4, 1), (6, 3), (2, 1), (8, 8), (6, 2)]


def _say(*a):
    print("[case]", *a, flush=True)


def _runs(rng, rows, base):
    """Split `rows` into 1-4 contiguous runs placed in a shuffled order at
    random gaps from `base`; with probability 1/4 a single strided run."""
    if rows > 1 and rng.random() < 0.25:
        return [(base + int(rng.integers(0, 50)), rows, int(rng.integers(2, 5)))]
    n = int(rng.integers(1, min(4, rows) + 1))
    cuts = np.sort(rng.choice(np.arange(1, rows), n - 1, replace=False)) if n > 1 else np.array([], int)
    lens = np.diff(np.concatenate([[0], cuts, [rows]])).astype(int)
    starts, p = {}, base
    for i in rng.permutation(n):
        p += int(rng.integers(0, 70))
        starts[i] = p
        p += int(lens[i])
    return [(starts[i], int(lens[i]), 1) for i in range(n)]


def _pos(segs):
    return np.concatenate([s + st * np.arange(n) for s, n, st in segs])


def _bf16(rng, shape, scale=1.0):
    bits = W.f32_to_bf16_bits((scale * rng.standard_normal(shape)).astype(np.float32))
    return bits, W.bf16_bits_to_f32(bits).astype(np.float64)


def _geometry(seed, max_rows=300, max_keys=400):
    rng = np.random.default_rng(10_000 + seed)
    hq, hkv = HEADS[int(rng.integers(0, len(HEADS)))]
    d = int(rng.choice([64, 128]))
    mask = int(rng.integers(0, 3))
    sq = int(rng.integers(1, max_rows + 1))
    sk = int(rng.integers(1, max_keys + 1))
    ksegs = _runs(rng, sk, int(rng.integers(0, 100)))
    # queries start around the keys so that causal and document masks cut tiles
    qsegs = _runs(rng, sq, int(rng.integers(0, int(_pos(ksegs).max()) + 60)))
    qpos, kpos = _pos(qsegs), _pos(ksegs)
    cu = None
    if mask == 2:
        end = int(max(qpos.max(), kpos.max())) + 1
        n_cut = int(rng.integers(0, min(8, end - 1) + 1))
        cuts = np.sort(rng.choice(np.arange(1, end), n_cut, replace=False)) if n_cut else np.array([], int)
        cu = np.concatenate([[0], cuts, [end]]).astype(np.int32)
    return rng, hq, hkv, d, mask, sq, sk, qsegs, ksegs, qpos, kpos, cu


def _attn(hq, hkv, d, mask, cu):
    scale = float(np.float32(1.0 / np.sqrt(d)))
    cu_dev = None if cu is None else torch.from_numpy(cu).to(DEV)
    return rba.attn_params(hq, hkv, d, scale, rba.RBA_BF16, mask, cu_dev, cu), scale


@pytest.mark.parametrize("seed", range(100))
def test_random_forward_step(seed):
    rng, hq, hkv, d, mask, sq, sk, qsegs, ksegs, qpos, kpos, cu = _geometry(seed)
    score = float(rng.choice([0.5, 1.0, 2.0, 3.0]))
    _say("random fwd", seed, dict(hq=hq, hkv=hkv, d=d, mask=mask, sq=sq, sk=sk, qsegs=qsegs, ksegs=ksegs,
                                  docs=None if cu is None else len(cu) - 1, score=score))
    qb, q64 = _bf16(rng, (sq, hq, d), score)
    kb, k64 = _bf16(rng, (sk, hkv, d), score)
    vb, v64 = _bf16(rng, (sk, hkv, d))
    a, scale = _attn(hq, hkv, d, mask, cu)
    q, k, v = (to_device(x, "bf16", DEV) for x in (qb, kb, vb))
    qs, ks = rba.make_segs(qsegs), rba.make_segs(ksegs)
    want_o, want_lse = oracle.attention(q64, k64, v64, qpos, kpos, mask, scale, cu)

    # plain step: every element of the partial is written
    o = torch.full((sq, hq, d), float("nan"), device=DEV)
    lse = torch.full((hq, sq), float("nan"), device=DEV)
    st = rba.rba_fwd_step(a, q, qs, k, v, ks, o, lse)
    torch.cuda.synchronize()
    if st == rba.RBA_STEP_EMPTY:
        assert np.isneginf(want_lse).all()
    else:
        assert_lse(lse.cpu().numpy(), want_lse, "lse")
        assert_close(o.cpu().numpy(), want_o, "bf16", "o_part")

    # merging step into a random earlier partial (some rows empty)
    o0 = rng.standard_normal((sq, hq, d)).astype(np.float32)
    l0 = rng.uniform(-3.0, 3.0, (hq, sq)).astype(np.float32)
    l0[:, rng.random(sq) < 0.2] = -np.inf
    o0[np.isneginf(l0).T] = 0.0
    o_acc = torch.from_numpy(o0).to(DEV)
    lse_acc = torch.from_numpy(l0).to(DEV)
    rba.rba_fwd_step_acc(a, q, qs, k, v, ks, o_acc, lse_acc)
    torch.cuda.synchronize()
    mo, ml = oracle.merge(o0.astype(np.float64), l0.astype(np.float64), want_o, want_lse)
    assert_lse(lse_acc.cpu().numpy(), ml, "lse_acc")
    assert_close(o_acc.cpu().numpy(), mo, "bf16", "o_acc")


@pytest.mark.parametrize("seed", range(50))
def test_random_backward_step(seed):
    """One KV chunk holding every key: the step's gradients are the whole
    gradients of attention over these positions."""
    rng, hq, hkv, d, mask, sq, sk, qsegs, ksegs, qpos, kpos, cu = _geometry(100 + seed, 200, 300)
    score = float(rng.choice([0.5, 1.0, 1.5]))
    _say("random bwd", seed, dict(hq=hq, hkv=hkv, d=d, mask=mask, sq=sq, sk=sk, qsegs=qsegs, ksegs=ksegs,
                                  docs=None if cu is None else len(cu) - 1, score=score))
    qb, q64 = _bf16(rng, (sq, hq, d), score)
    kb, k64 = _bf16(rng, (sk, hkv, d), score)
    vb, v64 = _bf16(rng, (sk, hkv, d))
    dob, do64 = _bf16(rng, (sq, hq, d))
    a, scale = _attn(hq, hkv, d, mask, cu)
    wdq, wdk, wdv, _, _, _ = oracle.attention_backward(q64, k64, v64, do64, qpos, kpos, mask, scale, cu)
    q, k, v, dO = (to_device(x, "bf16", DEV) for x in (qb, kb, vb, dob))
    qs, ks = rba.make_segs(qsegs), rba.make_segs(ksegs)
    o_acc = torch.empty((sq, hq, d), device=DEV)
    lse = torch.empty((hq, sq), device=DEV)
    st = rba.rba_fwd_step(a, q, qs, k, v, ks, o_acc, lse)
    if st == rba.RBA_STEP_EMPTY:
        assert not np.any(wdq) and not np.any(wdk) and not np.any(wdv)
        return
    delta = torch.empty((hq, sq), device=DEV)
    rba.rba_bwd_preprocess(o_acc, dO, delta)
    dq = torch.zeros((sq, hq, d), device=DEV)
    dk = torch.full((sk, hkv, d), float("nan"), device=DEV)
    dv = torch.full((sk, hkv, d), float("nan"), device=DEV)
    assert rba.rba_bwd_step(a, q, qs, k, v, ks, dO, lse, delta, dq, dk, dv) == rba.RBA_OK
    torch.cuda.synchronize()
    # A gradient element sums up to several hundred bf16-rounded products
    # here (few keys seen by many query rows and heads), so its size, and
    # the rounding error with it, can exceed 1: each gradient is compared
    # after dividing both sides by its RMS when that is above 1 (a tile
    # missed or counted twice still moves it by order 1).
    for name, got, want in (("dq", dq, wdq), ("dk", dk, wdk), ("dv", dv, wdv)):
        unit = max(1.0, float(np.sqrt(np.mean(want ** 2))))
        assert_close(got.cpu().numpy() / unit, want / unit, "bf16", name)


@pytest.mark.parametrize("seed", range(16))
def test_random_forward_step_workspace(seed):
    """Few query rows against 2K-5K keys, through rba_fwd_step_ws: whether or
    not the plan splits, the result matches the oracle, plain and merging."""
    rng, hq, hkv, d, mask, sq, sk, qsegs, ksegs, qpos, kpos, cu = _geometry(500 + seed, 160, 1)
    sk = int(rng.integers(2048, 5001))
    ksegs = _runs(rng, sk, int(rng.integers(0, 100)))
    qsegs = _runs(rng, sq, int(rng.integers(0, int(_pos(ksegs).max()) + 60)))
    qpos, kpos = _pos(qsegs), _pos(ksegs)
    if mask == 2:
        end = int(max(qpos.max(), kpos.max())) + 1
        cuts = np.sort(rng.choice(np.arange(1, end), int(rng.integers(1, 6)), replace=False))
        cu = np.concatenate([[0], cuts, [end]]).astype(np.int32)
    a, scale = _attn(hq, hkv, d, mask, cu)
    qs, ks = rba.make_segs(qsegs), rba.make_segs(ksegs)
    need = rba.rba_fwd_workspace_size(a, sq, qs, sk, ks)
    _say("random fwd ws", seed, dict(hq=hq, hkv=hkv, d=d, mask=mask, sq=sq, sk=sk, qsegs=qsegs, ksegs=ksegs,
                                     docs=None if cu is None else len(cu) - 1, workspace=need))
    qb, q64 = _bf16(rng, (sq, hq, d))
    kb, k64 = _bf16(rng, (sk, hkv, d))
    vb, v64 = _bf16(rng, (sk, hkv, d))
    q, k, v = (to_device(x, "bf16", DEV) for x in (qb, kb, vb))
    ws = torch.full((max(need, 16) // 4,), float("nan"), dtype=torch.float32, device=DEV)
    want_o, want_lse = oracle.attention(q64, k64, v64, qpos, kpos, mask, scale, cu)
    o = torch.full((sq, hq, d), float("nan"), device=DEV)
    lse = torch.full((hq, sq), float("nan"), device=DEV)
    st = rba.rba_fwd_step_ws(a, q, qs, k, v, ks, o, lse, False, None, rba.RBA_BF16, ws)
    torch.cuda.synchronize()
    if st == rba.RBA_STEP_EMPTY:
        assert np.isneginf(want_lse).all()
        return
    assert_lse(lse.cpu().numpy(), want_lse, "lse")
    assert_close(o.cpu().numpy(), want_o, "bf16", "o_part")
    o0 = rng.standard_normal((sq, hq, d)).astype(np.float32)
    l0 = rng.uniform(-3.0, 3.0, (hq, sq)).astype(np.float32)
    o_acc = torch.from_numpy(o0).to(DEV)
    lse_acc = torch.from_numpy(l0).to(DEV)
    rba.rba_fwd_step_ws(a, q, qs, k, v, ks, o_acc, lse_acc, True, None, rba.RBA_BF16, ws)
    torch.cuda.synchronize()
    mo, ml = oracle.merge(o0.astype(np.float64), l0.astype(np.float64), want_o, want_lse)
    assert_lse(lse_acc.cpu().numpy(), ml, "lse_acc")
    assert_close(o_acc.cpu().numpy(), mo, "bf16", "o_acc")


@pytest.mark.parametrize("seed", range(24))
def test_random_ring_replay(seed):
    """A ring of 2-5 KV chunks over random runs of one position range, taken
    in a random order: the merged forward (running O and LSE, then the bf16
    output) against attention over all the keys, and the backward steps'
    dQ (accumulated over the ring) and per-chunk dK / dV against the whole
    gradient.  A chunk may be empty for the mask (nothing launched)."""
    rng = np.random.default_rng(20_000 + seed)
    hq, hkv = HEADS[int(rng.integers(0, len(HEADS)))]
    d = int(rng.choice([64, 128]))
    mask = int(rng.integers(0, 3))
    n_chunks = int(rng.integers(2, 6))
    span = int(rng.integers(64, 600))
    # cut [0, span) into runs and deal them out to the chunks (at most 8 runs each)
    n_runs = int(rng.integers(n_chunks, min(span, 8 * n_chunks) + 1))
    cuts = np.sort(rng.choice(np.arange(1, span), n_runs - 1, replace=False))
    bounds = np.concatenate([[0], cuts, [span]])
    owner = np.concatenate([rng.permutation(n_chunks), rng.integers(0, n_chunks, n_runs - n_chunks)])
    chunks = [[(int(bounds[i]), int(bounds[i + 1] - bounds[i]))
               for i in range(n_runs) if owner[i] == c] for c in range(n_chunks)]
    sq = int(rng.integers(1, 201))
    qsegs = _runs(rng, sq, int(rng.integers(0, span)))
    qpos = _pos(qsegs)
    cu = None
    if mask == 2:
        end = int(max(qpos.max(), span - 1)) + 1
        n_cut = int(rng.integers(0, min(6, end - 1) + 1))
        cut = np.sort(rng.choice(np.arange(1, end), n_cut, replace=False)) if n_cut else np.array([], int)
        cu = np.concatenate([[0], cut, [end]]).astype(np.int32)
    order = [int(c) for c in rng.permutation(n_chunks)]
    _say("random ring", seed, dict(hq=hq, hkv=hkv, d=d, mask=mask, sq=sq, qsegs=qsegs, chunks=chunks,
                                   order=order, docs=None if cu is None else len(cu) - 1))
    a, scale = _attn(hq, hkv, d, mask, cu)
    qb, q64 = _bf16(rng, (sq, hq, d))
    dob, do64 = _bf16(rng, (sq, hq, d))
    ks_b, ks_64, vs_b, vs_64 = [], [], [], []
    for c in range(n_chunks):
        n = sum(l for _, l in chunks[c])
        kb, k64 = _bf16(rng, (n, hkv, d))
        vb, v64 = _bf16(rng, (n, hkv, d))
        ks_b.append(kb); ks_64.append(k64); vs_b.append(vb); vs_64.append(v64)
    kpos_all = np.concatenate([np.concatenate([s + np.arange(l) for s, l in ch]) for ch in chunks])
    k_all, v_all = np.concatenate(ks_64), np.concatenate(vs_64)
    want_o, want_lse = oracle.attention(q64, k_all, v_all, qpos, kpos_all, mask, scale, cu)
    wdq, wdk, wdv, _, _, _ = oracle.attention_backward(q64, k_all, v_all, do64, qpos, kpos_all, mask, scale, cu)

    q, dO = to_device(qb, "bf16", DEV), to_device(dob, "bf16", DEV)
    qs = rba.make_segs(qsegs)
    kd = [to_device(x, "bf16", DEV) for x in ks_b]
    vd = [to_device(x, "bf16", DEV) for x in vs_b]
    kss = [rba.make_segs(ch) for ch in chunks]
    o_acc = torch.zeros((sq, hq, d), device=DEV)
    lse_acc = torch.full((hq, sq), float("-inf"), device=DEV)
    for c in order:
        rba.rba_fwd_step_acc(a, q, qs, kd[c], vd[c], kss[c], o_acc, lse_acc)
    o_fin = torch.full((sq, hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    rba.rba_merge(o_acc, lse_acc, None, None, o_fin, rba.RBA_BF16)
    torch.cuda.synchronize()
    assert_lse(lse_acc.cpu().numpy(), want_lse, "lse_acc")
    assert_close(o_acc.cpu().numpy(), want_o, "bf16", "o_acc")
    assert_close(o_fin.float().cpu().numpy(), want_o, "bf16", "o_final")

    delta = torch.empty((hq, sq), device=DEV)
    rba.rba_bwd_preprocess(o_acc, dO, delta)
    dq = torch.zeros((sq, hq, d), device=DEV)
    dk_parts, dv_parts = {}, {}
    for c in order:
        n = kd[c].shape[0]
        dk = torch.zeros((n, hkv, d), device=DEV)
        dv = torch.zeros((n, hkv, d), device=DEV)
        rba.rba_bwd_step(a, q, qs, kd[c], vd[c], kss[c], dO, lse_acc, delta, dq, dk, dv)
        dk_parts[c], dv_parts[c] = dk, dv
    torch.cuda.synchronize()
    got_dk = np.concatenate([dk_parts[c].cpu().numpy() for c in range(n_chunks)])
    got_dv = np.concatenate([dv_parts[c].cpu().numpy() for c in range(n_chunks)])
    # gradients at unit scale, as in test_random_backward_step
    for name, got, want in (("dq", dq.cpu().numpy(), wdq), ("dk", got_dk, wdk), ("dv", got_dv, wdv)):
        unit = max(1.0, float(np.sqrt(np.mean(want ** 2))))
        assert_close(got / unit, want / unit, "bf16", name)
