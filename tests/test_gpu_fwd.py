"""GPU parity of the forward step and the merge against the fp64 oracle.

Each test prints its case before touching the GPU.  Small cases compare every
element of a step's partial (O, LSE) with the oracle restricted to the step's
keys; ring replays compare the merged output with unchunked attention; the
full-size workloads compare sampled rows."""
import numpy as np
import pytest
import torch

import oracle
from ring_sequence_parallelism_amd import rba
from ring_sequence_parallelism_amd import workloads as W
from ring_sequence_parallelism_amd.ring import RingReplay, ring_order, to_device

from _gpu_util import (BF16_MAX, BF16_MEAN, assert_close, assert_lse, chunk_positions, cu_or_none, full_kv_f64,
                       oracle_attention_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


def _segs_for(rng, rows, nseg, gap_max=40, base=0):
    nseg = max(1, min(nseg, rows))
    cuts = np.sort(rng.choice(np.arange(1, rows), nseg - 1, replace=False)) if nseg > 1 else np.array([], int)
    lens = np.diff(np.concatenate([[0], cuts, [rows]])).astype(int)
    order = rng.permutation(nseg)
    starts = {}
    p = base
    for i in order:
        p += int(rng.integers(0, gap_max))
        starts[i] = p
        p += int(lens[i])
    return [(starts[i], int(lens[i])) for i in range(nseg)]


def _pos(segs):
    """Positions of (start, length[, stride]) runs, in row order."""
    return np.concatenate([g[0] + (g[2] if len(g) > 2 else 1) * np.arange(g[1]) for g in segs])


def _rand_inputs(rng, n, h, d, dtype):
    x = rng.standard_normal((n, h, d)).astype(np.float32)
    if dtype == "bf16":
        bits = W.f32_to_bf16_bits(x)
        return bits, W.bf16_bits_to_f32(bits).astype(np.float64)
    return x, x.astype(np.float64)


def run_step(rng, sq, sk, hq, hkv, d, mask, dtype, qsegs, ksegs, cu=None):
    qb, q64 = _rand_inputs(rng, sq, hq, d, dtype)
    kb, k64 = _rand_inputs(rng, sk, hkv, d, dtype)
    vb, v64 = _rand_inputs(rng, sk, hkv, d, dtype)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    cu_dev = None if cu is None else torch.from_numpy(cu.astype(np.int32)).to(DEV)
    a = rba.attn_params(hq, hkv, d, scale, rba.RBA_BF16 if dtype == "bf16" else rba.RBA_F32, mask,
                        cu_dev, cu)
    q, k, v = (to_device(x, dtype, DEV) for x in (qb, kb, vb))
    o = torch.full((sq, hq, d), float("nan"), device=DEV)
    lse = torch.full((hq, sq), float("nan"), device=DEV)
    st = rba.rba_fwd_step(a, q, rba.make_segs(qsegs), k, v, rba.make_segs(ksegs), o, lse)
    torch.cuda.synchronize()
    want_o, want_lse = oracle.attention(q64, k64, v64, _pos(qsegs), _pos(ksegs), mask, scale, cu)
    return st, o.cpu().numpy(), lse.cpu().numpy(), want_o, want_lse


CASES = [
    # sq, sk, hq, hkv, d, n_qseg, n_kseg
    (200, 333, 8, 2, 128, 1, 1),
    (77, 129, 4, 4, 64, 2, 3),
    (300, 130, 6, 2, 128, 4, 2),
    (1, 77, 3, 1, 128, 1, 5),
    (96, 1, 4, 1, 64, 3, 1),
    (64, 64, 4, 2, 128, 16, 16),
    (513, 257, 2, 2, 64, 7, 9),
]


@pytest.mark.parametrize("mask", [0, 1, 2])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_step_bf16_small(case, mask):
    sq, sk, hq, hkv, d, nqs, nks = case
    _say("fwd bf16", case, "mask", mask)
    rng = np.random.default_rng(hash((case, mask)) % 2**32)
    # queries and keys interleave in position so every mask has mixed tiles
    qsegs = _segs_for(rng, sq, nqs)
    ksegs = _segs_for(rng, sk, nks, base=int(rng.integers(0, 60)))
    end = int(max(_pos(qsegs).max(), _pos(ksegs).max())) + 1
    cu = None
    if mask == 2:
        cuts = np.sort(rng.choice(np.arange(1, end), min(6, end - 1), replace=False))
        cu = np.concatenate([[0], cuts, [end]]).astype(np.int32)
    # keys may overlap queries' positions: the two chunks are different tensors
    st, o, lse, wo, wl = run_step(rng, sq, sk, hq, hkv, d, mask, "bf16", qsegs, ksegs, cu)
    if st == rba.RBA_STEP_EMPTY:
        assert np.isneginf(wl).all()
        return
    assert_lse(lse, wl, "lse")
    assert_close(o, wo, "bf16", "o_part")
    assert np.all(o[np.isneginf(wl).T] == 0)


@pytest.mark.parametrize("mask", [0, 1])
@pytest.mark.parametrize("d", [64, 128])
def test_step_f32_small(mask, d):
    _say("fwd f32 d", d, "mask", mask)
    rng = np.random.default_rng(5 + d + mask)
    qsegs = [(100, 150), (0, 50)]
    ksegs = [(40, 170), (300, 20)]
    st, o, lse, wo, wl = run_step(rng, 200, 190, 4, 2, d, mask, "f32", qsegs, ksegs)
    assert st == rba.RBA_OK
    assert_lse(lse, wl, "lse")
    assert_close(o, wo, "f32", "o_part")


def test_step_fully_masked_rows():
    _say("fwd rows without keys")
    rng = np.random.default_rng(3)
    # keys at positions 100..199; queries 50..149: the first 50 rows see nothing
    st, o, lse, wo, wl = run_step(rng, 100, 100, 4, 1, 128, 1, "bf16", [(50, 100)], [(100, 100)])
    assert st == rba.RBA_OK
    assert np.isneginf(lse[:, :50]).all() and np.all(o[:50] == 0)
    assert_lse(lse, wl, "lse")
    assert_close(o, wo, "bf16", "o_part")


def _run_scaled_keys(sq, sk, hq, hkv, d, mask, qsegs, ksegs, row_scale, seed):
    rng = np.random.default_rng(seed)
    qb, q64 = _rand_inputs(rng, sq, hq, d, "bf16")
    k = rng.standard_normal((sk, hkv, d)).astype(np.float32) * row_scale[:, None, None].astype(np.float32)
    kb = W.f32_to_bf16_bits(k)
    k64 = W.bf16_bits_to_f32(kb).astype(np.float64)
    vb, v64 = _rand_inputs(rng, sk, hkv, d, "bf16")
    scale = float(np.float32(1.0 / np.sqrt(d)))
    a = rba.attn_params(hq, hkv, d, scale, rba.RBA_BF16, mask)
    q, kd, v = (to_device(x, "bf16", DEV) for x in (qb, kb, vb))
    o = torch.full((sq, hq, d), float("nan"), device=DEV)
    lse = torch.full((hq, sq), float("nan"), device=DEV)
    st = rba.rba_fwd_step(a, q, rba.make_segs(qsegs), kd, v, rba.make_segs(ksegs), o, lse)
    torch.cuda.synchronize()
    wo, wl = oracle.attention(q64, k64, v64, _pos(qsegs), _pos(ksegs), mask, scale)
    return st, o.cpu().numpy(), lse.cpu().numpy(), wo, wl


@pytest.mark.parametrize("pattern", ["jump", "ramp", "drop"])
@pytest.mark.parametrize("mask", [0, 1])
def test_step_score_range(pattern, mask):
    # Key norms that change along the chunk move the row maximum by far more
    # than 2^16 between key tiles (jump, ramp) or leave later tiles far below
    # it (drop): exercises the lazy running maximum (moved only when a tile's
    # maximum exceeds it by more than 2^8) and the rescale of O and l.
    sq, sk, hq, hkv, d = 96, 448, 4, 2, 128
    _say("fwd score range", pattern, "mask", mask)
    rows = np.arange(sk)
    if pattern == "jump":
        row_scale = np.where(rows < 64, 0.05, 12.0)
    elif pattern == "ramp":
        row_scale = 0.05 + 20.0 * rows / sk
    else:
        row_scale = np.where(rows < 128, 12.0, 0.05)
    # queries after every key: every tile is full under the causal mask too
    st, o, lse, wo, wl = _run_scaled_keys(sq, sk, hq, hkv, d, mask, [(1000, sq)], [(0, sk)], row_scale,
                                          11 + mask + 3 * len(pattern))
    assert st == rba.RBA_OK
    assert_lse(lse, wl, "lse")
    assert_close(o, wo, "bf16", "o_part")


def test_step_deterministic():
    _say("fwd determinism")
    rng = np.random.default_rng(8)
    sq, sk, hq, hkv, d = 300, 500, 8, 2, 128
    qb, _ = _rand_inputs(rng, sq, hq, d, "bf16")
    kb, _ = _rand_inputs(rng, sk, hkv, d, "bf16")
    q, k, v = (to_device(x, "bf16", DEV) for x in (qb, kb, kb))
    a = rba.attn_params(hq, hkv, d, 0.088, rba.RBA_BF16, rba.RBA_MASK_CAUSAL)
    outs = []
    for _ in range(2):
        o = torch.empty((sq, hq, d), device=DEV)
        l = torch.empty((hq, sq), device=DEV)
        rba.rba_fwd_step(a, q, rba.make_segs([(400, 300)]), k, v, rba.make_segs([(0, 500)]), o, l)
        outs.append((o.cpu(), l.cpu()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


# ---------------------------------------------------------------------------
# merge

@pytest.mark.parametrize("d", [4, 36, 64, 128, 260, 1024])
def test_merge_kernel(d):
    # d = 36 and 260: pairs of 9 and 65 vectors, whose threads the merge's
    # thread map still keeps inside one wave (16 and 64 lanes per pair)
    _say("merge d", d)
    rng = np.random.default_rng(d)
    sq, hq = 333, 5
    oa, ob = rng.standard_normal((2, sq, hq, d)).astype(np.float32)
    la, lb = (rng.standard_normal((2, hq, sq)) * 3).astype(np.float32)
    la[0, :10] = -np.inf
    lb[0, 5:15] = -np.inf
    lb[1, 20:30] = -np.inf
    oa[:10, 0] = 0
    ob[5:15, 0] = 0
    ob[20:30, 1] = 0
    want_o, want_l = oracle.merge(oa, la, ob, lb)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    o_acc, l_acc, o_part, l_part = t(oa), t(la), t(ob), t(lb)
    fin = torch.empty((sq, hq, d), dtype=torch.bfloat16, device=DEV)
    rba.rba_merge(o_acc, l_acc, o_part, l_part, fin, rba.RBA_BF16)
    torch.cuda.synchronize()
    assert_close(o_acc.cpu().numpy(), want_o, "f32", "merged o")
    assert_lse(l_acc.cpu().numpy(), want_l, "merged lse")
    assert_close(fin.float().cpu().numpy(), want_o, "bf16", "bf16 final")
    # finalise only: fp32 copy
    fin32 = torch.empty((sq, hq, d), device=DEV)
    rba.rba_merge(o_acc, l_acc, None, None, fin32, rba.RBA_F32)
    torch.cuda.synchronize()
    assert torch.equal(fin32, o_acc)


# ---------------------------------------------------------------------------
# ring replays

def _check_replay(w, rank, rows=None, heads=None):
    rr = RingReplay(w, rank, DEV)
    rr.forward()
    torch.cuda.synchronize()
    qpos = chunk_positions(w, rr.r)
    q64 = W.to_f64(W.gen_rank_chunk(w, W.T_Q, rr.r), w.dtype)
    k64, v64 = full_kv_f64(w)
    if rows is not None:
        qpos, q64 = qpos[rows], q64[rows]
    want_o, want_l = oracle_attention_rows(q64, k64, v64, qpos, w.mask, w.scale, cu_or_none(w),
                                           block=64 if rows is None else 8)
    got = rr.o_final.float().cpu().numpy()
    got_l = rr.lse_acc.cpu().numpy()
    if rows is not None:
        got, got_l = got[rows], got_l[:, rows]
    cls = "bf16" if w.dtype == "bf16" else "f32"
    assert_lse(got_l, want_l, f"{w.name} lse")
    return assert_close(got, want_o, cls, f"{w.name} o")


def test_replay_c1_full():
    w = W.WORKLOADS["c1"]
    _say("replay", w.name)
    _check_replay(w, 0)


@pytest.mark.parametrize("rank", [0, 3, 7])
def test_replay_zigzag_scaled(rank):
    w = W.scaled_workload(W.WORKLOADS["c2"], 4096)
    _say("replay", w.name, "rank", rank)
    _check_replay(w, rank)


@pytest.mark.parametrize("rank", [2, 6])
def test_replay_zigzag_scaled_d64(rank):
    # head_dim 64 through the whole replay (merging epilogue included)
    w = W.scaled_workload(W.WORKLOADS["c2"], 4096, d=64, name="c2_s4096_d64")
    _say("replay", w.name, "rank", rank)
    _check_replay(w, rank)


@pytest.mark.parametrize("rank", [0, 9, 15])
def test_replay_packed_docs_scaled(rank):
    w = W.scaled_workload(W.WORKLOADS["c3"], 8192, hq=8, hkv=2)
    _say("replay", w.name, "rank", rank)
    _check_replay(w, rank)


def test_replay_c2_full():
    """The 32K causal zigzag workload: all 4096 rows of rank 3, all 32 heads,
    against unchunked attention over the whole sequence."""
    w = W.WORKLOADS["c2"]
    _say("replay full", w.name, "all rows")
    _check_replay(w, w.rank)


def test_replay_c3_full_all_ranks():
    """The 64K packed-document workload: every rank replays all 16 KV chunks
    (256 calls, the host skips the empty ones); the 16 ranks' outputs together
    are compared with the full 65536-row packed causal attention."""
    w = W.WORKLOADS["c3"]
    _say("replay full", w.name, "all 16 ranks")
    k64, v64 = full_kv_f64(w)
    cu = cu_or_none(w)
    shared = {"k": {j: to_device(W.gen_rank_chunk(w, W.T_K, j), w.dtype, DEV) for j in range(w.n_ranks)},
              "v": {j: to_device(W.gen_rank_chunk(w, W.T_V, j), w.dtype, DEV) for j in range(w.n_ranks)}}
    abs_sum, count, o_max, l_max, launched = 0.0, 0, 0.0, 0.0, 0
    for r in range(w.n_ranks):
        rr = RingReplay(w, r, DEV, kv=shared)
        launched += sum(s.status == rba.RBA_OK for s in rr.steps)
        rr.forward()
        torch.cuda.synchronize()
        got = rr.o_final.float().cpu().numpy().astype(np.float64)
        got_l = rr.lse_acc.cpu().numpy()
        qpos = chunk_positions(w, r)
        q64 = W.to_f64(W.gen_rank_chunk(w, W.T_Q, r), w.dtype)
        want_o, want_l = oracle_attention_rows(q64, k64, v64, qpos, w.mask, w.scale, cu)
        assert_lse(got_l, want_l, f"rank {r} lse")
        err = np.abs(got - want_o)
        assert np.isfinite(got).all(), f"rank {r}: non-finite output"
        abs_sum += float(err.sum())
        count += err.size
        o_max = max(o_max, float(err.max()))
        l_max = max(l_max, float(np.abs(got_l - want_l).max()))
        del rr
    mean = abs_sum / count
    print(f"[c3] {launched} non-empty calls of 256; o max {o_max:.3g} mean {mean:.3g}; lse max {l_max:.3g}",
          flush=True)
    assert o_max <= BF16_MAX and mean <= BF16_MEAN, (o_max, mean)


def test_replay_c4_full_sampled_rows():
    """The 512K causal zigzag workload: the 256 sampled query rows the
    workload names (first and last row of each piece, the rest drawn
    uniformly), all 32 heads, in fp64."""
    w = W.WORKLOADS["c4"]
    _say("replay full", w.name, "256 sampled rows")
    rows = W.gen_sampled_rows(w, 256, w.chunk_len)
    assert rows.size == 256
    _check_replay(w, w.rank, rows)


# ---------------------------------------------------------------------------
# replays that must fail, and replays that must pass, the comparison

def _teeth_workload():
    return W.scaled_workload(W.WORKLOADS["c2"], 4096, hq=8, hkv=2, name="c2_s4096_teeth")


def _replay_error(w, rank, order):
    rr = RingReplay(w, rank, DEV, order=order)
    rr.forward()
    torch.cuda.synchronize()
    q64 = W.to_f64(W.gen_rank_chunk(w, W.T_Q, rank), w.dtype)
    k64, v64 = full_kv_f64(w)
    want_o, want_l = oracle_attention_rows(q64, k64, v64, chunk_positions(w, rank), w.mask, w.scale)
    return rr, rr.o_final.float().cpu().numpy(), rr.lse_acc.cpu().numpy(), want_o, want_l


@pytest.mark.parametrize("change", ["drop", "duplicate"])
def test_replay_with_a_missing_or_repeated_step_fails(change):
    """A ring that skips one KV chunk, or visits one twice, is not exact
    attention: the comparison that the true ring passes must reject it."""
    w = _teeth_workload()
    rank = 5
    order = ring_order(rank, w.n_ranks)
    order = order[:3] + order[4:] if change == "drop" else order + [order[2]]
    _say("replay teeth", change, order)
    _, got, got_l, want_o, want_l = _replay_error(w, rank, order)
    with pytest.raises(AssertionError):
        assert_lse(got_l, want_l, "lse")
        assert_close(got, want_o, "bf16", "o")


@pytest.mark.parametrize("seed", [0, 1])
def test_replay_permuted_order_passes(seed):
    """The merge is order-free: the KV chunks in any order give the same
    attention (to rounding)."""
    w = _teeth_workload()
    rank = 2
    order = list(np.random.default_rng(seed).permutation(ring_order(rank, w.n_ranks)))
    _say("replay permuted", order)
    _, got, got_l, want_o, want_l = _replay_error(w, rank, order)
    assert_lse(got_l, want_l, "lse")
    assert_close(got, want_o, "bf16", "o")


@pytest.mark.parametrize("k", [1, 4, 7])
def test_replay_checkpoint_resume(k):
    """Stop after k steps, copy the running (O, LSE) to host memory, restore it
    into fresh buffers and finish the remaining steps: the result is bit for
    bit that of the uninterrupted replay."""
    w = _teeth_workload()
    rank = 6
    order = ring_order(rank, w.n_ranks)
    _say("replay checkpoint after", k, "steps")
    full = RingReplay(w, rank, DEV)
    full.forward()
    head = RingReplay(w, rank, DEV, order=order[:k])
    head.forward()
    torch.cuda.synchronize()
    saved_o, saved_l = head.o_acc.cpu().clone(), head.lse_acc.cpu().clone()
    del head
    tail = RingReplay(w, rank, DEV, order=order[k:])
    tail.o_acc.copy_(saved_o.to(DEV))
    tail.lse_acc.copy_(saved_l.to(DEV))
    tail.forward(resume=True)
    torch.cuda.synchronize()
    assert torch.equal(tail.o_acc, full.o_acc)
    assert torch.equal(tail.lse_acc, full.lse_acc)
    assert torch.equal(tail.o_final, full.o_final)


def test_per_step_partials_c2():
    """Each step's partial equals the oracle restricted to that KV chunk."""
    w = W.WORKLOADS["c2"]
    _say("per-step partials", w.name)
    rr = RingReplay(w, None, DEV)
    rows = W.gen_sampled_rows(w, 64, w.chunk_len)
    qpos = chunk_positions(w, rr.r)[rows]
    q64 = W.to_f64(W.gen_rank_chunk(w, W.T_Q, rr.r), w.dtype)[rows]
    for i in (0, 3, 4):
        s = rr.steps[i]
        rr.fwd_step(i, into_acc=False)
        torch.cuda.synchronize()
        k64 = W.to_f64(W.gen_rank_chunk(w, W.T_K, s.src), w.dtype)
        v64 = W.to_f64(W.gen_rank_chunk(w, W.T_V, s.src), w.dtype)
        kpos = chunk_positions(w, s.src)
        wo, wl = oracle.attention(q64, k64, v64, qpos, kpos, w.mask, w.scale)
        assert_lse(rr.lse_part.cpu().numpy()[:, rows], wl, f"step {i} lse")
        assert_close(rr.o_part.cpu().numpy()[rows], wo, "bf16", f"step {i} o")


# ---------------------------------------------------------------------------
# forward step with the merge in its epilogue (rba_fwd_step_acc)

@pytest.mark.parametrize("final", [None, "bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_fwd_step_acc_equals_step_plus_merge(final, d):
    """rba_fwd_step_acc gives what rba_fwd_step followed by rba_merge gives,
    including accumulator rows with LSE = -inf and step rows without keys."""
    _say("fwd step acc", d, final)
    rng = np.random.default_rng(40 + d)
    sq, sk, hq, hkv = 150, 200, 4, 2
    qb, _ = _rand_inputs(rng, sq, hq, d, "bf16")
    kb, _ = _rand_inputs(rng, sk, hkv, d, "bf16")
    vb, _ = _rand_inputs(rng, sk, hkv, d, "bf16")
    q, k, v = (to_device(x, "bf16", DEV) for x in (qb, kb, vb))
    a = rba.attn_params(hq, hkv, d, float(np.float32(1 / np.sqrt(d))), rba.RBA_BF16, rba.RBA_MASK_CAUSAL)
    qs, ks = rba.make_segs([(100, sq)]), rba.make_segs([(120, sk)])    # rows 0..19 (positions 100..119) see no key
    acc0 = torch.from_numpy(rng.standard_normal((sq, hq, d)).astype(np.float32)).to(DEV)
    lse0 = torch.from_numpy((rng.standard_normal((hq, sq)) * 2).astype(np.float32)).to(DEV)
    lse0[0, 0:30] = float("-inf")                                       # rows 0..19 empty on both sides
    acc0[0:30, 0] = 0
    # reference: partial, then the merge kernel
    o_part = torch.empty((sq, hq, d), device=DEV)
    l_part = torch.empty((hq, sq), device=DEV)
    assert rba.rba_fwd_step(a, q, qs, k, v, ks, o_part, l_part) == rba.RBA_OK
    o_ref, l_ref = acc0.clone(), lse0.clone()
    fdt = rba.RBA_BF16 if final != "f32" else rba.RBA_F32
    tdt = torch.bfloat16 if final != "f32" else torch.float32
    f_ref = torch.full((sq, hq, d), 7.0, dtype=tdt, device=DEV) if final else None
    rba.rba_merge(o_ref, l_ref, o_part, l_part, f_ref, fdt)
    # fused
    o_acc, l_acc = acc0.clone(), lse0.clone()
    f_acc = torch.full((sq, hq, d), 7.0, dtype=tdt, device=DEV) if final else None
    assert rba.rba_fwd_step_acc(a, q, qs, k, v, ks, o_acc, l_acc, f_acc, fdt) == rba.RBA_OK
    torch.cuda.synchronize()
    assert torch.allclose(o_acc, o_ref, rtol=2e-6, atol=2e-6)
    assert torch.equal(torch.isneginf(l_acc), torch.isneginf(l_ref))
    fin = ~torch.isneginf(l_ref)
    assert torch.allclose(l_acc[fin], l_ref[fin], rtol=1e-6, atol=1e-6)
    assert (o_acc[0:20, 0] == 0).all()                    # empty in both: (0, -inf)
    # an empty step row merges as the identity, bit for bit
    assert torch.equal(o_acc[0:20, 1:], acc0[0:20, 1:])
    assert torch.equal(l_acc[1:, 0:20], lse0[1:, 0:20])
    assert torch.isneginf(l_acc[0, 0:20]).all()
    assert torch.allclose(o_acc[20:30, 0], o_part[20:30, 0], rtol=1e-6, atol=1e-6)   # empty accumulator
    if final:
        assert torch.allclose(f_acc.float(), f_ref.float(), rtol=1e-2 if final == "bf16" else 2e-6, atol=2e-6)
    # an empty step changes nothing and writes no final output
    before_o, before_l = o_acc.clone(), l_acc.clone()
    f2 = torch.full((sq, hq, d), 7.0, dtype=tdt, device=DEV) if final else None
    st = rba.rba_fwd_step_acc(a, q, qs, k, v, rba.make_segs([(5000, sk)]), o_acc, l_acc, f2, fdt)
    torch.cuda.synchronize()
    assert st == rba.RBA_STEP_EMPTY
    assert torch.equal(o_acc, before_o) and torch.equal(l_acc, before_l)
    if final:
        assert (f2.float() == 7.0).all()


@pytest.mark.parametrize("final", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_fwd_step_acc_final_rows_without_keys(final, d):
    """A merging step that writes the final output, in which whole row groups
    see no key: their final output is the running result converted (bit for
    bit), their running result and LSE are left as they were, and the rest
    matches rba_fwd_step followed by rba_merge."""
    _say("fwd step acc final copy", d, final)
    rng = np.random.default_rng(70 + d)
    sq, sk, hq, hkv = 230, 180, 8, 2
    qb, _ = _rand_inputs(rng, sq, hq, d, "bf16")
    kb, _ = _rand_inputs(rng, sk, hkv, d, "bf16")
    vb, _ = _rand_inputs(rng, sk, hkv, d, "bf16")
    q, k, v = (to_device(x, "bf16", DEV) for x in (qb, kb, vb))
    a = rba.attn_params(hq, hkv, d, float(np.float32(1 / np.sqrt(d))), rba.RBA_BF16, rba.RBA_MASK_CAUSAL)
    qs, ks = rba.make_segs([(0, sq)]), rba.make_segs([(110, sk)])      # rows 0..109 see no key
    acc0 = torch.from_numpy(rng.standard_normal((sq, hq, d)).astype(np.float32)).to(DEV)
    lse0 = torch.from_numpy((rng.standard_normal((hq, sq)) * 2).astype(np.float32)).to(DEV)
    lse0[1, 0:40] = float("-inf")
    acc0[0:40, 1] = 0
    fdt, tdt = (rba.RBA_BF16, torch.bfloat16) if final == "bf16" else (rba.RBA_F32, torch.float32)
    o_part = torch.empty((sq, hq, d), device=DEV)
    l_part = torch.empty((hq, sq), device=DEV)
    assert rba.rba_fwd_step(a, q, qs, k, v, ks, o_part, l_part) == rba.RBA_OK
    o_ref, l_ref = acc0.clone(), lse0.clone()
    f_ref = torch.full((sq, hq, d), 7.0, dtype=tdt, device=DEV)
    rba.rba_merge(o_ref, l_ref, o_part, l_part, f_ref, fdt)
    o_acc, l_acc = acc0.clone(), lse0.clone()
    f_acc = torch.full((sq, hq, d), 7.0, dtype=tdt, device=DEV)
    assert rba.rba_fwd_step_acc(a, q, qs, k, v, ks, o_acc, l_acc, f_acc, fdt) == rba.RBA_OK
    torch.cuda.synchronize()
    assert torch.equal(o_acc[:110], acc0[:110]) and torch.equal(l_acc[:, :110], lse0[:, :110])
    assert torch.equal(f_acc[:110], acc0[:110].to(tdt))
    assert torch.allclose(o_acc, o_ref, rtol=2e-6, atol=2e-6)
    fin = ~torch.isneginf(l_ref)
    assert torch.equal(torch.isneginf(l_acc), torch.isneginf(l_ref))
    assert torch.allclose(l_acc[fin], l_ref[fin], rtol=1e-6, atol=1e-6)
    assert torch.allclose(f_acc.float(), f_ref.float(), rtol=1e-2 if final == "bf16" else 2e-6, atol=2e-6)


@pytest.mark.parametrize("fused", [True, False])
def test_replay_merge_paths_agree(fused):
    """The replay through rba_fwd_step_acc and through o_part + rba_merge both
    match unchunked attention."""
    w = W.scaled_workload(W.WORKLOADS["c2"], 4096, hq=8, hkv=2)
    _say("replay merge path", "fused" if fused else "separate")
    rr = RingReplay(w, 5, DEV)
    rr.forward(fused_merge=fused)
    torch.cuda.synchronize()
    qpos = chunk_positions(w, 5)
    q64 = W.to_f64(W.gen_rank_chunk(w, W.T_Q, 5), w.dtype)
    k64, v64 = full_kv_f64(w)
    want_o, want_l = oracle.attention(q64, k64, v64, qpos, np.arange(w.seq), w.mask, w.scale)
    assert_lse(rr.lse_acc.cpu().numpy(), want_l, "lse")
    assert_close(rr.o_final.float().cpu().numpy(), want_o, "bf16", "o")


# ---------------------------------------------------------------------------
# striped layout (strided position segments)

def _striped(w):
    import dataclasses
    return dataclasses.replace(w, layout="striped", name=w.name + "_striped")


@pytest.mark.parametrize("rank", [0, 5])
def test_replay_striped_scaled(rank):
    w = _striped(W.scaled_workload(W.WORKLOADS["c2"], 4096, hq=8, hkv=2))
    _say("replay", w.name, "rank", rank)
    _check_replay(w, rank)


def test_replay_striped_packed_docs_scaled():
    w = _striped(W.scaled_workload(W.WORKLOADS["c3"], 8192, hq=8, hkv=2))
    _say("replay", w.name, "rank", 7)
    _check_replay(w, 7)


@pytest.mark.parametrize("mask", [0, 1, 2])
@pytest.mark.parametrize("d", [64, 128])
def test_step_strided_segments(mask, d):
    """Mixed strided and unit-stride segments on both sides of one step."""
    _say("fwd strided step", d, "mask", mask)
    rng = np.random.default_rng(70 + 3 * d + mask)
    qsegs = [(3, 150, 5), (2000, 60, 1)]
    ksegs = [(1, 130, 5), (700, 70, 3), (1990, 33, 1)]
    end = 2100
    cu = None
    if mask == 2:
        cu = np.array([0, 250, 600, 1500, 1995, end], dtype=np.int32)
    sq, sk = sum(x[1] for x in qsegs), sum(x[1] for x in ksegs)
    st, o, lse, wo, wl = run_step(rng, sq, sk, 4, 2, d, mask, "bf16", qsegs, ksegs, cu)
    assert st == rba.RBA_OK
    assert_lse(lse, wl, "lse")
    assert_close(o, wo, "bf16", "o_part")


# Steps whose every visited key tile is full for every query row (tile-aligned
# KV segments wholly before the rows that see them, or no mask and whole
# tiles): the host launches the forward without tile classification or mask
# code.  Each case also gives the same KV positions split at a row that is
# not a tile boundary, which takes the general path; both must match the
# oracle, and each other bit for bit (the arithmetic is the same).
FULL_CASES = [
    # mask, d, q segments, k segments, the same keys split off a tile boundary
    (1, 128, [(4096, 256)], [(0, 512)], [(0, 100), (100, 412)]),
    (1, 128, [(1024, 128), (3072, 128)], [(512, 256), (2048, 256)], [(512, 37), (549, 219), (2048, 256)]),
    (1, 64, [(1024, 128), (3072, 128)], [(512, 256), (2048, 256)], [(512, 256), (2048, 70), (2118, 186)]),
    (1, 128, [(2048, 64, 8), (4000, 96)], [(1, 64, 4), (300, 128)], [(1, 30, 4), (121, 34, 4), (300, 128)]),
    (0, 128, [(0, 100)], [(5000, 128), (0, 64)], None),
]


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4)])
@pytest.mark.parametrize("case", FULL_CASES, ids=lambda c: f"m{c[0]}d{c[1]}k{len(c[3])}")
def test_step_full_tiles_path(case, hq, hkv):
    mask, d, qsegs, ksegs, ksplit = case
    _say("fwd full-tile path", case, hq, hkv)
    sq, sk = sum(x[1] for x in qsegs), sum(x[1] for x in ksegs)
    seed = 90 + d + 7 * mask + hq
    st, o, lse, wo, wl = run_step(np.random.default_rng(seed), sq, sk, hq, hkv, d, mask, "bf16", qsegs, ksegs)
    assert st == rba.RBA_OK
    assert_lse(lse, wl, "lse")
    assert_close(o, wo, "bf16", "o_part")
    if ksplit is None:
        return
    assert sum(x[1] for x in ksplit) == sk and np.array_equal(_pos(ksplit), _pos(ksegs))
    st2, o2, lse2, _, _ = run_step(np.random.default_rng(seed), sq, sk, hq, hkv, d, mask, "bf16", qsegs, ksplit)
    assert st2 == rba.RBA_OK
    assert np.array_equal(o2, o) and np.array_equal(lse2, lse)
