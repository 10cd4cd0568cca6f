"""GPU parity of the forward step with a workspace (rba_fwd_step_ws), whose
launches with few rows of work split each row group's key tiles over
several workgroups and merge the items' partials in a second launch (and
launches of between one and two rounds of workgroups halve their heaviest
row groups).

Each case checks that the step does split (rba_fwd_workspace_size > 0),
compares the result with the fp64 oracle at the forward's tolerances, and
with the unsplit entry point on the same inputs.  The split items sum P in
another order and against their own running maxima (so P is rounded to bf16
from other references), so the two agree to rounding, not bit for bit; a
key tile skipped or counted twice would move LSE by about 1e-2 at these
sizes (and O by about 1e-3 on average), far above what the comparison
allows (LSE within 1e-4; O within 2e-3, and 1e-4 on average)."""
import numpy as np
import pytest
import torch

import oracle
from ring_sequence_parallelism_amd import rba
from ring_sequence_parallelism_amd import workloads as W
from ring_sequence_parallelism_amd.ring import RingReplay, to_device

from _gpu_util import (BF16_MAX, BF16_MEAN, assert_close, assert_lse, chunk_positions, cu_or_none, full_kv_f64,
                       oracle_attention_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


def _pos(segs):
    return np.concatenate([g[0] + (g[2] if len(g) > 2 else 1) * np.arange(g[1]) for g in segs])


def _bf16(rng, shape, scale=1.0):
    bits = W.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))
    return bits, W.bf16_bits_to_f32(bits).astype(np.float64)


def _close_to_unsplit(o, o_ref):
    diff = (o - o_ref).abs()
    assert float(diff.max()) <= 2e-3 and float(diff.mean()) <= 1e-4, (float(diff.max()), float(diff.mean()))


def _workspace(a, sq, qs, sk, ks):
    need = rba.rba_fwd_workspace_size(a, sq, qs, sk, ks)
    return need, torch.full((max(need, 16) // 4,), float("nan"), dtype=torch.float32, device=DEV)


# sq, sk, hq, hkv, d, q segments, k segments, mask, document starts (mask 2)
SPLIT_CASES = [
    (64, 4096, 8, 2, 128, [(5000, 64)], [(0, 4096)], 1, None),            # every tile full, 64 tiles per row group
    (100, 3000, 32, 8, 128, [(2990, 100)], [(0, 3000)], 1, None),         # ragged last tile, diagonal rows
    (40, 2500, 4, 4, 64, [(0, 40)], [(100, 2500)], 0, None),              # no mask
    (96, 4096, 32, 8, 128, [(9000, 96)], [(0, 1000), (2000, 1500), (6000, 1596)], 1, None),   # items cross segments
    (150, 4096, 32, 8, 128, [(4096, 150)], [(0, 4096)], 2, [0, 700, 1000, 4180, 8192]),   # documents
    (33, 2048, 16, 4, 64, [(3000, 10, 7), (2100, 23)], [(0, 2048)], 1, None),   # strided query rows
    (2432, 4096, 32, 8, 64, [(5000, 2432)], [(0, 4096)], 1, None),   # 608 workgroups: the 12 heaviest row groups halved
]


@pytest.mark.parametrize("accumulate", [False, True])
@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: f"{c[0]}x{c[1]}h{c[2]}d{c[4]}m{c[7]}s{len(c[6])}")
def test_fwd_step_ws_split(case, accumulate):
    sq, sk, hq, hkv, d, qsegs, ksegs, mask, cu = case
    _say("fwd ws split", case, "acc" if accumulate else "part")
    rng = np.random.default_rng(sq * 31 + sk + mask)
    qb, q64 = _bf16(rng, (sq, hq, d))
    kb, k64 = _bf16(rng, (sk, hkv, d))
    vb, v64 = _bf16(rng, (sk, hkv, d))
    scale = float(np.float32(1 / np.sqrt(d)))
    cu_np = None if cu is None else np.asarray(cu, dtype=np.int32)
    cu_dev = None if cu is None else torch.from_numpy(cu_np).to(DEV)
    a = rba.attn_params(hq, hkv, d, scale, rba.RBA_BF16, mask, cu_dev, cu_np)
    q, k, v = (to_device(x, "bf16", DEV) for x in (qb, kb, vb))
    qs, ks = rba.make_segs(qsegs), rba.make_segs(ksegs)
    need, ws = _workspace(a, sq, qs, sk, ks)
    assert 0 < need <= 32 << 20, need
    want_o, want_l = oracle.attention(q64, k64, v64, _pos(qsegs), _pos(ksegs), mask, scale, cu_np)
    if not accumulate:
        o = torch.full((sq, hq, d), float("nan"), device=DEV)
        lse = torch.full((hq, sq), float("nan"), device=DEV)
        assert rba.rba_fwd_step_ws(a, q, qs, k, v, ks, o, lse, False, None, rba.RBA_BF16, ws) == rba.RBA_OK
        o_ref = torch.full_like(o, float("nan"))
        l_ref = torch.full_like(lse, float("nan"))
        assert rba.rba_fwd_step(a, q, qs, k, v, ks, o_ref, l_ref) == rba.RBA_OK
        torch.cuda.synchronize()
        assert_lse(lse.cpu().numpy(), want_l, "lse")
        assert_close(o.cpu().numpy(), want_o, "bf16", "o_part")
        fin = ~torch.isneginf(l_ref)
        assert torch.equal(torch.isneginf(lse), ~fin)
        assert torch.allclose(lse[fin], l_ref[fin], rtol=0, atol=1e-4)
        _close_to_unsplit(o, o_ref)
        return
    # accumulate: a running result of random partials, merged and finalised
    acc0 = torch.from_numpy(rng.standard_normal((sq, hq, d)).astype(np.float32)).to(DEV)
    lse0 = torch.from_numpy((rng.standard_normal((hq, sq)) * 2).astype(np.float32)).to(DEV)
    lse0[0, :5] = float("-inf")
    acc0[:5, 0] = 0
    o, lse = acc0.clone(), lse0.clone()
    fin_bf16 = torch.full((sq, hq, d), 7.0, dtype=torch.bfloat16, device=DEV)
    assert rba.rba_fwd_step_ws(a, q, qs, k, v, ks, o, lse, True, fin_bf16, rba.RBA_BF16, ws) == rba.RBA_OK
    o_ref, l_ref = acc0.clone(), lse0.clone()
    fin_ref = torch.full_like(fin_bf16, 7.0)
    assert rba.rba_fwd_step_acc(a, q, qs, k, v, ks, o_ref, l_ref, fin_ref, rba.RBA_BF16) == rba.RBA_OK
    torch.cuda.synchronize()
    # against the oracle: merge of the random running result with the step's attention
    wo, wl = oracle.merge(acc0.cpu().numpy(), lse0.cpu().numpy(), want_o, want_l)
    assert_lse(lse.cpu().numpy(), wl, "merged lse")
    assert_close(o.cpu().numpy(), wo, "bf16", "merged o")
    assert_close(fin_bf16.float().cpu().numpy(), wo, "bf16", "final bf16")
    fin = ~torch.isneginf(l_ref)
    assert torch.equal(torch.isneginf(lse), ~fin)
    assert torch.allclose(lse[fin], l_ref[fin], rtol=0, atol=1e-4)
    _close_to_unsplit(o, o_ref)


def test_fwd_step_ws_small_or_absent_workspace_does_not_split():
    """A NULL workspace, or one smaller than any split needs, runs the step
    unsplit (bit for bit the rba_fwd_step result)."""
    _say("fwd ws too small")
    rng = np.random.default_rng(77)
    sq, sk, hq, hkv, d = 64, 4096, 8, 2, 128
    qb, _ = _bf16(rng, (sq, hq, d))
    kb, _ = _bf16(rng, (sk, hkv, d))
    q, k = to_device(qb, "bf16", DEV), to_device(kb, "bf16", DEV)
    a = rba.attn_params(hq, hkv, d, 0.088, rba.RBA_BF16, rba.RBA_MASK_CAUSAL)
    qs, ks = rba.make_segs([(5000, sq)]), rba.make_segs([(0, sk)])
    assert rba.rba_fwd_workspace_size(a, sq, qs, sk, ks) > 0
    outs = []
    for ws in (None, torch.empty(1024, device=DEV)):
        o = torch.empty((sq, hq, d), device=DEV)
        l = torch.empty((hq, sq), device=DEV)
        assert rba.rba_fwd_step_ws(a, q, qs, k, k, ks, o, l, False, None, rba.RBA_BF16, ws) == rba.RBA_OK
        outs.append((o, l))
    o_ref = torch.empty((sq, hq, d), device=DEV)
    l_ref = torch.empty((hq, sq), device=DEV)
    rba.rba_fwd_step(a, q, qs, k, k, ks, o_ref, l_ref)
    torch.cuda.synchronize()
    for o, l in outs:
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref)


def test_replay_c3_full_all_ranks_split():
    """The 64K packed-document workload through rba_fwd_step_ws: every rank
    replays all 16 KV chunks with a workspace, so the calls with few rows of
    work split; the 16 ranks' outputs are compared with the full 65536-row
    packed causal attention."""
    w = W.WORKLOADS["c3"]
    _say("replay full split", w.name, "all 16 ranks")
    k64, v64 = full_kv_f64(w)
    cu = cu_or_none(w)
    shared = {"k": {j: to_device(W.gen_rank_chunk(w, W.T_K, j), w.dtype, DEV) for j in range(w.n_ranks)},
              "v": {j: to_device(W.gen_rank_chunk(w, W.T_V, j), w.dtype, DEV) for j in range(w.n_ranks)}}
    ws = torch.empty((32 << 20) // 4, dtype=torch.float32, device=DEV)
    abs_sum, count, o_max, n_split = 0.0, 0, 0.0, 0
    for r in range(w.n_ranks):
        rr = RingReplay(w, r, DEV, kv=shared, workspace=ws)
        for s in rr.steps:
            if s.status == rba.RBA_OK and rba.rba_fwd_workspace_size(
                    rr.attn, rr.q.shape[0], rr.q_segs, rr.k[s.src].shape[0], rr.kv_segs[s.src]) > 0:
                n_split += 1
        rr.forward()
        torch.cuda.synchronize()
        got = rr.o_final.float().cpu().numpy().astype(np.float64)
        got_l = rr.lse_acc.cpu().numpy()
        q64 = W.to_f64(W.gen_rank_chunk(w, W.T_Q, r), w.dtype)
        want_o, want_l = oracle_attention_rows(q64, k64, v64, chunk_positions(w, r), w.mask, w.scale, cu)
        assert_lse(got_l, want_l, f"rank {r} lse")
        assert np.isfinite(got).all()
        err = np.abs(got - want_o)
        abs_sum += float(err.sum())
        count += err.size
        o_max = max(o_max, float(err.max()))
        del rr
    mean = abs_sum / count
    print(f"[c3 split] {n_split} split calls; o max {o_max:.3g} mean {mean:.3g}", flush=True)
    assert n_split > 0
    assert o_max <= BF16_MAX and mean <= BF16_MEAN, (o_max, mean)
