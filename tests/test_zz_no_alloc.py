"""GPU check of rba_fwd_step_noalloc, the forward step whose split partials
live in the library's per-device array instead of a caller's workspace.

Its results must equal, bit for bit, those of rba_fwd_step_ws given a
32 MiB workspace (the same plan and the same kernels), and match the fp64
oracle at the forward's tolerances.  Two calls run in a row, the second on
a smaller input, so the second reads an array that still holds the first
call's partials; then the same with accumulation into a running result.
The file sorts last so that a failure here cannot hide the other GPU tests."""
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
WS_BYTES = 32 << 20

# sq, sk, hq, hkv, d, query segments, key segments, mask; the second smaller
CALLS = [
    (100, 3000, 32, 8, 128, [(2990, 100)], [(0, 3000)], rba.RBA_MASK_CAUSAL),
    (40, 2500, 4, 4, 64, [(0, 40)], [(100, 2500)], rba.RBA_MASK_NONE),
]


def _pos(segs):
    return np.concatenate([s + np.arange(n) for s, n in segs])


def _inputs(call, seed):
    sq, sk, hq, hkv, d, qsegs, ksegs, mask = call
    rng = np.random.default_rng(seed)
    bits = [W.f32_to_bf16_bits(rng.standard_normal(sh).astype(np.float32))
            for sh in ((sq, hq, d), (sk, hkv, d), (sk, hkv, d))]
    f64 = [W.bf16_bits_to_f32(b).astype(np.float64) for b in bits]
    scale = float(np.float32(1 / np.sqrt(d)))
    a = rba.attn_params(hq, hkv, d, scale, rba.RBA_BF16, mask)
    q, k, v = (to_device(b, "bf16", DEV) for b in bits)
    want = oracle.attention(*f64, _pos(qsegs), _pos(ksegs), mask, scale)
    return a, q, k, v, rba.make_segs(qsegs), rba.make_segs(ksegs), want, rng


def test_noalloc_matches_workspace_entry_point():
    ws = torch.full((WS_BYTES // 4,), float("nan"), dtype=torch.float32, device=DEV)
    for i, call in enumerate(CALLS):
        print("[case] noalloc partial", i, call[:5], flush=True)
        sq, sk, hq, hkv, d = call[:5]
        a, q, k, v, qs, ks, (want_o, want_l), _ = _inputs(call, 100 + i)
        assert rba.rba_fwd_workspace_size(a, sq, qs, sk, ks) > 0   # the call splits
        o = torch.full((sq, hq, d), float("nan"), device=DEV)
        lse = torch.full((hq, sq), float("nan"), device=DEV)
        assert rba.rba_fwd_step_noalloc(a, q, qs, k, v, ks, o, lse, False) == rba.RBA_OK
        o_ws, l_ws = torch.full_like(o, float("nan")), torch.full_like(lse, float("nan"))
        assert rba.rba_fwd_step_ws(a, q, qs, k, v, ks, o_ws, l_ws, False, None, rba.RBA_BF16, ws) == rba.RBA_OK
        torch.cuda.synchronize()
        assert torch.equal(o, o_ws) and torch.equal(lse, l_ws)
        assert_lse(lse.cpu().numpy(), want_l, "lse")
        assert_close(o.cpu().numpy(), want_o, "bf16", "o_part")


def test_noalloc_accumulate_matches_workspace_entry_point():
    ws = torch.full((WS_BYTES // 4,), float("nan"), dtype=torch.float32, device=DEV)
    for i, call in enumerate(CALLS):
        print("[case] noalloc accumulate", i, call[:5], flush=True)
        sq, sk, hq, hkv, d = call[:5]
        a, q, k, v, qs, ks, (want_o, want_l), rng = _inputs(call, 200 + i)
        acc0 = torch.from_numpy(rng.standard_normal((sq, hq, d)).astype(np.float32)).to(DEV)
        lse0 = torch.from_numpy((rng.standard_normal((hq, sq)) * 2).astype(np.float32)).to(DEV)
        outs = []
        for use_ws in (False, True):
            o, lse = acc0.clone(), lse0.clone()
            fin = torch.full((sq, hq, d), 7.0, dtype=torch.bfloat16, device=DEV)
            if use_ws:
                rc = rba.rba_fwd_step_ws(a, q, qs, k, v, ks, o, lse, True, fin, rba.RBA_BF16, ws)
            else:
                rc = rba.rba_fwd_step_noalloc(a, q, qs, k, v, ks, o, lse, True, fin, rba.RBA_BF16)
            assert rc == rba.RBA_OK
            outs.append((o, lse, fin))
        torch.cuda.synchronize()
        (o, lse, fin), (o_ws, l_ws, fin_ws) = outs
        assert torch.equal(o, o_ws) and torch.equal(lse, l_ws) and torch.equal(fin, fin_ws)
        wo, wl = oracle.merge(acc0.cpu().numpy(), lse0.cpu().numpy(), want_o, want_l)
        assert_lse(lse.cpu().numpy(), wl, "merged lse")
        assert_close(o.cpu().numpy(), wo, "bf16", "merged o")
        assert_close(fin.float().cpu().numpy(), wo, "bf16", "final bf16")


def test_noalloc_rejects_o_final_without_accumulate():
    call = CALLS[1]
    a, q, k, v, qs, ks, _, _ = _inputs(call, 300)
    o = torch.empty((call[0], call[2], call[4]), device=DEV)
    lse = torch.empty((call[2], call[0]), device=DEV)
    with pytest.raises(rba.RbaError) as e:
        rba.rba_fwd_step_noalloc(a, q, qs, k, v, ks, o, lse, False, torch.empty_like(o))
    assert e.value.code == rba.RBA_ERR_INVALID
