"""GPU parity of the document mask for document counts on both sides of the
register table's size: up to 63 documents the kernels look document starts
and ends up in a table held in the lanes of a wave, from 64 on they search
cu_seqlens in memory.  Forward steps (alone and merged into a running
result, where merging launches skip row groups without keys) and backward
steps, against the fp64 oracle."""
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
N_DOCS = [1, 2, 63, 64, 65, 200]


def _say(*a):
    print("[case]", *a, flush=True)


def _bf16(rng, shape):
    bits = W.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    return bits, W.bf16_bits_to_f32(bits).astype(np.float64)


def _cu(rng, end, n_docs):
    """n_docs documents of random lengths covering positions [0, end)."""
    cuts = np.sort(rng.choice(np.arange(1, end), n_docs - 1, replace=False)) if n_docs > 1 else np.array([], int)
    return np.concatenate([[0], cuts, [end]]).astype(np.int32)


def _setup(n_docs, seed, sq=320, sk=700, hq=8, hkv=2, d=128):
    rng = np.random.default_rng(seed)
    # queries at positions 500..819, keys in two chunks: 0..349 and 350..699
    qsegs = [(500, sq)]
    k1, k2 = [(0, sk // 2)], [(sk // 2, sk - sk // 2)]
    cu = _cu(rng, 500 + sq, n_docs)
    cu_dev = torch.from_numpy(cu).to(DEV)
    scale = float(np.float32(1 / np.sqrt(d)))
    a = rba.attn_params(hq, hkv, d, scale, rba.RBA_BF16, rba.RBA_MASK_DOC_CAUSAL, cu_dev, cu)
    qb, q64 = _bf16(rng, (sq, hq, d))
    kb, k64 = _bf16(rng, (sk, hkv, d))
    vb, v64 = _bf16(rng, (sk, hkv, d))
    dob, do64 = _bf16(rng, (sq, hq, d))
    dev = {n: to_device(x, "bf16", DEV) for n, x in (("q", qb), ("k", kb), ("v", vb), ("do", dob))}
    return a, cu, scale, qsegs, k1, k2, dev, (q64, k64, v64, do64)


@pytest.mark.parametrize("n_docs", N_DOCS)
def test_fwd_step_and_merging_step_many_documents(n_docs):
    _say("fwd documents", n_docs)
    a, cu, scale, qsegs, k1, k2, dev, (q64, k64, v64, _) = _setup(n_docs, 100 + n_docs)
    sq, hq, d = dev["q"].shape
    half = k1[0][1]
    qpos = np.arange(qsegs[0][0], qsegs[0][0] + sq)
    kpos = np.arange(k64.shape[0])
    qs, ks1, ks2 = rba.make_segs(qsegs), rba.make_segs(k1), rba.make_segs(k2)
    o = torch.full((sq, hq, d), float("nan"), device=DEV)
    lse = torch.full((hq, sq), float("nan"), device=DEV)
    st1 = rba.rba_fwd_step(a, dev["q"], qs, dev["k"][:half], dev["v"][:half], ks1, o, lse)
    torch.cuda.synchronize()
    w1o, w1l = oracle.attention(q64, k64[:half], v64[:half], qpos, kpos[:half], oracle.MASK_DOC_CAUSAL, scale, cu)
    if st1 == rba.RBA_OK:
        assert_lse(lse.cpu().numpy(), w1l, "lse, first chunk")
        assert_close(o.cpu().numpy(), w1o, "bf16", "o, first chunk")
    else:
        assert st1 == rba.RBA_STEP_EMPTY and np.isneginf(w1l).all()
        o.zero_()
        lse.fill_(float("-inf"))
    # merge the second chunk into the running result in the step's epilogue
    st2 = rba.rba_fwd_step_acc(a, dev["q"], qs, dev["k"][half:], dev["v"][half:], ks2, o, lse)
    torch.cuda.synchronize()
    wo, wl = oracle.attention(q64, k64, v64, qpos, kpos, oracle.MASK_DOC_CAUSAL, scale, cu)
    if st2 == rba.RBA_STEP_EMPTY:
        w2o, w2l = oracle.attention(q64, k64[half:], v64[half:], qpos, kpos[half:], oracle.MASK_DOC_CAUSAL, scale, cu)
        assert np.isneginf(w2l).all()
    fin = ~np.isneginf(wl)
    got_l = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(got_l), ~fin)
    assert_lse(got_l, wl, "merged lse")
    got_o = o.cpu().numpy()
    assert_close(got_o[fin.T], wo[fin.T], "bf16", "merged o")


@pytest.mark.parametrize("n_docs", [63, 64, 200])
def test_bwd_step_many_documents(n_docs):
    _say("bwd documents", n_docs)
    a, cu, scale, qsegs, k1, k2, dev, (q64, k64, v64, do64) = _setup(n_docs, 200 + n_docs)
    sq, hq, d = dev["q"].shape
    sk, hkv = dev["k"].shape[0], dev["k"].shape[1]
    qpos = np.arange(qsegs[0][0], qsegs[0][0] + sq)
    kpos = np.arange(sk)
    ks = rba.make_segs([(0, sk)])
    qs = rba.make_segs(qsegs)
    wdq, wdk, wdv, *_ = oracle.attention_backward(q64, k64, v64, do64, qpos, kpos, oracle.MASK_DOC_CAUSAL, scale, cu)
    o_acc = torch.empty((sq, hq, d), device=DEV)
    lse = torch.empty((hq, sq), device=DEV)
    assert rba.rba_fwd_step(a, dev["q"], qs, dev["k"], dev["v"], ks, o_acc, lse) == rba.RBA_OK
    delta = torch.empty((hq, sq), device=DEV)
    rba.rba_bwd_preprocess(o_acc, dev["do"], delta)
    dq = torch.zeros((sq, hq, d), device=DEV)
    dk = torch.full((sk, hkv, d), float("nan"), device=DEV)
    dv = torch.full((sk, hkv, d), float("nan"), device=DEV)
    assert rba.rba_bwd_step(a, dev["q"], qs, dev["k"], dev["v"], ks, dev["do"], lse, delta, dq, dk, dv) == rba.RBA_OK
    torch.cuda.synchronize()
    assert_close(dq.cpu().numpy(), wdq, "bf16", "dq")
    assert_close(dk.cpu().numpy(), wdk, "bf16", "dk")
    assert_close(dv.cpu().numpy(), wdv, "bf16", "dv")
