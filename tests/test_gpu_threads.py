"""The library from several host threads at once: two threads, each with
its own stream and inputs, run forward steps (plain and merging) and a
backward step over and over; every result must equal the same call made
alone beforehand: bit for bit, except dK / dV, which workgroups of the
same KV head may add in any order (fp32 atomics) and so agree to rounding."""
import threading

import numpy as np
import pytest
import torch

from ring_sequence_parallelism_amd import rba
from ring_sequence_parallelism_amd import workloads as W
from ring_sequence_parallelism_amd.ring import to_device

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(seed):
    rng = np.random.default_rng(seed)
    sq, sk, hq, hkv, d = 256, 1024, 8, 2, 128
    bits = [W.f32_to_bf16_bits(rng.standard_normal(sh).astype(np.float32))
            for sh in ((sq, hq, d), (sk, hkv, d), (sk, hkv, d), (sq, hq, d))]
    q, k, v, do = (to_device(b, "bf16", DEV) for b in bits)
    a = rba.attn_params(hq, hkv, d, float(np.float32(1 / np.sqrt(d))), rba.RBA_BF16, rba.RBA_MASK_CAUSAL)
    qs, ks = rba.make_segs([(1000, sq)]), rba.make_segs([(300, sk)])
    return a, q, k, v, do, qs, ks


def _run(case, stream):
    a, q, k, v, do, qs, ks = case
    sq, hq, d = q.shape
    sk, hkv = k.shape[0], k.shape[1]
    with torch.cuda.stream(stream):
        o = torch.empty((sq, hq, d), device=DEV)
        lse = torch.empty((hq, sq), device=DEV)
        assert rba.rba_fwd_step(a, q, qs, k, v, ks, o, lse, stream=stream) == rba.RBA_OK
        o2, l2 = o.clone(), lse.clone()
        fin = torch.empty((sq, hq, d), dtype=torch.bfloat16, device=DEV)
        assert rba.rba_fwd_step_acc(a, q, qs, k, v, ks, o2, l2, fin, rba.RBA_BF16, stream=stream) == rba.RBA_OK
        delta = torch.empty((hq, sq), device=DEV)
        assert rba.rba_bwd_preprocess(fin, do, delta, stream=stream) == rba.RBA_OK
        dq = torch.zeros((sq, hq, d), device=DEV)
        dk = torch.empty((sk, hkv, d), device=DEV)
        dv = torch.empty((sk, hkv, d), device=DEV)
        assert rba.rba_bwd_step(a, q, qs, k, v, ks, do, l2, delta, dq, dk, dv, stream=stream) == rba.RBA_OK
    stream.synchronize()
    return [x.clone() for x in (o, lse, o2, l2, fin, delta, dq, dk, dv)]


def test_two_threads_two_streams():
    print("[case] two host threads, two streams", flush=True)
    cases = [_case(11), _case(12)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    want = [_run(c, s) for c, s in zip(cases, streams)]
    errors = []

    def worker(i):
        try:
            torch.cuda.set_device(0)
            for _ in range(20):
                got = _run(cases[i], streams[i])
                for j, (g, w_) in enumerate(zip(got, want[i])):
                    same = torch.allclose(g, w_, rtol=1e-5, atol=1e-6) if j >= 7 else torch.equal(g, w_)
                    if not same:
                        raise AssertionError(f"thread {i}: output {j} differs from the call made alone")
        except Exception as e:   # re-raised in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[0]
