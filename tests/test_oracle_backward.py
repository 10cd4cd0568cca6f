"""Pins of the oracle's attention backward.

* the hand-derived worked example in tests/golden/worked_examples.json;
* central finite differences of L = sum dO * O in fp64;
* a library special case: torch fp64 autograd through
  scaled_dot_product_attention with an explicit mask;
* invariants: per KV head sum_j dK_j = 0 (each row of dS sums to 0) and
  sum_j dV_j = sum of dO over the rows that have keys, per head group.
A planted sign slip in dS is shown to fail the finite-difference pin.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attn as oatt

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _val(x):
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, {"ln3": math.log(3.0)}))
    return float(x)


def _arr(x):
    if isinstance(x, list):
        return np.array([_arr(e) for e in x])
    return _val(x)


def _case(rng, nq, nk, hq, hkv, d, mask):
    q = rng.standard_normal((nq, hq, d))
    k = rng.standard_normal((nk, hkv, d))
    v = rng.standard_normal((nk, hkv, d))
    do = rng.standard_normal((nq, hq, d))
    kpos = np.arange(nk)
    qpos = np.sort(rng.choice(nk, nq, replace=False))
    cu = np.array([0, nk // 3, nk // 2 + 1, nk]) if mask == 2 else None
    return q, k, v, do, qpos, kpos, cu


def _loss(q, k, v, do, qpos, kpos, mask, scale, cu):
    o, _ = oracle.attention(q, k, v, qpos, kpos, mask, scale, cu)
    return float((o * do).sum())


def test_worked_backward():
    with open(GOLDEN) as f:
        case = json.load(f)["backward_cases"][0]
    dq, dk, dv, *_ = oracle.attention_backward(
        _arr(case["q"]), _arr(case["k"]), _arr(case["v"]), _arr(case["do"]),
        np.array(case["qpos"]), np.array(case["kpos"]), case["mask"], case["scale"])
    np.testing.assert_allclose(dq, _arr(case["dq"]), atol=1e-12)
    np.testing.assert_allclose(dk, _arr(case["dk"]), atol=1e-12)
    np.testing.assert_allclose(dv, _arr(case["dv"]), atol=1e-12)


def _fd_check(q, k, v, do, qpos, kpos, mask, scale, cu, h=1e-6, tol=1e-6):
    dq, dk, dv, *_ = oracle.attention_backward(q, k, v, do, qpos, kpos, mask, scale, cu)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, qpos, kpos, mask, scale, cu)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, qpos, kpos, mask, scale, cu)
            num[idx] = (lp - lm) / (2 * h)
        if not np.allclose(g, num, rtol=tol, atol=tol):
            return False, name, np.abs(g - num).max()
    return True, None, 0.0


@pytest.mark.parametrize("mask", [0, 1, 2])
def test_finite_differences(mask):
    rng = np.random.default_rng(40 + mask)
    q, k, v, do, qpos, kpos, cu = _case(rng, 5, 7, 4, 2, 3, mask)
    ok, name, err = _fd_check(q, k, v, do, qpos, kpos, mask, 0.6, cu)
    assert ok, f"d{name} off by {err}"


@pytest.mark.parametrize("mask", [0, 1, 2])
def test_torch_autograd_fp64(mask):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(60 + mask)
    nq, nk, hq, hkv, d = 24, 32, 4, 2, 8
    q, k, v, do, _, kpos, cu = _case(rng, nq, nk, hq, hkv, d, mask)
    qpos = np.arange(nk - nq, nk)
    allow = np.ones((nq, nk), dtype=bool)
    for i in range(nq):
        for j in range(nk):
            if mask >= 1 and kpos[j] > qpos[i]:
                allow[i, j] = False
            if mask == 2:
                di = max(t for t in range(len(cu) - 1) if cu[t] <= qpos[i])
                dj = max(t for t in range(len(cu) - 1) if cu[t] <= kpos[j])
                if di != dj:
                    allow[i, j] = False
    scale = 1.0 / math.sqrt(d)
    group = hq // hkv
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(1, 0, 2)[None],
        tk.repeat_interleave(group, dim=1).permute(1, 0, 2)[None],
        tv.repeat_interleave(group, dim=1).permute(1, 0, 2)[None],
        attn_mask=torch.from_numpy(allow), scale=scale)
    (out[0].permute(1, 0, 2) * torch.from_numpy(do)).sum().backward()
    dq, dk, dv, *_ = oracle.attention_backward(q, k, v, do, qpos, kpos, mask, scale, cu)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("mask", [0, 1, 2])
def test_gradient_invariants(mask):
    rng = np.random.default_rng(80 + mask)
    nq, nk, hq, hkv, d = 20, 30, 4, 2, 6
    q, k, v, do, qpos, kpos, cu = _case(rng, nq, nk, hq, hkv, d, mask)
    dq, dk, dv, delta, o, lse = oracle.attention_backward(q, k, v, do, qpos, kpos, mask, 0.5, cu)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    has = ~np.isneginf(lse)                      # [hq, nq]
    group = hq // hkv
    for g in range(hkv):
        want = sum((do[:, h, :] * has[h][:, None]).sum(axis=0) for h in range(g * group, (g + 1) * group))
        np.testing.assert_allclose(dv[:, g, :].sum(axis=0), want, atol=1e-12)
    np.testing.assert_allclose(delta, (do * o).sum(axis=2).T, atol=1e-13)


def test_planted_sign_slip_is_caught(monkeypatch):
    rng = np.random.default_rng(41)
    q, k, v, do, qpos, kpos, cu = _case(rng, 4, 6, 2, 1, 3, 1)
    assert _fd_check(q, k, v, do, qpos, kpos, 1, 0.6, cu)[0]
    monkeypatch.setattr(oatt, "_score_grad", lambda p, dp, delta: p * (dp + delta[:, None]))
    assert not _fd_check(q, k, v, do, qpos, kpos, 1, 0.6, cu)[0]


@pytest.mark.parametrize("mask", [0, 1, 2])
def test_sampled_backward_equals_full(mask):
    rng = np.random.default_rng(90 + mask)
    q, k, v, do, qpos, kpos, cu = _case(rng, 30, 40, 6, 2, 8, mask)
    dq, dk, dv, *_ = oracle.attention_backward(q, k, v, do, qpos, kpos, mask, 0.4, cu)
    rows = np.array([0, 7, 29])
    keys = np.array([1, 2, 33, 39])
    sdq, sdk, sdv = oracle.attention_backward_sampled(q, k, v, do, qpos, kpos, mask, 0.4, cu,
                                                      rows=rows, keys=keys, heads=[3, 4, 5], row_block=7)
    np.testing.assert_allclose(sdq, dq[rows][:, 3:6], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sdk[:, 1], dk[keys][:, 1], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sdv[:, 1], dv[keys][:, 1], rtol=1e-12, atol=1e-13)
    assert np.all(sdk[:, 0] == 0) and np.all(sdv[:, 0] == 0)
