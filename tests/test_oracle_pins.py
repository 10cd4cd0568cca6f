"""Pins of the CPU oracle's forward and merge against facts outside itself.

* hand-derived worked examples (tests/golden/worked_examples.json);
* brute force: pure-Python loops over tiny inputs, with the mask decided by
  scanning the document table and the softmax summed with math.fsum;
* a library special case: torch's fp64 CPU scaled_dot_product_attention with
  an explicit boolean mask;
* closed forms (uniform scores -> mean of the allowed values, LSE = ln count;
  a single allowed key -> that key's value, LSE = its score);
* invariants (rows of P sum to 1, merging any chunking of the keys equals
  unchunked attention, merge is commutative and associative);
* reductions (one document = causal, GQA = MHA with repeated KV heads).
Planted mistakes at the end show that these pins catch the plausible slips.
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
        env = {"ln2": math.log(2.0), "ln3": math.log(3.0), "ln4": math.log(4.0)}
        if x == "-inf":
            return -math.inf
        return float(eval(x, {"__builtins__": {}}, env))
    return float(x)


def _arr(x):
    if x is None:
        return None
    if isinstance(x, list):
        return np.array([_arr(e) for e in x]) if x and isinstance(x[0], list) else np.array([_val(e) for e in x])
    return _val(x)


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Worked examples

@pytest.mark.parametrize("case", _golden()["cases"], ids=lambda c: c["name"])
def test_worked_example(case):
    cu = None if case["cu_seqlens"] is None else np.array(case["cu_seqlens"])
    o, lse = oracle.attention(_arr(case["q"]), _arr(case["k"]), _arr(case["v"]),
                              np.array(case["qpos"]), np.array(case["kpos"]),
                              case["mask"], case["scale"], cu)
    np.testing.assert_allclose(o, _arr(case["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, _arr(case["lse"]), rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", _golden()["merge_cases"], ids=lambda c: c["name"])
def test_worked_merge(case):
    o, lse = oracle.merge(_arr(case["o_a"]), _arr(case["lse_a"]), _arr(case["o_b"]), _arr(case["lse_b"]))
    np.testing.assert_allclose(o, _arr(case["o"]), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(_arr(case["lse"])))
    fin = ~np.isneginf(lse)
    np.testing.assert_allclose(lse[fin], _arr(case["lse"])[fin], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Brute force

def _brute_doc(p, cu):
    t = 0
    while not (cu[t] <= p < cu[t + 1]):
        t += 1
    return t


def _brute_attention(q, k, v, qpos, kpos, mask, scale, cu):
    nq, hq, d = q.shape
    nk, hkv, _ = k.shape
    per = hq // hkv
    o = [[[0.0] * d for _ in range(hq)] for _ in range(nq)]
    lse = [[-math.inf] * nq for _ in range(hq)]
    for i in range(nq):
        for h in range(hq):
            g = h // per
            keys = []
            for j in range(nk):
                ok = True
                if mask >= 1 and not (kpos[j] <= qpos[i]):
                    ok = False
                if mask == 2 and ok and _brute_doc(qpos[i], cu) != _brute_doc(kpos[j], cu):
                    ok = False
                if ok:
                    keys.append(j)
            if not keys:
                continue
            s = {j: scale * math.fsum(float(q[i, h, c]) * float(k[j, g, c]) for c in range(d)) for j in keys}
            top = max(s.values())
            w = {j: math.exp(s[j] - top) for j in keys}
            tot = math.fsum(w.values())
            lse[h][i] = top + math.log(tot)
            for c in range(d):
                o[i][h][c] = math.fsum(w[j] / tot * float(v[j, g, c]) for j in keys)
    return np.array(o), np.array(lse)


def _rand_case(rng, nq, nk, hq, hkv, d, mask):
    q = rng.standard_normal((nq, hq, d))
    k = rng.standard_normal((nk, hkv, d))
    v = rng.standard_normal((nk, hkv, d))
    total = max(nq, nk) + 4
    qpos = np.sort(rng.choice(total, nq, replace=False))
    kpos = np.sort(rng.choice(total, nk, replace=False))
    cu = None
    if mask == 2:
        cuts = np.sort(rng.choice(np.arange(1, total), 3, replace=False))
        cu = np.concatenate([[0], cuts, [total]])
    return q, k, v, qpos, kpos, cu


@pytest.mark.parametrize("mask", [0, 1, 2])
@pytest.mark.parametrize("shape", [(7, 11, 2, 2, 4), (12, 9, 4, 2, 8), (5, 24, 2, 1, 3)])
def test_brute_force(mask, shape):
    nq, nk, hq, hkv, d = shape
    rng = np.random.default_rng(100 + mask * 7 + nq)
    q, k, v, qpos, kpos, cu = _rand_case(rng, nq, nk, hq, hkv, d, mask)
    # shuffled row order: positions need not be sorted within a chunk
    perm = rng.permutation(nk)
    k, v, kpos = k[perm], v[perm], kpos[perm]
    scale = 0.37
    o, lse = oracle.attention(q, k, v, qpos, kpos, mask, scale, cu, row_block=4)
    bo, blse = _brute_attention(q, k, v, qpos, kpos, mask, scale, cu)
    np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(blse))
    fin = ~np.isneginf(blse)
    np.testing.assert_allclose(lse[fin], blse[fin], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# Library special case: torch fp64 CPU SDPA with an explicit mask

@pytest.mark.parametrize("mask", [0, 1, 2])
def test_torch_sdpa_fp64(mask):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7 + mask)
    nq, nk, hq, hkv, d = 40, 56, 4, 2, 16
    q, k, v, _, _, _ = _rand_case(rng, nq, nk, hq, hkv, d, mask)
    # queries are the last nq key positions, so every row has its own key
    kpos = np.arange(nk)
    qpos = np.arange(nk - nq, nk)
    cu = np.array([0, 10, 30, nk]) if mask == 2 else None
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attention(q, k, v, qpos, kpos, mask, scale, cu)
    allow = np.ones((nq, nk), dtype=bool)
    for i in range(nq):
        for j in range(nk):
            if mask >= 1 and kpos[j] > qpos[i]:
                allow[i, j] = False
            if mask == 2 and _brute_doc(qpos[i], cu) != _brute_doc(kpos[j], cu):
                allow[i, j] = False
    assert allow.any(axis=1).all()
    group = hq // hkv
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(np.repeat(k, group, axis=1)).permute(1, 0, 2)[None]
    tv = torch.from_numpy(np.repeat(v, group, axis=1)).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(allow), scale=scale)
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# Closed forms

@pytest.mark.parametrize("mask", [0, 1, 2])
@pytest.mark.parametrize("zero", ["q", "k"])
def test_uniform_scores_closed_form(mask, zero):
    rng = np.random.default_rng(3)
    nq, nk, hq, hkv, d = 16, 20, 4, 2, 8
    q, k, v, _, _, _ = _rand_case(rng, nq, nk, hq, hkv, d, mask)
    if zero == "q":
        q[:] = 0
    else:
        k[:] = 0
    qpos = np.arange(4, 4 + nq)
    kpos = np.arange(nk)
    cu = np.array([0, 9, 17, 40]) if mask == 2 else None
    o, lse = oracle.attention(q, k, v, qpos, kpos, mask, 0.5, cu)
    for i in range(nq):
        if mask == 0:
            keys = list(range(nk))
        else:
            keys = [j for j in range(nk) if kpos[j] <= qpos[i]]
            if mask == 2:
                keys = [j for j in keys if _brute_doc(kpos[j], cu) == _brute_doc(qpos[i], cu)]
        for h in range(hq):
            g = h // (hq // hkv)
            np.testing.assert_allclose(o[i, h], v[keys, g].mean(axis=0), rtol=1e-12, atol=1e-13)
            assert abs(lse[h, i] - math.log(len(keys))) < 1e-12


def test_single_allowed_key_closed_form():
    rng = np.random.default_rng(11)
    d = 8
    q = rng.standard_normal((3, 2, d))
    k = rng.standard_normal((3, 1, d))
    v = rng.standard_normal((3, 1, d))
    # row 0 at position 0 (causal): only key 0; row 2 opens a one-token document
    pos = np.array([0, 1, 2])
    for mask, cu, rows in [(1, None, [0]), (2, np.array([0, 2, 3]), [0, 2])]:
        o, lse = oracle.attention(q, k, v, pos, pos, mask, 0.3, cu)
        for i in rows:
            for h in range(2):
                np.testing.assert_allclose(o[i, h], v[i, 0], rtol=1e-13, atol=1e-14)
                assert abs(lse[h, i] - 0.3 * float(q[i, h] @ k[i, 0])) < 1e-13


def test_empty_row_is_zero_and_neg_inf():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((2, 1, 4))
    k = rng.standard_normal((3, 1, 4))
    v = rng.standard_normal((3, 1, 4))
    o, lse = oracle.attention(q, k, v, np.array([0, 10]), np.array([5, 6, 7]), 1, 1.0)
    assert np.all(o[0] == 0) and np.isneginf(lse[0, 0])
    assert np.isfinite(lse[0, 1])


# ---------------------------------------------------------------------------
# Invariants

@pytest.mark.parametrize("mask", [0, 1, 2])
def test_rows_of_p_sum_to_one(mask):
    # With one-hot values v_j = e_j the output row is the probability row P_i.
    rng = np.random.default_rng(5)
    nq, nk = 9, 12
    q = rng.standard_normal((nq, 2, 6))
    k = rng.standard_normal((nk, 1, 6))
    v = np.eye(nk)[:, None, :]
    qpos = np.arange(3, 3 + nq)
    kpos = np.arange(nk)
    cu = np.array([0, 5, 12, 20]) if mask == 2 else None
    o, _ = oracle.attention(q, k, v, qpos, kpos, mask, 0.8, cu)
    np.testing.assert_allclose(o.sum(axis=2), 1.0, rtol=0, atol=1e-13)
    assert (o >= 0).all()
    allow = oracle.allowed_mask(qpos, kpos, mask, cu)
    assert np.all(o[:, 0, :][~allow] == 0) and np.all(o[:, 1, :][~allow] == 0)


@pytest.mark.parametrize("mask", [0, 1, 2])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_merge_of_any_chunking_equals_unchunked(mask, seed):
    rng = np.random.default_rng(50 + seed)
    nq, nk, hq, hkv, d = 14, 40, 4, 2, 8
    q, k, v, qpos, kpos, cu = _rand_case(rng, nq, nk, hq, hkv, d, mask)
    perm = rng.permutation(nk)
    k, v, kpos = k[perm], v[perm], kpos[perm]
    scale = 0.4
    full_o, full_lse = oracle.attention(q, k, v, qpos, kpos, mask, scale, cu)
    cuts = [0] + sorted(rng.choice(np.arange(1, nk), 5, replace=False).tolist()) + [nk]
    if seed == 2:
        cuts = list(range(nk + 1))          # size-1 chunks
    parts = [oracle.attention(q, k[a:b], v[a:b], qpos, kpos[a:b], mask, scale, cu)
             for a, b in zip(cuts[:-1], cuts[1:])]
    # some chunks are fully masked for some rows: they carry LSE = -inf
    o, lse = oracle.merge_many(parts)
    np.testing.assert_allclose(o, full_o, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(full_lse))
    fin = ~np.isneginf(lse)
    np.testing.assert_allclose(lse[fin], full_lse[fin], rtol=1e-12, atol=1e-12)
    # order-free: reversed and a tree reduction give the same result
    o_r, lse_r = oracle.merge_many(parts[::-1])
    np.testing.assert_allclose(o_r, full_o, rtol=1e-12, atol=1e-12)
    left = oracle.merge_many(parts[:3])
    right = oracle.merge_many(parts[3:])
    o_t, _ = oracle.merge(*left, *right)
    np.testing.assert_allclose(o_t, full_o, rtol=1e-12, atol=1e-12)


def test_merge_commutes():
    rng = np.random.default_rng(9)
    oa, ob = rng.standard_normal((2, 5, 3, 4))
    la, lb = rng.standard_normal((2, 3, 5))
    la[0, 1] = -np.inf
    o1, l1 = oracle.merge(oa, la, ob, lb)
    o2, l2 = oracle.merge(ob, lb, oa, la)
    np.testing.assert_allclose(o1, o2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)


# ---------------------------------------------------------------------------
# Reductions

def test_one_document_equals_causal():
    rng = np.random.default_rng(21)
    q, k, v, qpos, kpos, _ = _rand_case(rng, 10, 15, 2, 2, 4, 1)
    total = max(qpos.max(), kpos.max()) + 1
    a = oracle.attention(q, k, v, qpos, kpos, 1, 0.5)
    b = oracle.attention(q, k, v, qpos, kpos, 2, 0.5, np.array([0, total]))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_zigzag_one_rank_is_plain_causal():
    assert np.array_equal(oracle.zigzag_positions(64, 1, 0), np.arange(64))


@pytest.mark.parametrize("mask", [0, 1, 2])
def test_gqa_equals_mha_with_repeated_kv(mask):
    rng = np.random.default_rng(31)
    q, k, v, qpos, kpos, cu = _rand_case(rng, 8, 12, 6, 2, 4, mask)
    a = oracle.attention(q, k, v, qpos, kpos, mask, 0.5, cu)
    b = oracle.attention(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), qpos, kpos, mask, 0.5, cu)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=0)
    np.testing.assert_array_equal(a[1], b[1])


# ---------------------------------------------------------------------------
# Planted mistakes: each slip in the oracle must fail one of the pins above.

def _brute_pin_passes():
    rng = np.random.default_rng(123)
    for mask in (0, 1, 2):
        q, k, v, qpos, kpos, cu = _rand_case(rng, 6, 9, 4, 2, 3, mask)
        o, lse = oracle.attention(q, k, v, qpos, kpos, mask, 0.37, cu)
        bo, blse = _brute_attention(q, k, v, qpos, kpos, mask, 0.37, cu)
        if not np.allclose(o, bo, rtol=1e-12, atol=1e-13):
            return False
        if not np.array_equal(np.isneginf(lse), np.isneginf(blse)):
            return False
        fin = ~np.isneginf(blse)
        if not np.allclose(lse[fin], blse[fin], rtol=1e-12, atol=1e-13):
            return False
    return True


def test_planted_mistakes_are_caught(monkeypatch):
    assert _brute_pin_passes()
    real_allowed = oatt.allowed_mask
    real_doc = oatt.doc_of
    real_probs = oatt._head_probs

    def strict_causal(qpos, kpos, mask, cu=None):
        a = real_allowed(qpos, kpos, mask, cu)
        if mask >= 1:
            a &= np.asarray(kpos)[None, :] != np.asarray(qpos)[:, None]
        return a

    def doc_left(pos, cu):
        return np.searchsorted(np.asarray(cu), np.asarray(pos), side="left") - 1

    def unnormalised(s, allow):          # forgets to divide by the row sum
        _, lse = real_probs(s, allow)
        has = allow.any(axis=1)
        sm = np.where(allow, s, -np.inf)
        m = np.where(has, sm.max(axis=1, initial=-np.inf), 0.0)
        return np.where(allow, np.exp(sm - m[:, None]), 0.0), lse

    def no_max_shift_bug(s, allow):      # drops the max in the LSE
        p, lse = real_probs(s, allow)
        m = np.where(allow, s, -np.inf).max(axis=1, initial=-np.inf)
        return p, np.where(np.isfinite(lse), lse - np.where(np.isfinite(m), m, 0), lse)

    for name, fn in [("allowed_mask", strict_causal), ("doc_of", doc_left),
                     ("_head_probs", unnormalised), ("_head_probs", no_max_shift_bug)]:
        monkeypatch.setattr(oatt, name, fn)
        try:
            caught = not _brute_pin_passes()
        except Exception:
            caught = True
        monkeypatch.setattr(oatt, "allowed_mask", real_allowed)
        monkeypatch.setattr(oatt, "doc_of", real_doc)
        monkeypatch.setattr(oatt, "_head_probs", real_probs)
        assert caught, f"planted mistake in {name} was not caught"


def test_planted_merge_mistake_is_caught():
    rng = np.random.default_rng(77)
    q, k, v, qpos, kpos, cu = _rand_case(rng, 6, 10, 2, 2, 4, 1)
    full = oracle.attention(q, k, v, qpos, kpos, 1, 0.5, cu)
    a = oracle.attention(q, k[:5], v[:5], qpos, kpos[:5], 1, 0.5, cu)
    b = oracle.attention(q, k[5:], v[5:], qpos, kpos[5:], 1, 0.5, cu)
    good, _ = oracle.merge(*a, *b)
    np.testing.assert_allclose(good, full[0], atol=1e-12)
    # swapped weights (a slip in the merge formula) must disagree
    bad, _ = oracle.merge(a[0], b[1], b[0], a[1])
    assert not np.allclose(bad, full[0], atol=1e-6)
