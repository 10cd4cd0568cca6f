"""C-ABI checks that need no GPU: the library loads and exports every entry
point include/rba.h declares, argument validation rejects bad calls before
any device work, and the host planner's exact pair counts equal the oracle's
brute-force count of allowed pairs."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from ring_sequence_parallelism_amd import rba
from ring_sequence_parallelism_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rba.h")

pytestmark = pytest.mark.skipif(not os.path.exists(rba.LIB_PATH), reason="librba.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rba_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = rba.load()
    names = declared_functions()
    assert set(names) == set(rba.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert rba.rba_version().startswith("rba ")


def test_struct_layout_matches_header():
    # rba_segs: int32 n, pad, int64 start[16], len[16], stride[16]; rba_attn ends with n_docs
    assert ctypes.sizeof(rba.rba_segs) == 8 + 16 * 8 * 3
    assert rba.rba_segs.stride.offset == 8 + 16 * 8 * 2
    assert rba.rba_attn.cu_seqlens_dev.offset == 24
    assert rba.rba_attn.n_docs.offset == 40


FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails or plans only


def _fwd(a, sq, qs, sk, ks, q=FAKE, o=FAKE):
    lib = rba.load()
    return lib.rba_fwd_step(ctypes.byref(a), q, sq, ctypes.byref(qs), FAKE, FAKE, sk,
                            ctypes.byref(ks), o, FAKE, None)


def _attn(**kw):
    base = dict(hq=4, hkv=2, d=128, scale=0.088, dtype=rba.RBA_BF16, mask=rba.RBA_MASK_CAUSAL)
    base.update(kw)
    return rba.attn_params(**base)


SEG64 = rba.make_segs([(0, 64)])


@pytest.mark.parametrize("kw,code", [
    (dict(hq=3, hkv=2), rba.RBA_ERR_INVALID),
    (dict(hq=0), rba.RBA_ERR_INVALID),
    (dict(d=96), rba.RBA_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), rba.RBA_ERR_INVALID),
    (dict(scale=-1.0), rba.RBA_ERR_INVALID),
    (dict(dtype=7), rba.RBA_ERR_INVALID),
    (dict(mask=9), rba.RBA_ERR_INVALID),
    (dict(mask=rba.RBA_MASK_DOC_CAUSAL), rba.RBA_ERR_INVALID),   # no cu_seqlens
])
def test_fwd_rejects_bad_params(kw, code):
    assert _fwd(_attn(**kw), 64, SEG64, 64, SEG64) == code
    assert rba.rba_last_error() != ""


def test_fwd_rejects_bad_segments():
    a = _attn()
    assert _fwd(a, 64, rba.make_segs([(0, 32)]), 64, SEG64) == rba.RBA_ERR_INVALID      # sum != rows
    assert _fwd(a, 64, rba.make_segs([(0, 40), (30, 24)]), 64, SEG64) == rba.RBA_ERR_INVALID  # overlap
    assert _fwd(a, 64, rba.make_segs([(-5, 64)]), 64, SEG64) == rba.RBA_ERR_INVALID
    s = rba.make_segs([(0, 64)])
    s.n = 17
    assert _fwd(a, 64, s, 64, SEG64) == rba.RBA_ERR_INVALID
    assert _fwd(a, 64, rba.make_segs([(2**31 - 10, 64)]), 64, SEG64) == rba.RBA_ERR_UNSUPPORTED


def test_fwd_alignment_and_null():
    a = _attn(mask=rba.RBA_MASK_NONE)
    assert _fwd(a, 64, SEG64, 64, SEG64, q=ctypes.c_void_p(0x10008)) == rba.RBA_ERR_ALIGNMENT
    assert _fwd(a, 64, SEG64, 64, SEG64, o=None) == rba.RBA_ERR_INVALID


def test_empty_steps_launch_nothing():
    a = _attn()
    # keys entirely after the queries: causal step is empty
    assert _fwd(a, 64, SEG64, 64, rba.make_segs([(64, 64)])) == rba.RBA_STEP_EMPTY
    # zero rows
    assert _fwd(a, 0, rba.make_segs([]), 64, SEG64) == rba.RBA_STEP_EMPTY
    # document mask: keys in an earlier document
    cu = np.array([0, 100, 200], dtype=np.int32)
    ad = _attn(mask=rba.RBA_MASK_DOC_CAUSAL, cu_seqlens_dev=None, cu_seqlens_host=cu)
    ad.cu_seqlens_dev = 0x20000
    assert _fwd(ad, 50, rba.make_segs([(120, 50)]), 64, rba.make_segs([(0, 64)])) == rba.RBA_STEP_EMPTY
    # position past the packed buffer
    assert _fwd(ad, 50, rba.make_segs([(180, 50)]), 64, SEG64) == rba.RBA_ERR_INVALID


def test_merge_and_preprocess_validation():
    lib = rba.load()
    assert lib.rba_merge(8, 2, 6, FAKE, FAKE, FAKE, FAKE, None, 0, None) == rba.RBA_ERR_UNSUPPORTED
    assert lib.rba_merge(8, 2, 64, FAKE, FAKE, FAKE, None, None, 0, None) == rba.RBA_ERR_INVALID
    assert lib.rba_merge(8, 2, 64, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == rba.RBA_ERR_INVALID  # alias
    assert lib.rba_merge(8, 2, 64, FAKE, FAKE, None, None, None, 0, None) == rba.RBA_OK          # nothing to do
    assert lib.rba_bwd_preprocess(8, 2, 96, 0, 0, FAKE, FAKE, FAKE, None) == rba.RBA_ERR_UNSUPPORTED
    assert lib.rba_bwd_preprocess(8, 2, 64, 0, 5, FAKE, FAKE, FAKE, None) == rba.RBA_ERR_INVALID


@pytest.mark.parametrize("fn", ["rba_bwd_step", "rba_bwd_step_acc"])
def test_bwd_rejects_f32(fn):
    lib = rba.load()
    a = _attn(dtype=rba.RBA_F32)
    rc = getattr(lib, fn)(ctypes.byref(a), FAKE, 64, ctypes.byref(SEG64), FAKE, FAKE, 64,
                          ctypes.byref(SEG64), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert rc == rba.RBA_ERR_UNSUPPORTED


@pytest.mark.parametrize("fn", ["rba_bwd_step", "rba_bwd_step_acc"])
def test_bwd_null_and_empty(fn):
    lib = rba.load()
    a = _attn()
    f = getattr(lib, fn)
    args = [ctypes.byref(a), FAKE, 64, ctypes.byref(SEG64), FAKE, FAKE, 64, ctypes.byref(SEG64),
            FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None]
    bad = list(args)
    bad[12] = None                          # dk
    assert f(*bad) == rba.RBA_ERR_INVALID
    assert "dk" in rba.rba_last_error()
    # keys after every query: nothing is launched
    empty = list(args)
    empty[7] = ctypes.byref(rba.make_segs([(64, 64)]))
    assert f(*empty) == rba.RBA_STEP_EMPTY


# ---------------------------------------------------------------------------
# Host planner vs the oracle's explicit-mask count

def _positions(segs):
    return np.concatenate([np.arange(s, s + n) for s, n in segs]) if segs else np.zeros(0, np.int64)


def _random_segs(rng, total, rows, max_segs):
    n = int(rng.integers(1, max_segs + 1))
    n = min(n, rows)
    cuts = np.sort(rng.choice(np.arange(1, rows), n - 1, replace=False)) if n > 1 else np.array([], int)
    lens = np.diff(np.concatenate([[0], cuts, [rows]]))
    # place the runs at disjoint random positions
    gaps = rng.integers(0, 20, size=n)
    starts, p = [], 0
    order = rng.permutation(n)
    placed = {}
    for i in order:
        p += int(gaps[i])
        placed[i] = p
        p += int(lens[i])
    return [(placed[i], int(lens[i])) for i in range(n)]


@pytest.mark.parametrize("mask", [0, 1, 2])
@pytest.mark.parametrize("seed", range(6))
def test_plan_pairs_match_oracle(mask, seed):
    rng = np.random.default_rng(1000 + 10 * mask + seed)
    qsegs = _random_segs(rng, 0, int(rng.integers(1, 300)), 16)
    ksegs = _random_segs(rng, 0, int(rng.integers(1, 300)), 16)
    qpos, kpos = _positions(qsegs), _positions(ksegs)
    end = int(max(qpos.max(), kpos.max())) + 1
    cu = None
    if mask == 2:
        cuts = np.sort(rng.choice(np.arange(1, end), min(12, end - 1), replace=False))
        cu = np.concatenate([[0], cuts, [end]]).astype(np.int32)
    a = _attn(mask=mask, cu_seqlens_host=cu)
    if mask == 2:
        a.cu_seqlens_dev = 0x20000
    st, pairs = rba.rba_plan_step(a, qpos.size, rba.make_segs(qsegs), kpos.size, rba.make_segs(ksegs))
    want = oracle.count_pairs(qpos, kpos, mask, cu)
    assert pairs == want
    assert st == (rba.RBA_OK if want else rba.RBA_STEP_EMPTY)


def test_plan_workload_totals():
    # the 32K zigzag rank 3 and the 512K zigzag rank 0 totals over their rings
    for key, want in (("c2", 67_110_912), ("c4", 17_179_901_952)):
        w = W.WORKLOADS[key]
        a = _attn(hq=w.hq, hkv=w.hkv, mask=rba.RBA_MASK_CAUSAL)
        qs = rba.make_segs(w.rank_segments(w.rank))
        tot = 0
        for j in range(w.n_ranks):
            _, p = rba.rba_plan_step(a, w.chunk_len, qs, w.chunk_len, rba.make_segs(w.rank_segments(j)))
            tot += p
        assert tot == want


def test_plan_packed_docs_total():
    w = W.WORKLOADS["c3"]
    cu = W.gen_cu_seqlens(w)
    a = _attn(mask=rba.RBA_MASK_DOC_CAUSAL, cu_seqlens_host=cu)
    a.cu_seqlens_dev = 0x20000
    tot = 0
    nonempty = 0
    for r in range(w.n_ranks):
        for j in range(w.n_ranks):
            st, p = rba.rba_plan_step(a, w.chunk_len, rba.make_segs(w.rank_segments(r)), w.chunk_len,
                                      rba.make_segs(w.rank_segments(j)))
            tot += p
            nonempty += st == rba.RBA_OK
    lens = np.diff(cu.astype(np.int64))
    assert tot == int((lens * (lens + 1) // 2).sum())
    assert 16 <= nonempty < 256


def test_fwd_step_acc_validation():
    lib = rba.load()
    a = _attn(mask=rba.RBA_MASK_NONE)
    f = lib.rba_fwd_step_acc
    args = [ctypes.byref(a), FAKE, 64, ctypes.byref(SEG64), FAKE, FAKE, 64, ctypes.byref(SEG64),
            ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000), None, rba.RBA_BF16, None]
    bad = list(args)
    bad[10], bad[11] = ctypes.c_void_p(0x40000), 9          # final dtype unknown
    assert f(*bad) == rba.RBA_ERR_INVALID
    bad = list(args)
    bad[10] = ctypes.c_void_p(0x20000)                       # o_final aliases o_acc
    assert f(*bad) == rba.RBA_ERR_INVALID
    bad = list(args)
    bad[9] = None                                            # no lse_acc
    assert f(*bad) == rba.RBA_ERR_INVALID
    assert "lse_acc" in rba.rba_last_error()
    ac = _attn()
    empty = list(args)
    empty[0] = ctypes.byref(ac)
    empty[7] = ctypes.byref(rba.make_segs([(64, 64)]))       # keys after every query
    assert f(*empty) == rba.RBA_STEP_EMPTY


# ---------------------------------------------------------------------------
# strided segments

def _plan_rc(a, segs):
    lib = rba.load()
    pairs = ctypes.c_int64(0)
    qs = rba.make_segs(segs)
    return lib.rba_plan_step(ctypes.byref(a), sum(x[1] for x in segs), ctypes.byref(qs), 64,
                             ctypes.byref(SEG64), ctypes.byref(pairs))


def test_strided_segment_overlap_checks():
    a = _attn(mask=rba.RBA_MASK_NONE)
    plan = lambda segs: _plan_rc(a, segs)
    assert plan([(0, 10, 2), (1, 10, 2)]) == rba.RBA_OK              # evens and odds interleave
    assert plan([(0, 6, 3), (1, 6, 3), (2, 6, 3)]) == rba.RBA_OK
    for bad in ([(0, 10, 2), (4, 3, 1)],          # 4 is even
                [(0, 10, 3), (6, 2, 2)],          # 6 = 0 + 2*3
                [(5, 4, 4), (13, 1, 1)],          # 13 = 5 + 2*4
                [(0, 5, 6), (9, 5, 4)]):          # 0,6,...,24 vs 9,13,...,25: disjoint
        rc = _plan_rc(a, bad)
        share = len(set(_strided_positions(bad))) < sum(x[1] for x in bad)
        assert (rc == rba.RBA_ERR_INVALID) == share, (bad, rc)
    assert plan([(0, 5, 6), (3, 5, 6)]) == rba.RBA_OK
    assert _plan_rc(a, [(0, 4, -1)]) == rba.RBA_ERR_INVALID
    assert _plan_rc(a, [(2**30, 4, 2**29)]) == rba.RBA_ERR_UNSUPPORTED       # past position 2^31 - 2


def _strided_positions(segs):
    return np.concatenate([s + d * np.arange(n) for s, n, d in segs]) if segs else np.zeros(0, np.int64)


@pytest.mark.parametrize("mask", [0, 1, 2])
@pytest.mark.parametrize("seed", range(5))
def test_plan_pairs_match_oracle_strided(mask, seed):
    rng = np.random.default_rng(500 + 10 * mask + seed)
    # striped query rows of one rank, and strided or contiguous key runs
    n = int(rng.integers(2, 9))
    qsegs = [(int(rng.integers(0, n)), int(rng.integers(1, 120)), n)]
    r0 = int(rng.integers(0, n))
    ksegs = [(r0, int(rng.integers(1, 80)), n), (int(rng.integers(2000, 2100)), int(rng.integers(1, 50)), 1)]
    qpos, kpos = _strided_positions(qsegs), _strided_positions(ksegs)
    end = int(max(qpos.max(), kpos.max())) + 1
    cu = None
    if mask == 2:
        cuts = np.sort(rng.choice(np.arange(1, end), min(12, end - 1), replace=False))
        cu = np.concatenate([[0], cuts, [end]]).astype(np.int32)
    a = _attn(mask=mask, cu_seqlens_host=cu)
    if mask == 2:
        a.cu_seqlens_dev = 0x20000
    st, pairs = rba.rba_plan_step(a, qpos.size, rba.make_segs(qsegs), kpos.size, rba.make_segs(ksegs))
    want = oracle.count_pairs(qpos, kpos, mask, cu)
    assert pairs == want
    assert st == (rba.RBA_OK if want else rba.RBA_STEP_EMPTY)


@pytest.mark.parametrize("seed", range(8))
def test_strided_overlap_matches_brute_force(seed):
    # the host's progression-intersection test against explicit position sets
    rng = np.random.default_rng(900 + seed)
    a = _attn(mask=rba.RBA_MASK_NONE)
    for _ in range(60):
        k = int(rng.integers(2, 4))
        segs = [(int(rng.integers(0, 60)), int(rng.integers(1, 12)), int(rng.integers(1, 9))) for _ in range(k)]
        pos = _strided_positions(segs)
        share = len(set(pos.tolist())) < pos.size
        rc = _plan_rc(a, segs)
        assert (rc == rba.RBA_ERR_INVALID) == share, segs


def test_merge_thread_map_keeps_each_pair_in_one_wave():
    """For every d rba_merge accepts, the thread map it launches puts all
    threads of a (row, head) pair in one 64-lane wave (the pair's LSE is read
    by all of them and then overwritten in place by one of them), and covers
    each of the pair's d / 4 vectors exactly once.  Every other d is refused
    by both the layout query and rba_merge itself."""
    lib = rba.load()
    for d in range(-8, 1100):
        rc, lpp, vpl, tpw = rba.rba_merge_layout(d)
        accepted = d >= 4 and d <= 1024 and d % 4 == 0
        if not accepted:
            assert rc == rba.RBA_ERR_UNSUPPORTED, d
            assert lib.rba_merge(8, 2, d, FAKE, FAKE, FAKE, FAKE, None, 0, None) == rba.RBA_ERR_UNSUPPORTED, d
            continue
        assert rc == rba.RBA_OK, d
        nv = d // 4
        assert tpw % 64 == 0 and tpw % lpp == 0, (d, lpp, tpw)
        covered = {}
        for t in range(tpw):
            slot, c0 = t // lpp, t % lpp
            covered.setdefault(slot, []).append(t // 64)
            for i in range(vpl):
                c = c0 + i * lpp
                if c < nv:
                    covered.setdefault(("vec", slot), []).append(c)
        for slot in range(tpw // lpp):
            waves = set(covered[slot])
            assert len(waves) == 1, f"d={d}: pair slot {slot} spans waves {sorted(waves)}"
            vecs = sorted(covered[("vec", slot)])
            assert vecs == list(range(nv)), f"d={d}: pair slot {slot} vectors {vecs[:8]}..."


def test_probe_library_exports_its_header():
    """librba_probe.so (the benchmark's measurement probes) exports every
    entry point include/rba_probe.h declares, and rejects bad arguments
    before any launch."""
    from ring_sequence_parallelism_amd import probe
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "rba_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(rba_[a-z_0-9]+)\s*\(", text)))
    assert set(names) == set(probe.EXPORTS)
    lib = probe.load()
    for n in names:
        assert hasattr(lib, n), n
    fl = ctypes.c_double(0)
    assert lib.rba_probe_mfma_bf16(0, 10, FAKE, ctypes.byref(fl), None) == rba.RBA_ERR_INVALID
    assert lib.rba_probe_mfma_bf16(4, 0, FAKE, ctypes.byref(fl), None) == rba.RBA_ERR_INVALID
    assert lib.rba_probe_copy(FAKE, FAKE, 64, 4, None) == rba.RBA_ERR_INVALID          # overlap
    assert lib.rba_probe_copy(FAKE, ctypes.c_void_p(1 << 40), 20, 4, None) == rba.RBA_ERR_INVALID   # not x16


def test_fwd_workspace_size_of_the_packed_document_steps():
    """The host's split plan for the 64K packed-document replay: the steps
    with few rows of work ask for a workspace, never more than 32 MiB; steps
    that already fill the chip ask for none; empty steps report
    RBA_STEP_EMPTY.  Host only (the compute-unit count of a missing device
    reads as 256)."""
    w = W.WORKLOADS["c3"]
    cu = W.gen_cu_seqlens(w)
    a = rba.attn_params(w.hq, w.hkv, w.d, w.scale, rba.RBA_BF16, rba.RBA_MASK_DOC_CAUSAL, None, cu)
    a.cu_seqlens_dev = 0x10000
    lib = rba.load()
    sizes = {}
    for r in range(w.n_ranks):
        for s in range(w.n_ranks):
            j = (r - s) % w.n_ranks
            qs, ks = rba.make_segs(w.rank_runs(r)), rba.make_segs(w.rank_runs(j))
            n = ctypes.c_int64(-1)
            rc = lib.rba_fwd_workspace_size(ctypes.byref(a), 4096, ctypes.byref(qs), 4096, ctypes.byref(ks),
                                            ctypes.byref(n))
            st, pairs = rba.rba_plan_step(a, 4096, qs, 4096, ks)
            assert rc == st
            if st == rba.RBA_STEP_EMPTY:
                assert n.value == 0
                continue
            assert 0 <= n.value <= 32 << 20
            sizes[(r, j)] = (n.value, pairs)
    assert any(b > 0 for b, _ in sizes.values())
    # the whole 4096 x 4096 block of one long document fills the chip: no split
    full = [b for (b, p) in sizes.values() if p == 4096 * 4096]
    assert full and all(b == 0 for b in full)
    # fp32 steps never split
    a32 = rba.attn_params(2, 2, 64, 0.125, rba.RBA_F32, rba.RBA_MASK_NONE)
    n = ctypes.c_int64(-1)
    assert lib.rba_fwd_workspace_size(ctypes.byref(a32), 64, ctypes.byref(rba.make_segs([(0, 64)])), 4096,
                                      ctypes.byref(rba.make_segs([(0, 4096)])), ctypes.byref(n)) == rba.RBA_OK
    assert n.value == 0


def test_fwd_workspace_size_split_regimes():
    """The split planner's two regimes on steps whose tiles are all full
    (queries after every key, causal; 32 q / 8 kv heads, so 8 head groups of
    32-row workgroups, and 512 slots on a missing device's 256 compute
    units): fewer workgroups than one round split (within the 32 MiB
    workspace bound); 608 workgroups of 64
    tiles (1.19 rounds) halve their 12 heaviest row groups, whose partials
    take 2 x 12 x 8 slots of (4 x 32 x 128 + 128) floats; exactly two rounds,
    more than two, or lists shorter than 32 tiles do not split."""
    lib = rba.load()
    a = rba.attn_params(32, 8, 128, 128 ** -0.5, rba.RBA_BF16, rba.RBA_MASK_CAUSAL)

    def size(row_groups, sk):
        n = ctypes.c_int64(-1)
        qs, ks = rba.make_segs([(100000, 32 * row_groups)]), rba.make_segs([(0, sk)])
        assert lib.rba_fwd_workspace_size(ctypes.byref(a), 32 * row_groups, ctypes.byref(qs), sk,
                                          ctypes.byref(ks), ctypes.byref(n)) == rba.RBA_OK
        return n.value

    slot_bytes = (4 * 32 * 128 + 4 * 32) * 4
    assert size(20, 4096) > 0                        # 160 workgroups: under one round
    assert size(76, 4096) == 2 * 12 * 8 * slot_bytes  # 608 workgroups: 12 row groups halved
    assert size(128, 4096) == 0                      # 1024 workgroups: two whole rounds
    assert size(130, 4096) == 0                      # more than two rounds
    assert size(76, 1024) == 0                       # 16 tiles per row group: too short


def test_host_calls_from_several_threads():
    """The planner and the error string are per call / per thread: several
    host threads planning steps at once get each their own pair counts, and
    a thread's error text is not overwritten by another thread's calls."""
    import threading
    lib = rba.load()
    errors, results = [], {}

    def worker(i):
        try:
            a = _attn(mask=rba.RBA_MASK_CAUSAL)
            for rep in range(200):
                n = 64 + i
                st, pairs = rba.rba_plan_step(a, n, rba.make_segs([(0, n)]), n, rba.make_segs([(0, n)]))
                assert st == rba.RBA_OK and pairs == n * (n + 1) // 2
                bad = _attn(d=96)   # rejected: unsupported head dimension
                assert _fwd(bad, 64, SEG64, 64, SEG64) == rba.RBA_ERR_UNSUPPORTED
                msg = lib.rba_last_error().decode()
                assert "96" in msg, msg
            results[i] = True
        except Exception as e:   # collected and re-raised in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[0]
    assert len(results) == 8
