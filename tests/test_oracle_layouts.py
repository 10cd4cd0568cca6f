"""Pins of the oracle's layouts and pair counts, and checks of the seeded inputs.

Layouts are pinned to the workload text: 16 pieces of 2048 tokens over 8
ranks, rank 3 holds pieces 3 and 12 (positions 6144-8191 and 24576-26623).
Pair counts are pinned to closed forms: a zigzag rank with pieces of n_p
tokens over n ranks has 2 n n_p^2 + n_p causal pairs per head, and a packed
buffer of documents L_t has sum L_t (L_t + 1) / 2 document-causal pairs.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from ring_sequence_parallelism_amd import workloads as W


def test_zigzag_rank3_of_8():
    pos = oracle.zigzag_positions(32768, 8, 3)
    assert pos.size == 4096
    assert np.array_equal(pos[:2048], np.arange(6144, 8192))
    assert np.array_equal(pos[2048:], np.arange(24576, 26624))


def test_zigzag_covers_sequence_once():
    seq, n = 96, 3
    allpos = np.concatenate([oracle.zigzag_positions(seq, n, r) for r in range(n)])
    assert np.array_equal(np.sort(allpos), np.arange(seq))


def test_contiguous():
    assert np.array_equal(oracle.contiguous_positions(2048, 4, 2), np.arange(1024, 1536))


def test_ring_order_rank3():
    assert [oracle.ring_source(3, s, 8) for s in range(8)] == [3, 2, 1, 0, 7, 6, 5, 4]


@pytest.mark.parametrize("n,n_p", [(1, 8), (2, 5), (3, 7), (4, 16)])
def test_zigzag_pair_count_closed_form(n, n_p):
    seq = 2 * n * n_p
    for r in range(n):
        qpos = oracle.zigzag_positions(seq, n, r)
        assert oracle.count_pairs(qpos, np.arange(seq), oracle.MASK_CAUSAL) == 2 * n * n_p * n_p + n_p


def test_workload_pair_counts():
    # rank 3 of the 32K zigzag workload against all keys: 67,110,912 per head
    qpos = oracle.zigzag_positions(32768, 8, 3)
    assert oracle.count_pairs(qpos, np.arange(32768), oracle.MASK_CAUSAL) == 67_110_912
    # 512K zigzag: each row at position p sees p + 1 keys
    qpos = oracle.zigzag_positions(524288, 8, 0)
    assert int((qpos + 1).sum()) == 17_179_901_952


def test_doc_pair_count_closed_form():
    rng = np.random.default_rng(0)
    lens = rng.integers(1, 40, size=9)
    cu = np.concatenate([[0], np.cumsum(lens)])
    pos = np.arange(cu[-1])
    assert oracle.count_pairs(pos, pos, oracle.MASK_DOC_CAUSAL, cu) == int((lens * (lens + 1) // 2).sum())


# ---------------------------------------------------------------------------
# Seeded inputs (shared by both sides; inputs only)

def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 3,
                        np.array([1.00390625, 1.01171875, -2.00781250, 65504.0, 1e-40], dtype=np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_pieces_are_reproducible_and_independent():
    w = W.scaled_workload(W.WORKLOADS["c2"], 1024, hq=4, hkv=2, d=16)
    a = W.gen_piece(w, W.T_K, 3)
    b = W.gen_piece(w, W.T_K, 3)
    c = W.gen_piece(w, W.T_K, 4)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    chunk = W.gen_rank_chunk(w, W.T_K, 1)
    assert np.array_equal(chunk[: w.piece_len], W.gen_piece(w, W.T_K, 1))
    assert np.array_equal(chunk[w.piece_len:], W.gen_piece(w, W.T_K, 2 * w.n_ranks - 2))


def test_value_scale_and_distribution():
    w = W.WORKLOADS["c1"]
    x = W.gen_piece(w, W.T_Q, 0)
    assert x.dtype == np.float32 and x.shape == (512, 2, 64)
    assert abs(x.std() - 0.5) < 0.02


def test_doc_sampler():
    w = W.WORKLOADS["c3"]
    lens = W.gen_doc_lengths(w)
    assert lens.sum() == 65536
    assert (lens[:-1] >= 256).all() and (lens <= 16384).all()
    cu = W.gen_cu_seqlens(w)
    assert cu[0] == 0 and cu[-1] == 65536 and np.all(np.diff(cu) > 0)
    assert np.array_equal(cu, W.gen_cu_seqlens(w))


def test_sampled_rows():
    w = W.WORKLOADS["c4"]
    rows = W.gen_sampled_rows(w, 256, w.chunk_len)
    assert rows.size == 256 and len(set(rows.tolist())) == 256
    for r in (0, 32767, 32768, 65535):
        assert r in rows


def test_workload_segments_match_oracle_layouts():
    for key, w in W.WORKLOADS.items():
        for r in range(w.n_ranks):
            segs = w.rank_segments(r)
            pos = np.concatenate([np.arange(s, s + n) for s, n in segs])
            if w.layout == "zigzag":
                ref = oracle.zigzag_positions(w.seq, w.n_ranks, r)
            else:
                ref = oracle.contiguous_positions(w.seq, w.n_ranks, r)
            assert np.array_equal(pos, ref), (key, r)


# ---------------------------------------------------------------------------
# striped layout (token i on rank i mod n)

@pytest.mark.parametrize("seq,n", [(32, 4), (4096, 8), (96, 3)])
def test_striped_positions_partition_and_residues(seq, n):
    allp = np.concatenate([oracle.striped_positions(seq, n, r) for r in range(n)])
    assert np.array_equal(np.sort(allp), np.arange(seq))
    for r in range(n):
        p = oracle.striped_positions(seq, n, r)
        assert (p % n == r).all() and np.all(np.diff(p) == n)


@pytest.mark.parametrize("r", [0, 3, 7])
def test_striped_causal_pairs_closed_form(r):
    # rank r's queries against the whole sequence, causal: the row at
    # position r + n a sees r + n a + 1 keys, so the total is
    # c (r + 1) + n c (c - 1) / 2 for c = S / n rows
    seq, n = 512, 8
    c = seq // n
    qpos = oracle.striped_positions(seq, n, r)
    want = c * (r + 1) + n * c * (c - 1) // 2
    assert oracle.count_pairs(qpos, np.arange(seq), oracle.MASK_CAUSAL) == want


def test_striped_workload_chunk_rows():
    # the generator's striped chunk is every n-th row of the position-ordered sequence
    w = W.scaled_workload(W.WORKLOADS["c2"], 256, hq=2, hkv=1, d=64)
    w = dataclasses.replace(w, layout="striped")
    full = W.gen_pieces(w, W.T_K, range(w.n_pieces))
    for r in (0, 5):
        chunk = W.gen_rank_chunk(w, W.T_K, r)
        assert np.array_equal(chunk, full[oracle.striped_positions(w.seq, w.n_ranks, r)])
    assert w.rank_runs(5) == [(5, w.chunk_len, w.n_ranks)]
