"""Oracle-side token layouts of the sequence-parallel split (test infrastructure).

Written independently of the product's segment builder; tests check that the
two agree.

* Contiguous split: rank r of n holds global positions [r*S/n, (r+1)*S/n).
* Zigzag split (the causal load-balancing variant Zigzag-Ring Attention,
  named in TASP: Topology-aware Sequence Parallelism, experiment highlights):
  the sequence is cut into 2n equal pieces and rank r holds piece r followed
  by piece 2n-1-r.
* Striped split (Striped Attention, in the TASP citation map; only its title
  is on the pages, so the plainest reading of "striped" is taken): token i
  goes to rank i mod n, so rank r holds positions r, r + n, r + 2n, ...
* Ring order (TASP abstract: KV chunks travel around a ring, one per
  iteration): at step s rank r holds the KV chunk of rank (r - s) mod n, so
  step 0 is its own chunk.  The direction is not stated on the pages; the
  merge is order-free, so this only changes rounding.
"""
import numpy as np


def contiguous_positions(seq: int, n: int, r: int) -> np.ndarray:
    if seq % n:
        raise ValueError("sequence length must divide evenly")
    c = seq // n
    return np.arange(r * c, (r + 1) * c, dtype=np.int64)


def zigzag_positions(seq: int, n: int, r: int) -> np.ndarray:
    if seq % (2 * n):
        raise ValueError("sequence length must divide into 2n pieces")
    p = seq // (2 * n)
    first = np.arange(r * p, (r + 1) * p, dtype=np.int64)
    j = 2 * n - 1 - r
    second = np.arange(j * p, (j + 1) * p, dtype=np.int64)
    return np.concatenate([first, second])


def striped_positions(seq: int, n: int, r: int) -> np.ndarray:
    if seq % n:
        raise ValueError("sequence length must divide evenly")
    return np.arange(r, seq, n, dtype=np.int64)


def ring_source(r: int, s: int, n: int) -> int:
    return (r - s) % n
