"""rba — ring block attention on MI355X (gfx950).

The per-device hot path of Ring Attention and TASP: one query chunk against
one arriving KV chunk, emitting a partial output and its log-sum-exp, the
LSE-weighted merge of partials, and the matching backward step.  The compute
runs in hand-written HIP kernels behind a C ABI (``include/rba.h``); the
Python side only marshals arguments (``ring_sequence_parallelism_amd.rba``)
and replays one rank's ring on one GPU (``ring_sequence_parallelism_amd.ring``).

Submodules are imported on demand so that loading the seeded input
generator does not load the HIP library.
"""
__version__ = "0.1.0"
