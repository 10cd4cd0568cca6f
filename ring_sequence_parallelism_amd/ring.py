"""One rank's ring, replayed on one GPU.

Ring Attention (TASP: Topology-aware Sequence Parallelism, abstract) keeps a
rank's query chunk in place while the KV chunks of all ranks pass by, one
per ring iteration.  Here every KV chunk is resident on the one GPU and the
iterations are replayed in ring order: at step s rank r holds the KV chunk
of rank (r - s) mod n.  Each step calls rba_fwd_step; the partials are
folded with rba_merge (the last merge also writes the bf16/fp32 output), and
steps the host proves empty launch nothing.  The backward replays the same
steps with rba_bwd_step after one rba_bwd_preprocess.

Device memory comes from torch; every arithmetic step runs in librba.so.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch

from . import rba
from . import workloads as W

_MASKS = {W.MASK_NONE: rba.RBA_MASK_NONE, W.MASK_CAUSAL: rba.RBA_MASK_CAUSAL,
          W.MASK_DOC_CAUSAL: rba.RBA_MASK_DOC_CAUSAL}


def to_device(x: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Upload generator output: uint16 bf16 bits -> torch.bfloat16, float32 as is."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def ring_order(r: int, n: int) -> List[int]:
    return [(r - s) % n for s in range(n)]


@dataclasses.dataclass
class StepInfo:
    src: int           # KV chunk (source rank) of this step
    status: int        # RBA_OK or RBA_STEP_EMPTY from host planning
    pairs: int         # allowed (query, key) pairs per query head


class RingReplay:
    """Device-resident inputs and buffers of one rank's ring replay."""

    def __init__(self, w: W.Workload, rank: Optional[int] = None, device="cuda",
                 kv_sources: Optional[List[int]] = None, with_grad: bool = False,
                 order: Optional[List[int]] = None, kv: Optional[Dict[str, Dict[int, torch.Tensor]]] = None,
                 workspace: Optional[torch.Tensor] = None):
        """``order``: the KV chunks of the steps in replay order (default: ring
        order; a caller may permute, drop or repeat chunks).  ``kv``: device
        K / V chunks already made for this workload ({"k": {j: tensor},
        "v": {j: tensor}}), shared instead of generated again.
        ``workspace``: a device buffer handed to rba_fwd_step_ws, which lets
        steps with few rows of work split their key ranges over more
        workgroups (None: rba_fwd_step / rba_fwd_step_acc, never split)."""
        self.workspace = workspace
        self.w = w
        self.r = w.rank if rank is None else rank
        self.device = torch.device(device)
        self.dtype = rba.RBA_BF16 if w.dtype == "bf16" else rba.RBA_F32
        n = w.n_ranks
        self.order = ring_order(self.r, n) if order is None else list(order)
        srcs = sorted(set(self.order if kv_sources is None else kv_sources))
        # inputs
        self.q = to_device(W.gen_rank_chunk(w, W.T_Q, self.r), w.dtype, self.device)
        self.q_segs = rba.make_segs(w.rank_runs(self.r))
        self._shared_kv = kv
        self.order = self._build_kv(srcs)
        self.cu_host = None
        self.cu_dev = None
        if w.mask == W.MASK_DOC_CAUSAL:
            self.cu_host = W.gen_cu_seqlens(w)
            self.cu_dev = torch.from_numpy(self.cu_host.astype(np.int32)).to(self.device)
        self.attn = rba.attn_params(w.hq, w.hkv, w.d, w.scale, self.dtype, _MASKS[w.mask],
                                    self.cu_dev, self.cu_host)
        # host plan of every step
        sq = self.q.shape[0]
        self.steps: List[StepInfo] = []
        for j in self.order:
            if kv_sources is not None and j not in self.k:
                continue
            st, pairs = rba.rba_plan_step(self.attn, sq, self.q_segs, self.k[j].shape[0], self.kv_segs[j])
            self.steps.append(StepInfo(j, st, pairs))
        # forward buffers
        hq, d = w.hq, w.d
        f32 = dict(dtype=torch.float32, device=self.device)
        self.o_acc = torch.empty((sq, hq, d), **f32)
        self.lse_acc = torch.empty((hq, sq), **f32)
        self.o_part = torch.empty((sq, hq, d), **f32)
        self.lse_part = torch.empty((hq, sq), **f32)
        out_dtype = torch.bfloat16 if self.dtype == rba.RBA_BF16 else torch.float32
        self.o_final = torch.empty((sq, hq, d), dtype=out_dtype, device=self.device)
        self.with_grad = with_grad
        if with_grad:
            self.d_o = to_device(W.gen_rank_chunk(w, W.T_DO, self.r), w.dtype, self.device)
            self.delta = torch.empty((hq, sq), **f32)
            self.dq = torch.empty((sq, hq, d), **f32)
            self.dk = {s.src: torch.empty((self.k[s.src].shape[0], w.hkv, d), **f32) for s in self.steps}
            self.dv = {s.src: torch.empty((self.k[s.src].shape[0], w.hkv, d), **f32) for s in self.steps}

    def _build_kv(self, srcs):
        """Device K / V and segments of every step, keyed as the steps are;
        returns the step keys in replay order."""
        w = self.w
        shared = self._shared_kv or {"k": {}, "v": {}}
        self.k = {j: shared["k"][j] if j in shared["k"] else to_device(W.gen_rank_chunk(w, W.T_K, j), w.dtype,
                                                                        self.device) for j in srcs}
        self.v = {j: shared["v"][j] if j in shared["v"] else to_device(W.gen_rank_chunk(w, W.T_V, j), w.dtype,
                                                                        self.device) for j in srcs}
        self.kv_segs = {j: rba.make_segs(w.rank_runs(j)) for j in srcs}
        return self.order

    # -- forward -----------------------------------------------------------
    @property
    def effective_pairs(self) -> int:
        return sum(s.pairs for s in self.steps)

    def fwd_flops(self) -> int:
        """Effective forward FLOPs: 4*d per allowed pair and query head."""
        return 4 * self.w.d * self.w.hq * self.effective_pairs

    def bwd_flops(self) -> int:
        """Effective backward FLOPs: 10*d per allowed pair and query head (5 contractions)."""
        return 10 * self.w.d * self.w.hq * self.effective_pairs

    def fwd_step(self, i: int, into_acc: bool, stream=None) -> int:
        s = self.steps[i]
        o, l = (self.o_acc, self.lse_acc) if into_acc else (self.o_part, self.lse_part)
        if self.workspace is not None:
            return rba.rba_fwd_step_ws(self.attn, self.q, self.q_segs, self.k[s.src], self.v[s.src],
                                       self.kv_segs[s.src], o, l, False, None, rba.RBA_BF16, self.workspace, stream)
        return rba.rba_fwd_step(self.attn, self.q, self.q_segs, self.k[s.src], self.v[s.src],
                                self.kv_segs[s.src], o, l, stream)

    def fwd_step_acc(self, i: int, o_final=None, final_dtype: int = rba.RBA_BF16, stream=None) -> int:
        s = self.steps[i]
        if self.workspace is not None:
            return rba.rba_fwd_step_ws(self.attn, self.q, self.q_segs, self.k[s.src], self.v[s.src],
                                       self.kv_segs[s.src], self.o_acc, self.lse_acc, True, o_final, final_dtype,
                                       self.workspace, stream)
        return rba.rba_fwd_step_acc(self.attn, self.q, self.q_segs, self.k[s.src], self.v[s.src],
                                    self.kv_segs[s.src], self.o_acc, self.lse_acc, o_final, final_dtype, stream)

    def forward(self, stream=None, on_step=None, fused_merge: bool = True, resume: bool = False) -> torch.Tensor:
        """Replay all steps; returns o_final (merged output in the input dtype).

        The first live step writes the running result (o_acc, lse_acc); each
        later one is merged into it by rba_fwd_step_acc in the same launch
        (``fused_merge``, the last one also writing o_final), or, with
        ``fused_merge=False``, goes through o_part / lse_part and rba_merge.
        With ``resume`` (fused merges only) (o_acc, lse_acc) already hold the
        result of earlier steps, restored by the caller, and every step is
        merged into it.
        ``on_step(kind, i)`` is called before each launch ("fwd" / "merge") so
        a caller can bracket launches with events.
        """
        live = [i for i, s in enumerate(self.steps) if s.status == rba.RBA_OK]
        final_dtype = rba.RBA_BF16 if self.dtype == rba.RBA_BF16 else rba.RBA_F32
        if resume and not fused_merge:
            raise ValueError("resume merges every step in its launch (fused_merge=True)")
        if not live:
            if not resume:
                self.o_acc.zero_()
                self.lse_acc.fill_(float("-inf"))
            rba.rba_merge(self.o_acc, self.lse_acc, None, None, self.o_final, final_dtype, stream)
            return self.o_final
        for n_done, i in enumerate(live):
            first = n_done == 0 and not resume
            last = n_done == len(live) - 1
            if on_step:
                on_step("fwd", i)
            if first or not fused_merge:
                st = self.fwd_step(i, into_acc=first, stream=stream)
            else:
                st = self.fwd_step_acc(i, self.o_final if last else None, final_dtype, stream)
            assert st == rba.RBA_OK, "host plan and step status disagree"
            if not first and not fused_merge:
                if on_step:
                    on_step("merge", i)
                rba.rba_merge(self.o_acc, self.lse_acc, self.o_part, self.lse_part,
                              self.o_final if last else None, final_dtype, stream)
        if len(live) == 1 and not resume:
            rba.rba_merge(self.o_acc, self.lse_acc, None, None, self.o_final, final_dtype, stream)
        return self.o_final

    # -- backward ----------------------------------------------------------
    def backward(self, o_saved: Optional[torch.Tensor] = None, lse_saved: Optional[torch.Tensor] = None,
                 stream=None, on_step=None, dk_acc=None, dv_acc=None):
        """dq (fp32, accumulated over steps) and per-step dk / dv by step key.

        Uses the forward's merged output (the fp32 accumulator by default) and
        merged LSE.  Steps the host proves empty leave their dk / dv zero.
        With ``dk_acc`` / ``dv_acc`` (dicts by step key of [sk, hkv, d] fp32
        tensors, the accumulators that travel with each KV chunk) the steps
        add into those with rba_bwd_step_acc instead, and those are returned.
        """
        assert self.with_grad
        o_saved = self.o_acc if o_saved is None else o_saved
        lse_saved = self.lse_acc if lse_saved is None else lse_saved
        acc = dk_acc is not None
        if on_step:
            on_step("prep", -1)
        rba.rba_bwd_preprocess(o_saved, self.d_o, self.delta, stream)
        self.dq.zero_()
        for i, s in enumerate(self.steps):
            if s.status != rba.RBA_OK:
                if not acc:
                    self.dk[s.src].zero_()
                    self.dv[s.src].zero_()
                continue
            if on_step:
                on_step("bwd", i)
            step = rba.rba_bwd_step_acc if acc else rba.rba_bwd_step
            dk = dk_acc[s.src] if acc else self.dk[s.src]
            dv = dv_acc[s.src] if acc else self.dv[s.src]
            st = step(self.attn, self.q, self.q_segs, self.k[s.src], self.v[s.src], self.kv_segs[s.src],
                      self.d_o, lse_saved, self.delta, self.dq, dk, dv, stream)
            assert st == rba.RBA_OK
        return (self.dq, dk_acc, dv_acc) if acc else (self.dq, self.dk, self.dv)


class TaspReplay(RingReplay):
    """One rank's ring under TASP's decomposed schedule (see tasp.py).

    Iteration 0 is the rank's own chunk; iteration s >= 1 is the union of the
    n - 1 slices the rank holds then, one per Hamiltonian cycle, assembled in
    cycle order into one KV buffer (standing in for the receive buffer the
    transfers would fill) and passed to rba_fwd_step / rba_bwd_step with the
    slices' position segments.  Steps are keyed by iteration: ``k[s]``,
    ``v[s]``, ``kv_segs[s]``, ``dk[s]``, ``dv[s]`` and ``slices[s]``.
    """

    def __init__(self, w: W.Workload, rank: Optional[int] = None, device="cuda", with_grad: bool = False,
                 schedule=None):
        from . import tasp
        self.schedule = schedule if schedule is not None else tasp.TaspSchedule(w.n_ranks)
        if self.schedule.n != w.n_ranks:
            raise ValueError("schedule is for a different number of ranks")
        r = w.rank if rank is None else rank
        self.slices = [self.schedule.step_slices(r, it, w.chunk_len) for it in range(w.n_ranks)]
        segs = [tasp.step_segments(w, sl) for sl in self.slices]
        if max(len(x) for x in segs) > rba.RBA_MAX_SEGS:
            raise ValueError("a step has more position segments than rba_segs holds")
        self._tasp_segs = segs
        super().__init__(w, r, device, kv_sources=None, with_grad=with_grad)

    def _build_kv(self, srcs):
        w = self.w
        chunk_k = {j: to_device(W.gen_rank_chunk(w, W.T_K, j), w.dtype, self.device) for j in range(w.n_ranks)}
        chunk_v = {j: to_device(W.gen_rank_chunk(w, W.T_V, j), w.dtype, self.device) for j in range(w.n_ranks)}
        self.k, self.v, self.kv_segs = {}, {}, {}
        for it, sl in enumerate(self.slices):
            self.k[it] = torch.cat([chunk_k[x.src][x.rows[0]:x.rows[1]] for x in sl]).contiguous()
            self.v[it] = torch.cat([chunk_v[x.src][x.rows[0]:x.rows[1]] for x in sl]).contiguous()
            self.kv_segs[it] = rba.make_segs(self._tasp_segs[it])
        del chunk_k, chunk_v
        return list(range(w.n_ranks))


def full_ring_backward(w: W.Workload, device="cuda", stream=None):
    """The backward of every rank's ring on one GPU, KV-side gradients summed
    at their owners: returns dq per rank and dk, dv per chunk (fp32), i.e. the
    gradients of sum dO * O over the whole sequence.  Each rank's replay adds
    into the accumulators of the chunks it meets (rba_bwd_step_acc), as the
    accumulators travelling with the KV chunks would in a real ring."""
    dk_acc: Dict[int, torch.Tensor] = {}
    dv_acc: Dict[int, torch.Tensor] = {}
    dq = {}
    for r in range(w.n_ranks):
        rr = RingReplay(w, r, device, with_grad=True)
        if not dk_acc:
            for j in range(w.n_ranks):
                dk_acc[j] = torch.zeros((w.chunk_len, w.hkv, w.d), dtype=torch.float32, device=rr.device)
                dv_acc[j] = torch.zeros_like(dk_acc[j])
        rr.forward(stream)
        d, _, _ = rr.backward(stream=stream, dk_acc=dk_acc, dv_acc=dv_acc)
        dq[r] = d.clone()
        del rr
    return dq, dk_acc, dv_acc
