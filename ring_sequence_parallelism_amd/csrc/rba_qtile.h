// Query-stationary tiling shared by the forward step and the backward dQ
// kernel: a workgroup of 4 waves owns query rows of one or more query heads
// that share a KV head, and walks the key tiles that may hold an allowed key
// for its rows.
#pragma once

#include "rba_device.h"

namespace rba {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBN = kFwdTileKeys;  // keys per tile

// Which rows and head a wave owns, and the
// allowed key interval of the workgroup.
struct WaveTask {
  int g, h, row0;           // kv head, query head, first row of the wave
  int hg;                   // head group of the workgroup
  int wg_row0, wg_rows;     // workgroup row range
  bool wave_any;            // the wave has at least one valid row
  int32_t wq_lo, wq_hi;     // wave query position range
  int32_t wds_lo, wds_hi;   // document starts of wq_lo / wq_hi (doc mask)
  int64_t k_lo, k_hi;       // allowed key positions for the workgroup
  // split launches: the workgroup computes visited tiles [skip, skip +
  // count) of its row group and writes its partial to workspace slot `slot`
  // (-1: the whole visit list, written to the output)
  int skip, count, slot;
  // document mask: start of the document of this lane's row (row0 + lane %
  // 32), INT32_MIN for rows past the chunk and other masks
  int32_t lane_ds;
};

// Which head group and row group a workgroup works on, and for a split
// item the run of tiles and the workspace slot: the first, cheap part of
// the task (no position ranges, no document lookups), enough to address
// the workgroup's query rows.
struct TaskHead {
  int hg, rg;
  int skip, count, slot;
};

// Entry i of a 16-bit table in the kernel arguments, read as the aligned
// 32-bit word that holds it: with a uniform index this is one scalar load,
// where a 16-bit element read is a vector load and a wait on vector memory.
__device__ __forceinline__ int karg_u16(const uint16_t* a, int i) {
  const uint32_t w = reinterpret_cast<const uint32_t*>(a)[i >> 1];
  return (int)((w >> ((i & 1) * 16)) & 0xffffu);
}

__device__ __forceinline__ TaskHead task_head(const FwdParams& p, int logical) {
  TaskHead t;
  t.skip = 0;
  t.count = INT32_MAX;
  t.slot = -1;
  int hg, rg;
  if (!p.split) {
    hg = logical / p.n_rg_launch;       // head group (query heads hg*hpw ...)
    const int rg_i = logical % p.n_rg_launch;
    rg = p.n_order ? karg_u16(p.order, rg_i)
                   : (p.order_reverse ? p.n_row_groups - 1 - rg_i : rg_i);   // heavy first when ordered
  } else {
    // per head group: the split items, the other active row groups, then
    // the row groups without work
    const int per_hg = p.n_items + p.n_row_groups - p.n_active;
    hg = logical / per_hg;
    const int it = logical % per_hg;
    const int n_split_items = karg_u16(p.item_start, p.n_split_rg);
    int i;
    if (it < n_split_items) {
      int lo = 0, hi = p.n_split_rg - 1;   // the last i with item_start[i] <= it
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (karg_u16(p.item_start, mid) <= it) lo = mid; else hi = mid - 1;
      }
      i = lo;
      t.skip = (it - karg_u16(p.item_start, i)) * karg_u16(p.split_len, i);
      t.count = karg_u16(p.split_len, i);
      t.slot = it * p.n_head_groups + hg;
    } else if (it < p.n_items) {
      i = p.n_split_rg + (it - n_split_items);
    } else {
      i = p.n_active + (it - p.n_items);
    }
    rg = karg_u16(p.order, i);
  }
  t.hg = hg;
  t.rg = rg;
  return t;
}

// First query row and query head of a wave of the task.
template <int QR>
__device__ __forceinline__ int task_row0(const FwdParams& p, const TaskHead& th, int wave) {
  return th.rg * p.rbw * QR + (wave / p.hpw) * QR;
}
__device__ __forceinline__ int task_head_index(const FwdParams& p, const TaskHead& th, int wave) {
  return th.hg * p.hpw + wave % p.hpw;
}

// The rest of the task: row and key position ranges, document starts.
template <int QR>
__device__ __forceinline__ WaveTask make_task_from(const FwdParams& p, int wave, const TaskHead& th) {
  WaveTask t;
  t.skip = th.skip;
  t.count = th.count;
  t.slot = th.slot;
  const int hg = th.hg, rg = th.rg;
  t.hg = hg;
  const int hw = wave % p.hpw, rb = wave / p.hpw;
  t.h = hg * p.hpw + hw;
  t.g = t.h / p.group;
  t.wg_row0 = rg * p.rbw * QR;
  t.wg_rows = min(p.rbw * QR, p.sq - t.wg_row0);
  t.row0 = t.wg_row0 + rb * QR;
  const int wr1 = min(t.row0 + QR, p.sq);
  t.wave_any = t.row0 < wr1;
  t.wq_lo = INT32_MAX; t.wq_hi = INT32_MIN; t.wds_lo = INT32_MIN; t.wds_hi = INT32_MIN;
  t.lane_ds = INT32_MIN;
  if (t.wave_any) {
    PosRange r = pos_range(p.qs, t.row0, wr1);
    t.wq_lo = r.lo; t.wq_hi = r.hi;
  }
  PosRange wr = pos_range(p.qs, t.wg_row0, t.wg_row0 + t.wg_rows);
  t.k_lo = kPosNegInf; t.k_hi = kPosPosInf;
  if (p.mask != kMaskNone) t.k_hi = wr.hi;
  if (p.mask == kMaskDoc) {
    // every document lookup of the task, from the table in registers
    const DocLanes dl = doc_lanes(p.cu, p.n_docs, threadIdx.x & 63);
    t.k_lo = doc_start_u(dl, p.cu, p.n_docs, wr.lo);
    if (t.wave_any) {
      t.wds_lo = doc_start_u(dl, p.cu, p.n_docs, t.wq_lo);
      t.wds_hi = doc_start_u(dl, p.cu, p.n_docs, t.wq_hi);
      // the lane's row (rows past the chunk look up the wave's first position)
      const int row = t.row0 + (int)(threadIdx.x & 31);
      const bool ok = row < p.sq;
      const int32_t ds = t.wds_lo == t.wds_hi
                             ? t.wds_lo
                             : doc_start_v(dl, p.cu, p.n_docs, ok ? row_to_pos(p.qs, row) : t.wq_lo);
      t.lane_ds = ok ? ds : INT32_MIN;
    }
  }
  return t;
}

template <int QR>
__device__ __forceinline__ WaveTask make_task(const FwdParams& p, int wave, int block) {
  return make_task_from<QR>(p, wave, task_head(p, xcd_remap(block, p.n_wg)));
}

// Document start of a query row at position qpos of the wave: the wave's
// own document start when all its rows lie in one document (positions
// between wq_lo and wq_hi, whose documents start at wds_lo = wds_hi), else a
// search of cu_seqlens for this row.
__device__ __forceinline__ int32_t wave_doc_start(const FwdParams& p, const WaveTask& t, int32_t qpos) {
  return t.wds_lo == t.wds_hi ? t.wds_lo : doc_start(p.cu, p.n_docs, qpos);
}

// Visits, in row order, every key tile that may hold an allowed key for the
// workgroup: for each KV segment, the rows whose positions fall in
// [k_lo, k_hi].  `body(kt)` is called once per tile.
template <typename F>
__device__ __forceinline__ void for_each_tile(const FwdParams& p, const WaveTask& t, F&& body) {
  int next_tile = 0;
  for (int s = 0; s < p.ks.n; ++s) {
    const int r0 = p.ks.row0[s];
    const RowSpan rs = rows_in(p.ks.start[s], p.ks.stride[s], p.ks.row0[s + 1] - r0, t.k_lo, t.k_hi);
    const int64_t a = rs.a, b = rs.b;
    if (a >= b) continue;
    const int t0 = max((int)((r0 + a) / kBN), next_tile);
    const int t1 = (int)((r0 + b + kBN - 1) / kBN);
    for (int kt = t0; kt < t1; ++kt) body(kt);
    next_tile = max(next_tile, t1);
  }
}

// Iterator over the key tiles for_each_tile visits (same order), so that the
// next tile's loads can be issued before the current tile is computed.
struct TileIter {
  int s, kt, t1, next_tile;
  int valid;   // int, not bool: a padding-free struct stays in registers
  int seg_r0, seg_r1, seg_st, seg_sd;   // rows [seg_r0, seg_r1), first position and stride of segment s
};

__device__ __forceinline__ void tile_next(TileIter& it, const FwdParams& p, const WaveTask& t) {
  ++it.kt;
  while (it.kt >= it.t1) {
    ++it.s;
    if (it.s >= p.ks.n) {
      it.valid = 0;
      return;
    }
    const int r0 = p.ks.row0[it.s];
    it.seg_r0 = r0;
    it.seg_r1 = p.ks.row0[it.s + 1];
    it.seg_st = p.ks.start[it.s];
    it.seg_sd = p.ks.stride[it.s];
    const RowSpan rs = rows_in(it.seg_st, it.seg_sd, it.seg_r1 - r0, t.k_lo, t.k_hi);
    const int64_t a = rs.a, b = rs.b;
    if (a >= b) {
      it.kt = 0;
      it.t1 = 0;
      continue;
    }
    it.kt = max((int)((r0 + a) / kBN), it.next_tile);
    it.t1 = (int)((r0 + b + kBN - 1) / kBN);
    it.next_tile = max(it.next_tile, it.t1);
  }
}

// Position range of key rows [r0, r1) of the tile the iterator is on: from
// the current segment's fields when the rows lie inside it (the common case),
// else from the segment table.
// ONESEG: the caller knows that no key tile spans two KV segments.
template <bool ONESEG = false>
__device__ __forceinline__ PosRange tile_pos_range(const TileIter& it, const SegTable& t, int r0, int r1) {
  if (ONESEG || (r0 >= it.seg_r0 && r1 <= it.seg_r1))
    return PosRange{it.seg_st + (r0 - it.seg_r0) * it.seg_sd, it.seg_st + (r1 - 1 - it.seg_r0) * it.seg_sd, true,
                    it.seg_sd};
  return pos_range(t, r0, r1);
}

// Direct-to-LDS loads of K and V key tiles (kBN rows of one KV head) into
// double-buffered LDS tiles of unpadded, swizzled rows: [buffer][K, V][tile].
// The lane addresses (which row and chunk each lane fetches, and the clamp
// of the last, ragged tile to the chunk's last row) are KvTileAddr's; the
// per-lane offsets of a whole tile are loop invariant and a tile adds a
// uniform base.
template <int D>
struct KvLoader {
  using A = KvTileAddr<D, kBN, kWaves>;
  static constexpr int RB = D * 2;                  // bytes per tile row
  static constexpr int TILE = kBN * RB;             // bytes per K or V tile
  static constexpr int LOADS = A::LOADS;            // per wave per tensor per tile

  const char* kg;       // K and V rows of the KV head (uniform)
  const char* vg;
  uint32_t row_bytes;   // stride of a K/V row in global memory
  int sk, r_lane;
  uint32_t loff0;       // lane offset of load 0 inside a tile
  uint32_t loffs[LOADS];   // lane offset of load i from the tile's first row
  uint32_t lds_wave;    // LDS byte address of this wave's part of buffer 0's K tile

  __device__ __forceinline__ KvLoader(const FwdParams& p, int g, int wave, int lane, uint32_t lds_base) {
    row_bytes = (uint32_t)p.hkv * RB;
    kg = uniform_ptr(static_cast<const char*>(p.k) + (uint32_t)(g * RB));
    vg = uniform_ptr(static_cast<const char*>(p.v) + (uint32_t)(g * RB));
    sk = p.sk;
    r_lane = A::r_lane(wave, lane);
    loff0 = A::loff0(wave, lane, row_bytes);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) loffs[i] = A::whole_off(loff0, i, row_bytes);
    lds_wave = lds_base + wave * LOADS * 1024;
  }

  // Loads key tile kt into buffer b.
  __device__ __forceinline__ void issue(int kt, int b) const {
    const uint32_t dst = lds_wave + b * 2 * TILE;
    const size_t tb = A::tile_base(kt, row_bytes);
    if ((kt + 1) * kBN <= sk) {
      // one scalar base per tensor; the row steps are in the lane offsets
      dma16_kv<LOADS>(kg + tb, vg + tb, loffs, dst, dst + TILE);
      return;
    }
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const uint32_t off = A::ragged_off(kt, i, r_lane, loff0, row_bytes, sk);
      dma16(kg + tb, off, dst + i * 1024);
      dma16(vg + tb, off, dst + TILE + i * 1024);
    }
  }
};

// Sets to -inf the elements of a 32-key block of an S^T accumulator (keys of
// tile rows kb * 32 .. + 31, this lane's query at position qpos with document
// start qd) that the mask does not allow, or that lie past the chunk.  Lane
// (col, half) holds keys kb * 32 + 8 * (j / 4) + 4 * half + j % 4 in element
// j.  Every element is rewritten through a select (no conditional stores
// into the vector).  ONESEG: no key tile spans two KV segments (kr.single
// holds), so the per-element segment search is not compiled in.
template <bool ONESEG = false>
__device__ __forceinline__ void mask_block(f32x16& s, const FwdParams& p, const PosRange& kr, int kr0, int kb,
                                           int half, int32_t qpos, int32_t qd) {
  if (kr.single && kr.stride == 1) {
    // Contiguous positions: element j holds tile row base + c_j (c_j = 8 (j / 4)
    // + j % 4) at position kr.lo + base + c_j, so the mask is a window
    // lo <= c_j <= hi on the lane's row offsets.
    const int base = kb * 32 + 4 * half;
    int hi = p.sk - 1 - kr0 - base;                       // inside the chunk
    int lo = INT32_MIN;
    if (p.mask != kMaskNone) {
      hi = qpos == kPosNone ? -1 : min(hi, qpos - kr.lo - base);   // at or before the query
      if (p.mask == kMaskDoc) lo = qd - kr.lo - base;                // in the query's document
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int c = 8 * (j >> 2) + (j & 3);
      s[j] = (c <= hi && c >= lo) ? s[j] : -INFINITY;
    }
    return;
  }
  int32_t kp[16];
  if (ONESEG || kr.single) {
#pragma unroll
    for (int j = 0; j < 16; ++j) kp[j] = kr.lo + (kb * 32 + 8 * (j >> 2) + 4 * half + (j & 3)) * kr.stride;
  } else {
    for (int j = 0; j < 16; ++j) {
      const int krow = kr0 + kb * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
      kp[j] = krow < p.sk ? row_to_pos(p.ks, krow) : 0;
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const bool kin = kr0 + kb * 32 + 8 * (j >> 2) + 4 * half + (j & 3) < p.sk;
    const bool ok = kin && visible(p.mask, kp[j], qpos, qd);
    s[j] = ok ? s[j] : -INFINITY;
  }
}

// Writes one lane's share of a query row's step result: O = oacc / l (this
// lane's 16 elements of each 32-column block db: d = 32 db + 8 (j / 4) +
// 4 half + j % 4, four consecutive d per vector) and the row's LSE.  Rows
// with no allowed key have inv = 0 and lse = -inf.  In accumulate mode the
// result is merged into the running (O, LSE) instead (merge_weights), and
// the merged O is also written to o_final when one is given.  Both lanes of
// a row read the running LSE before either writes it (the write depends on
// the read's value).
template <int D>
__device__ __forceinline__ void write_step_output(const FwdParams& p, int row, int h, int half,
                                                  const f32x16 (&oacc)[D / 32], float inv, float lse) {
  if (row >= p.sq) return;
  const size_t li = (size_t)h * p.sq + row;
  const size_t oi = ((size_t)row * p.hq + h) * D;
  float* dst = p.o + oi;
  if (!p.accumulate) {
    if (half == 0) p.lse[li] = lse;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 val = {oacc[db][4 * jj] * inv, oacc[db][4 * jj + 1] * inv, oacc[db][4 * jj + 2] * inv,
                           oacc[db][4 * jj + 3] * inv};
        *reinterpret_cast<f32x4*>(dst + db * 32 + 8 * jj + 4 * half) = val;
      }
    return;
  }
  // An empty partial merges as the identity: the row's running result is
  // neither read nor written, and only read for the final output when that
  // is due (the merge weights are then exactly 1 and 0).
  const bool empty = lse == -INFINITY;
  if (empty && !p.o_final) return;
  f32x4 old[D / 32][4];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) old[db][jj] = *reinterpret_cast<const f32x4*>(dst + db * 32 + 8 * jj + 4 * half);
  const MergeWeights w = merge_weights(p.lse[li], lse);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 part = {oacc[db][4 * jj] * inv, oacc[db][4 * jj + 1] * inv, oacc[db][4 * jj + 2] * inv,
                          oacc[db][4 * jj + 3] * inv};
      const f32x4 o = w.wa * old[db][jj] + w.wb * part;
      const int c = db * 32 + 8 * jj + 4 * half;
      if (!empty) *reinterpret_cast<f32x4*>(dst + c) = o;
      if (p.o_final) {
        if (p.final_bf16) {
          const u32x2 b = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o_final) + oi + c) = b;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.o_final) + oi + c) = o;
        }
      }
    }
  if (half == 0 && !empty) p.lse[li] = w.L;
}

// The final output of a merging step's workgroup whose row group has no key
// in the step: the running result unchanged (an empty partial merges as the
// identity), converted.  Each wave copies its 32 rows of one head with
// consecutive lanes on consecutive 16-byte pieces of a row.
template <int D, int QR>
__device__ __forceinline__ void copy_running_to_final(const FwdParams& p, const TaskHead& th, int wave, int lane) {
  constexpr int CPR4 = D / 4;   // f32x4 pieces per row
  static_assert(QR * CPR4 % 64 == 0, "whole passes of the wave");
  const int row0 = task_row0<QR>(p, th, wave), h = task_head_index(p, th, wave);
#pragma unroll 4
  for (int i = 0; i < QR * CPR4 / 64; ++i) {
    const int c = i * 64 + lane;
    const int row = row0 + c / CPR4;
    if (row >= p.sq) continue;
    const size_t oi = ((size_t)row * p.hq + h) * D + 4 * (c % CPR4);
    const f32x4 o = *reinterpret_cast<const f32x4*>(p.o + oi);
    if (p.final_bf16) {
      const u32x2 b = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o_final) + oi) = b;
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(p.o_final) + oi) = o;
    }
  }
}

// The merging epilogue of one wave (32 rows of one head) with coalesced
// global accesses.  Each lane scales its accumulator share by the partial's
// merge weight (wb / l) into the wave's 32 x D fp32 block of LDS (16-byte
// pieces XOR-swizzled by row); after a workgroup barrier lane l takes piece
// l % 32 of rows 2 i + l / 32, i = 0..15: it loads the running output of
// all 16 at once, then adds wa times each to the partial and stores the
// merged rows (and the final output), each half-wave one whole row per
// instruction.  A row whose partial is empty keeps its running output and
// LSE untouched (weights exactly 1 and 0).  All four waves call it (it
// holds two workgroup barriers); `w_lds` is the wave's LDS block.
template <int D>
__device__ __forceinline__ void merge_step_output_coalesced(const FwdParams& p, int row0, int h, int lane,
                                                            const f32x16 (&oacc)[D / 32], float inv, float lse,
                                                            float* w_lds) {
  constexpr int P = D / 4;                  // 16-byte pieces per row
  const int col = lane & 31, half = lane >> 5, q = lane & 31;
  const int row = row0 + col;
  const bool row_ok = row < p.sq;
  const size_t li = (size_t)h * p.sq + (row_ok ? row : 0);
  const float la = row_ok ? p.lse[li] : -INFINITY;
  const bool empty = lse == -INFINITY;
  const MergeWeights w = merge_weights(la, lse);
  const float sb = w.wb * inv;
  // per row, read by the other lanes through a shuffle: wa; -1 for a row
  // that keeps its running result and writes nothing (and rows past the
  // chunk); with the final output due and an empty partial, 2 (the running
  // result is final as it is) or 3 (neither side has a key: zeros)
  const float wa_row = (!row_ok || (empty && !p.o_final)) ? -1.f : (empty ? (la == -INFINITY ? 3.f : 2.f) : w.wa);
  __syncthreads();   // every wave is done with the tile buffers
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int pc = db * 8 + 2 * jj + half;   // piece of d = 4 pc .. 4 pc + 3
      const f32x4 v = {oacc[db][4 * jj] * sb, oacc[db][4 * jj + 1] * sb, oacc[db][4 * jj + 2] * sb,
                       oacc[db][4 * jj + 3] * sb};
      *reinterpret_cast<f32x4*>(w_lds + col * D + 4 * (pc ^ (col % P))) = v;
    }
  if (half == 0 && row_ok && !empty) p.lse[li] = w.L;
  __syncthreads();
  // every load first (rows past the chunk read its last row, unused), then
  // the merge and the stores
  float wa[16];
  f32x4 old[16], part[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 2 * i + half;
    wa[i] = __shfl(wa_row, r);
    const size_t oi = ((size_t)min(row0 + r, p.sq - 1) * p.hq + h) * D + 4 * min(q, P - 1);
    old[i] = *reinterpret_cast<const f32x4*>(p.o + oi);
    part[i] = *reinterpret_cast<const f32x4*>(w_lds + r * D + 4 * (min(q, P - 1) ^ (r % P)));
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 2 * i + half;
    if (q >= P || wa[i] < 0.f) continue;
    const size_t oi = ((size_t)(row0 + r) * p.hq + h) * D + 4 * q;
    f32x4 o;
    if (wa[i] > 1.5f) {
      o = wa[i] > 2.5f ? f32x4{0.f, 0.f, 0.f, 0.f} : old[i];   // empty partial, final output due
    } else {
      o = wa[i] * old[i] + part[i];
      *reinterpret_cast<f32x4*>(p.o + oi) = o;
    }
    if (p.o_final) {
      if (p.final_bf16) {
        const u32x2 b = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o_final) + oi) = b;
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(p.o_final) + oi) = o;
      }
    }
  }
}

// Writes one lane's share of a split item's partial (O = oacc / l, the
// row's LSE) into its workspace slot: wave w's rows at floats
// [w * 32 * D, (w + 1) * 32 * D) (row-major, D per row), their LSE at
// 128 * D + w * 32 + row.  Rows past the chunk hold (0, -inf).
template <int D>
__device__ __forceinline__ void write_split_partial(const FwdParams& p, int slot, int wave, int col, int half,
                                                    const f32x16 (&oacc)[D / 32], float inv, float lse) {
  float* base = p.ws + (size_t)slot * split_slot_floats(D);
  float* dst = base + (size_t)(wave * 32 + col) * D;
  if (half == 0) base[128 * D + wave * 32 + col] = lse;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 val = {oacc[db][4 * jj] * inv, oacc[db][4 * jj + 1] * inv, oacc[db][4 * jj + 2] * inv,
                         oacc[db][4 * jj + 3] * inv};
      *reinterpret_cast<f32x4*>(dst + db * 32 + 8 * jj + 4 * half) = val;
    }
}

}  // namespace rba
