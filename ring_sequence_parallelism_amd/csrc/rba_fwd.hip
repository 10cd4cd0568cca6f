// Forward ring step: blockwise exact softmax attention of a query chunk
// against one KV chunk, emitting the partial output and its log-sum-exp.
//
// What is computed (TASP: Topology-aware Sequence Parallelism, abstract: a
// query chunk attends to one arriving KV chunk per ring iteration; the
// blockwise exact scheme with a running maximum and sum is that of
// FlashAttention / FlashAttention-2, named in its citation map):
//   for each query row i and head h, over the allowed keys j of this chunk,
//   O_i = sum_j softmax_j(scale * <q_i, k_j>) v_j  and  LSE_i = ln sum_j e^{s_ij}.
//
// gfx950 design
//   * A workgroup is 4 waves sharing one KV head: wave w takes query head
//     (w % hpw) of the group's heads and row block (w / hpw), so every K/V
//     tile staged in LDS feeds 4 waves (4 GQA heads of the same rows when the
//     group has 4 or more heads).
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: each lane owns one query column, so the row
//     max and sum over the 32 keys of a block are 15 in-lane ops plus one
//     v_permlane32_swap, and the fp32 accumulator of S^T converts in place to
//     the B operand of O^T += V^T P^T (no LDS round trip for P).
//   * Q^T stays in registers for the whole key loop.  K and V tiles stream
//     from HBM straight into double-buffered LDS (global_load_lds, 16 bytes
//     per lane, no register staging) while the previous tile is computed;
//     rows are unpadded with an XOR swizzle of their 16-byte chunks.  V is
//     read as the A operand of PV through the LDS transpose load, in the
//     key order the P^T accumulator rows imply.  One barrier per tile.
//   * Key tiles outside the allowed position interval of the workgroup are
//     never visited; inside it, each wave classifies a tile as full (no mask
//     arithmetic) or partial (per-element mask; a tile wholly masked for
//     one wave but needed by another is computed masked, so the tile body
//     has no branch around it).
//     Steps whose visited tiles the host has shown to be all full run an
//     instantiation with no classification and no mask code.
//   * Scheduling groups keep 6 K reads in flight ahead of the score MFMAs.
//   * Softmax runs in base 2 with scale*log2(e) folded into one FMA per score,
//     and a lazy running maximum that rarely rescales O.
#include <type_traits>

#include "rba_qtile.h"

namespace rba {

// floor(a / b) for b > 0.
__device__ __forceinline__ int floor_div_i32(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// FULL: every visited tile is full for every wave (shown on the host), so
// the tile body has no classification and no mask code.  ONESEG: no key tile
// spans two KV segments (every segment boundary on a tile boundary, shown on
// the host), so the masked path has no per-element segment search.
template <int D, int NQB, bool FULL, bool ONESEG>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(FwdParams p) {
  constexpr int QR = 32 * NQB;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int RB = D * 2;                  // bytes per row (no padding: swizzled)
  constexpr int TILE = kBN * RB;             // bytes per K or V tile
  // [buffer][K, V] tiles, double-buffered: tile t is computed from buffer t % 2
  // while tile t + 1 streams into the other one.
  __shared__ __attribute__((aligned(16))) char lds[2][2][TILE];
  // the merging epilogue reuses the tile buffers: one 32-row fp32 block per wave
  static_assert(kWaves * 32 * D * sizeof(float) <= sizeof(lds), "epilogue blocks fit the tile buffers");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: task setup stays scalar
  const int col = lane & 31, half = lane >> 5;
  const int logical = xcd_remap(blockIdx.x, p.n_wg);
  // A merging step leaves the running result of rows that see no key as it
  // is (an empty partial merges as the identity): workgroups the host has
  // listed after every row group with work end at once, or only convert
  // that result when the final output is due.
  if (!p.split && (p.n_order || p.order_reverse) && p.accumulate && logical % p.n_rg_launch >= p.n_active) {
    if (p.o_final) copy_running_to_final<D, QR>(p, task_head(p, logical), wave, lane);
    return;
  }
  const TaskHead th = task_head(p, logical);

  // Q^T as the B operand: lane holds query `col`, d = 16*ks + 8*half + 0..7.
  // Loaded first, so that the rest of the task setup runs while it lands.
  // Lanes of rows past the chunk load row 0 (their results are never
  // written): unconditional loads leave the load count the same on every
  // path, so the setup's waits need not cover these loads.
  bf16x8 qreg[NQB][D / 16];
  {
    const int row0 = task_row0<QR>(p, th, wave), h = task_head_index(p, th, wave);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int row = row0 + qb * 32 + col;
      const bf16x8* src = reinterpret_cast<const bf16x8*>(
          static_cast<const uint16_t*>(p.q) + ((size_t)(row < p.sq ? row : 0) * p.hq + h) * D);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) qreg[qb][ks] = src[2 * ks + half];
    }
  }
  const WaveTask t = make_task_from<QR>(p, wave, th);
  TileIter it{-1, 0, 0, 0, 1};
  tile_next(it, p, t);
  // a split item starts t.skip tiles into its row group's visit list and
  // computes at most t.count tiles
  for (int i = 0; i < t.skip && it.valid; ++i) tile_next(it, p, t);
  int left = t.count;
  // A merging step whose rows see no key tile leaves the running result as
  // it is (an empty partial merges as the identity).
  if (!it.valid && t.slot < 0 && p.accumulate && !p.o_final) return;

  int32_t qpos[NQB], qds[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int row = t.row0 + qb * 32 + col;
    const bool ok = row < p.sq;
    qpos[qb] = (ok && !FULL) ? row_to_pos(p.qs, row) : kPosNone;
    // the lane's own row's document start comes with the task (NQB = 1)
    const int32_t ds = qb == 0 ? t.lane_ds : wave_doc_start(p, t, qpos[qb]);
    qds[qb] = (ok && !FULL && p.mask == kMaskDoc) ? ds : INT32_MIN;
  }

  const KvLoader<D> loader(p, t.g, wave, lane, lds_addr(&lds[0][0][0]));

  f32x16 oacc[NQB][D / 32];
  // Running maximum in base-2 units (m_run), the same with -inf read as 0
  // (m_use, the reference the exponentials subtract) and the raw score
  // above which the lazy maximum must move ((m_run + 8) / scale_log2).
  float m_run[NQB], m_use[NQB], thr_raw[NQB], l_run[NQB];
  const float inv_c = 1.f / p.scale_log2;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m_run[qb] = -INFINITY;
    m_use[qb] = 0.f;
    thr_raw[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[qb][db] = f32x16{};
  }

  if (it.valid) loader.issue(it.kt, 0);
  // With one contiguous KV run, the key tiles that are full for this wave
  // (every key at or before its first row, at or after the latest document
  // start of its rows, inside the chunk) are the tile indices [f_lo, f_hi].
  bool iv = false;
  int f_lo = 1, f_hi = 0;
  if (!FULL && p.ks.n == 1 && p.ks.stride[0] == 1) {
    iv = true;
    if (t.wave_any) {
      const int32_t st = p.ks.start[0];          // position of key row 0
      int lo = 0, hi = p.sk / kBN - 1;          // tiles not past the chunk
      if (p.mask != kMaskNone) hi = min(hi, floor_div_i32(t.wq_lo - st - (kBN - 1), kBN));
      if (p.mask == kMaskDoc) lo = max(lo, -floor_div_i32(st - t.wds_hi, kBN));
      f_lo = lo;
      f_hi = hi;
    }
  }
  // The body of one key tile, for a compile-time buffer index (the loop is
  // unrolled by two so LDS addresses of either buffer are immediate offsets).
  auto tile = [&](auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    const int kt = it.kt;
    const int kr0 = kt * kBN;
    const int kr1 = min(kr0 + kBN, p.sk);
    // This wave's loads of tile kt have landed; after the barrier every
    // wave's have, and every wave is done with the other buffer.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    TileIter nx = it;
    tile_next(nx, p, t);
    if (--left == 0) nx.valid = 0;
    if (nx.valid) loader.issue(nx.kt, buf ^ 1);

    // A tile this wave may skip (another wave of the workgroup needs it) is
    // computed fully masked instead: no branch around the tile body.
    PosRange kr{0, 0, true, 1};
    int cls = kFull;
    if (!FULL) {
      if (iv) {
        cls = (kt >= f_lo && kt <= f_hi) ? kFull : kPartial;
      } else {
        kr = tile_pos_range<ONESEG>(it, p.ks, kr0, kr1);
        const int cls0 = classify(p.mask, kr, kr1 - kr0 < kBN, t.wq_lo, t.wq_hi, t.wds_lo, t.wds_hi, t.wave_any);
        cls = cls0 == kSkip ? kPartial : cls0;
      }
    }
    {
      const char* kt_lds = lds[buf][0];
      const char* vt_lds = lds[buf][1];
      // S^T = K Q^T for two 32-key blocks.
      f32x16 sacc[2][NQB];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) sacc[kb][qb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int r = kb * 32 + col;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              kt_lds + r * RB + (((2 * ks + half) ^ tile_swz<CPR>(r)) << 4));
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
            sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[qb][ks], sacc[kb][qb], 0, 0, 0);
        }
      }
      if (NQB == 1) {
        // 6 K reads in flight ahead of the score MFMAs (2 by the compiler's
        // own schedule, which leaves the MFMAs waiting on LDS latency)
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int i = 0; i < 10; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
      }

      if (!FULL && cls == kPartial) {
        if (iv) kr = tile_pos_range<ONESEG>(it, p.ks, kr0, kr1);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) mask_block<ONESEG>(sacc[kb][qb], p, kr, kr0, kb, half, qpos[qb], qds[qb]);
      }

      // Online softmax (base 2) per query column with a lazy maximum: the
      // running maximum only moves (and O, l are only rescaled) when some
      // lane's tile maximum exceeds it by more than 2^8, so P stays below
      // 256 and most tiles skip the rescale.
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        // The tile maximum is compared in raw score units; it is scaled only
        // when the running maximum moves.  Both lanes of a query share its
        // threshold, so each tests its own 32 of the tile's 64 keys; the two
        // are combined only when the maximum moves.
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[kb][qb][j]);
        if (__any(mx > thr_raw[qb])) {
          mx = half_max(mx);
          const float m_new = fmaxf(m_run[qb], mx * p.scale_log2);
          const float alpha = fast_exp2(m_run[qb] - (m_new == -INFINITY ? 0.f : m_new));
          m_run[qb] = m_new;
          m_use[qb] = m_new == -INFINITY ? 0.f : m_new;
          thr_raw[qb] = (m_new + 8.f) * inv_c;
          l_run[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) oacc[qb][db] *= alpha;
        }
        // four partial sums: shorter dependency chains for the scheduler
        float ls[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float e = fast_exp2(fmaf(sacc[kb][qb][j], p.scale_log2, -m_use[qb]));
            sacc[kb][qb][j] = e;
            const int i = (16 * kb + j) & 3;
            ls[i] = (kb == 0 && j < 4) ? e : ls[i] + e;
          }
        l_run[qb] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
      }

      // O^T += V^T P^T.  The k-slot of P^T register j maps to key
      // 16*t2 + 8*(i/4) + 4*half + i%4; the transpose load reads V rows in
      // that order straight from the row-major tile.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          bf16x8 pb[NQB];
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            u32x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              w[i] = pack_bf16x2(sacc[kb][qb][8 * t2 + 2 * i], sacc[kb][qb][8 * t2 + 2 * i + 1]);
            pb[qb] = __builtin_bit_cast(bf16x8, w);
          }
          const int rA = kb * 32 + 16 * t2 + 4 * half;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const bf16x8 a = tr_operand_swz<CPR>(vt_lds, rA, rA + 8, db * 32, lane);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
              oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb], oacc[qb][db], 0, 0, 0);
          }
        }
      }
    }
    it = nx;
  };
  while (it.valid) {
    tile(std::integral_constant<int, 0>{});
    if (!it.valid) break;
    tile(std::integral_constant<int, 1>{});
  }

  // Epilogue: O = O_acc / l, LSE = m ln 2 + ln l; rows with no key: (0, -inf).
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float l = half_sum(l_run[qb]);
    const bool has = l > 0.f;
    const float inv = has ? 1.f / l : 0.f;
    const float lse = has ? m_run[qb] * kLn2 + __logf(l) : -INFINITY;
    if (t.slot >= 0)
      write_split_partial<D>(p, t.slot, wave, col, half, oacc[qb], inv, lse);
    else if (p.accumulate && NQB == 1)
      merge_step_output_coalesced<D>(p, t.row0 + qb * 32, t.h, lane, oacc[qb], inv, lse,
                                     reinterpret_cast<float*>(&lds[0][0][0]) + wave * 32 * D);
    else
      write_step_output<D>(p, t.row0 + qb * 32 + col, t.h, half, oacc[qb], inv, lse);
  }
}

// ---------------------------------------------------------------------------
// Merge of split items: one workgroup per (split row group, head group) with
// the forward workgroup's 4 (head, row block) waves; 8 lanes per row (D / 32
// f32x4 vectors each), so a wave covers 8 rows and runs 4 passes over its 32.
// The items' partials (O_s normalized, LSE_s) combine as
//   L = m + ln sum_s e^{LSE_s - m},  O = sum_s e^{LSE_s - L} O_s   (m = max LSE_s),
// the LSE-weighted merge of all items at once; items with LSE = -inf weigh 0.
// The LSE values are read first and then every O_s load is issued before
// any is used (the kernel is bound by load latency).  The result goes to the
// output as write_step_output would write an unsplit partial.

template <int D>
__global__ __launch_bounds__(256) void split_merge_kernel(FwdParams p) {
  constexpr int VPL = D / 32;                      // f32x4 vectors per lane
  constexpr int MAXI = 8;                          // items read per batch
  const int hg = blockIdx.x % p.n_head_groups;
  const int i = blockIdx.x / p.n_head_groups;      // order index, < n_split_rg
  const int rg = karg_u16(p.order, i);
  const int it0 = karg_u16(p.item_start, i), n_it = karg_u16(p.item_start, i + 1) - it0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = hg * p.hpw + wave % p.hpw;
  const int v0 = (lane & 7) * VPL;
  const size_t slot_stride = (size_t)p.n_head_groups * split_slot_floats(D);
  const float* slot0 = p.ws + (size_t)(it0 * p.n_head_groups + hg) * split_slot_floats(D);
  for (int pass = 0; pass < 4; ++pass) {
    const int rin = pass * 8 + (lane >> 3);
    const int row = rg * p.rbw * 32 + (wave / p.hpw) * 32 + rin;
    // largest item LSE of the row
    float m = -INFINITY;
    for (int s = 0; s < n_it; ++s) m = fmaxf(m, slot0[s * slot_stride + 128 * D + wave * 32 + rin]);
    f32x4 o[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) o[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (m != -INFINITY) {
      for (int s0 = 0; s0 < n_it; s0 += MAXI) {
        const int ns = min(MAXI, n_it - s0);
        float w[MAXI];
        f32x4 os[MAXI][VPL];
#pragma unroll
        for (int s = 0; s < MAXI; ++s)
          if (s < ns) {
            const float* slot = slot0 + (s0 + s) * slot_stride;
            w[s] = __expf(slot[128 * D + wave * 32 + rin] - m);
#pragma unroll
            for (int v = 0; v < VPL; ++v)
              os[s][v] = reinterpret_cast<const f32x4*>(slot + (size_t)(wave * 32 + rin) * D)[v0 + v];
          }
#pragma unroll
        for (int s = 0; s < MAXI; ++s)
          if (s < ns) {
            wsum += w[s];
#pragma unroll
            for (int v = 0; v < VPL; ++v) o[v] += w[s] * os[s][v];
          }
      }
      const float inv = 1.f / wsum;
#pragma unroll
      for (int v = 0; v < VPL; ++v) o[v] *= inv;
    }
    const float L = m == -INFINITY ? -INFINITY : m + __logf(wsum);
    if (row >= p.sq) continue;
    const size_t li = (size_t)h * p.sq + row;
    const size_t oi = ((size_t)row * p.hq + h) * D + 4 * v0;
    float* dst = p.o + oi;
    if (!p.accumulate) {
      if ((lane & 7) == 0) p.lse[li] = L;
#pragma unroll
      for (int v = 0; v < VPL; ++v) reinterpret_cast<f32x4*>(dst)[v] = o[v];
      continue;
    }
    // The 8 lanes of the row (one wave) read the running LSE before one of
    // them writes it.
    if (L == -INFINITY && !p.o_final) continue;
    const MergeWeights mw = merge_weights(p.lse[li], L);
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const f32x4 r = mw.wa * reinterpret_cast<const f32x4*>(dst)[v] + mw.wb * o[v];
      reinterpret_cast<f32x4*>(dst)[v] = r;
      if (p.o_final) {
        if (p.final_bf16) {
          const u32x2 b = {pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
          reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o_final) + oi)[v] = b;
        } else {
          reinterpret_cast<f32x4*>(static_cast<float*>(p.o_final) + oi)[v] = r;
        }
      }
    }
    if ((lane & 7) == 0) p.lse[li] = mw.L;
  }
}

// ---------------------------------------------------------------------------
// fp32: v_mfma_f32_32x32x2_f32, P kept in fp32.  Same structure; the V tile
// needs no transpose because each PV k-step reads one key per lane half.

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_f32_kernel(FwdParams p) {
  constexpr int QR = 32;
  constexpr int KST = D + 2;   // conflict-free column reads of K
  constexpr int VST = D + 8;   // lane halves 4 keys apart land on disjoint banks
  __shared__ __attribute__((aligned(16))) float k_lds[kBN * KST];
  __shared__ __attribute__((aligned(16))) float v_lds[kBN * VST];

  const int tid = threadIdx.x, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const WaveTask t = make_task<QR>(p, __builtin_amdgcn_readfirstlane(tid >> 6), blockIdx.x);
  const float* kbase = static_cast<const float*>(p.k);
  const float* vbase = static_cast<const float*>(p.v);

  const int row = t.row0 + col;
  const bool row_ok = row < p.sq;
  float qreg[D / 2];
  {
    const float* src = static_cast<const float*>(p.q) + ((size_t)(row_ok ? row : 0) * p.hq + t.h) * D;
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) qreg[ks] = row_ok ? src[2 * ks + half] : 0.f;
  }
  const int32_t qpos = row_ok ? row_to_pos(p.qs, row) : kPosNone;
  const int32_t qds = (row_ok && p.mask == kMaskDoc) ? t.lane_ds : INT32_MIN;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  for_each_tile(p, t, [&](int kt) {
    const int kr0 = kt * kBN;
    const int kr1 = min(kr0 + kBN, p.sk);
    __syncthreads();
    for (int c = tid; c < kBN * D / 4; c += kThreads) {
      const int r = c / (D / 4), c4 = c % (D / 4);
      const int krow = kr0 + r;
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (krow < p.sk) {
        const size_t off = ((size_t)krow * p.hkv + t.g) * D + c4 * 4;
        kv = *reinterpret_cast<const f32x4*>(kbase + off);
        vv = *reinterpret_cast<const f32x4*>(vbase + off);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) k_lds[r * KST + c4 * 4 + i] = kv[i];
      *reinterpret_cast<f32x4*>(&v_lds[r * VST + c4 * 4]) = vv;
    }
    __syncthreads();

    const PosRange kr = pos_range(p.ks, kr0, kr1);
    const int cls = classify(p.mask, kr, kr1 - kr0 < kBN, t.wq_lo, t.wq_hi, t.wds_lo, t.wds_hi, t.wave_any);
    if (cls == kSkip) return;

    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(
            k_lds[(kb * 32 + col) * KST + 2 * ks + half], qreg[ks], sacc[kb], 0, 0, 0);

    if (cls == kPartial) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) mask_block(sacc[kb], p, kr, kr0, kb, half, qpos, qds);
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[kb][j]);
    mx = half_max(mx) * p.scale_log2;
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float e = fast_exp2(fmaf(sacc[kb][j], p.scale_log2, -m_use));
        sacc[kb][j] = e;
        lsum += e;
      }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;

    // O^T += V^T P^T: k-step j pairs key (8(j/4) + j%4) in the low lane half
    // with the key 4 above it in the high half, exactly the keys this lane's
    // accumulator register j holds.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kk = kb * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(v_lds[kk * VST + db * 32 + col], sacc[kb][j],
                                                          oacc[db], 0, 0, 0);
      }
  });

  const float l = half_sum(l_run);
  const bool has = l > 0.f;
  const float inv = has ? 1.f / l : 0.f;
  const float lse = has ? m_run * kLn2 + __logf(l) : -INFINITY;
  write_step_output<D>(p, row, t.h, half, oacc, inv, lse);
}

// ---------------------------------------------------------------------------

constexpr int kFwdNQB = 1;

int fwd_rows_per_wave(int d, int dtype_bf16) {
  (void)d;
  return dtype_bf16 ? 32 * kFwdNQB : 32;
}

hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t s) {
  dim3 grid(p.n_wg), block(kThreads);
  if (d == 128 && p.all_full)
    hipLaunchKernelGGL((fwd_bf16_kernel<128, kFwdNQB, true, true>), grid, block, 0, s, p);
  else if (d == 128 && p.one_seg)
    hipLaunchKernelGGL((fwd_bf16_kernel<128, kFwdNQB, false, true>), grid, block, 0, s, p);
  else if (d == 128)
    hipLaunchKernelGGL((fwd_bf16_kernel<128, kFwdNQB, false, false>), grid, block, 0, s, p);
  else if (d == 64 && p.all_full)
    hipLaunchKernelGGL((fwd_bf16_kernel<64, kFwdNQB, true, true>), grid, block, 0, s, p);
  else if (d == 64 && p.one_seg)
    hipLaunchKernelGGL((fwd_bf16_kernel<64, kFwdNQB, false, true>), grid, block, 0, s, p);
  else if (d == 64)
    hipLaunchKernelGGL((fwd_bf16_kernel<64, kFwdNQB, false, false>), grid, block, 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_split_merge(const FwdParams& p, int d, hipStream_t s) {
  dim3 grid(p.n_split_rg * p.n_head_groups), block(256);
  if (d == 128)
    hipLaunchKernelGGL((split_merge_kernel<128>), grid, block, 0, s, p);
  else if (d == 64)
    hipLaunchKernelGGL((split_merge_kernel<64>), grid, block, 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdParams& p, int d, hipStream_t s) {
  dim3 grid(p.n_wg), block(kThreads);
  if (d == 64)
    hipLaunchKernelGGL((fwd_f32_kernel<64>), grid, block, 0, s, p);
  else if (d == 128)
    hipLaunchKernelGGL((fwd_f32_kernel<128>), grid, block, 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace rba
