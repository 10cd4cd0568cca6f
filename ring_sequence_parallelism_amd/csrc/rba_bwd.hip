// Backward ring step, dK / dV part: gradients of L = sum dO * O with
// respect to the keys and values of one KV chunk.
//
// The pages name training as the workload (HSAP methodology and results;
// TASP abstract) but print no backward; this is the gradient of the softmax
// attention definition.  With P_ij = exp(s_ij - LSE_i) (LSE from the merged
// forward) and delta_i = <dO_i, O_i>:
//   dV_j  = sum_i P_ij dO_i
//   dS_ij = P_ij (<dO_i, v_j> - delta_i)
//   dK_j  = scale * sum_i dS_ij q_i
// summing dK / dV over the query heads that share a KV head (GQA).  dQ is
// computed by the query-stationary pass in rba_bwd_dq.h; both passes run in
// one launch (bwd_kernel below).
//
// gfx950 design
//   * A workgroup owns 128 keys of one KV head and one query head of its
//     group (4 waves x 32 keys).  Each wave keeps its V rows in registers as
//     MFMA B operands, and its dK / dV accumulators in registers
//     for the whole pass over the 32-row query blocks that can see those
//     keys.  Splitting the group's query heads over workgroups balances the
//     causal work (low key tiles see every query block); the group's partial
//     dK / dV are summed with fp32 atomics into zeroed outputs.  When every
//     key tile sees the same query rows (a chunk wholly before or after the
//     queries, or no mask) and there are workgroups to spare, a workgroup
//     instead takes several heads of the group in turn and sums them in its
//     accumulators (all of them: plain stores, no zero fill).  Workgroups
//     are ordered KV head, key tile, query head, so the heavier low key tiles
//     are dispatched first on every XCD.
//   * Scores are computed as S = Q K^T (v_mfma_f32_32x32x16_bf16) so a lane
//     owns one key column: P and dS then feed dV += P^T dO and dK += dS^T Q as
//     A operands straight from the accumulator registers.  The matching B
//     operands (dO and Q with the query index along k) come from the same
//     row-major LDS tiles through the LDS transpose load, with the k order
//     permuted to match the accumulator rows.  K^T (the B operand of S) is
//     read from the K tile; V stays in registers.
//   * The K tile, and each query block's Q, dO, LSE and delta rows, stream
//     from HBM straight into LDS (direct loads; Q / dO double-buffered, rows
//     unpadded with the XOR chunk swizzle).  Iteration i: wait for block i's
//     loads and barrier; issue block i + 1's loads; compute block i.
#include <type_traits>

#include "rba_bwd_dq.h"
#include "rba_device.h"

namespace rba {

constexpr int kBwdThreads = 256;
constexpr int kBK = 128;   // keys per workgroup
constexpr int kBQ = 32;    // query rows per block

// End (exclusive) of the document holding position p.
__device__ __forceinline__ int32_t doc_end(const int32_t* cu, int32_t n_docs, int32_t p) {
  int lo = 0, hi = n_docs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= p) lo = mid; else hi = mid - 1;
  }
  return cu[lo + 1];
}

// The same from the document table in registers (see DocLanes), for a
// wave-uniform position and for a position per lane.
__device__ __forceinline__ int32_t doc_end_u(const DocLanes& d, const int32_t* cu, int32_t n_docs, int32_t p) {
  if (!d.ok) return doc_end(cu, n_docs, p);
  return __builtin_amdgcn_readlane(d.v, doc_index_u(d, p) + 1);
}
__device__ __forceinline__ int32_t doc_end_v(const DocLanes& d, const int32_t* cu, int32_t n_docs, int32_t p) {
  if (!d.ok) return doc_end(cu, n_docs, p);
  return __shfl(d.v, doc_index_v(d, n_docs, p) + 1);
}

// Walks the 32-row query blocks whose positions fall in [q_lo, q_hi] (per
// query segment, in row order, each block once).  All fields are
// workgroup-uniform.
struct QIter {
  int s, qbk, b1, next_blk;
  int valid;   // int, not bool: a padding-free struct stays in registers
  int seg_r0, seg_r1, seg_st, seg_sd;   // rows [seg_r0, seg_r1), first position and stride of segment s
};

__device__ __forceinline__ void qiter_next(QIter& it, const BwdParams& p, int64_t q_lo, int64_t q_hi) {
  ++it.qbk;
  while (it.qbk >= it.b1) {
    ++it.s;
    if (it.s >= p.qs.n) {
      it.valid = 0;
      return;
    }
    const int r0 = p.qs.row0[it.s];
    it.seg_r0 = r0;
    it.seg_r1 = p.qs.row0[it.s + 1];
    it.seg_st = p.qs.start[it.s];
    it.seg_sd = p.qs.stride[it.s];
    const RowSpan rs = rows_in(it.seg_st, it.seg_sd, it.seg_r1 - r0, q_lo, q_hi);
    const int64_t a = rs.a, b = rs.b;
    if (a >= b) {
      it.qbk = 0;
      it.b1 = 0;
      continue;
    }
    const int b0 = max((int)((r0 + a) / kBQ), it.next_blk);
    it.b1 = (int)((r0 + b + kBQ - 1) / kBQ);
    it.next_blk = max(it.next_blk, it.b1);
    it.qbk = b0;
  }
}

// Class of a wave's keys (positions k, `k_bad` if ragged or split across
// segments) against a query block (positions q).  Key-side form of the
// document rule: key k is visible from query q iff k <= q < doc_end(k), with
// kend_lo / kend_hi the document ends of k.lo / k.hi.
__device__ __forceinline__ int classify_keys(int mask, PosRange k, bool k_bad, int32_t kend_lo, int32_t kend_hi,
                                             PosRange q, bool k_any) {
  if (!k_any) return kSkip;
  if (mask == kMaskNone) return k_bad ? kPartial : kFull;
  if (k.lo > q.hi) return kSkip;
  if (mask == kMaskDoc && q.lo >= kend_hi) return kSkip;
  const bool full = k.hi <= q.lo && (mask != kMaskDoc || q.hi < kend_lo);
  return (full && !k_bad) ? kFull : kPartial;
}

// LDS bytes of the dK / dV body: the K tile, double-buffered Q / dO tiles
// and LSE / delta rows.
template <int D>
constexpr int dkdv_lds_bytes() { return kBK * D * 2 + 2 * 2 * kBQ * D * 2 + 2 * 2 * 64 * 4; }

// One workgroup (4 waves, number `wg` of p.n_wg) of the dK / dV pass, with
// `smem` the workgroup's LDS (dkdv_lds_bytes<D>() bytes, 16-byte aligned).
// FULL: every visited (key wave, query block) pair is full (shown on the
// host), so blocks need no classification and no per-element mask.
template <int D, bool FULL, bool ONESEG = false>
__device__ __forceinline__ void bwd_dkdv_body(const BwdParams& p, int wg, char* smem) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per tile row
  constexpr int RB = D * 2;                  // bytes per tile row (swizzled, unpadded)
  constexpr int QT = kBQ * RB;               // bytes of a Q or dO block tile
  using A = DkdvAddr<D, kBK, kBQ, 4>;        // lane addresses of the tile loads
  // K tile (once), double-buffered Q / dO tiles and LSE / delta rows (loaded
  // straight from HBM into LDS).
  char* k_lds = smem;
  char (*qd_lds)[2][QT] = reinterpret_cast<char (*)[2][QT]>(smem + kBK * RB);          // [buffer][Q, dO]
  float (*ld_lds)[2][64] = reinterpret_cast<float (*)[2][64]>(smem + kBK * RB + 4 * QT);   // [buffer][lse, delta][row]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const int col = lane & 31, half = lane >> 5;
  const int logical = xcd_remap(wg, p.n_wg);
  const int sets = p.group / p.heads_per_wg;      // workgroups per key tile
  const int g = logical / (p.n_key_tiles * sets);
  const int kt = (logical / sets) % p.n_key_tiles;
  const int h0 = g * p.group + (logical % sets) * p.heads_per_wg;   // first query head of this workgroup
  const int kr0 = kt * kBK;
  const int kr1 = min(kr0 + kBK, p.sk);
  const uint16_t* vbase = static_cast<const uint16_t*>(p.v);
  // Uniform bases of this workgroup's heads and 32-bit row strides in bytes
  // (q, dO and k are each smaller than 4 GiB, checked on the host).
  const uint32_t q_row_bytes = (uint32_t)p.hq * RB, k_row_bytes = (uint32_t)p.hkv * RB;
  const char* qg = nullptr;
  const char* dog = nullptr;
  const char* kg = uniform_ptr(static_cast<const char*>(p.k) + (uint32_t)(g * RB));

  // This wave's 32 keys: rows kr0 + 32*wave + col.
  const int wk0 = kr0 + 32 * wave;
  const int wk1 = min(wk0 + 32, p.sk);
  const bool wave_any = wk0 < wk1;
  PosRange wkr{0, -1, true};
  if (wave_any) wkr = pos_range(p.ks, wk0, wk1);
  const bool wave_ragged = wk1 - wk0 < 32;

  // Query positions that can see a key of this tile; a workgroup with no
  // query block in that range loads nothing (and, unless it must store its
  // zero gradients, writes nothing).
  const PosRange tkr = pos_range(p.ks, kr0, kr1);
  const int my_krow = wk0 + col;
  const int32_t my_kpos = (my_krow < p.sk && !FULL) ? row_to_pos(p.ks, my_krow) : INT32_MAX;
  int64_t q_lo = kPosNegInf, q_hi = kPosPosInf;
  if (p.mask != kMaskNone) q_lo = tkr.lo;
  // document ends (document mask): of the tile's last key, of this lane's
  // key and of the wave's key range, all looked up before any tile load
  int32_t my_kend = INT32_MAX, wkend_lo = INT32_MAX, wkend_hi = INT32_MAX;
  if (p.mask == kMaskDoc) {
    const DocLanes dl = doc_lanes(p.cu, p.n_docs, lane);
    q_hi = (int64_t)doc_end_u(dl, p.cu, p.n_docs, tkr.hi) - 1;
    if (!FULL) {
      // every lane looks up (keys past the chunk: the tile's first key)
      const int32_t e = doc_end_v(dl, p.cu, p.n_docs, my_krow < p.sk ? my_kpos : tkr.lo);
      if (my_krow < p.sk) my_kend = e;
      if (wave_any) {
        wkend_lo = doc_end_u(dl, p.cu, p.n_docs, wkr.lo);
        wkend_hi = doc_end_u(dl, p.cu, p.n_docs, wkr.hi);
      }
    }
  }
  QIter first{-1, 0, 0, 0, 1};
  qiter_next(first, p, q_lo, q_hi);
  const bool stores = p.heads_per_wg == p.group && !p.accumulate;
  if (!first.valid && !stores) return;

  // K tile rows [kr0, kr0 + 128) (rows past the chunk re-read its last row).
  if (first.valid) {
#pragma unroll
    for (int i = 0; i < A::KLOADS; ++i)
      dma16(kg, A::k_off(kr0, wave, i, lane, p.sk, k_row_bytes), lds_addr(k_lds) + (wave * A::KLOADS + i) * 1024);
  }

  // V rows as B operands of dP = dO V^T (lane: key col, d = 16*ks + 8*half + 0..7).
  bf16x8 vreg[D / 16] = {};
  if (first.valid) {
    const int krow = min(wk0 + col, p.sk - 1);
    const bf16x8* src = reinterpret_cast<const bf16x8*>(vbase + ((size_t)krow * p.hkv + g) * D);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) vreg[ks] = src[2 * ks + half];
  }

  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) { dkacc[db] = f32x16{}; dvacc[db] = f32x16{}; }

  // Direct-to-LDS loads of query block b into buffer `buf`: Q and dO rows
  // (rows past the end re-read the last row and are masked) and, from wave
  // 0, the block's LSE and delta rows.  The per-lane
  // byte offsets inside a full block are loop invariant.
  constexpr int QLOADS = A::QLOADS;
  uint32_t qoff[QLOADS];
#pragma unroll
  for (int i = 0; i < QLOADS; ++i) qoff[i] = A::q_whole_off(wave, i, lane, q_row_bytes);
  const uint32_t qd_wave = lds_addr(&qd_lds[0][0][0]) + wave * QLOADS * 1024;
  const float* lse_h = nullptr;
  const float* dlt_h = nullptr;
  auto issue = [&](const QIter& b, int buf) {
    const int qr0 = b.qbk * kBQ;
    const uint32_t dst = qd_wave + buf * 2 * QT;
    if (qr0 + kBQ <= p.sq) {
      const size_t bb = A::block_base(qr0, q_row_bytes);
#pragma unroll
      for (int i = 0; i < QLOADS; ++i) {
        dma16(qg + bb, qoff[i], dst + i * 1024);
        dma16(dog + bb, qoff[i], dst + QT + i * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < QLOADS; ++i) {
        const uint32_t off = A::q_ragged_off(qr0, wave, i, lane, p.sq, q_row_bytes);
        dma16(qg, off, dst + i * 1024);
        dma16(dog, off, dst + QT + i * 1024);
      }
    }
    if (wave == 0) {
      // lanes l and l + 32 both fetch row qr0 + l (rows past the end: the last row)
      const uint32_t off = A::lse_off(qr0, lane, p.sq);
      dma4(lse_h, off, lds_addr(ld_lds[buf][0]));
      dma4(dlt_h, off, lds_addr(ld_lds[buf][1]));
    }
  };

  // Lane offsets inside the tiles: the Q / dO A operands (row `col`), the
  // K^T B operand (row kr = this wave's key `col`) and the transpose-load
  // rows 4 * half.. (A part) and 4 * half + 8.. (B part) of k-step t2 = 0
  // (t2 = 1 is 16 rows further: an immediate offset).
  // (Recomputed from the lane id in every iteration rather than held in
  // registers across the loop: the general instantiation is at its register
  // limit.  The full-block one holds the transpose-load offsets, which
  // leaves it at 246 VGPRs; holding the others too would spill.)

  QIter it{};
  int visited = 0;   // some block of this wave had allowed pairs (wave-uniform)
  // One query block, for a compile-time buffer index (the loop is unrolled
  // by two so LDS addresses of either buffer are immediate offsets).
  auto block = [&](auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    const int qr0 = it.qbk * kBQ;
    const int qr1 = min(qr0 + kBQ, p.sq);
    // This block's loads have landed; after the barrier every wave's loads
    // are visible and the other buffers are free.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    QIter nx = it;
    qiter_next(nx, p, q_lo, q_hi);
    if (nx.valid) issue(nx, buf ^ 1);

    PosRange qr{0, 0, true, 1};
    int cls = wave_any ? kFull : kSkip;
    if (!FULL) {
      qr = (ONESEG || (qr0 >= it.seg_r0 && qr1 <= it.seg_r1))
               ? PosRange{it.seg_st + (qr0 - it.seg_r0) * it.seg_sd,
                          it.seg_st + (qr1 - 1 - it.seg_r0) * it.seg_sd, true, it.seg_sd}
               : pos_range(p.qs, qr0, qr1);
      cls = classify_keys(p.mask, wkr, wave_ragged || !wkr.single, wkend_lo, wkend_hi, qr, wave_any);
      const bool q_ragged = qr1 - qr0 < kBQ;
      if (cls == kFull && q_ragged) cls = kPartial;
    }
    const char* qt = qd_lds[buf][0];
    const char* dot = qd_lds[buf][1];

    if (cls != kSkip) {
      visited = 1;
      f32x16 sacc = {}, dpacc = {};
      const int ln = (int)opaque((uint32_t)lane);
      const uint32_t qo = row_read_offset<CPR>(ln & 31, ln >> 5);
      const uint32_t ko = row_read_offset<CPR>(32 * wave + (ln & 31), ln >> 5);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const uint32_t oq = qo ^ (ks << 5), okk = ko ^ (ks << 5);
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(qt + oq);
        const bf16x8 ad = *reinterpret_cast<const bf16x8*>(dot + oq);
        const bf16x8 bk = *reinterpret_cast<const bf16x8*>(k_lds + okk);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, bk, sacc, 0, 0, 0);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, vreg[ks], dpacc, 0, 0, 0);
      }
      // P and dS in place (rows: queries 8*(j/4) + 4*half + j%4; column: my key).
      const float* lse_b = ld_lds[buf][0];
      const float* dlt_b = ld_lds[buf][1];
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int qb0 = 8 * j4 + 4 * half;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse_b[qb0]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&dlt_b[qb0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * j4 + i;
          float pv = fast_exp2(fmaf(sacc[j], p.scale_log2, -l4[i] * 1.4426950408889634f));
          if (!FULL && cls == kPartial) {
            const int qrow = qr0 + qb0 + i;
            bool ok = my_krow < p.sk && qrow < p.sq;
            if (p.mask != kMaskNone) {
              const int32_t qp = (ONESEG || qr.single) ? qr.lo + (qrow - qr0) * qr.stride : row_to_pos(p.qs, min(qrow, p.sq - 1));
              ok = ok && my_kpos <= qp && qp < my_kend;
            }
            pv = ok ? pv : 0.f;
          }
          sacc[j] = pv;
          dpacc[j] = pv * (dpacc[j] - d4[i]);
        }
      }
      // dV += P^T dO ; dK += dS^T Q  (k-step t2: queries 16*t2 + ...)
      const int ln2 = FULL ? lane : (int)opaque((uint32_t)lane);
      const uint32_t ta = tr_lane_offset<CPR>(4 * (ln2 >> 5), ln2);
      const uint32_t tb = tr_lane_offset<CPR>(4 * (ln2 >> 5) + 8, ln2);
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        u32x4 pw, sw;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pw[i] = pack_bf16x2(sacc[8 * t2 + 2 * i], sacc[8 * t2 + 2 * i + 1]);
          sw[i] = pack_bf16x2(dpacc[8 * t2 + 2 * i], dpacc[8 * t2 + 2 * i + 1]);
        }
        const bf16x8 pa = __builtin_bit_cast(bf16x8, pw);
        const bf16x8 sa = __builtin_bit_cast(bf16x8, sw);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const uint32_t oa = ta ^ (db << 6), ob = tb ^ (db << 6);
          const bf16x8 bdo = tr_read(dot + t2 * 16 * RB, oa, ob);
          const bf16x8 bq = tr_read(qt + t2 * 16 * RB, oa, ob);
          dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, bdo, dvacc[db], 0, 0, 0);
          dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa, bq, dkacc[db], 0, 0, 0);
        }
      }
    }
    it = nx;
  };
  // The workgroup's query heads one after another, their dK / dV summed in
  // the accumulators.
  for (int hh = 0; hh < p.heads_per_wg; ++hh) {
    const int h = h0 + hh;
    qg = uniform_ptr(static_cast<const char*>(p.q) + (uint32_t)(h * RB));
    dog = uniform_ptr(static_cast<const char*>(p.d_o) + (uint32_t)(h * RB));
    lse_h = p.lse + (size_t)h * p.sq;
    dlt_h = p.delta + (size_t)h * p.sq;
    // every wave is done with the previous head's buffers
    if (hh > 0) __syncthreads();
    it = first;
    if (it.valid) issue(it, 0);
    while (it.valid) {
      block(std::integral_constant<int, 0>{});
      if (!it.valid) break;
      block(std::integral_constant<int, 1>{});
    }
  }

  // dK = scale * acc, dV = acc for this wave's keys (rows: keys 8*(j/4)+4*half+j%4).
  // When the workgroup sums every query head of the group it owns its keys'
  // gradients and stores (or adds) them; otherwise the group's workgroups add
  // with atomics, into zeroed outputs or into the accumulators (a wave that
  // saw no allowed pair has nothing to add).
  if (!wave_any || (!visited && !stores)) return;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int krow = wk0 + 8 * (j >> 2) + 4 * half + (j & 3);
      if (krow < p.sk) {
        float* dkp = p.dk + ((size_t)krow * p.hkv + g) * D + db * 32 + col;
        float* dvp = p.dv + ((size_t)krow * p.hkv + g) * D + db * 32 + col;
        if (p.heads_per_wg == p.group && !p.accumulate) {
          *dkp = dkacc[db][j] * p.scale;
          *dvp = dvacc[db][j];
        } else if (p.heads_per_wg == p.group) {
          *dkp += dkacc[db][j] * p.scale;
          *dvp += dvacc[db][j];
        } else {
          unsafeAtomicAdd(dkp, dkacc[db][j] * p.scale);
          unsafeAtomicAdd(dvp, dvacc[db][j]);
        }
      }
    }
}

// Zero two fp32 arrays of n elements (n a multiple of 4, 16-byte aligned).
__global__ __launch_bounds__(256) void zero2_kernel(float* a, float* b, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    reinterpret_cast<f32x4*>(a)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    reinterpret_cast<f32x4*>(b)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

hipError_t launch_zero_f32(float* a, float* b, int64_t n, hipStream_t s) {
  const int64_t n4 = n / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(zero2_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a, b, n4);
  return hipGetLastError();
}

int bwd_keys_per_wg(int d) {
  (void)d;
  return kBK;
}

// The backward step in one launch: workgroups [0, p.n_wg) run the dK / dV
// pass (heaviest key tiles first), the following dp.f.n_wg the dQ pass, which
// fills the CUs as the dK / dV tail drains.  The two passes share no output
// and read the same inputs.  LDS is one buffer sized for the larger body.
// FULL: both passes visit only full tiles / blocks (shown on the host).
template <int D, bool FULL, bool ONESEG>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_kernel(BwdParams p, DqParams dp) {
  constexpr int SMEM = dkdv_lds_bytes<D>() > dq_lds_bytes<D>() ? dkdv_lds_bytes<D>() : dq_lds_bytes<D>();
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  const int b = blockIdx.x;
  if (b < p.n_wg)
    bwd_dkdv_body<D, FULL, ONESEG>(p, b, smem);
  else
    bwd_dq_body<D, FULL, ONESEG>(dp, b - p.n_wg, smem);
}

hipError_t launch_bwd(const BwdParams& p, const DqParams& dp, int d, hipStream_t s) {
  dim3 grid(p.n_wg + dp.f.n_wg), block(kBwdThreads);
  bool one_seg = dp.f.one_seg != 0;
  for (int i = 1; i < p.qs.n; ++i)
    if (p.qs.row0[i] % kBQ) one_seg = false;
  const bool full = p.all_full && dp.f.all_full;
  if (d == 128 && full)
    hipLaunchKernelGGL((bwd_kernel<128, true, true>), grid, block, 0, s, p, dp);
  else if (d == 128 && one_seg)
    hipLaunchKernelGGL((bwd_kernel<128, false, true>), grid, block, 0, s, p, dp);
  else if (d == 128)
    hipLaunchKernelGGL((bwd_kernel<128, false, false>), grid, block, 0, s, p, dp);
  else if (d == 64 && full)
    hipLaunchKernelGGL((bwd_kernel<64, true, true>), grid, block, 0, s, p, dp);
  else if (d == 64 && one_seg)
    hipLaunchKernelGGL((bwd_kernel<64, false, true>), grid, block, 0, s, p, dp);
  else if (d == 64)
    hipLaunchKernelGGL((bwd_kernel<64, false, false>), grid, block, 0, s, p, dp);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace rba
