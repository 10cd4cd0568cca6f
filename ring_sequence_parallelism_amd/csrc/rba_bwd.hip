// Backward ring step: gradients of L = sum dO * O through one KV chunk.
//
// The pages name training as the workload (HSAP methodology and results;
// TASP abstract) but print no backward; this is the gradient of the softmax
// attention definition.  With P_ij = exp(s_ij - LSE_i) (LSE from the merged
// forward) and delta_i = <dO_i, O_i>:
//   dV_j  = sum_i P_ij dO_i
//   dS_ij = P_ij (<dO_i, v_j> - delta_i)
//   dK_j  = scale * sum_i dS_ij q_i
//   dQ_i += scale * sum_j dS_ij k_j
// summing dK / dV over the query heads that share a KV head (GQA).
//
// gfx950 design
//   * A workgroup owns 128 keys of one KV head and one query head of its
//     group (4 waves x 32 keys).  Each wave keeps its K and V rows in
//     registers as MFMA B operands, and its dK / dV accumulators in registers
//     for the whole pass over the 32-row query blocks that can see those
//     keys.  Splitting the group's query heads over workgroups balances the
//     causal work (low key tiles see every query block); the group's partial
//     dK / dV are summed with fp32 atomics into zeroed outputs.  Workgroups
//     are ordered KV head, key tile, query head, so the heavier low key tiles
//     are dispatched first on every XCD.
//   * Scores are computed as S = Q K^T (v_mfma_f32_32x32x16_bf16) so a lane
//     owns one key column: P and dS then feed dV += P^T dO and dK += dS^T Q as
//     A operands straight from the accumulator registers.  The matching B
//     operands (dO and Q with the query index along k) come from the same
//     row-major LDS tiles through the LDS transpose load, with the k order
//     permuted to match the accumulator rows.
//   * dQ = dS K needs the other orientation: dS goes through LDS once, and
//     each wave computes a 32-column slice of dQ over all 128 keys (K read
//     from a row-major LDS tile through the transpose load), then adds it to
//     dq_acc with fp32 atomics (consecutive lanes hit consecutive addresses).
//   * Software pipeline with one barrier per block: block i is staged into
//     one half of double-buffered LDS tiles, then (after the barrier) the
//     dQ of block i - 1 is computed and its atomics issued, the loads of
//     block i + 1 are issued, and block i is computed.  Loads retire in issue
//     order, so waiting for block i + 1's data never waits for atomics that
//     were issued after it.
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

// Walks the 32-row query blocks whose positions fall in [q_lo, q_hi] (per
// query segment, in row order, each block once).  All fields are
// workgroup-uniform.
struct QIter {
  int s, qbk, b1, next_blk;
  bool valid;
};

__device__ __forceinline__ void qiter_next(QIter& it, const BwdParams& p, int64_t q_lo, int64_t q_hi) {
  ++it.qbk;
  while (it.qbk >= it.b1) {
    ++it.s;
    if (it.s >= p.qs.n) {
      it.valid = false;
      return;
    }
    const int64_t st = p.qs.start[it.s];
    const int r0 = p.qs.row0[it.s];
    const int64_t len = p.qs.row0[it.s + 1] - r0;
    const int64_t a = min(max(q_lo - st, (int64_t)0), len);
    const int64_t b = min(max(q_hi - st + 1, (int64_t)0), len);
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

template <int D>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_bf16_kernel(BwdParams p) {
  constexpr int TS = D + 16;       // row stride of the Q, dO and K tiles
  constexpr int SST = kBK + 8;     // dS tile (per query row)
  constexpr int NCH = (kBQ * D / 8 + kBwdThreads - 1) / kBwdThreads;   // 16-byte chunks per thread
  // Q, dO and dS tiles are double-buffered: block i is staged and computed in
  // buffer i % 2 while the dQ of block i - 1 still reads dS buffer (i-1) % 2.
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[2][kBQ * TS];
  __shared__ __attribute__((aligned(16))) uint16_t do_lds[2][kBQ * TS];
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kBK * TS];
  __shared__ __attribute__((aligned(16))) uint16_t ds_lds[2][kBQ * SST];
  __shared__ __attribute__((aligned(16))) float lse_lds[2][kBQ];
  __shared__ __attribute__((aligned(16))) float dlt_lds[2][kBQ];
  __shared__ int32_t qpos_lds[2][kBQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int logical = xcd_remap(blockIdx.x, p.n_wg);
  const int g = logical / (p.n_key_tiles * p.group);
  const int kt = (logical / p.group) % p.n_key_tiles;
  const int h = g * p.group + logical % p.group;   // the query head of this workgroup
  const int kr0 = kt * kBK;
  const int kr1 = min(kr0 + kBK, p.sk);
  const uint16_t* qbase = static_cast<const uint16_t*>(p.q);
  const uint16_t* kbase = static_cast<const uint16_t*>(p.k);
  const uint16_t* vbase = static_cast<const uint16_t*>(p.v);
  const uint16_t* dobase = static_cast<const uint16_t*>(p.d_o);

  // This wave's 32 keys: rows kr0 + 32*wave + col.
  const int wk0 = kr0 + 32 * wave;
  const int wk1 = min(wk0 + 32, p.sk);
  const bool wave_any = wk0 < wk1;
  PosRange wkr{0, -1, true};
  if (wave_any) wkr = pos_range(p.ks, wk0, wk1);
  const bool wave_ragged = wk1 - wk0 < 32;

  // K and V rows as B operands (lane: key col, d = 16*ks + 8*half + 0..7).
  bf16x8 kreg[D / 16], vreg[D / 16];
  {
    const int krow = wk0 + col;
    const bool ok = krow < p.sk;
    const size_t off = ((size_t)(ok ? krow : 0) * p.hkv + g) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      bf16x8 z = {};
      kreg[ks] = ok ? reinterpret_cast<const bf16x8*>(kbase + off)[2 * ks + half] : z;
      vreg[ks] = ok ? reinterpret_cast<const bf16x8*>(vbase + off)[2 * ks + half] : z;
    }
  }
  const int my_krow = wk0 + col;
  const int32_t my_kpos = my_krow < p.sk ? row_to_pos(p.ks, my_krow) : INT32_MAX;
  // document ends (document mask): of this lane's key and of the wave's key range
  int32_t my_kend = INT32_MAX, wkend_lo = INT32_MAX, wkend_hi = INT32_MAX;
  if (p.mask == kMaskDoc) {
    if (my_krow < p.sk) my_kend = doc_end(p.cu, p.n_docs, my_kpos);
    if (wave_any) {
      wkend_lo = doc_end(p.cu, p.n_docs, wkr.lo);
      wkend_hi = doc_end(p.cu, p.n_docs, wkr.hi);
    }
  }

  // Row-major K tile of the workgroup (dQ's B operand, via the transpose load).
  for (int c = tid; c < kBK * D / 8; c += kBwdThreads) {
    const int r = c / (D / 8), c8 = c % (D / 8);
    const int krow = kr0 + r;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (krow < p.sk) val = *reinterpret_cast<const u32x4*>(kbase + ((size_t)krow * p.hkv + g) * D + c8 * 8);
    *reinterpret_cast<u32x4*>(&k_lds[r * TS + c8 * 8]) = val;
  }

  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) { dkacc[db] = f32x16{}; dvacc[db] = f32x16{}; }

  // Query positions that can see a key of this tile.
  const PosRange tkr = pos_range(p.ks, kr0, kr1);
  int64_t q_lo = kPosNegInf, q_hi = kPosPosInf;
  if (p.mask != kMaskNone) q_lo = tkr.lo;
  if (p.mask == kMaskDoc) q_hi = (int64_t)doc_end(p.cu, p.n_docs, tkr.hi) - 1;

  // Prefetch registers for one query block.  Nothing reads them before the
  // block is staged one iteration later, so the loads stay in flight during
  // a whole block of compute.
  u32x4 pq[NCH], pdo[NCH];
  float plse = 0.f, pdlt = 0.f;
  auto fetch = [&](const QIter& b) {
    const int qr0 = b.qbk * kBQ;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + kBwdThreads * i;
      const int r = c / (D / 8), c8 = c % (D / 8);
      const int qrow = qr0 + r;
      pq[i] = u32x4{0u, 0u, 0u, 0u};
      pdo[i] = u32x4{0u, 0u, 0u, 0u};
      if (c < kBQ * D / 8 && qrow < p.sq) {
        const size_t off = ((size_t)qrow * p.hq + h) * D + c8 * 8;
        pq[i] = *reinterpret_cast<const u32x4*>(qbase + off);
        pdo[i] = *reinterpret_cast<const u32x4*>(dobase + off);
      }
    }
    if (tid < kBQ && qr0 + tid < p.sq) {
      plse = p.lse[(size_t)h * p.sq + qr0 + tid];
      pdlt = p.delta[(size_t)h * p.sq + qr0 + tid];
    }
  };

  // dQ[:, slice] += scale * dS K over the 128 keys of the tile, for the block
  // whose dS sits in buffer `buf` (rows qr0..).
  auto dq_block = [&](int buf, int qr0) {
    constexpr int NDB = D / 32;                    // column slices
    constexpr int KSPLIT = 4 / NDB;                // waves per slice
    constexpr int KEYS = kBK / KSPLIT;
    constexpr int NKS = KEYS / 16;
    const int wd = wave % NDB, kh = wave / NDB;
    // all operands first, then two independent accumulation chains
    bf16x8 a[NKS], b[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int key0 = kh * KEYS + 16 * ks + 8 * half;
      a[ks] = *reinterpret_cast<const bf16x8*>(&ds_lds[buf][col * SST + key0]);
      b[ks] = tr_operand(k_lds, TS, key0, key0 + 4, wd * 32, lane);
    }
    f32x16 q0 = {}, q1 = {};
#pragma unroll
    for (int ks = 0; ks < NKS; ks += 2) {
      q0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], b[ks], q0, 0, 0, 0);
      q1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks + 1], b[ks + 1], q1, 0, 0, 0);
    }
    // rows: queries 8*(j/4) + 4*half + j%4; column: d = 32*wd + col.
    // 32-bit element offsets from the uniform base (dq_acc is below 2^32
    // bytes, checked on the host); the row offsets are scalar multiples.
    const uint32_t row_stride = (uint32_t)p.hq * D;
    float* base = p.dq + (((uint32_t)(qr0 + 4 * half) * p.hq + h) * D + wd * 32 + col);
    if (qr0 + kBQ <= p.sq) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t r = 8 * (j >> 2) + (j & 3);
        unsafeAtomicAdd(base + r * row_stride, (q0[j] + q1[j]) * p.scale);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t r = 8 * (j >> 2) + (j & 3);
        if (qr0 + 4 * half + (int)r < p.sq) unsafeAtomicAdd(base + r * row_stride, (q0[j] + q1[j]) * p.scale);
      }
    }
  };

  QIter it{-1, 0, 0, 0, true};
  qiter_next(it, p, q_lo, q_hi);
  if (it.valid) fetch(it);
  int buf = 0;
  int prev_qr0 = -1;      // block whose dQ is pending

  while (it.valid) {
    const int qr0 = it.qbk * kBQ;
    const int qr1 = min(qr0 + kBQ, p.sq);
    // Stage block i into buffer `buf`.  Its previous readers (block i - 2)
    // finished before the last barrier.
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + kBwdThreads * i;
      if (c < kBQ * D / 8) {
        const int r = c / (D / 8), c8 = c % (D / 8);
        *reinterpret_cast<u32x4*>(&q_lds[buf][r * TS + c8 * 8]) = pq[i];
        *reinterpret_cast<u32x4*>(&do_lds[buf][r * TS + c8 * 8]) = pdo[i];
      }
    }
    const PosRange qr = pos_range(p.qs, qr0, qr1);
    if (tid < kBQ) {
      const int qrow = qr0 + tid;
      const bool ok = qrow < p.sq;
      // log2-domain LSE; rows past the end get +inf so that P = 0
      lse_lds[buf][tid] = ok ? plse * 1.4426950408889634f : INFINITY;
      dlt_lds[buf][tid] = ok ? pdlt : 0.f;
      qpos_lds[buf][tid] = !ok ? kPosNone : (qr.single ? qr.lo + tid : row_to_pos(p.qs, qrow));
    }
    __syncthreads();
    // dQ of the previous block (its dS is complete in the other buffer),
    // then the next block's loads: both stay in flight while this block runs.
    if (prev_qr0 >= 0) dq_block(buf ^ 1, prev_qr0);
    QIter nx = it;
    qiter_next(nx, p, q_lo, q_hi);
    if (nx.valid) fetch(nx);

    // Class of this wave's keys against the block's queries.
    const int cls = classify_keys(p.mask, wkr, wave_ragged || !wkr.single, wkend_lo, wkend_hi, qr, wave_any);
    const uint16_t* qt = q_lds[buf];
    const uint16_t* dot = do_lds[buf];

    f32x16 sacc = {}, dpacc = {};
    if (cls != kSkip) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&qt[col * TS + 16 * ks + 8 * half]);
        const bf16x8 ad = *reinterpret_cast<const bf16x8*>(&dot[col * TS + 16 * ks + 8 * half]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kreg[ks], sacc, 0, 0, 0);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, vreg[ks], dpacc, 0, 0, 0);
      }
      // P and dS in place (rows: queries 8*(j/4) + 4*half + j%4; column: my key).
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int qb0 = 8 * j4 + 4 * half;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse_lds[buf][qb0]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&dlt_lds[buf][qb0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * j4 + i;
          float pv = fast_exp2(fmaf(sacc[j], p.scale_log2, -l4[i]));
          if (cls == kPartial) {
            const int32_t qp = qpos_lds[buf][qb0 + i];
            const bool ok = my_krow < p.sk && (p.mask == kMaskNone || (my_kpos <= qp && qp < my_kend));
            pv = ok ? pv : 0.f;
          }
          sacc[j] = pv;
          dpacc[j] = pv * (dpacc[j] - d4[i]);
        }
      }
      // dV += P^T dO ; dK += dS^T Q  (k-step t2: queries 16*t2 + ...)
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
        const int rA = 16 * t2 + 4 * half, rB = rA + 8;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 bdo = tr_operand(dot, TS, rA, rB, db * 32, lane);
          const bf16x8 bq = tr_operand(qt, TS, rA, rB, db * 32, lane);
          dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, bdo, dvacc[db], 0, 0, 0);
          dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa, bq, dkacc[db], 0, 0, 0);
        }
      }
    }
    // dS (bf16) to LDS as ds_lds[buf][query][key]; skipped waves write zeros.
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int qq = 8 * (j >> 2) + 4 * half + (j & 3);
      const __bf16 v = (__bf16)(cls != kSkip ? dpacc[j] : 0.f);
      ds_lds[buf][qq * SST + 32 * wave + col] = __builtin_bit_cast(uint16_t, v);
    }
    prev_qr0 = qr0;
    buf ^= 1;
    it = nx;
  }
  if (prev_qr0 >= 0) {
    __syncthreads();
    dq_block(buf ^ 1, prev_qr0);
  }

  // dK = scale * acc, dV = acc for this wave's keys (rows: keys 8*(j/4)+4*half+j%4).
  // With one query head per KV head the workgroup owns its keys' gradients
  // and stores them; otherwise the group's workgroups add into zeroed outputs.
  if (!wave_any) return;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int krow = wk0 + 8 * (j >> 2) + 4 * half + (j & 3);
      if (krow < p.sk) {
        float* dkp = p.dk + ((size_t)krow * p.hkv + g) * D + db * 32 + col;
        float* dvp = p.dv + ((size_t)krow * p.hkv + g) * D + db * 32 + col;
        if (p.group == 1) {
          *dkp = dkacc[db][j] * p.scale;
          *dvp = dvacc[db][j];
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

hipError_t launch_bwd_bf16(const BwdParams& p, int d, hipStream_t s) {
  dim3 grid(p.n_wg), block(kBwdThreads);
  if (d == 128)
    hipLaunchKernelGGL(bwd_bf16_kernel<128>, grid, block, 0, s, p);
  else if (d == 64)
    hipLaunchKernelGGL(bwd_bf16_kernel<64>, grid, block, 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace rba
