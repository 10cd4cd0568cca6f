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
//   * A workgroup owns 128 keys of one KV head (4 waves x 32 keys).  Each wave
//     keeps its K and V rows in registers as MFMA B operands, and its dK / dV
//     accumulators in registers for the whole pass over every query head of
//     the group and every query block that can see those keys.
//   * Scores are computed as S = Q K^T (v_mfma_f32_32x32x16_bf16) so a lane
//     owns one key column: P and dS then feed dV += P^T dO and dK += dS^T Q as
//     A operands straight from the accumulator registers, with Q^T and dO^T
//     read from transposed LDS tiles whose query order inside each 16-row
//     group is permuted (bits 2 and 3 swapped) to match the accumulator rows.
//   * dQ = dS K needs the other orientation: dS goes through LDS once, and
//     each wave computes a 32-column slice of dQ over all 128 keys against a
//     transposed K tile staged once per workgroup, then adds it to dq_acc with
//     fp32 atomics (consecutive lanes hit consecutive addresses).
#include "rba_device.h"

namespace rba {

constexpr int kBwdThreads = 256;
constexpr int kBK = 128;   // keys per workgroup
constexpr int kBQ = 32;    // query rows per block

__device__ __forceinline__ int q_slot(int r) {   // rows inside a 32-row block
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// End (exclusive) of the document holding position p.
__device__ __forceinline__ int32_t doc_end(const int32_t* cu, int32_t n_docs, int32_t p) {
  int lo = 0, hi = n_docs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= p) lo = mid; else hi = mid - 1;
  }
  return cu[lo + 1];
}

template <int D>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_bf16_kernel(BwdParams p) {
  constexpr int QST = D + 8;       // row-major Q / dO tiles
  constexpr int TST = kBQ + 8;     // transposed Q / dO tiles (per d row)
  constexpr int KTST = kBK + 8;    // transposed K tile (per d row)
  constexpr int SST = kBK + 8;     // dS tile (per query row)
  __shared__ __attribute__((aligned(16))) uint16_t q_lds[kBQ * QST];
  __shared__ __attribute__((aligned(16))) uint16_t do_lds[kBQ * QST];
  __shared__ __attribute__((aligned(16))) uint16_t qt_lds[D * TST];
  __shared__ __attribute__((aligned(16))) uint16_t dot_lds[D * TST];
  __shared__ __attribute__((aligned(16))) uint16_t kt_lds[D * KTST];
  __shared__ __attribute__((aligned(16))) uint16_t ds_lds[kBQ * SST];
  __shared__ __attribute__((aligned(16))) float lse_lds[kBQ];
  __shared__ __attribute__((aligned(16))) float dlt_lds[kBQ];
  __shared__ int32_t qpos_lds[kBQ], qds_lds[kBQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int logical = xcd_remap(blockIdx.x, p.n_wg);
  const int g = logical / p.n_key_tiles;
  const int kt = logical % p.n_key_tiles;
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
  // Positions of this lane's key (the accumulator column it owns).
  const int my_krow = wk0 + col;
  const int32_t my_kpos = my_krow < p.sk ? row_to_pos(p.ks, my_krow) : INT32_MAX;

  // Transposed K tile for dQ = dS K: kt_lds[d][key], units of 4 keys x 8 dims.
  for (int u = tid; u < (kBK / 4) * (D / 8); u += kBwdThreads) {
    const int dg = u % (D / 8), kg = u / (D / 8);
    u32x4 rows[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int krow = kr0 + 4 * kg + i;
      rows[i] = u32x4{0u, 0u, 0u, 0u};
      if (krow < p.sk) rows[i] = *reinterpret_cast<const u32x4*>(kbase + ((size_t)krow * p.hkv + g) * D + dg * 8);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      u32x2 lo = {(rows[0][w] & 0xffffu) | (rows[1][w] << 16), (rows[2][w] & 0xffffu) | (rows[3][w] << 16)};
      u32x2 hi = {(rows[0][w] >> 16) | (rows[1][w] & 0xffff0000u), (rows[2][w] >> 16) | (rows[3][w] & 0xffff0000u)};
      *reinterpret_cast<u32x2*>(&kt_lds[(dg * 8 + 2 * w) * KTST + 4 * kg]) = lo;
      *reinterpret_cast<u32x2*>(&kt_lds[(dg * 8 + 2 * w + 1) * KTST + 4 * kg]) = hi;
    }
  }

  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) { dkacc[db] = f32x16{}; dvacc[db] = f32x16{}; }

  // Query positions that can see a key of this tile.
  const PosRange tkr = pos_range(p.ks, kr0, kr1);
  int64_t q_lo = kPosNegInf, q_hi = kPosPosInf;
  if (p.mask != kMaskNone) q_lo = tkr.lo;
  if (p.mask == kMaskDoc) q_hi = (int64_t)doc_end(p.cu, p.n_docs, tkr.hi) - 1;

  for (int hh = 0; hh < p.group; ++hh) {
    const int h = g * p.group + hh;
    int next_blk = 0;
    for (int s = 0; s < p.qs.n; ++s) {
      const int64_t st = p.qs.start[s];
      const int r0 = p.qs.row0[s];
      const int64_t len = p.qs.row0[s + 1] - r0;
      const int64_t a = min(max(q_lo - st, (int64_t)0), len);
      const int64_t b = min(max(q_hi - st + 1, (int64_t)0), len);
      if (a >= b) continue;
      const int b0 = max((int)((r0 + a) / kBQ), next_blk);
      const int b1 = (int)((r0 + b + kBQ - 1) / kBQ);
      next_blk = max(next_blk, b1);
      for (int qbk = b0; qbk < b1; ++qbk) {
        const int qr0 = qbk * kBQ;
        const int qr1 = min(qr0 + kBQ, p.sq);
        __syncthreads();   // previous block's LDS reads are done
        // Q and dO rows [qr0, qr0+32) of head h: row-major and transposed.
        {
          const int which = tid / 128;          // 0: Q, 1: dO
          const int u = tid % 128;
          if (u < (kBQ / 4) * (D / 8)) {
            const uint16_t* base = which ? dobase : qbase;
            uint16_t* rm = which ? do_lds : q_lds;
            uint16_t* tr = which ? dot_lds : qt_lds;
            const int dg = u % (D / 8), rg = u / (D / 8);
            u32x4 rows[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int qrow = qr0 + 4 * rg + i;
              rows[i] = u32x4{0u, 0u, 0u, 0u};
              if (qrow < p.sq)
                rows[i] = *reinterpret_cast<const u32x4*>(base + ((size_t)qrow * p.hq + h) * D + dg * 8);
              *reinterpret_cast<u32x4*>(&rm[(4 * rg + i) * QST + dg * 8]) = rows[i];
            }
            const int slot = q_slot(4 * rg);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              u32x2 lo = {(rows[0][w] & 0xffffu) | (rows[1][w] << 16), (rows[2][w] & 0xffffu) | (rows[3][w] << 16)};
              u32x2 hi = {(rows[0][w] >> 16) | (rows[1][w] & 0xffff0000u),
                          (rows[2][w] >> 16) | (rows[3][w] & 0xffff0000u)};
              *reinterpret_cast<u32x2*>(&tr[(dg * 8 + 2 * w) * TST + slot]) = lo;
              *reinterpret_cast<u32x2*>(&tr[(dg * 8 + 2 * w + 1) * TST + slot]) = hi;
            }
          }
        }
        if (tid < kBQ) {
          const int qrow = qr0 + tid;
          const bool ok = qrow < p.sq;
          const float l = ok ? p.lse[(size_t)h * p.sq + qrow] : INFINITY;
          // log2-domain LSE; a row with no key anywhere (-inf) or past the end
          // (+inf) yields P = 0 or is masked.
          lse_lds[tid] = l * 1.4426950408889634f;
          dlt_lds[tid] = ok ? p.delta[(size_t)h * p.sq + qrow] : 0.f;
          const int32_t qp = ok ? row_to_pos(p.qs, qrow) : kPosNone;
          qpos_lds[tid] = qp;
          qds_lds[tid] = (ok && p.mask == kMaskDoc) ? doc_start(p.cu, p.n_docs, qp) : INT32_MIN;
        }
        __syncthreads();

        // Class of this wave's keys against the block's queries.
        const PosRange qr = pos_range(p.qs, qr0, qr1);
        int32_t ds_lo = INT32_MIN, ds_hi = INT32_MIN;
        if (p.mask == kMaskDoc) {
          ds_lo = doc_start(p.cu, p.n_docs, qr.lo);
          ds_hi = doc_start(p.cu, p.n_docs, qr.hi);
        }
        const int cls = classify(p.mask, wkr, wave_ragged || !wkr.single, qr.lo, qr.hi, ds_lo, ds_hi, wave_any);

        f32x16 sacc = {}, dpacc = {};
        if (cls != kSkip) {
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) {
            const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&q_lds[col * QST + 16 * ks + 8 * half]);
            const bf16x8 ad = *reinterpret_cast<const bf16x8*>(&do_lds[col * QST + 16 * ks + 8 * half]);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kreg[ks], sacc, 0, 0, 0);
            dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, vreg[ks], dpacc, 0, 0, 0);
          }
          // P and dS in place (rows: queries 8*(j/4) + 4*half + j%4; column: my key).
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4) {
            const int qb0 = 8 * j4 + 4 * half;
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse_lds[qb0]);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(&dlt_lds[qb0]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = 4 * j4 + i;
              // rows past the end carry LSE = +inf and get P = 0 without a mask
              float pv = fast_exp2(fmaf(sacc[j], p.scale_log2, -l4[i]));
              if (cls == kPartial) {
                const int qq = qb0 + i;
                const bool ok = my_krow < p.sk && qr0 + qq < p.sq &&
                                visible(p.mask, my_kpos, qpos_lds[qq], qds_lds[qq]);
                if (!ok) pv = 0.f;
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
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
              const bf16x8 bdo = *reinterpret_cast<const bf16x8*>(&dot_lds[(db * 32 + col) * TST + 16 * t2 + 8 * half]);
              const bf16x8 bq = *reinterpret_cast<const bf16x8*>(&qt_lds[(db * 32 + col) * TST + 16 * t2 + 8 * half]);
              dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, bdo, dvacc[db], 0, 0, 0);
              dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa, bq, dkacc[db], 0, 0, 0);
            }
          }
        }
        // dS (bf16) to LDS as ds_lds[query][key]; skipped waves write zeros.
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int qq = 8 * (j >> 2) + 4 * half + (j & 3);
          const __bf16 v = (__bf16)(cls != kSkip ? dpacc[j] : 0.f);
          ds_lds[qq * SST + 32 * wave + col] = __builtin_bit_cast(uint16_t, v);
        }
        __syncthreads();

        // dQ[:, slice] += scale * dS K over the 128 keys of the tile.
        {
          constexpr int NDB = D / 32;                    // column slices
          constexpr int KSPLIT = 4 / NDB;                // waves per slice
          constexpr int KEYS = kBK / KSPLIT;
          const int wd = wave % NDB, kh = wave / NDB;
          f32x16 qacc = {};
#pragma unroll
          for (int ks = 0; ks < KEYS / 16; ++ks) {
            const int key0 = kh * KEYS + 16 * ks + 8 * half;
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&ds_lds[col * SST + key0]);
            const bf16x8 b = *reinterpret_cast<const bf16x8*>(&kt_lds[(wd * 32 + col) * KTST + key0]);
            qacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, qacc, 0, 0, 0);
          }
          // rows: queries 8*(j/4) + 4*half + j%4; column: d = 32*wd + col
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int qrow = qr0 + 8 * (j >> 2) + 4 * half + (j & 3);
            if (qrow < p.sq)
              unsafeAtomicAdd(p.dq + ((size_t)qrow * p.hq + h) * D + wd * 32 + col, qacc[j] * p.scale);
          }
        }
      }
    }
  }

  // dK = scale * acc, dV = acc for this wave's keys (rows: keys 8*(j/4)+4*half+j%4).
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int krow = wk0 + 8 * (j >> 2) + 4 * half + (j & 3);
      if (krow < p.sk) {
        const size_t off = ((size_t)krow * p.hkv + g) * D + db * 32 + col;
        p.dk[off] = dkacc[db][j] * p.scale;
        p.dv[off] = dvacc[db][j];
      }
    }
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
