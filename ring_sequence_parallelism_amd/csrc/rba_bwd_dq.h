// Backward ring step, dQ part: dQ_i += scale * sum_j dS_ij k_j over the keys of
// one KV chunk, with dS_ij = P_ij (<dO_i, v_j> - delta_i) and
// P_ij = exp(s_ij - LSE_i) from the final merged LSE (the gradient of the
// softmax attention definition; the pages name training as the workload,
// HSAP methodology and TASP abstract, but print no backward).
//
// gfx950 design: the query-stationary tiling of the forward step.  A
// workgroup is 4 waves over one KV head; each wave owns 32 query rows of one
// query head and keeps Q^T and dO^T in registers as MFMA B operands.  K and V
// tiles of 64 keys stream into double-buffered LDS; each 32-key half of a tile
// is computed in transposed form (lane = query column) so the softmax-side
// math stays in-lane:
//   S^T  = K Q^T      (A: K rows from LDS)
//   dP^T = V dO^T     (A: V rows from LDS)
//   P^T  = 2^(scale_log2 s - LSE log2 e),  dS^T = P^T (dP^T - delta)
//   dQ^T += K^T dS^T  (A: K through the LDS transpose load, B: dS^T packed
//                      to bf16 in the key order of the accumulator rows)
// Each (row, head) of dq_acc belongs to one wave: the kernel adds its
// contribution with one read-modify-write at the end, no atomics.
//
// This is a device-side body: the backward step runs it in the same launch
// as the dK / dV pass (rba_bwd.hip).
#pragma once

#include <type_traits>

#include "rba_qtile.h"

namespace rba {

// LDS bytes of the dQ body: double-buffered K and V tiles.
template <int D>
constexpr int dq_lds_bytes() { return 2 * 2 * kBN * D * 2; }

// One workgroup (4 waves, number `block` of dp.f.n_wg) of the dQ pass, with
// `smem` the workgroup's LDS (dq_lds_bytes<D>() bytes, 16-byte aligned).
// FULL: every visited tile is full for every wave (shown on the host), so
// tiles need no classification and no mask.
template <int D, bool FULL, bool ONESEG = false>
__device__ __forceinline__ void bwd_dq_body(const DqParams& dp, int block, char* smem) {
  const FwdParams& p = dp.f;
  constexpr int CPR = D / 8;
  constexpr int RB = D * 2;
  constexpr int TILE = kBN * RB;
  char (*lds)[2][TILE] = reinterpret_cast<char (*)[2][TILE]>(smem);   // [buffer][K, V]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const WaveTask t = make_task<32>(p, wave, block);
  // A workgroup whose rows see no key tile adds nothing to dq_acc.
  TileIter it{-1, 0, 0, 0, 1};
  tile_next(it, p, t);
  if (!it.valid) return;
  const KvLoader<D> loader(p, t.g, wave, lane, lds_addr(&lds[0][0][0]));

  // Q^T and dO^T as B operands: lane holds query `col`, d = 16*ks + 8*half + 0..7.
  const int row = t.row0 + col;
  const bool row_ok = row < p.sq;
  bf16x8 qreg[D / 16], doreg[D / 16];
  {
    const size_t off = ((size_t)(row_ok ? row : 0) * p.hq + t.h) * D;
    const bf16x8* qs = reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(p.q) + off);
    const bf16x8* ds = reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(dp.d_o) + off);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 z = {};
      qreg[ks] = row_ok ? qs[2 * ks + half] : z;
      doreg[ks] = row_ok ? ds[2 * ks + half] : z;
    }
  }
  const int32_t qpos = (row_ok && !FULL) ? row_to_pos(p.qs, row) : kPosNone;
  const int32_t qds = (row_ok && !FULL && p.mask == kMaskDoc) ? t.lane_ds : INT32_MIN;
  // LSE in base 2 (rows without any allowed key, LSE = -inf, get P = 0 like
  // rows past the chunk), and delta.
  float lse2 = INFINITY, dlt = 0.f;
  if (row_ok) {
    const float l = dp.lse[(size_t)t.h * p.sq + row];
    lse2 = l == -INFINITY ? INFINITY : l * 1.4426950408889634f;
    dlt = dp.delta[(size_t)t.h * p.sq + row];
  }

  f32x16 dqacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dqacc[db] = f32x16{};
  // Lane offsets in the K / V tiles (XOR-linear swizzle: see row_read_offset
  // and tr_lane_offset): row `col` for the A operands of S^T and dP^T, and
  // the transpose-load rows 4*half.. / 4*half + 8.. for K^T.
  const uint32_t row_off = row_read_offset<CPR>(col, half);
  const uint32_t tr_a = tr_lane_offset<CPR>(4 * half, lane);
  const uint32_t tr_b = tr_lane_offset<CPR>(4 * half + 8, lane);

  int visited = 0;   // some tile of this wave had allowed pairs (wave-uniform)
  loader.issue(it.kt, 0);
  auto tile = [&](auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    const int kt = it.kt;
    const int kr0 = kt * kBN;
    const int kr1 = min(kr0 + kBN, p.sk);
    // Tile kt has landed for every wave, which are all done with the other buffer.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    TileIter nx = it;
    tile_next(nx, p, t);
    if (nx.valid) loader.issue(nx.kt, buf ^ 1);

    PosRange kr{0, 0, true, 1};
    int cls = t.wave_any ? kFull : kSkip;
    if (!FULL) {
      kr = tile_pos_range<ONESEG>(it, p.ks, kr0, kr1);
      cls = classify(p.mask, kr, kr1 - kr0 < kBN, t.wq_lo, t.wq_hi, t.wds_lo, t.wds_hi, t.wave_any);
    }
    if (cls != kSkip) {
      visited = 1;
      const char* kt_lds = lds[buf][0];
      const char* vt_lds = lds[buf][1];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // S^T and dP^T for keys kb*32 .. +31 (rows of the A operands).
        f32x16 sacc = {}, dpacc = {};
        // rows kb*32 + col: the swizzle ignores row bit 5, so half kb is a
        // plain byte offset from half 0
        const uint32_t ro = row_off;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const uint32_t c = ro ^ (ks << 5);
          const bf16x8 ak = *reinterpret_cast<const bf16x8*>(kt_lds + kb * 32 * RB + c);
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(vt_lds + kb * 32 * RB + c);
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qreg[ks], sacc, 0, 0, 0);
          dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, doreg[ks], dpacc, 0, 0, 0);
        }
        if (!FULL && cls == kPartial) mask_block<ONESEG>(sacc, p, kr, kr0, kb, half, qpos, qds);
        // dS^T in place, packed to bf16 pairs in accumulator order.
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p0 = fast_exp2(fmaf(sacc[2 * i], p.scale_log2, -lse2));
          const float p1 = fast_exp2(fmaf(sacc[2 * i + 1], p.scale_log2, -lse2));
          w[i] = pack_bf16x2(p0 * (dpacc[2 * i] - dlt), p1 * (dpacc[2 * i + 1] - dlt));
        }
        // dQ^T += K^T dS^T.  k-slot of dS^T register j <-> key
        // 16*t2 + 8*(i/4) + 4*half + i%4 (as P^T in the forward's PV).
        const uint32_t ta = tr_a, tb = tr_b;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const u32x4 wv = {w[4 * t2], w[4 * t2 + 1], w[4 * t2 + 2], w[4 * t2 + 3]};
          const bf16x8 b = __builtin_bit_cast(bf16x8, wv);
          const int rA0 = kb * 32 + 16 * t2;   // rows rA0 + 4*half.. (+8): same swizzle as rows 4*half..
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const bf16x8 a = tr_read(kt_lds + rA0 * RB, ta ^ (db << 6), tb ^ (db << 6));
            dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, dqacc[db], 0, 0, 0);
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

  // dq_acc[row, h, :] += scale * dQ^T[:, row] (accumulator rows: d =
  // 32*db + 8*(j/4) + 4*half + j%4, four consecutive d per f32x4).
  if (row_ok && visited) {
    float* dst = dp.dq + ((size_t)row * p.hq + t.h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4* q4 = reinterpret_cast<f32x4*>(dst + db * 32 + 8 * jj + 4 * half);
        const f32x4 add = {dqacc[db][4 * jj], dqacc[db][4 * jj + 1], dqacc[db][4 * jj + 2], dqacc[db][4 * jj + 3]};
        *q4 = *q4 + add * dp.scale;
      }
  }
}

}  // namespace rba
