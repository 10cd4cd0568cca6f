// Lane address arithmetic of the direct-to-LDS tile loads.
//
// Every tile load of the step kernels reads 16 bytes per lane from a
// wave-uniform base (an SGPR pair) plus a 32-bit per-lane byte offset.  The
// functions below compute those bases and offsets; the kernels call them
// and so does a host program in the CPU test suite, which enumerates every
// tile, load, lane and ragged chunk length and checks that each byte read
// lies inside its tensor.  They are __host__ __device__ for that reason and
// hold no other logic.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rba {

// XOR swizzle of 16-byte chunks inside a row of a bf16 tile that has no
// padding (rows of CPR chunks, CPR = 16 for d = 128, 8 for d = 64): chunk c of
// row r is stored at chunk position c ^ tile_swz(r).  The map is linear over
// GF(2) in the row bits (tile_swz(a ^ b) = tile_swz(a) ^ tile_swz(b)).  For
// CPR = 16 (bit k of the result from row bits: 0 <- 2, 1 <- 1, 2 <- 0,
// 3 <- 1 ^ 3):
//   * 16-byte row reads (one chunk of 16 consecutive rows per 16 lanes, 8 per
//     8) land on 16 (8) distinct chunk positions modulo 16 (8);
//   * transpose reads (4 consecutive rows, 2 or 4 consecutive chunks from an
//     aligned pair / quad) land on distinct positions modulo 8 / 16,
// so neither access pattern has a bank conflict with 32 or with 64 banks of
// 4 bytes.  CPR = 8 keeps the analogous (2 * (r & 3)) | ((r >> 2) & 1).
template <int CPR>
__host__ __device__ __forceinline__ constexpr int tile_swz(int r) {
  if (CPR == 16) {
    const int b1 = (r >> 1) & 1;
    return ((r >> 2) & 1) | (b1 << 1) | ((r & 1) << 2) | ((b1 ^ ((r >> 3) & 1)) << 3);
  }
  return (2 * (r & 3)) | ((r >> 2) & 1);
}

// K / V key tiles of the query-stationary kernels (forward step, dQ pass):
// BN rows of one KV head, loaded by WAVES waves.  Load i of a wave fills
// tile rows (wave * LOADS + i) * ROWS_PER_LOAD + lane / CPR: lane l writes
// chunk position l % CPR of its row and fetches the global chunk that the
// swizzle stores there.  Load i covers rows r_lane + ROWS_PER_LOAD * i,
// where the two terms share no set bit, so its row term is a uniform step of
// load 0's and, tile_swz being XOR-linear, its swizzled chunk is load 0's XOR
// tile_swz(ROWS_PER_LOAD * i).
//
// Addresses are relative to the KV head's first row (K or V + head * 2d
// bytes); rows are row_bytes = hkv * 2d apart.
template <int D, int BN, int WAVES>
struct KvTileAddr {
  static constexpr int CPR = D / 8;                     // 16-byte chunks per row
  static constexpr int ROWS_PER_LOAD = 64 / CPR;        // rows one wave-wide load covers
  static constexpr int LOADS = BN / ROWS_PER_LOAD / WAVES;   // per wave per tensor per tile
  static_assert(LOADS * ROWS_PER_LOAD * WAVES == BN, "tile rows");

  // Tile row of load 0 for this lane.
  __host__ __device__ static constexpr int r_lane(int wave, int lane) {
    return wave * LOADS * ROWS_PER_LOAD + lane / CPR;
  }
  // Lane offset of load 0 from its tile's first row.
  __host__ __device__ static constexpr uint32_t loff0(int wave, int lane, uint32_t row_bytes) {
    return (uint32_t)r_lane(wave, lane) * row_bytes +
           (uint32_t)(((lane % CPR) ^ tile_swz<CPR>(r_lane(wave, lane))) << 4);
  }
  // Whole tile (every row inside the chunk): load i reads tile_base + this
  // offset.  Load i's row step is folded into the lane offset; it stays
  // below BN rows of K or V, so under the 4 GiB the host allows for a
  // tensor, and cannot wrap.
  __host__ __device__ static constexpr uint32_t whole_off(uint32_t l0, int i, uint32_t row_bytes) {
    return (l0 ^ ((uint32_t)tile_swz<CPR>(ROWS_PER_LOAD * i) << 4)) + (uint32_t)(i * ROWS_PER_LOAD) * row_bytes;
  }
  // Uniform base of tile kt (whole or ragged).
  __host__ __device__ static constexpr size_t tile_base(int kt, uint32_t row_bytes) {
    return (size_t)kt * BN * row_bytes;
  }
  // Last, ragged tile (the chunk of sk rows ends inside it): load i reads
  // tile_base + this offset.  Lanes whose row lies past the chunk step back
  // to its last row (finite values, masked out).  The offset is taken from
  // the tile's first row, not from load i's own first row (which may lie
  // past the end of the chunk): the clamped row is at or after the tile's
  // first row, so the unsigned offset never goes negative.
  __host__ __device__ static constexpr uint32_t ragged_off(int kt, int i, int rl, uint32_t l0, uint32_t row_bytes,
                                                           int sk) {
    uint32_t off = (l0 ^ ((uint32_t)tile_swz<CPR>(ROWS_PER_LOAD * i) << 4)) + (uint32_t)(i * ROWS_PER_LOAD) * row_bytes;
    const int over = kt * BN + rl + i * ROWS_PER_LOAD - (sk - 1);
    if (over > 0) off -= (uint32_t)over * row_bytes;
    return off;
  }
};

// Loads of the key-stationary dK / dV pass: the K tile of BK keys (once per
// workgroup), and per 32-row query block the Q and dO rows of one query head
// and its LSE and delta values.
template <int D, int BK, int BQ, int WAVES>
struct DkdvAddr {
  static constexpr int CPR = D / 8;
  static constexpr int ROWS_PER_LOAD = 64 / CPR;
  static constexpr int KLOADS = BK / ROWS_PER_LOAD / WAVES;   // K loads per wave
  static constexpr int QLOADS = BQ / ROWS_PER_LOAD / WAVES;   // Q (and dO) loads per wave per block
  static_assert(KLOADS * ROWS_PER_LOAD * WAVES == BK && QLOADS * ROWS_PER_LOAD * WAVES == BQ, "tile rows");

  // K tile load i of a wave: byte offset from the KV head's first row (rows
  // past the chunk re-read its last row).
  __host__ __device__ static constexpr uint32_t k_off(int kr0, int wave, int i, int lane, int sk,
                                                      uint32_t k_row_bytes) {
    const int ld = wave * KLOADS + i;
    const int r = ld * ROWS_PER_LOAD + lane / CPR;
    const int c = (lane % CPR) ^ tile_swz<CPR>(r);
    const int row = kr0 + r < sk - 1 ? kr0 + r : sk - 1;
    return (uint32_t)row * k_row_bytes + (uint32_t)(c << 4);
  }
  // Q / dO load i of a wave inside a whole block: offset from the block's
  // first row (loop invariant; the block base is block_base).
  __host__ __device__ static constexpr uint32_t q_whole_off(int wave, int i, int lane, uint32_t q_row_bytes) {
    const int r = (wave * QLOADS + i) * ROWS_PER_LOAD + lane / CPR;
    return (uint32_t)r * q_row_bytes + (uint32_t)(((lane % CPR) ^ tile_swz<CPR>(r)) << 4);
  }
  __host__ __device__ static constexpr size_t block_base(int qr0, uint32_t q_row_bytes) {
    return (size_t)qr0 * q_row_bytes;
  }
  // Q / dO load i of a wave in the last, ragged block (the chunk of sq rows
  // ends inside it): offset from the query head's first row; rows past the
  // chunk re-read its last row.
  __host__ __device__ static constexpr uint32_t q_ragged_off(int qr0, int wave, int i, int lane, int sq,
                                                             uint32_t q_row_bytes) {
    const int r = (wave * QLOADS + i) * ROWS_PER_LOAD + lane / CPR;
    const int row = qr0 + r < sq - 1 ? qr0 + r : sq - 1;
    return (uint32_t)row * q_row_bytes + (uint32_t)(((lane % CPR) ^ tile_swz<CPR>(r)) << 4);
  }
  // LSE / delta of the block (4-byte loads from one wave, lanes l and l + 32
  // both fetch row qr0 + l % 32): offset from the head's first row.
  __host__ __device__ static constexpr uint32_t lse_off(int qr0, int lane, int sq) {
    const int row = qr0 + (lane & 31) < sq - 1 ? qr0 + (lane & 31) : sq - 1;
    return 4u * (uint32_t)row;
  }
};

}  // namespace rba
