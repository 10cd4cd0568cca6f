// Device-side helpers shared by the forward and backward step kernels:
// chunk row -> global position, document starts, position ranges of row
// ranges, and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rba_addr.h"
#include "rba_kernels.h"

namespace rba {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaskNone = 0, kMaskCausal = 1, kMaskDoc = 2;
constexpr int kPosNone = INT32_MIN;   // "no position": masks every key
constexpr float kLn2 = 0.69314718055994530942f;
// Unbounded ends of a position interval.  Positions are below 2^31, so
// differences with these never overflow int64.
constexpr int64_t kPosNegInf = -(int64_t(1) << 40);
constexpr int64_t kPosPosInf = int64_t(1) << 40;

// Global position of chunk row `row` (0 <= row < rows of the chunk).
__device__ __forceinline__ int32_t row_to_pos(const SegTable& t, int32_t row) {
  int s = 0;
  while (s + 1 < t.n && row >= t.row0[s + 1]) ++s;
  return t.start[s] + (row - t.row0[s]) * t.stride[s];
}

// Start of the document holding position p: the largest cu[t] <= p, t < n_docs.
__device__ __forceinline__ int32_t doc_start(const int32_t* cu, int32_t n_docs, int32_t p) {
  int lo = 0, hi = n_docs - 1;           // answer index in [lo, hi]
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= p) lo = mid; else hi = mid - 1;
  }
  return cu[lo];
}

// The document table in registers: lane l of a wave holds cu[l] for
// l <= n_docs (INT32_MAX above), when the whole table fits one wave
// (n_docs < 64).  A document lookup is then a compare and a ballot (or, for
// a position per lane, a 6-step search over the lanes) instead of a chain
// of dependent loads from global memory.  `ok` is wave-uniform; without it
// the lookups fall back to the binary search over cu.  Every lane of the
// wave must take part in the lookups (they read other lanes' entries).
struct DocLanes {
  int32_t v;
  bool ok;
};

__device__ __forceinline__ DocLanes doc_lanes(const int32_t* cu, int32_t n_docs, int lane) {
  DocLanes d;
  d.ok = cu != nullptr && n_docs > 0 && n_docs < 64;
  d.v = (d.ok && lane <= n_docs) ? cu[lane] : INT32_MAX;
  // The lookups use the table at once; waiting here (vmcnt(0) alone) also
  // tells the compiler that no load into it is pending on the paths that
  // join this one, so code after them need not wait on vector memory.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  return d;
}

// Index t < n_docs of the document holding the wave-uniform position p (the
// largest t with cu[t] <= p): the entries <= p form a prefix of the lanes.
__device__ __forceinline__ int doc_index_u(const DocLanes& d, int32_t p) {
  return __popcll(__ballot(d.v <= p)) - 1;
}

// The same for a position per lane: binary search over the lanes' entries.
__device__ __forceinline__ int doc_index_v(const DocLanes& d, int32_t n_docs, int32_t p) {
  int lo = 0;
#pragma unroll
  for (int step = 32; step > 0; step >>= 1) {
    const int cand = lo + step;
    const int32_t c = __shfl(d.v, min(cand, 63));
    if (cand < n_docs && c <= p) lo = cand;
  }
  return lo;
}

// Document start of a wave-uniform position p (any n_docs).
__device__ __forceinline__ int32_t doc_start_u(const DocLanes& d, const int32_t* cu, int32_t n_docs, int32_t p) {
  if (!d.ok) return doc_start(cu, n_docs, p);
  return __builtin_amdgcn_readlane(d.v, doc_index_u(d, p));
}

// Document start of a position per lane (any n_docs).
__device__ __forceinline__ int32_t doc_start_v(const DocLanes& d, const int32_t* cu, int32_t n_docs, int32_t p) {
  if (!d.ok) return doc_start(cu, n_docs, p);
  return __shfl(d.v, doc_index_v(d, n_docs, p));
}

// Minimum and maximum global position over chunk rows [r0, r1) (r0 < r1),
// and whether those rows lie in a single segment (then row r0 + i is at
// position lo + i * stride).
struct PosRange {
  int32_t lo, hi;
  bool single;
  int32_t stride;
};

__device__ __forceinline__ PosRange pos_range(const SegTable& t, int32_t r0, int32_t r1) {
  PosRange out{INT32_MAX, INT32_MIN, true, 1};
  int hits = 0;
  for (int s = 0; s < t.n; ++s) {
    int32_t a = max(r0, t.row0[s]);
    int32_t b = min(r1, t.row0[s + 1]);
    if (a < b) {
      ++hits;
      out.lo = min(out.lo, t.start[s] + (a - t.row0[s]) * t.stride[s]);
      out.hi = max(out.hi, t.start[s] + (b - 1 - t.row0[s]) * t.stride[s]);
      out.stride = t.stride[s];
    }
  }
  out.single = hits <= 1;
  return out;
}

// Rows [a, b) of a segment (start st, stride sd, len rows) whose positions
// lie in [lo, hi]; a >= b when none do.
struct RowSpan {
  int64_t a, b;
};
__device__ __forceinline__ RowSpan rows_in(int64_t st, int64_t sd, int64_t len, int64_t lo, int64_t hi) {
  // first row at or after lo, one past the last row at or before hi (floor division)
  const int64_t da = lo - st, db = hi - st;
  if (sd == 1)   // contiguous positions: no division
    return RowSpan{min(max(da, (int64_t)0), len), min(max(db + 1, (int64_t)0), len)};
  int64_t a = da <= 0 ? 0 : (da + sd - 1) / sd;
  int64_t b = db < 0 ? 0 : db / sd + 1;
  a = min(a, len);
  b = min(b, len);
  return RowSpan{a, b};
}

// 8 XCDs: consecutive workgroup ids are dealt round-robin to the XCDs.  Map
// them so that every XCD works through one contiguous range of the logical
// order, which keeps workgroups that read the same K/V head on one L2.
__device__ __forceinline__ int xcd_remap(int wg, int n) {
  constexpr int X = 8;
  int per = n / X, rem = n % X;
  int x = wg % X, idx = wg / X;
  int base = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  return base + idx;
}

// Tile classes.
constexpr int kSkip = 0, kFull = 1, kPartial = 2;

// Class of a key tile (positions [k.lo, k.hi], `k.single` if in one segment,
// `ragged` if it runs past the end of the chunk) for query rows whose
// positions lie in [q_lo, q_hi] with document starts in [ds_lo, ds_hi].
__device__ __forceinline__ int classify(int mask, PosRange k, bool ragged,
                                        int32_t q_lo, int32_t q_hi,
                                        int32_t ds_lo, int32_t ds_hi, bool q_any) {
  if (!q_any) return kSkip;
  if (mask == kMaskNone) return ragged ? kPartial : kFull;
  if (k.lo > q_hi) return kSkip;
  if (mask == kMaskDoc && k.hi < ds_lo) return kSkip;
  bool full = k.hi <= q_lo && (mask != kMaskDoc || k.lo >= ds_hi);
  return (full && k.single && !ragged) ? kFull : kPartial;
}

// Is key position kp visible from query position qp with document start qd?
__device__ __forceinline__ bool visible(int mask, int32_t kp, int32_t qp, int32_t qd) {
  if (mask == kMaskNone) return true;
  return kp <= qp && kp >= qd;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Weights of the LSE-weighted merge of two partial results over disjoint key
// sets (blockwise exact attention, FlashAttention in the TASP citation map):
// with L = ln(e^la + e^lb), O = wa Oa + wb Ob for wa = e^(la - L),
// wb = e^(lb - L).  A side with LSE = -inf has weight 0; two such sides give
// weights 0 and L = -inf.  Shared by the merge kernel and the forward step's
// merging epilogue, so both round alike.
struct MergeWeights {
  float wa, wb, L;
};
__device__ __forceinline__ MergeWeights merge_weights(float la, float lb) {
  const float mx = fmaxf(la, lb);
  MergeWeights w{0.f, 0.f, -INFINITY};
  if (mx != -INFINITY) {
    const float a = __expf(la - mx), b = __expf(lb - mx);
    const float s = a + b;
    w.L = mx + __logf(s);
    const float inv = 1.f / s;
    w.wa = a * inv;
    w.wb = b * inv;
  }
  return w;
}

// Both halves of a wave: lane l gets {v[l % 32], v[l % 32 + 32]}.
__device__ __forceinline__ float half_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// MFMA operand read with the LDS transpose load (ds_read_b64_tr_b16).
//
// For a row-major bf16 tile X[row][col] (row stride `stride` elements), this
// returns the operand of a 32x32x16 MFMA whose k index runs along rows and
// whose m (or n) index is the column: lane l gets column n0 + l % 32 and the
// 8 rows rowA + 0..3 (k-slots 0..3 of its half) and rowB + 0..3 (k-slots
// 4..7).  The transpose load works on groups of 16 lanes: each source lane
// supplies the address of 4 consecutive elements, and lane i of the group
// receives element i, 16 + i, 32 + i and 48 + i of the group's 64 elements
// in (source lane, element) order.  Source lane j of a group therefore
// points at row (base + j / 4), column (group column + 4 * (j % 4)), and lane i
// receives rows base..base+3 of column (group column + i).
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* tile, int stride, int rowA, int rowB, int n0,
                                             int lane) {
  typedef __attribute__((address_space(3))) i16x4* lds_i16x4;
  const int j = lane & 15;
  const int colx = n0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const uint16_t* pa = tile + (rowA + (j >> 2)) * stride + colx;
  const uint16_t* pb = tile + (rowB + (j >> 2)) * stride + colx;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(pa));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(pb));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// tile_swz (the XOR swizzle of 16-byte chunks in a tile row) is in rba_addr.h.

// tr_operand for a swizzled, unpadded tile (base = byte address of row 0).
template <int CPR>
__device__ __forceinline__ bf16x8 tr_operand_swz(const char* base, int rowA, int rowB, int n0, int lane) {
  typedef __attribute__((address_space(3))) i16x4* lds_i16x4;
  const int j = lane & 15;
  const int colx = n0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);   // element column
  const int c = colx >> 3, within = (colx & 7) * 2;
  const int ra = rowA + (j >> 2), rb = rowB + (j >> 2);
  const char* pa = base + ra * (CPR * 16) + ((c ^ tile_swz<CPR>(ra)) << 4) + within;
  const char* pb = base + rb * (CPR * 16) + ((c ^ tile_swz<CPR>(rb)) << 4) + within;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(pa));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(pb));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Round-to-nearest-even fp32 -> bf16 pair packed in one dword (lo = a): one
// v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Per-lane byte offsets into a swizzled, unpadded tile for the XOR-linear
// swizzle (the chunk and column-block terms below occupy bits that the row
// term leaves clear, so XOR equals addition there):
//  * row_read_offset: the 16-byte chunk (2 * ks + half) of tile row `row` is
//    at row_read_offset(row, half) ^ (ks << 5).
//  * tr_lane_offset: the transpose-load operand rows row.. row + 3 (source
//    lane j: row + j / 4, column 16 * ((lane >> 4) & 1) + 4 * (j % 4), see
//    tr_operand) at column block 0; column block db (32 * db elements) is
//    at tr_lane_offset(row, lane) ^ (db << 6).
template <int CPR>
__device__ __forceinline__ uint32_t row_read_offset(int row, int half) {
  return (uint32_t)row * (CPR * 16) + ((uint32_t)(half ^ tile_swz<CPR>(row)) << 4);
}
template <int CPR>
__device__ __forceinline__ uint32_t tr_lane_offset(int row, int lane) {
  const int j = lane & 15;
  const int colx = 16 * ((lane >> 4) & 1) + 4 * (j & 3);   // element column in block 0
  const int ra = row + (j >> 2);
  return (uint32_t)ra * (CPR * 16) + ((uint32_t)((colx >> 3) ^ tile_swz<CPR>(ra)) << 4) + (colx & 7) * 2;
}

// The transpose-load operand whose two row groups sit at byte addresses
// base + offA and base + offB (k-slots 0..3 and 4..7 of the lane's half).
__device__ __forceinline__ bf16x8 tr_read(const char* base, uint32_t offA, uint32_t offB) {
  typedef __attribute__((address_space(3))) i16x4* lds_i16x4;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(base + offA));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(base + offB));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Keeps the compiler from hoisting work derived from `x` out of a loop (no
// instruction is emitted): used on lane offsets so that per-iteration XORs
// are recomputed instead of occupying registers for the whole loop.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Direct-to-LDS load, 16 bytes per lane, in the scalar-base form: lane l
// reads global address sbase + voff (voff a 32-bit byte offset) and its data
// lands at LDS byte address lds + 16 * l.  sbase and lds must be uniform
// over the wave.
//
// Written as inline assembly so that the compiler does not see an LDS write:
// it would otherwise make every later LDS read wait for all outstanding
// direct loads (it cannot tell the double buffers apart), which stalls each
// tile on the prefetch of the next.  The caller orders these loads against
// LDS reads itself: s_waitcnt vmcnt(0) and a workgroup barrier before a
// buffer is read, and a barrier before a buffer that was read is refilled.
// M0 carries the LDS address; it is saved and restored around the load.
// A wave-uniform pointer, pinned to SGPRs (readfirstlane is free when the
// value already is scalar; 64-bit address arithmetic otherwise tends to stay
// in VGPRs).
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t b = reinterpret_cast<uint64_t>(p);
  return reinterpret_cast<const char*>(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                                       (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b));
}

__device__ __forceinline__ void dma16(const void* sbase_in, uint32_t voff, uint32_t lds_in) {
  // sbase and lds are uniform by contract; pin them to SGPRs.
  const char* sbase = uniform_ptr(sbase_in);
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_in);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}

// A whole K and V tile pair of direct-to-LDS loads (same ordering contract
// as dma16): load i of K reads kbase + off[i] and lands at LDS byte address
// lds_k + 1024 * i + 16 * lane, and likewise for V at lds_v.  One M0 save
// and restore for all of them, M0 stepped by 1 KiB between loads (each M0
// write is followed by the wait state the load needs).  N is 2 or 4.
template <int N>
__device__ __forceinline__ void dma16_kv(const void* kbase_in, const void* vbase_in, const uint32_t (&off)[N],
                                         uint32_t lds_k_in, uint32_t lds_v_in) {
  const char* kbase = uniform_ptr(kbase_in);
  const char* vbase = uniform_ptr(vbase_in);
  const uint32_t lds_k = __builtin_amdgcn_readfirstlane(lds_k_in);
  const uint32_t lds_v = __builtin_amdgcn_readfirstlane(lds_v_in);
  uint32_t saved;
  if constexpr (N == 4) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %7\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %5\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %5\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %5\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %4, %5\n\t"
        "s_mov_b32 m0, %8\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %6\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %6\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %6\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %4, %6\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(kbase), "s"(vbase), "s"(lds_k), "s"(lds_v)
        : "memory", "scc");
  } else {
    static_assert(N == 2, "2 or 4 loads per tensor");
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %5\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %3\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %6\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %4\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %4\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off[0]), "v"(off[1]), "s"(kbase), "s"(vbase), "s"(lds_k), "s"(lds_v)
        : "memory", "scc");
  }
}

// Direct-to-LDS load of 4 bytes per lane in the scalar-base form: lane l
// reads sbase + voff and its dword lands at LDS byte address lds + 4 * l
// (sbase, lds uniform).  Same ordering contract as dma16.
__device__ __forceinline__ void dma4(const void* sbase_in, uint32_t voff, uint32_t lds_in) {
  const char* sbase = uniform_ptr(sbase_in);
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_in);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

}  // namespace rba
