// Internal interface between the C-ABI host layer (rba_host.cpp) and the HIP
// kernels.  Parameter blocks are passed to kernels by value, so everything a
// kernel needs about a chunk's positions travels in the kernel arguments.
#pragma once

#include <cstddef>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rba {

constexpr int kMaxSegs = 16;
constexpr int kMaxOrder = 512;   // longest host-computed workgroup order passed in kernel arguments
constexpr int kMaxSplitRg = 128; // most row groups whose key range a forward launch splits
constexpr int kFwdTileKeys = 64;   // keys per tile of the query-stationary kernels
constexpr int kMergeThreads = 256;  // threads per workgroup of the merge and preprocess kernels

// A chunk's rows mapped to global positions: rows [row0[s], row0[s+1]) hold
// positions start[s], start[s] + stride[s], ...  (row0[n] = number of rows).
struct SegTable {
  int32_t n;
  int32_t start[kMaxSegs];
  int32_t stride[kMaxSegs];
  int32_t row0[kMaxSegs + 1];
};

// Forward step.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  float* o;            // [sq, hq, d] fp32 partial output, or the running output (accumulate)
  float* lse;          // [hq, sq] fp32 partial log-sum-exp, or the running one
  int32_t accumulate;  // 1: merge the step's partial into (o, lse) in place
  void* o_final;       // accumulate only, may be null: also write the merged output
  int32_t final_bf16;  // 1: o_final is bf16, 0: fp32
  int32_t sq, sk, hq, hkv, group;
  float scale_log2;    // softmax scale * log2(e): scores are exponentiated in base 2
  int32_t mask;        // RBA_MASK_*
  const int32_t* cu;   // device cu_seqlens (document mask)
  int32_t n_docs;
  SegTable qs, ks;
  // launch geometry: each workgroup runs 4 waves; wave w takes query head
  // (w % hpw) of its head group and row block (w / hpw) of its row group.
  int32_t hpw;         // query heads per workgroup (1, 2 or 4)
  int32_t rbw;         // row blocks per workgroup (4 / hpw)
  int32_t n_row_groups;
  // Row groups per head group that get a workgroup (unsplit launches): all
  // of them, or in a merging step with a heavy-first order (`order` or
  // `order_reverse`) only the first n_active (the others have no key to
  // merge).
  int32_t n_rg_launch;
  int32_t n_head_groups;   // hq / hpw
  int32_t n_wg;
  // Heavy-first order of the row groups (host-computed from the masks and
  // segments), used when 0 < n_order (== n_row_groups <= kMaxOrder); the
  // i-th row group a head group's workgroups take is order[i].
  int32_t n_order;
  uint16_t order[kMaxOrder];
  // 1 (only when n_order = 0): row groups are taken last to first, the
  // heavy-first order when work rises with the row index.
  int32_t order_reverse;
  // 1: the host has shown that every key tile a workgroup visits is full
  // (no masked pair, inside the chunk, in one segment) for every wave of it,
  // so the kernel needs no tile classification and no per-element mask.
  int32_t all_full;
  int32_t one_seg;    // no key tile spans two KV segments (launch choice)
  // Split key ranges (forward only; split = 0 elsewhere).  For a launch with
  // too few workgroups for the chip, `order` lists the row groups by
  // decreasing number of key tiles; the first n_active have work, and the
  // first n_split_rg of those are cut into items of split_len[i] tiles
  // (consecutive runs of their visit list).  Item j of order index i < n_split_rg is work item
  // item_start[i] + j; it runs in its own workgroup (per head group) and
  // writes its partial result to workspace slot (item * n_head_groups +
  // head group) of split_slot_floats floats; split_merge_kernel merges the
  // slots of each split row group into the output.  The other active row
  // groups are one item each, numbered after the split ones, and write the
  // output directly; row groups without work follow (one workgroup each).
  int32_t split;
  // Row groups with work (the first n_active of `order` when it is given;
  // set for unsplit launches too, where the rest end at once in a merging
  // step).
  int32_t n_active;
  int32_t n_split_rg;
  int32_t n_items;        // items of the n_active row groups
  uint16_t item_start[kMaxSplitRg + 2];   // one spare entry keeps split_len 4-byte aligned
  uint16_t split_len[kMaxSplitRg];   // tiles per item of each split row group (the last may have fewer)
  float* ws;              // workspace of the split items
};

// The 16-bit tables are read on the device as aligned 32-bit words.
static_assert(offsetof(FwdParams, order) % 4 == 0 && offsetof(FwdParams, item_start) % 4 == 0 &&
                  offsetof(FwdParams, split_len) % 4 == 0 && kMaxOrder % 2 == 0 && kMaxSplitRg % 2 == 0,
              "16-bit kernel-argument tables must start and end on 4-byte boundaries");

// Floats of one split item's workspace slot: the partial (O normalized, LSE)
// of the 4 waves x 32 rows of a query-stationary workgroup.
constexpr int64_t split_slot_floats(int d) { return 4 * 32 * (int64_t)d + 4 * 32; }

// Backward step, dK / dV kernel (key-stationary).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* d_o;
  const float* lse;    // [hq, sq] final log-sum-exp (natural log)
  const float* delta;  // [hq, sq]
  float* dk;           // [sk, hkv, d]: overwritten, or added into (accumulate)
  float* dv;           // [sk, hkv, d]
  int32_t accumulate;  // 1: dk / dv are accumulators (+=); 0: zero-filled outputs
  int32_t sq, sk, hq, hkv, group;
  float scale;
  float scale_log2;
  int32_t mask;
  const int32_t* cu;
  int32_t n_docs;
  SegTable qs, ks;
  int32_t n_key_tiles;
  int32_t heads_per_wg;   // query heads of a group one workgroup sums over (divides group)
  // 1: the host has shown that every (key wave, query block) pair a
  // workgroup visits is full, so the pass needs no classification or mask.
  int32_t all_full;
  int32_t n_wg;      // n_key_tiles * hkv * group / heads_per_wg: one workgroup per (key tile, head set)
};

// Backward dQ kernel: the query-stationary geometry of a forward step (the
// o and lse members of `f` are unused) plus the backward operands.
struct DqParams {
  FwdParams f;
  const void* d_o;     // [sq, hq, d] bf16
  const float* lse;    // [hq, sq] final log-sum-exp (natural log)
  const float* delta;  // [hq, sq]
  float* dq;           // [sq, hq, d] fp32, dq += scale * dS K
  float scale;
};

struct MergeParams {
  float* o_acc;
  float* lse_acc;
  const float* o_part;   // may be null (finalise only)
  const float* lse_part;
  void* o_final;         // may be null
  int32_t final_bf16;    // 1: o_final is bf16, 0: fp32
  int64_t n_pairs;       // sq * hq
  int32_t sq, hq, d;
  // thread map (merge_lanes): a pair's lanes_per_pair consecutive threads
  // (a power of two dividing 64) each move vecs_per_lane 16-byte vectors
  int32_t lanes_per_pair, vecs_per_lane;
};

// Thread map of the merge kernel for head dimension d (a multiple of 4 in
// [4, 1024]): lanes per pair = the smallest power of two >= d / 4, at most
// 64; vectors per lane = ceil(d / 4 / lanes per pair).
inline void merge_lanes(int d, int* lanes_per_pair, int* vecs_per_lane) {
  const int nv = d / 4;
  int lpp = 1;
  while (lpp < nv && lpp < 64) lpp *= 2;
  *lanes_per_pair = lpp;
  *vecs_per_lane = (nv + lpp - 1) / lpp;
}

struct PrepParams {
  const void* o;
  const void* d_o;
  float* delta;
  int64_t n_pairs;
  int32_t sq, hq, d;
  int32_t o_bf16, do_bf16;   // element types of O and dO (1: bf16, 0: fp32)
};

// Launchers (defined next to their kernels).  Each returns the launch status.
hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t s);
// Merges the split items' partials into the output (after launch_fwd_bf16
// of a split launch, on the same stream).
hipError_t launch_split_merge(const FwdParams& p, int d, hipStream_t s);
hipError_t launch_fwd_f32(const FwdParams& p, int d, hipStream_t s);
hipError_t launch_merge(const MergeParams& p, hipStream_t s);
hipError_t launch_bwd_preprocess(const PrepParams& p, hipStream_t s);
// The backward step's dK / dV and dQ passes, in one launch.
hipError_t launch_bwd(const BwdParams& p, const DqParams& dp, int d, hipStream_t s);
hipError_t launch_zero_f32(float* a, float* b, int64_t n, hipStream_t s);

// Rows of the forward workgroup tile per wave (32 * fwd_row_blocks).
int fwd_rows_per_wave(int d, int dtype_bf16);
// Keys per backward workgroup.
int bwd_keys_per_wg(int d);

}  // namespace rba
