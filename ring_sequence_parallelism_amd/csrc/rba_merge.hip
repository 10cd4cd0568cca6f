// LSE-weighted merge of ring-step partials, and the backward preprocess.
//
// Merge (blockwise exact attention, FlashAttention in the TASP citation map;
// the merge of two partial softmax results over disjoint key sets follows from
// the definition): with L = ln(e^{La} + e^{Lb}),
//   O = e^{La - L} Oa + e^{Lb - L} Ob,  LSE = L,
// and a side with LSE = -inf carrying weight 0.
//
// Both kernels stream memory once; they are bound by HBM bandwidth.
//
// Merge thread map.  A (row, head) pair of d / 4 16-byte vectors is handled
// by a group of `lpp` consecutive threads, lpp = the smallest power of two
// >= d / 4, capped at 64 (merge_lanes in the host layer); thread t of a
// workgroup takes pair slot t / lpp and vectors (t % lpp) + i * lpp for
// i < vpl = ceil(d / 4 / lpp).  Since lpp divides 64, a pair's threads are
// lanes of one wave: they all read the pair's two LSE values before the
// wave's single store of the merged LSE (program order within a wave, and
// the stored value depends on the loaded ones), so no thread of the pair
// can read an LSE that is already merged, whatever d is.
#include "rba_device.h"

namespace rba {

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeParams p) {
  const int lpp = p.lanes_per_pair, vpl = p.vecs_per_lane;
  const int ppb = kMergeThreads / lpp;            // pairs per block per sweep
  const int sub = threadIdx.x / lpp, c0 = threadIdx.x % lpp;
  const int nv = p.d >> 2;                        // 16-byte vectors per pair
  for (int64_t pair = (int64_t)blockIdx.x * ppb + sub; pair < p.n_pairs; pair += (int64_t)gridDim.x * ppb) {
    const int row = (int)(pair / p.hq), h = (int)(pair % p.hq);
    const size_t li = (size_t)h * p.sq + row;
    MergeWeights w{1.f, 0.f, 0.f};
    if (p.o_part) w = merge_weights(p.lse_acc[li], p.lse_part[li]);
    for (int i = 0; i < vpl; ++i) {
      const int c4 = c0 + i * lpp;
      if (c4 >= nv) break;
      const size_t oi = (size_t)pair * p.d + 4 * c4;
      f32x4 o = *reinterpret_cast<const f32x4*>(p.o_acc + oi);
      if (p.o_part) {
        const f32x4 ob = *reinterpret_cast<const f32x4*>(p.o_part + oi);
        o = w.wa * o + w.wb * ob;
        *reinterpret_cast<f32x4*>(p.o_acc + oi) = o;
      }
      if (p.o_final) {
        if (p.final_bf16) {
          u32x2 b = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o_final) + oi) = b;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.o_final) + oi) = o;
        }
      }
    }
    if (p.o_part && c0 == 0) p.lse_acc[li] = w.L;
  }
}

// delta[h, i] = sum_c dO[i, h, c] * O[i, h, c].  Each thread takes 4
// consecutive elements of one (row, head) pair from both tensors (8 or 16
// bytes per load, by element type).
__device__ __forceinline__ f32x4 load4(const void* base, size_t i, bool bf16) {
  if (bf16) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(base) + i);
    return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                 __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
  }
  return *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + i);
}

__global__ __launch_bounds__(kMergeThreads) void bwd_preprocess_kernel(PrepParams p) {
  const int tpp = p.d / 4;                        // threads per pair (power of two, <= 32)
  const int ppb = kMergeThreads / tpp;
  const int sub = threadIdx.x / tpp, c = threadIdx.x % tpp;
  for (int64_t base = (int64_t)blockIdx.x * ppb; base < p.n_pairs; base += (int64_t)gridDim.x * ppb) {
    const int64_t pair = base + sub;
    float acc = 0.f;
    if (pair < p.n_pairs) {
      const size_t i = (size_t)pair * p.d + (size_t)c * 4;
      const f32x4 a = load4(p.o, i, p.o_bf16), b = load4(p.d_o, i, p.do_bf16);
      acc = a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
    }
    // reduce over the tpp consecutive lanes of the pair
    for (int off = tpp >> 1; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (pair < p.n_pairs && c == 0) {
      const int row = (int)(pair / p.hq), h = (int)(pair % p.hq);
      p.delta[(size_t)h * p.sq + row] = acc;
    }
  }
}

static int grid_for(int64_t n_pairs, int ppb) {
  int64_t blocks = (n_pairs + ppb - 1) / ppb;
  const int64_t cap = 256 * 16;   // enough resident waves to saturate HBM
  return (int)(blocks < cap ? (blocks > 0 ? blocks : 1) : cap);
}

hipError_t launch_merge(const MergeParams& p, hipStream_t s) {
  const int ppb = kMergeThreads / p.lanes_per_pair;
  hipLaunchKernelGGL(merge_kernel, dim3(grid_for(p.n_pairs, ppb)), dim3(kMergeThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_preprocess(const PrepParams& p, hipStream_t s) {
  const int ppb = kMergeThreads / (p.d / 4);
  hipLaunchKernelGGL(bwd_preprocess_kernel, dim3(grid_for(p.n_pairs, ppb)), dim3(kMergeThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace rba
