// Host-side enumeration of the lane addresses of every direct-to-LDS tile
// load the step kernels issue (rba_addr.h, the same functions the kernels
// call): for each tile / block, wave, lane, load and ragged chunk length, the
// 16-byte (or 4-byte) read must lie inside its tensor and inside the rows of
// the head it loads, and must fetch the row and chunk that the lane's LDS
// destination holds.  Built and run by tests/test_addr_cpu.py.
//
// With -DPLANT_OLD_RAGGED the ragged K / V tile offset is computed the way an
// earlier version did (the scalar base includes load i's own row step, so the
// clamped lane offset goes negative and wraps when the chunk ends before
// that row); the test requires this variant to report violations, which
// shows the enumeration reaches the case that once faulted.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "rba_addr.h"

using namespace rba;

struct Tally {
  const char* name;
  uint64_t checked = 0, bad = 0, misplaced = 0;
  void report() const {
    std::printf("%s checked=%llu bad=%llu misplaced=%llu\n", name, (unsigned long long)checked,
                (unsigned long long)bad, (unsigned long long)misplaced);
  }
};

// A read of `bytes` at byte address `addr` of a [rows, heads, row_elems]
// tensor (row stride row_bytes) must stay inside the tensor and inside head
// `h`'s part of one row.
static void check_read(Tally& t, uint64_t addr, uint64_t bytes, uint64_t rows, uint32_t row_bytes, int h,
                       uint32_t head_bytes) {
  ++t.checked;
  const uint64_t size = rows * (uint64_t)row_bytes;
  if (addr + bytes > size) {
    ++t.bad;
    return;
  }
  const uint64_t in_row = addr % row_bytes;
  if (in_row < (uint64_t)h * head_bytes || in_row + bytes > (uint64_t)(h + 1) * head_bytes) ++t.bad;
}

template <int D>
static void kv_tiles(Tally& t, int sk, int hkv, int g, int kt_from) {
  using A = KvTileAddr<D, 64, 4>;
  constexpr int CPR = D / 8;
  const uint32_t head_bytes = D * 2, row_bytes = (uint32_t)hkv * head_bytes;
  const int tiles = (sk + 63) / 64;
  for (int kt = kt_from < 0 ? 0 : kt_from; kt < tiles; ++kt)
    for (int wave = 0; wave < 4; ++wave)
      for (int lane = 0; lane < 64; ++lane) {
        const int rl = A::r_lane(wave, lane);
        const uint32_t l0 = A::loff0(wave, lane, row_bytes);
        for (int i = 0; i < A::LOADS; ++i) {
          const uint64_t head0 = (uint64_t)g * head_bytes;
          uint64_t addr;
          if ((kt + 1) * 64 <= sk) {
            addr = head0 + A::tile_base(kt, row_bytes) + A::whole_off(l0, i, row_bytes);
          } else {
#ifdef PLANT_OLD_RAGGED
            const uint64_t tb = ((uint64_t)kt * 64 + (uint64_t)i * A::ROWS_PER_LOAD) * row_bytes;
            uint32_t off = l0 ^ ((uint32_t)tile_swz<CPR>(A::ROWS_PER_LOAD * i) << 4);
            const int over = kt * 64 + rl + i * A::ROWS_PER_LOAD - (sk - 1);
            if (over > 0) off -= (uint32_t)over * row_bytes;
            addr = head0 + tb + off;
#else
            addr = head0 + A::tile_base(kt, row_bytes) + A::ragged_off(kt, i, rl, l0, row_bytes, sk);
#endif
          }
          check_read(t, addr, 16, (uint64_t)sk, row_bytes, g, head_bytes);
          // the lane's LDS slot is chunk lane % CPR of tile row rl + i * ROWS_PER_LOAD:
          // it must hold that row (clamped to the chunk) and the chunk the swizzle puts there
          const int trow = rl + i * A::ROWS_PER_LOAD;
          const int64_t want_row = (int64_t)kt * 64 + trow < sk - 1 ? (int64_t)kt * 64 + trow : sk - 1;
          const int want_chunk = (lane % CPR) ^ tile_swz<CPR>(trow);
          if (addr + 16 <= (uint64_t)sk * row_bytes) {
            const int64_t got_row = (int64_t)(addr / row_bytes);
            const int got_chunk = (int)((addr % row_bytes - head0) / 16);
            if (got_row != want_row || got_chunk != want_chunk) ++t.misplaced;
          }
        }
      }
}

template <int D>
static void dkdv_loads(Tally& tk, Tally& tq, Tally& tl, int sk, int sq, int hkv, int hq, int g, int h) {
  using A = DkdvAddr<D, 128, 32, 4>;
  constexpr int CPR = D / 8;
  const uint32_t head_bytes = D * 2;
  const uint32_t k_row_bytes = (uint32_t)hkv * head_bytes, q_row_bytes = (uint32_t)hq * head_bytes;
  // K tile of each key workgroup
  for (int kr0 = 0; kr0 < sk; kr0 += 128)
    for (int wave = 0; wave < 4; ++wave)
      for (int lane = 0; lane < 64; ++lane)
        for (int i = 0; i < A::KLOADS; ++i) {
          const uint64_t addr = (uint64_t)g * head_bytes + A::k_off(kr0, wave, i, lane, sk, k_row_bytes);
          check_read(tk, addr, 16, (uint64_t)sk, k_row_bytes, g, head_bytes);
          const int r = (wave * A::KLOADS + i) * A::ROWS_PER_LOAD + lane / CPR;
          const int64_t want_row = kr0 + r < sk - 1 ? kr0 + r : sk - 1;
          const int want_chunk = (lane % CPR) ^ tile_swz<CPR>(r);
          if (addr + 16 <= (uint64_t)sk * k_row_bytes &&
              ((int64_t)(addr / k_row_bytes) != want_row ||
               (int)((addr % k_row_bytes - (uint64_t)g * head_bytes) / 16) != want_chunk))
            ++tk.misplaced;
        }
  // Q / dO rows and LSE / delta of each query block
  for (int qr0 = 0; qr0 < sq; qr0 += 32) {
    const bool whole = qr0 + 32 <= sq;
    for (int wave = 0; wave < 4; ++wave)
      for (int lane = 0; lane < 64; ++lane) {
        for (int i = 0; i < A::QLOADS; ++i) {
          const uint64_t off = whole ? A::block_base(qr0, q_row_bytes) + A::q_whole_off(wave, i, lane, q_row_bytes)
                                     : (uint64_t)A::q_ragged_off(qr0, wave, i, lane, sq, q_row_bytes);
          const uint64_t addr = (uint64_t)h * head_bytes + off;
          check_read(tq, addr, 16, (uint64_t)sq, q_row_bytes, h, head_bytes);
          const int r = (wave * A::QLOADS + i) * A::ROWS_PER_LOAD + lane / CPR;
          const int64_t want_row = qr0 + r < sq - 1 ? qr0 + r : sq - 1;
          const int want_chunk = (lane % CPR) ^ tile_swz<CPR>(r);
          if (addr + 16 <= (uint64_t)sq * q_row_bytes &&
              ((int64_t)(addr / q_row_bytes) != want_row ||
               (int)((addr % q_row_bytes - (uint64_t)h * head_bytes) / 16) != want_chunk))
            ++tq.misplaced;
        }
        if (wave == 0) {
          // LSE / delta [hq, sq] fp32: head h's row of sq values
          const uint64_t addr = (uint64_t)h * sq * 4 + A::lse_off(qr0, lane, sq);
          ++tl.checked;
          if (addr < (uint64_t)h * sq * 4 || addr + 4 > (uint64_t)(h + 1) * sq * 4) ++tl.bad;
          const int64_t want = qr0 + (lane & 31) < sq - 1 ? qr0 + (lane & 31) : sq - 1;
          if ((int64_t)((addr - (uint64_t)h * sq * 4) / 4) != want) ++tl.misplaced;
        }
      }
  }
}

int main() {
  Tally kv64{"kv_tiles_d64"}, kv128{"kv_tiles_d128"};
  Tally dk64{"dkdv_k_d64"}, dq64{"dkdv_q_do_d64"}, dl64{"dkdv_lse_d64"};
  Tally dk128{"dkdv_k_d128"}, dq128{"dkdv_q_do_d128"}, dl128{"dkdv_lse_d128"};
  const int hkvs[] = {1, 2, 8};
  // every chunk length up to 320 rows (every ragged remainder of the 64-,
  // 32- and 128-row tiles, several tiles deep), plus long chunks
  std::vector<int> lens;
  for (int n = 1; n <= 320; ++n) lens.push_back(n);
  for (int n : {4095, 4096, 4097, 8191, 65535, 65536, 65537}) lens.push_back(n);
  for (int hkv : hkvs)
    for (int g : {0, hkv - 1})
      for (int n : lens) {
        kv_tiles<64>(kv64, n, hkv, g, 0);
        kv_tiles<128>(kv128, n, hkv, g, 0);
      }
  // K / V near the 4 GiB the host allows per tensor (d = 128, 8 KV heads:
  // 2 KiB rows): the last tiles only
  for (int n : {2097151, 2097089, 2097100})
    for (int g : {0, 7}) kv_tiles<128>(kv128, n, 8, g, (n + 63) / 64 - 3);
  const int hqs[] = {1, 4, 32};
  for (int hi = 0; hi < 3; ++hi) {
    const int hq = hqs[hi], hkv = hkvs[hi];
    for (int n = 1; n <= 260; ++n) {
      dkdv_loads<64>(dk64, dq64, dl64, n, n + 3, hkv, hq, hkv - 1, hq - 1);
      dkdv_loads<128>(dk128, dq128, dl128, n, n + 3, hkv, hq, 0, 0);
      dkdv_loads<128>(dk128, dq128, dl128, n + 5, n, hkv, hq, hkv - 1, hq - 1);
    }
  }
  for (const Tally* t : {&kv64, &kv128, &dk64, &dq64, &dl64, &dk128, &dq128, &dl128}) t->report();
  return 0;
}
