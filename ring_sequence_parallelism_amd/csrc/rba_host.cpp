// C-ABI host layer of the ring block-attention library: argument validation,
// host-side step planning (exact pair counts, empty-step detection), launch
// geometry.  The entry points and their contracts are declared in rba.h.
#include "rba.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "rba_kernels.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// Segments

struct Seg {
  int64_t start, len, row0, stride;
  int64_t last() const { return start + (len - 1) * stride; }   // last position
};

// Do the position progressions of two segments share a position?  Solved
// with the Chinese remainder theorem: a0 + i sa = b0 + j sb has solutions
// x = x0 (mod lcm) iff gcd(sa, sb) divides b0 - a0; then the smallest such x
// in the intersection of the two ranges decides.
bool segs_overlap(const Seg& a, const Seg& b) {
  const int64_t lo = std::max(a.start, b.start), hi = std::min(a.last(), b.last());
  if (lo > hi) return false;
  // extended Euclid on (sa, sb)
  int64_t r0 = a.stride, r1 = b.stride, s0 = 1, s1 = 0;
  while (r1) {
    const int64_t q = r0 / r1, t = r0 - q * r1;
    r0 = r1; r1 = t;
    const int64_t u = s0 - q * s1;
    s0 = s1; s1 = u;
  }
  const int64_t g = r0;                       // s0 * sa = g (mod sb)
  const int64_t diff = b.start - a.start;
  if (diff % g) return false;
  const int64_t m = b.stride / g;             // solutions i = i0 (mod m)
  const __int128 i0 = (((__int128)(diff / g) * s0) % m + m) % m;
  const __int128 L = (__int128)a.stride * m;  // lcm
  const __int128 x0 = (__int128)a.start + i0 * a.stride;
  __int128 x = x0;
  if (x < lo) x += ((lo - x + L - 1) / L) * L;
  return x <= hi;
}

// Validates a chunk's segment list against its row count.  rows == 0 allows
// n == 0.  On success fills `out` (in row order).
int check_segs(const rba_segs* s, int64_t rows, const char* what, std::vector<Seg>& out) {
  out.clear();
  if (!s) return fail(RBA_ERR_INVALID, "%s: segment list is NULL", what);
  if (s->n < 0 || s->n > RBA_MAX_SEGS)
    return fail(RBA_ERR_INVALID, "%s: segment count %d outside [0, %d]", what, s->n, RBA_MAX_SEGS);
  if (s->n == 0 && rows != 0) return fail(RBA_ERR_INVALID, "%s: no segments for %lld rows", what, (long long)rows);
  int64_t total = 0;
  for (int i = 0; i < s->n; ++i) {
    if (s->len[i] < 1) return fail(RBA_ERR_INVALID, "%s: segment %d has length %lld", what, i, (long long)s->len[i]);
    if (s->start[i] < 0) return fail(RBA_ERR_INVALID, "%s: segment %d starts at %lld", what, i, (long long)s->start[i]);
    if (s->stride[i] < 0)
      return fail(RBA_ERR_INVALID, "%s: segment %d has stride %lld", what, i, (long long)s->stride[i]);
    const int64_t stride = s->stride[i] ? s->stride[i] : 1;
    if (stride > (int64_t)INT32_MAX || s->len[i] > (int64_t)INT32_MAX ||
        s->start[i] + (s->len[i] - 1) * stride >= (int64_t)INT32_MAX)
      return fail(RBA_ERR_UNSUPPORTED, "%s: segment %d reaches past position 2^31-2", what, i);
    out.push_back({s->start[i], s->len[i], total, stride});
    total += s->len[i];
  }
  if (total != rows)
    return fail(RBA_ERR_INVALID, "%s: segment lengths sum to %lld, expected %lld rows", what, (long long)total,
                (long long)rows);
  for (size_t i = 0; i < out.size(); ++i)
    for (size_t j = i + 1; j < out.size(); ++j)
      if (segs_overlap(out[i], out[j])) return fail(RBA_ERR_INVALID, "%s: segments overlap in position", what);
  return RBA_OK;
}

rba::SegTable to_table(const std::vector<Seg>& segs) {
  rba::SegTable t{};
  t.n = (int32_t)segs.size();
  int64_t r = 0;
  for (size_t i = 0; i < segs.size(); ++i) {
    t.start[i] = (int32_t)segs[i].start;
    t.stride[i] = (int32_t)segs[i].stride;
    t.row0[i] = (int32_t)r;
    r += segs[i].len;
  }
  t.row0[segs.size()] = (int32_t)r;
  return t;
}

// ---------------------------------------------------------------------------
// Pair counting.  sum_{p = p0}^{p1 - 1} clamp(p - lo + 1, 0, cap): the number
// of keys in [lo, lo + cap) at or before each position p, summed over p.
int64_t sum_clamp(int64_t p0, int64_t p1, int64_t lo, int64_t cap) {
  if (p1 <= p0 || cap <= 0) return 0;
  int64_t total = 0;
  // ramp: p in [lo, lo + cap - 1) contributes p - lo + 1
  const int64_t r0 = std::max(p0, lo), r1 = std::min(p1, lo + cap - 1);
  if (r1 > r0) {
    const int64_t a = r0 - lo + 1, b = r1 - 1 - lo + 1;  // first and last term
    total += (a + b) * (r1 - r0) / 2;
  }
  // plateau: p >= lo + cap - 1 contributes cap
  const int64_t f0 = std::max(p0, lo + cap - 1);
  if (p1 > f0) total += (p1 - f0) * cap;
  return total;
}

struct DocTable {
  const int32_t* cu = nullptr;
  int32_t n = 0;
};

int check_docs(const rba_attn* a, DocTable& dt) {
  if (!a->cu_seqlens_dev) return fail(RBA_ERR_INVALID, "document mask: cu_seqlens_dev is NULL");
  if (a->n_docs < 1) return fail(RBA_ERR_INVALID, "document mask: n_docs = %d", a->n_docs);
  if (a->cu_seqlens_host) {
    const int32_t* cu = a->cu_seqlens_host;
    if (cu[0] != 0) return fail(RBA_ERR_INVALID, "cu_seqlens[0] = %d, expected 0", cu[0]);
    for (int t = 0; t < a->n_docs; ++t)
      if (cu[t + 1] <= cu[t]) return fail(RBA_ERR_INVALID, "cu_seqlens not strictly ascending at %d", t);
    dt.cu = cu;
    dt.n = a->n_docs;
  }
  return RBA_OK;
}

int check_positions_in_docs(const std::vector<Seg>& segs, const DocTable& dt, const char* what) {
  if (!dt.cu) return RBA_OK;
  for (const Seg& s : segs)
    if (s.last() >= dt.cu[dt.n])
      return fail(RBA_ERR_INVALID, "%s: position %lld is past the packed buffer (%d tokens)", what,
                  (long long)s.last(), dt.cu[dt.n]);
  return RBA_OK;
}

int64_t floor_div(int64_t a, int64_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// Keys of segment k at positions in [lo, hi].
int64_t keys_in(const Seg& k, int64_t lo, int64_t hi) {
  const int64_t b0 = std::max<int64_t>(0, -floor_div(k.start - lo, k.stride));   // first index with pos >= lo
  const int64_t b1 = std::min<int64_t>(k.len - 1, floor_div(hi - k.start, k.stride));
  return b1 >= b0 ? b1 - b0 + 1 : 0;
}

// Exact allowed-pair count of a step (per query head).
int64_t count_pairs(int mask, const std::vector<Seg>& qs, const std::vector<Seg>& ks, const DocTable& dt) {
  int64_t total = 0;
  for (const Seg& q : qs)
    for (const Seg& k : ks) {
      if (mask == RBA_MASK_NONE) {
        total += q.len * k.len;
      } else if (q.stride != 1 || k.stride != 1) {
        // strided positions: per query row, the keys in [doc start, q]
        for (int64_t a = 0; a < q.len; ++a) {
          const int64_t qp = q.start + a * q.stride;
          int64_t lo = INT64_MIN / 4;
          if (mask == RBA_MASK_DOC_CAUSAL) lo = std::upper_bound(dt.cu, dt.cu + dt.n + 1, (int32_t)qp)[-1];
          total += keys_in(k, lo, qp);
        }
      } else if (mask == RBA_MASK_CAUSAL) {
        total += sum_clamp(q.start, q.start + q.len, k.start, k.len);
      } else {
        // documents intersecting the query segment
        int t = (int)(std::upper_bound(dt.cu, dt.cu + dt.n + 1, (int32_t)q.start) - dt.cu) - 1;
        for (; t < dt.n && dt.cu[t] < q.start + q.len; ++t) {
          const int64_t ds = dt.cu[t], de = dt.cu[t + 1];
          const int64_t p0 = std::max(q.start, ds), p1 = std::min(q.start + q.len, de);
          const int64_t lo = std::max(k.start, ds);
          const int64_t cap = std::min(k.start + k.len, de) - lo;
          total += sum_clamp(p0, p1, lo, cap);
        }
      }
    }
  return total;
}

// ---------------------------------------------------------------------------
// Common argument checks of fwd/bwd steps.

int check_attn(const rba_attn* a, bool backward) {
  if (!a) return fail(RBA_ERR_INVALID, "attention parameters are NULL");
  if (a->hq < 1 || a->hkv < 1) return fail(RBA_ERR_INVALID, "hq = %d, hkv = %d must be >= 1", a->hq, a->hkv);
  if (a->hq % a->hkv) return fail(RBA_ERR_INVALID, "hq = %d is not a multiple of hkv = %d", a->hq, a->hkv);
  if (a->d != 64 && a->d != 128) return fail(RBA_ERR_UNSUPPORTED, "head dimension %d (supported: 64, 128)", a->d);
  if (!(std::isfinite(a->scale) && a->scale > 0.f)) return fail(RBA_ERR_INVALID, "scale must be finite and > 0");
  if (a->dtype != RBA_BF16 && a->dtype != RBA_F32) return fail(RBA_ERR_INVALID, "unknown dtype %d", (int)a->dtype);
  if (backward && a->dtype != RBA_BF16) return fail(RBA_ERR_UNSUPPORTED, "backward step supports bf16 only");
  if (a->mask != RBA_MASK_NONE && a->mask != RBA_MASK_CAUSAL && a->mask != RBA_MASK_DOC_CAUSAL)
    return fail(RBA_ERR_INVALID, "unknown mask %d", (int)a->mask);
  return RBA_OK;
}

int check_rows(int64_t rows, const char* what) {
  if (rows < 0) return fail(RBA_ERR_INVALID, "%s: negative row count", what);
  if (rows > (int64_t)INT32_MAX) return fail(RBA_ERR_UNSUPPORTED, "%s: %lld rows (limit 2^31-1)", what, (long long)rows);
  return RBA_OK;
}

int check_ptr(const void* p, const char* what) {
  if (!p) return fail(RBA_ERR_INVALID, "%s is NULL", what);
  if (!aligned16(p)) return fail(RBA_ERR_ALIGNMENT, "%s is not 16-byte aligned", what);
  return RBA_OK;
}

// gfx950 check, cached per device (devices 0..63; others are checked on
// every call).  The caches are atomics: calls from several host threads
// may fill them at once, with the same values.
int check_device() {
  static std::atomic<int> state[64];  // 0 unknown, 1 ok, -1 unsupported
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RBA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  const bool cached = dev >= 0 && dev < 64;
  int st = cached ? state[dev].load(std::memory_order_relaxed) : 0;
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(RBA_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    if (cached) state[dev].store(st, std::memory_order_relaxed);
  }
  if (st < 0) return fail(RBA_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return RBA_OK;
}

// Compute units of the current device (cached per device; 256 if unknown).
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(RBA_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return RBA_OK;
}

// Shared preparation of a fwd or bwd step: validates, plans, fills geometry.
struct StepPlan {
  std::vector<Seg> qs, ks;
  DocTable dt;
  bool empty = false;
};

int prepare_step(const rba_attn* a, int64_t sq, const rba_segs* q_segs, int64_t sk, const rba_segs* kv_segs,
                 bool backward, StepPlan& plan) {
  int rc;
  if ((rc = check_attn(a, backward))) return rc;
  if ((rc = check_rows(sq, "query chunk"))) return rc;
  if ((rc = check_rows(sk, "KV chunk"))) return rc;
  if ((rc = check_segs(q_segs, sq, "query chunk", plan.qs))) return rc;
  if ((rc = check_segs(kv_segs, sk, "KV chunk", plan.ks))) return rc;
  if (a->mask == RBA_MASK_DOC_CAUSAL) {
    if ((rc = check_docs(a, plan.dt))) return rc;
    if ((rc = check_positions_in_docs(plan.qs, plan.dt, "query chunk"))) return rc;
    if ((rc = check_positions_in_docs(plan.ks, plan.dt, "KV chunk"))) return rc;
  }
  plan.empty = sq == 0 || sk == 0;
  if (!plan.empty) {
    if (a->mask == RBA_MASK_CAUSAL) {
      int64_t kmin = INT64_MAX, qmax = INT64_MIN;
      for (const Seg& s : plan.ks) kmin = std::min(kmin, s.start);
      for (const Seg& s : plan.qs) qmax = std::max(qmax, s.last());
      plan.empty = kmin > qmax;
    } else if (a->mask == RBA_MASK_DOC_CAUSAL && plan.dt.cu) {
      plan.empty = count_pairs(a->mask, plan.qs, plan.ks, plan.dt) == 0;
    }
  }
  return RBA_OK;
}

// Global position range [lo, hi] of chunk rows [r0, r1) (r0 < r1).
std::pair<int64_t, int64_t> host_pos_range(const std::vector<Seg>& segs, int64_t r0, int64_t r1) {
  int64_t lo = INT64_MAX, hi = INT64_MIN;
  for (const Seg& s : segs) {
    const int64_t a = std::max(r0, s.row0), b = std::min(r1, s.row0 + s.len);
    if (a < b) {
      lo = std::min(lo, s.start + (a - s.row0) * s.stride);
      hi = std::max(hi, s.start + (b - 1 - s.row0) * s.stride);
    }
  }
  return {lo, hi};
}

// Start of the document holding position p (host copy of cu_seqlens).
int64_t host_doc_start(const DocTable& dt, int64_t p) {
  const int32_t* it = std::upper_bound(dt.cu, dt.cu + dt.n + 1, (int32_t)p);
  return it[-1];
}

// Heavy-first order of the row groups of a query-stationary launch: the
// work of a row group is the number of key rows in its allowed position
// interval (the interval its workgroup walks: up to the group's last
// position, from the document start of its first position under the
// document mask), and groups are sorted by decreasing work (stable).  Left
// in natural order without a mask (all equal) or without the host copy of
// cu_seqlens.  Beyond kMaxOrder groups only the reversed natural order is
// available (when it is heavy-first).
void fill_row_order(const rba_attn* a, const StepPlan& plan, int64_t sq, rba::FwdParams& p, int64_t rows_per_wg) {
  p.n_order = 0;
  p.order_reverse = 0;
  p.n_active = p.n_row_groups;
  if (a->mask == RBA_MASK_NONE) return;
  if (a->mask == RBA_MASK_DOC_CAUSAL && !plan.dt.cu) return;
  std::vector<std::pair<int64_t, int>> work(p.n_row_groups);
  for (int rg = 0; rg < p.n_row_groups; ++rg) {
    const int64_t r0 = rg * rows_per_wg, r1 = std::min(sq, r0 + rows_per_wg);
    const auto pr = host_pos_range(plan.qs, r0, r1);
    const int64_t k_hi = pr.second;
    const int64_t k_lo = a->mask == RBA_MASK_DOC_CAUSAL ? host_doc_start(plan.dt, pr.first) : INT64_MIN;
    int64_t w = 0;
    for (const Seg& s : plan.ks) w += keys_in(s, std::max(k_lo, INT64_MIN / 4), k_hi);
    work[rg] = {w, rg};
  }
  if (p.n_row_groups > rba::kMaxOrder) {
    // Too many groups to list in the kernel arguments.  When the work never
    // decreases along the rows (a causal chunk whose positions ascend, such
    // as a zigzag rank's own step) and is not all equal, the reversed
    // natural order is heavy-first: each XCD then starts groups of similar
    // length together, whose workgroups walk the same key tiles at the same
    // time and share them in L2.
    bool rising = true, equal = true;
    for (int rg = 1; rg < p.n_row_groups; ++rg) {
      rising = rising && work[rg].first >= work[rg - 1].first;
      equal = equal && work[rg].first == work[0].first;
    }
    p.order_reverse = (rising && !equal) ? 1 : 0;
    if (p.order_reverse) {
      // the row groups with work are a suffix, taken first
      int n_active = 0;
      while (n_active < p.n_row_groups && work[p.n_row_groups - 1 - n_active].first > 0) ++n_active;
      p.n_active = n_active;
    }
    return;
  }
  std::stable_sort(work.begin(), work.end(), [](const std::pair<int64_t, int>& x, const std::pair<int64_t, int>& y) {
    return x.first > y.first;
  });
  for (int i = 0; i < p.n_row_groups; ++i) p.order[i] = (uint16_t)work[i].second;
  p.n_order = p.n_row_groups;
  // the row groups with work come first; the others visit no key tile
  int n_active = 0;
  while (n_active < p.n_row_groups && work[n_active].first > 0) ++n_active;
  p.n_active = n_active;
}

// Does every key tile that a query-stationary workgroup visits hold only
// pairs that the mask allows for every row of the workgroup (and no row past
// the chunk, and rows of one segment)?  A workgroup of rows with positions
// in [wlo, whi] visits, in each KV segment, the tiles of the rows at
// positions up to whi (causal); they are all full when none of those keys
// lies after wlo and the visited rows end on a tile boundary (or at the end
// of the segment).  Without a mask every tile is full unless it is ragged.
// The document mask is never taken as full.
bool all_tiles_full(const rba_attn* a, const StepPlan& plan, int64_t sq, int64_t sk, int64_t rows_per_wg) {
  constexpr int64_t BN = rba::kFwdTileKeys;
  if (a->mask == RBA_MASK_DOC_CAUSAL || sk % BN) return false;
  if (a->mask == RBA_MASK_NONE) return true;
  for (const Seg& k : plan.ks)
    if (k.row0 % BN || k.len % BN) return false;
  for (int64_t r0 = 0; r0 < sq; r0 += rows_per_wg) {
    const auto w = host_pos_range(plan.qs, r0, std::min(sq, r0 + rows_per_wg));
    for (const Seg& k : plan.ks) {
      // visited rows: positions start + i * stride <= whi
      const int64_t v = w.second < k.start ? 0 : std::min(k.len, (w.second - k.start) / k.stride + 1);
      if (v == 0) continue;
      if (k.start + (v - 1) * k.stride > w.first) return false;
      if (v < k.len && v % BN) return false;
    }
  }
  return true;
}

// Query heads of a query-stationary workgroup (4 waves): 4, 2 or 1 heads of
// one KV head, times 4 / that many row blocks.
int query_heads_per_wg(int group) { return (group % 4 == 0) ? 4 : (group % 2 == 0 ? 2 : 1); }
int64_t query_rows_per_wg(int group, int rows_per_wave) {
  return (int64_t)(4 / query_heads_per_wg(group)) * rows_per_wave;
}

// Sizes, mask, segments and the launch geometry of the query-stationary
// kernels (forward step, backward dQ): workgroups of 4 waves, each wave
// `rows_per_wave` query rows of one head; a workgroup takes 4, 2 or 1 query
// heads of one KV head (hpw) times 1, 2 or 4 row blocks (rbw).
int fill_query_tiling(const rba_attn* a, int64_t sq, int64_t sk, const StepPlan& plan, int rows_per_wave,
                      rba::FwdParams& p) {
  p.sq = (int32_t)sq; p.sk = (int32_t)sk; p.hq = a->hq; p.hkv = a->hkv; p.group = a->hq / a->hkv;
  p.scale_log2 = a->scale * 1.4426950408889634f;
  p.mask = a->mask;
  p.cu = a->mask == RBA_MASK_DOC_CAUSAL ? a->cu_seqlens_dev : nullptr;
  p.n_docs = a->mask == RBA_MASK_DOC_CAUSAL ? a->n_docs : 0;
  p.qs = to_table(plan.qs);
  p.ks = to_table(plan.ks);
  p.hpw = query_heads_per_wg(p.group);
  p.rbw = 4 / p.hpw;
  const int64_t rows_per_wg = query_rows_per_wg(p.group, rows_per_wave);
  p.n_row_groups = (int32_t)((sq + rows_per_wg - 1) / rows_per_wg);
  p.n_head_groups = a->hq / p.hpw;
  p.n_rg_launch = p.n_row_groups;
  const int64_t n_wg = (int64_t)p.n_row_groups * p.n_head_groups;
  if (n_wg > INT32_MAX) return fail(RBA_ERR_UNSUPPORTED, "too many workgroups");
  p.n_wg = (int32_t)n_wg;
  fill_row_order(a, plan, sq, p, rows_per_wg);
  p.all_full = all_tiles_full(a, plan, sq, sk, rows_per_wg) ? 1 : 0;
  // every KV segment boundary on a tile boundary: no tile spans two segments
  p.one_seg = 1;
  for (const Seg& k : plan.ks)
    if (k.row0 % rba::kFwdTileKeys) p.one_seg = 0;
  return RBA_OK;
}

// Rows [a, b) of segment k whose positions lie in [lo, hi] (a >= b: none),
// as the device's rows_in computes them.
std::pair<int64_t, int64_t> host_rows_in(const Seg& k, int64_t lo, int64_t hi) {
  const int64_t a = std::min(k.len, std::max<int64_t>(0, -floor_div(k.start - lo, k.stride)));
  const int64_t b = std::min(k.len, std::max<int64_t>(0, floor_div(hi - k.start, k.stride) + 1));
  return {a, b};
}

// Number of key tiles the query-stationary workgroup of rows [r0, r1)
// visits: the host form of the device's tile iterator (per KV segment in row
// order, the tiles holding rows whose positions lie in the workgroup's
// allowed interval, each tile once).
int64_t visited_tiles(const rba_attn* a, const StepPlan& plan, int64_t r0, int64_t r1) {
  constexpr int64_t BN = rba::kFwdTileKeys;
  const auto pr = host_pos_range(plan.qs, r0, r1);
  int64_t k_lo = INT64_MIN / 4, k_hi = INT64_MAX / 4;
  if (a->mask != RBA_MASK_NONE) k_hi = pr.second;
  if (a->mask == RBA_MASK_DOC_CAUSAL) k_lo = host_doc_start(plan.dt, pr.first);
  int64_t next_tile = 0, count = 0;
  for (const Seg& k : plan.ks) {
    const auto rs = host_rows_in(k, k_lo, k_hi);
    if (rs.first >= rs.second) continue;
    const int64_t t0 = std::max((k.row0 + rs.first) / BN, next_tile);
    const int64_t t1 = (k.row0 + rs.second + BN - 1) / BN;
    if (t1 > t0) count += t1 - t0;
    next_tile = std::max(next_tile, t1);
  }
  return count;
}

// Largest workspace a forward launch splits into (bytes).
constexpr int64_t kSplitMaxBytes = int64_t(32) << 20;
// A launch splits only when its heaviest row group visits at least this many
// key tiles: each workgroup's tiles follow one another at about the latency
// of one tile load, and a split adds the partials' round trip and a merge
// launch (roughly the time of 8-10 such tiles), so shorter lists gain nothing.
constexpr int64_t kSplitMinTiles = 32;

// Fixed cost of a forward workgroup (setup, first tile, epilogue) and of the
// split merge launch, in key-tile times, for the launch-length estimate.
constexpr int64_t kWgFixedTiles = 4;
constexpr int64_t kMergeTiles = 10;

// Length of a forward launch in key-tile times, estimated by replaying the
// hardware's dispatch: workgroups in logical order (per head group, `len`
// holds the row groups' or items' tile counts in launch order), each XCD
// taking a contiguous eighth of that order (xcd_remap) onto its share of the
// slots, each workgroup starting on the slot that frees first.
int64_t launch_length(const std::vector<int64_t>& len, int n_head_groups, int64_t slots) {
  const int64_t n = (int64_t)len.size() * n_head_groups;
  constexpr int64_t X = 8;
  const int64_t per = n / X, rem = n % X, xslots = std::max<int64_t>(1, slots / X);
  int64_t end = 0;
  for (int64_t x = 0, base = 0; x < X; ++x) {
    const int64_t cnt = per + (x < rem ? 1 : 0);
    std::vector<int64_t> free_at(xslots, 0);
    for (int64_t j = base; j < base + cnt; ++j) {
      auto it = std::min_element(free_at.begin(), free_at.end());
      *it += len[j % len.size()] + kWgFixedTiles;
      end = std::max(end, *it);
    }
    base += cnt;
  }
  return end;
}

// Split plan of a forward launch (see FwdParams): when the row groups with
// work give fewer workgroups than one round of the chip (two per compute
// unit) and the heaviest visits at least kSplitMinTiles tiles, each heavy
// row group's visit list is cut into items so that the launch has about one
// round, each item at least 2 tiles; the items' partials then need
// split_slot_floats(d) floats of workspace per item and head group, at most
// `ws_limit` bytes (fewer, longer items otherwise).  When they give more
// than one round but at most two, the heaviest row groups, as many as make
// the rest fit one round, are cut in two halves, if the dispatch estimate
// (launch_length) says the launch gets at least a tenth shorter, merge
// launch included: a second round of whole row groups would otherwise run
// on a few slots while the others wait.
// Returns the workspace bytes the plan uses (0: no split, p unchanged).
int64_t plan_split(const rba_attn* a, const StepPlan& plan, int64_t sq, rba::FwdParams& p, int64_t ws_limit) {
  p.split = 0;
  if (a->dtype != RBA_BF16 || p.n_row_groups > rba::kMaxOrder) return 0;
  if (a->mask == RBA_MASK_DOC_CAUSAL && !plan.dt.cu) return 0;
  const int64_t rows_per_wg = (int64_t)p.rbw * 32;
  std::vector<std::pair<int64_t, int>> tiles(p.n_row_groups);
  int64_t total = 0, n_active = 0;
  for (int rg = 0; rg < p.n_row_groups; ++rg) {
    const int64_t r0 = rg * rows_per_wg;
    tiles[rg] = {visited_tiles(a, plan, r0, std::min(sq, r0 + rows_per_wg)), rg};
    total += tiles[rg].first;
    n_active += tiles[rg].first > 0;
  }
  const int64_t slots = 2 * (int64_t)device_cus();
  const int64_t H = p.n_head_groups;
  if (n_active == 0 || n_active * H > 2 * slots) return 0;
  int64_t max_tiles = 0;
  for (const auto& t : tiles) max_tiles = std::max(max_tiles, t.first);
  if (max_tiles < kSplitMinTiles) return 0;
  std::stable_sort(tiles.begin(), tiles.end(), [](const std::pair<int64_t, int>& x, const std::pair<int64_t, int>& y) {
    return x.first > y.first;
  });
  const int64_t slot_bytes = rba::split_slot_floats(a->d) * 4;
  if (n_active * H >= slots) {
    // a second round: halve the k heaviest so that the rest fit one round
    const int64_t k = (n_active * H - slots + H - 1) / H;
    if (k < 1 || k > n_active || k > rba::kMaxSplitRg) return 0;
    std::vector<int64_t> whole, halved;
    for (int i = 0; i < p.n_row_groups; ++i) whole.push_back(tiles[i].first);
    for (int i = 0; i < k; ++i) {
      halved.push_back((tiles[i].first + 1) / 2);
      halved.push_back((tiles[i].first + 1) / 2);
    }
    for (int i = (int)k; i < p.n_row_groups; ++i) halved.push_back(tiles[i].first);
    if (10 * (launch_length(halved, (int)H, slots) + kMergeTiles) > 9 * launch_length(whole, (int)H, slots))
      return 0;
    const int64_t bytes = 2 * k * H * slot_bytes;
    if (bytes > std::min(ws_limit, kSplitMaxBytes)) return 0;
    for (int i = 0; i < p.n_row_groups; ++i) p.order[i] = (uint16_t)tiles[i].second;
    p.item_start[0] = 0;
    for (int i = 0; i < k; ++i) {
      p.split_len[i] = (uint16_t)((tiles[i].first + 1) / 2);
      p.item_start[i + 1] = (uint16_t)(p.item_start[i] + 2);
    }
    p.split = 1;
    p.n_active = (int32_t)n_active;
    p.n_split_rg = (int32_t)k;
    p.n_items = (int32_t)(2 * k + (n_active - k));
    p.n_wg = (int32_t)(H * (p.n_items + p.n_row_groups - n_active));
    return bytes;
  }
  int64_t L = std::max<int64_t>(2, (total * p.n_head_groups + slots - 1) / slots);
  for (;; L *= 2) {
    int n_split = 0;
    int64_t items = 0;
    while (n_split < n_active && (tiles[n_split].first + L - 1) / L > 1) {
      items += (tiles[n_split].first + L - 1) / L;
      ++n_split;
    }
    if (n_split == 0) return 0;
    const int64_t bytes = items * p.n_head_groups * slot_bytes;
    if (n_split > rba::kMaxSplitRg || items > 60000 || bytes > std::min(ws_limit, kSplitMaxBytes)) continue;
    // the plan
    for (int i = 0; i < p.n_row_groups; ++i) p.order[i] = (uint16_t)tiles[i].second;
    p.item_start[0] = 0;
    for (int i = 0; i < n_split; ++i) {
      const int64_t t = tiles[i].first, n = (t + L - 1) / L;
      p.split_len[i] = (uint16_t)((t + n - 1) / n);   // n items of nearly equal length
      p.item_start[i + 1] = (uint16_t)(p.item_start[i] + n);
    }
    p.split = 1;
    p.n_active = (int32_t)n_active;
    p.n_split_rg = n_split;
    p.n_items = (int32_t)(items + (n_active - n_split));
    p.n_wg = (int32_t)((int64_t)p.n_head_groups * (p.n_items + p.n_row_groups - n_active));
    return bytes;
  }
}

// Workspace of rba_fwd_step_noalloc: the split partials of one forward
// step, in a fixed device array instead of caller memory.  Each device the
// library runs on holds its own copy for the life of the process.  In host
// code `scratch` names a host-side stand-in, never the device array: kernels
// and copies get the per-device address from scratch_address().
constexpr int64_t kScratchBytes = kSplitMaxBytes;
constexpr int kMaxScratchDevices = 64;
static_assert(kScratchBytes % 256 == 0, "scratch size");

}  // namespace

static __device__ __align__(256) float scratch[kScratchBytes / 4];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (the device is current during the lookup) and kept.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RBA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(RBA_ERR_UNSUPPORTED, "device %d: the no-allocation workspace serves devices 0..%d", dev,
                kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(RBA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return RBA_OK;
}

// Shared body of the forward entry points: the partial written to o / lse,
// or merged into the running o / lse (accumulate); with a workspace of
// ws_bytes bytes (or, with use_scratch, the device's `scratch` array) a
// launch with too few workgroups may be split (plan_split).
int fwd_step(const rba_attn* a, const void* q, int64_t sq, const rba_segs* q_segs, const void* k, const void* v,
             int64_t sk, const rba_segs* kv_segs, float* o, float* lse, bool accumulate, void* o_final,
             int32_t final_dtype, void* stream, void* ws = nullptr, int64_t ws_bytes = 0,
             bool use_scratch = false) {
  g_err.clear();
  StepPlan plan;
  int rc = prepare_step(a, sq, q_segs, sk, kv_segs, false, plan);
  if (rc) return rc;
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) ||
      (rc = check_ptr(o, accumulate ? "o_acc" : "o_part")) || (rc = check_ptr(lse, accumulate ? "lse_acc" : "lse_part")))
    return rc;
  if (o_final) {
    if (final_dtype != RBA_BF16 && final_dtype != RBA_F32)
      return fail(RBA_ERR_INVALID, "unknown final dtype %d", final_dtype);
    if ((rc = check_ptr(o_final, "o_final"))) return rc;
    if (o_final == (void*)o) return fail(RBA_ERR_INVALID, "o_final aliases o_acc");
  }
  const bool bf16 = a->dtype == RBA_BF16;
  if (bf16 && sk * a->hkv * a->d * 2 >= ((int64_t)1 << 32))
    return fail(RBA_ERR_UNSUPPORTED, "forward step: k and v must each be smaller than 4 GiB");
  if (plan.empty) return RBA_STEP_EMPTY;
  if ((rc = check_device())) return rc;

  rba::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.accumulate = accumulate ? 1 : 0;
  p.o_final = o_final;
  p.final_bf16 = final_dtype == RBA_BF16;
  if ((rc = fill_query_tiling(a, sq, sk, plan, rba::fwd_rows_per_wave(a->d, bf16), p))) return rc;
  if (use_scratch) {
    if ((rc = scratch_address(&ws))) return rc;
    ws_bytes = kScratchBytes;
  }
  if (ws) {
    if ((rc = check_ptr(ws, "workspace"))) return rc;
    if (ws_bytes < 0) return fail(RBA_ERR_INVALID, "negative workspace size");
    const int64_t need = plan_split(a, plan, sq, p, ws_bytes);
    if (need > ws_bytes)
      return fail(RBA_ERR_INVALID, "forward step: split plan needs %lld workspace bytes, %lld given",
                  (long long)need, (long long)ws_bytes);
    if (need > 0) p.ws = static_cast<float*>(ws);
  }
  // A merging step launches no workgroup for the row groups listed after
  // every one with work: they have no key to merge.
  if (!p.split && (p.n_order || p.order_reverse) && accumulate && !o_final && p.n_active < p.n_row_groups) {
    p.n_rg_launch = p.n_active;
    p.n_wg = p.n_head_groups * p.n_active;
  }
  hipError_t e = bf16 ? rba::launch_fwd_bf16(p, a->d, (hipStream_t)stream) : rba::launch_fwd_f32(p, a->d, (hipStream_t)stream);
  if (e == hipSuccess && p.split) e = rba::launch_split_merge(p, a->d, (hipStream_t)stream);
  return hip_status(e, "forward step");
}

// Workspace bytes a forward step would split into (0: it would not split).
int fwd_workspace_size(const rba_attn* a, int64_t sq, const rba_segs* q_segs, int64_t sk, const rba_segs* kv_segs,
                       int64_t* bytes) {
  if (!bytes) return fail(RBA_ERR_INVALID, "bytes is NULL");
  *bytes = 0;
  StepPlan plan;
  int rc = prepare_step(a, sq, q_segs, sk, kv_segs, false, plan);
  if (rc) return rc;
  if (plan.empty) return RBA_STEP_EMPTY;
  rba::FwdParams p{};
  if ((rc = fill_query_tiling(a, sq, sk, plan, rba::fwd_rows_per_wave(a->d, a->dtype == RBA_BF16), p))) return rc;
  *bytes = plan_split(a, plan, sq, p, kSplitMaxBytes);
  return RBA_OK;
}

}  // namespace

extern "C" {

const char* rba_last_error(void) { return g_err.c_str(); }

const char* rba_version(void) { return "rba 0.1.0 gfx950"; }

int rba_plan_step(const rba_attn* a, int64_t sq, const rba_segs* q_segs, int64_t sk, const rba_segs* kv_segs,
                  int64_t* pairs) {
  g_err.clear();
  if (!pairs) return fail(RBA_ERR_INVALID, "pairs is NULL");
  StepPlan plan;
  int rc = prepare_step(a, sq, q_segs, sk, kv_segs, false, plan);
  if (rc) return rc;
  if (a->mask == RBA_MASK_DOC_CAUSAL && !plan.dt.cu)
    return fail(RBA_ERR_INVALID, "planning a document-masked step needs cu_seqlens_host");
  *pairs = (sq == 0 || sk == 0) ? 0 : count_pairs(a->mask, plan.qs, plan.ks, plan.dt);
  return *pairs == 0 ? RBA_STEP_EMPTY : RBA_OK;
}

int rba_fwd_step(const rba_attn* a, const void* q, int64_t sq, const rba_segs* q_segs, const void* k, const void* v,
                 int64_t sk, const rba_segs* kv_segs, float* o_part, float* lse_part, void* stream) {
  return fwd_step(a, q, sq, q_segs, k, v, sk, kv_segs, o_part, lse_part, false, nullptr, 0, stream);
}

int rba_fwd_step_acc(const rba_attn* a, const void* q, int64_t sq, const rba_segs* q_segs, const void* k,
                     const void* v, int64_t sk, const rba_segs* kv_segs, float* o_acc, float* lse_acc,
                     void* o_final, int32_t final_dtype, void* stream) {
  return fwd_step(a, q, sq, q_segs, k, v, sk, kv_segs, o_acc, lse_acc, true, o_final, final_dtype, stream);
}

int rba_fwd_workspace_size(const rba_attn* a, int64_t sq, const rba_segs* q_segs, int64_t sk,
                           const rba_segs* kv_segs, int64_t* bytes) {
  g_err.clear();
  return fwd_workspace_size(a, sq, q_segs, sk, kv_segs, bytes);
}

int rba_fwd_step_ws(const rba_attn* a, const void* q, int64_t sq, const rba_segs* q_segs, const void* k,
                    const void* v, int64_t sk, const rba_segs* kv_segs, float* o, float* lse, int32_t accumulate,
                    void* o_final, int32_t final_dtype, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!accumulate && o_final) {
    g_err.clear();
    return fail(RBA_ERR_INVALID, "o_final is written only when accumulating");
  }
  return fwd_step(a, q, sq, q_segs, k, v, sk, kv_segs, o, lse, accumulate != 0, o_final, final_dtype, stream,
                  workspace, workspace_bytes);
}

int rba_fwd_step_noalloc(const rba_attn* a, const void* q, int64_t sq, const rba_segs* q_segs, const void* k,
                         const void* v, int64_t sk, const rba_segs* kv_segs, float* o, float* lse,
                         int32_t accumulate, void* o_final, int32_t final_dtype, void* stream) {
  if (!accumulate && o_final) {
    g_err.clear();
    return fail(RBA_ERR_INVALID, "o_final is written only when accumulating");
  }
  return fwd_step(a, q, sq, q_segs, k, v, sk, kv_segs, o, lse, accumulate != 0, o_final, final_dtype, stream,
                  nullptr, 0, true);
}

int rba_merge(int64_t sq, int32_t hq, int32_t d, float* o_acc, float* lse_acc, const float* o_part,
              const float* lse_part, void* o_final, int32_t final_dtype, void* stream) {
  g_err.clear();
  int rc;
  if ((rc = check_rows(sq, "merge"))) return rc;
  if (hq < 1) return fail(RBA_ERR_INVALID, "hq = %d", hq);
  if (d < 4 || d > 1024 || d % 4) return fail(RBA_ERR_UNSUPPORTED, "merge: d = %d (multiple of 4, <= 1024)", d);
  if ((o_part == nullptr) != (lse_part == nullptr))
    return fail(RBA_ERR_INVALID, "o_part and lse_part must both be given or both be NULL");
  if (o_final && final_dtype != RBA_BF16 && final_dtype != RBA_F32)
    return fail(RBA_ERR_INVALID, "unknown final dtype %d", final_dtype);
  if ((rc = check_ptr(o_acc, "o_acc")) || (rc = check_ptr(lse_acc, "lse_acc"))) return rc;
  if (o_part && ((rc = check_ptr(o_part, "o_part")) || (rc = check_ptr(lse_part, "lse_part")))) return rc;
  if (o_final && (rc = check_ptr(o_final, "o_final"))) return rc;
  if (o_part && (const float*)o_acc == o_part) return fail(RBA_ERR_INVALID, "o_acc aliases o_part");
  if (o_final && (o_final == (void*)o_acc || o_final == (const void*)o_part))
    return fail(RBA_ERR_INVALID, "o_final aliases an input");
  if (sq == 0 || (!o_part && !o_final)) return RBA_OK;
  if ((rc = check_device())) return rc;
  rba::MergeParams p{};
  p.o_acc = o_acc; p.lse_acc = lse_acc; p.o_part = o_part; p.lse_part = lse_part;
  p.o_final = o_final; p.final_bf16 = final_dtype == RBA_BF16;
  p.n_pairs = sq * hq; p.sq = (int32_t)sq; p.hq = hq; p.d = d;
  rba::merge_lanes(d, &p.lanes_per_pair, &p.vecs_per_lane);
  return hip_status(rba::launch_merge(p, (hipStream_t)stream), "merge");
}

int rba_merge_layout(int32_t d, int32_t* lanes_per_pair, int32_t* vecs_per_lane, int32_t* threads_per_wg) {
  g_err.clear();
  if (!lanes_per_pair || !vecs_per_lane || !threads_per_wg) return fail(RBA_ERR_INVALID, "output pointer is NULL");
  if (d < 4 || d > 1024 || d % 4) return fail(RBA_ERR_UNSUPPORTED, "merge: d = %d (multiple of 4, <= 1024)", d);
  int lpp = 0, vpl = 0;
  rba::merge_lanes(d, &lpp, &vpl);
  *lanes_per_pair = lpp;
  *vecs_per_lane = vpl;
  *threads_per_wg = rba::kMergeThreads;
  return RBA_OK;
}

int rba_bwd_preprocess(int64_t sq, int32_t hq, int32_t d, int32_t o_dtype, int32_t do_dtype, const void* o,
                       const void* d_o, float* delta, void* stream) {
  g_err.clear();
  int rc;
  if ((rc = check_rows(sq, "preprocess"))) return rc;
  if (hq < 1) return fail(RBA_ERR_INVALID, "hq = %d", hq);
  if (d != 64 && d != 128) return fail(RBA_ERR_UNSUPPORTED, "head dimension %d (supported: 64, 128)", d);
  if (o_dtype != RBA_BF16 && o_dtype != RBA_F32) return fail(RBA_ERR_INVALID, "unknown O dtype %d", o_dtype);
  if (do_dtype != RBA_BF16 && do_dtype != RBA_F32) return fail(RBA_ERR_INVALID, "unknown dO dtype %d", do_dtype);
  if ((rc = check_ptr(o, "o")) || (rc = check_ptr(d_o, "d_o")) || (rc = check_ptr(delta, "delta"))) return rc;
  if (sq == 0) return RBA_OK;
  if ((rc = check_device())) return rc;
  rba::PrepParams p{};
  p.o = o; p.d_o = d_o; p.delta = delta;
  p.n_pairs = sq * hq; p.sq = (int32_t)sq; p.hq = hq; p.d = d;
  p.o_bf16 = o_dtype == RBA_BF16;
  p.do_bf16 = do_dtype == RBA_BF16;
  return hip_status(rba::launch_bwd_preprocess(p, (hipStream_t)stream), "backward preprocess");
}

}  // extern "C"

namespace {

// Query heads a dK / dV workgroup sums over.  Summing several heads of a GQA
// group in one workgroup replaces their atomic adds (and, with the whole
// group, the zero fill) but makes fewer, longer workgroups, so it is used
// only when every key tile sees the same number of query rows (one long
// workgroup cannot be balanced by the heavy-first order) and there are still
// enough workgroups to give every CU two.
int choose_heads_per_wg(const rba_attn* a, const StepPlan& plan, int64_t sk, int bk) {
  const int group = a->hq / a->hkv;
  if (group == 1) return 1;
  if (a->mask == RBA_MASK_DOC_CAUSAL && !plan.dt.cu) return 1;
  const int64_t tiles = (sk + bk - 1) / bk;
  int64_t lo_rows = INT64_MAX, hi_rows = 0;
  for (int64_t t = 0; t < tiles; ++t) {
    const auto pr = host_pos_range(plan.ks, t * bk, std::min<int64_t>((t + 1) * bk, sk));
    int64_t q_lo = INT64_MIN / 4, q_hi = INT64_MAX / 4;
    if (a->mask != RBA_MASK_NONE) q_lo = pr.first;
    if (a->mask == RBA_MASK_DOC_CAUSAL)
      q_hi = (int64_t)*std::upper_bound(plan.dt.cu, plan.dt.cu + plan.dt.n + 1, (int32_t)pr.second) - 1;
    int64_t rows = 0;
    for (const Seg& q : plan.qs) rows += keys_in(q, q_lo, q_hi);
    lo_rows = std::min(lo_rows, rows);
    hi_rows = std::max(hi_rows, rows);
  }
  if (lo_rows != hi_rows) return 1;
  const int64_t slots = 2 * (int64_t)device_cus();
  int best = 1;
  for (int hpw = 2; hpw <= group; ++hpw)
    if (group % hpw == 0 && tiles * a->hq / hpw >= slots) best = hpw;
  return best;
}

// Key-stationary counterpart of all_tiles_full for the dK / dV pass: is every
// (32-key wave, 32-row query block) pair that a workgroup of `bk` keys
// visits full?  A workgroup whose keys have positions in [klo, khi] visits,
// in each query segment, the blocks of the rows at positions from klo on
// (causal); they are all full when the first such row starts a block (or
// the segment) and lies at or after khi.  Query blocks and key waves must be
// whole (no ragged block or wave) and lie in one segment.  The document mask
// is never taken as full.
bool all_blocks_full(const rba_attn* a, const StepPlan& plan, int64_t sq, int64_t sk, int64_t bk) {
  constexpr int64_t BQ = 32, WK = 32;
  if (a->mask == RBA_MASK_DOC_CAUSAL || sq % BQ || sk % WK) return false;
  for (const Seg& k : plan.ks)
    if (k.row0 % WK || k.len % WK) return false;
  if (a->mask == RBA_MASK_NONE) return true;
  for (const Seg& q : plan.qs)
    if (q.row0 % BQ || q.len % BQ) return false;
  for (int64_t r0 = 0; r0 < sk; r0 += bk) {
    const auto kr = host_pos_range(plan.ks, r0, std::min(sk, r0 + bk));
    for (const Seg& q : plan.qs) {
      // first visited row: the first position >= klo
      const int64_t a0 = kr.first <= q.start ? 0 : (kr.first - q.start + q.stride - 1) / q.stride;
      if (a0 >= q.len) continue;
      if (a0 % BQ) return false;
      if (q.start + a0 * q.stride < kr.second) return false;
    }
  }
  return true;
}

// Shared body of rba_bwd_step (dK / dV overwritten) and rba_bwd_step_acc
// (dK / dV added into accumulators).
int bwd_step(const rba_attn* a, const void* q, int64_t sq, const rba_segs* q_segs, const void* k, const void* v,
             int64_t sk, const rba_segs* kv_segs, const void* d_o, const float* lse, const float* delta,
             float* dq_acc, float* dk, float* dv, bool accumulate, void* stream) {
  g_err.clear();
  StepPlan plan;
  int rc = prepare_step(a, sq, q_segs, sk, kv_segs, true, plan);
  if (rc) return rc;
  if ((rc = check_ptr(q, "q")) || (rc = check_ptr(k, "k")) || (rc = check_ptr(v, "v")) ||
      (rc = check_ptr(d_o, "d_o")) || (rc = check_ptr(lse, "lse")) || (rc = check_ptr(delta, "delta")) ||
      (rc = check_ptr(dq_acc, "dq_acc")) || (rc = check_ptr(dk, accumulate ? "dk_acc" : "dk_step")) ||
      (rc = check_ptr(dv, accumulate ? "dv_acc" : "dv_step")))
    return rc;
  if ((int64_t)sq * a->hq * a->d * 2 >= ((int64_t)1 << 32))
    return fail(RBA_ERR_UNSUPPORTED, "backward step: q and d_o must each be smaller than 4 GiB");
  if (sk * a->hkv * a->d * 2 >= ((int64_t)1 << 32))
    return fail(RBA_ERR_UNSUPPORTED, "backward step: k and v must each be smaller than 4 GiB");
  if (plan.empty) return RBA_STEP_EMPTY;
  if ((rc = check_device())) return rc;
  rba::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.d_o = d_o; p.lse = lse; p.delta = delta;
  p.dk = dk; p.dv = dv;
  p.accumulate = accumulate ? 1 : 0;
  p.sq = (int32_t)sq; p.sk = (int32_t)sk; p.hq = a->hq; p.hkv = a->hkv; p.group = a->hq / a->hkv;
  p.scale = a->scale;
  p.scale_log2 = a->scale * 1.4426950408889634f;
  p.mask = a->mask;
  p.cu = a->mask == RBA_MASK_DOC_CAUSAL ? a->cu_seqlens_dev : nullptr;
  p.n_docs = a->mask == RBA_MASK_DOC_CAUSAL ? a->n_docs : 0;
  p.qs = to_table(plan.qs);
  p.ks = to_table(plan.ks);
  const int bk = rba::bwd_keys_per_wg(a->d);
  p.n_key_tiles = (int32_t)((sk + bk - 1) / bk);
  p.heads_per_wg = choose_heads_per_wg(a, plan, sk, bk);
  const int64_t n_wg = (int64_t)p.n_key_tiles * a->hq / p.heads_per_wg;
  if (n_wg > INT32_MAX) return fail(RBA_ERR_UNSUPPORTED, "too many workgroups");
  p.n_wg = (int32_t)n_wg;
  p.all_full = all_blocks_full(a, plan, sq, sk, bk) ? 1 : 0;
  rba::DqParams dp{};
  dp.f.q = q; dp.f.k = k; dp.f.v = v;
  if ((rc = fill_query_tiling(a, sq, sk, plan, 32, dp.f))) return rc;
  dp.d_o = d_o; dp.lse = lse; dp.delta = delta; dp.dq = dq_acc; dp.scale = a->scale;
  if ((int64_t)p.n_wg + dp.f.n_wg > INT32_MAX) return fail(RBA_ERR_UNSUPPORTED, "too many workgroups");
  // every check is done: launches from here on
  if (p.heads_per_wg < p.group && !accumulate) {
    // the group's workgroups add their partial dK / dV into zeroed outputs
    hipError_t e = rba::launch_zero_f32(dk, dv, sk * a->hkv * a->d, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "backward zero fill");
  }
  return hip_status(rba::launch_bwd(p, dp, a->d, (hipStream_t)stream), "backward step");
}

}  // namespace

extern "C" {

int rba_step_full_tiles(const rba_attn* a, int64_t sq, const rba_segs* q_segs, int64_t sk, const rba_segs* kv_segs,
                        int32_t* fwd_full, int32_t* bwd_full) {
  g_err.clear();
  if (!fwd_full || !bwd_full) return fail(RBA_ERR_INVALID, "fwd_full / bwd_full is NULL");
  StepPlan plan;
  int rc = prepare_step(a, sq, q_segs, sk, kv_segs, false, plan);
  if (rc) return rc;
  // the row groups of the forward and dQ launches (fill_query_tiling) and
  // the key tiles of the dK/dV launch (bwd_step)
  const int group = a->hq / a->hkv;
  const int64_t fwd_rows = query_rows_per_wg(group, rba::fwd_rows_per_wave(a->d, 1));
  const int64_t dq_rows = query_rows_per_wg(group, 32);
  // only the bf16 kernels have mask-free instantiations (the backward is bf16 only)
  const bool bf16 = a->dtype == RBA_BF16;
  *fwd_full = (bf16 && all_tiles_full(a, plan, sq, sk, fwd_rows)) ? 1 : 0;
  *bwd_full = (bf16 && all_tiles_full(a, plan, sq, sk, dq_rows) &&
               all_blocks_full(a, plan, sq, sk, rba::bwd_keys_per_wg(a->d)))
                  ? 1 : 0;
  return RBA_OK;
}

int rba_bwd_step(const rba_attn* a, const void* q, int64_t sq, const rba_segs* q_segs, const void* k, const void* v,
                 int64_t sk, const rba_segs* kv_segs, const void* d_o, const float* lse, const float* delta,
                 float* dq_acc, float* dk_step, float* dv_step, void* stream) {
  return bwd_step(a, q, sq, q_segs, k, v, sk, kv_segs, d_o, lse, delta, dq_acc, dk_step, dv_step, false, stream);
}

int rba_bwd_step_acc(const rba_attn* a, const void* q, int64_t sq, const rba_segs* q_segs, const void* k,
                     const void* v, int64_t sk, const rba_segs* kv_segs, const void* d_o, const float* lse,
                     const float* delta, float* dq_acc, float* dk_acc, float* dv_acc, void* stream) {
  return bwd_step(a, q, sq, q_segs, k, v, sk, kv_segs, d_o, lse, delta, dq_acc, dk_acc, dv_acc, true, stream);
}

}  // extern "C"
