/*
 * rba.h — ring block attention on MI355X (gfx950): the per-device step of
 * Ring Attention and TASP, as a C ABI.
 *
 * What a ring step computes (TASP: Topology-aware Sequence Parallelism,
 * abstract: each query chunk stays on its accelerator and must attend to every
 * KV chunk, which arrive one per ring iteration; Zigzag-Ring Attention, named
 * in its experiment highlights, is the causal load-balanced split):
 *
 *   For one query chunk Q and one KV chunk (K, V), exact softmax attention of
 *   every query row against the keys of that chunk that its mask allows, as a
 *   partial result (O_part, LSE_part).  Merging the partials of all KV chunks
 *   with log-sum-exp weights gives exact attention over the whole sequence
 *   (blockwise exact attention: FlashAttention and "Self-attention Does Not
 *   Need O(n^2) Memory", both in the TASP citation map).
 *
 *   allowed(i, j):  NONE        always
 *                   CAUSAL      pos(k_j) <= pos(q_i)
 *                   DOC_CAUSAL  CAUSAL and both positions in the same packed
 *                               document (HSAP: A Hierarchical Sequence-aware
 *                               Parallelism for Hybrid-Context Generative
 *                               Models, abstract and methodology: causal
 *                               attention on packed sequences without
 *                               attention across documents)
 *   s_ij   = scale * <q_i, k_j>
 *   LSE_i  = ln sum_{allowed j} exp(s_ij)         (-inf: row has no key here)
 *   O_i    = sum_{allowed j} exp(s_ij - LSE_i) v_j (0: row has no key here)
 *
 * Conventions shared by every entry point
 *   - Tensors are tokens-major and contiguous: Q, dO [sq, hq, d];
 *     K, V [sk, hkv, d]; O / dQ [sq, hq, d]; dK, dV [sk, hkv, d];
 *     LSE and delta [hq, sq].  Element (t, h, c) sits at (t*H + h)*d + c.
 *   - Query head h reads KV head h / (hq / hkv) (contiguous GQA groups; GQA is
 *     named in the TASP citation map).
 *   - Every tensor pointer is a DEVICE pointer of the current HIP device and
 *     must be 16-byte aligned.  Struct pointers (rba_attn, rba_segs) and
 *     cu_seqlens_host are HOST pointers, read only during the call.
 *   - The caller owns every buffer.  The library allocates no device memory,
 *     keeps no pointer after it returns and launches on `stream` (a
 *     hipStream_t; NULL = the legacy default stream).  Launches are
 *     asynchronous: buffers must stay alive until the stream's work is done.
 *   - All arguments are validated before anything is launched.  On any
 *     negative status nothing was launched and no output was touched; the
 *     reason is in rba_last_error().
 *   - The library keeps no state between calls apart from a thread-local
 *     error string, per-device caches of the device's architecture and
 *     compute-unit count, and the per-device workspace array of
 *     rba_fwd_step_noalloc.  It is safe to call from several threads on
 *     different streams, except rba_fwd_step_noalloc calls that overlap on
 *     one device (see there).
 */
#ifndef RBA_H
#define RBA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RBA_OK = 0,
  RBA_STEP_EMPTY = 1,          /* not an error: no (query, key) pair of this step is
                                  allowed; nothing was launched, outputs untouched */
  RBA_ERR_INVALID = -1,        /* bad argument (null pointer, shape, segments, ...) */
  RBA_ERR_UNSUPPORTED = -2,    /* valid but not implemented (d, dtype, sizes) */
  RBA_ERR_ALIGNMENT = -3,      /* a tensor pointer is not 16-byte aligned */
  RBA_ERR_HIP = -4             /* the HIP runtime reported an error at launch */
} rba_status;

typedef enum { RBA_BF16 = 0, RBA_F32 = 1 } rba_dtype;

typedef enum { RBA_MASK_NONE = 0, RBA_MASK_CAUSAL = 1, RBA_MASK_DOC_CAUSAL = 2 } rba_mask;

#define RBA_MAX_SEGS 16

/*
 * Chunk offsets: where a chunk's rows sit in the global sequence.  Row r of
 * the chunk has global position start[s] + (r - row0(s)) * stride[s] where s
 * is the segment holding row r and row0(s) = len[0] + ... + len[s-1].  A
 * contiguous split uses one segment, the zigzag split two (pieces r and
 * 2n-1-r), a TASP step whose KV arrives in slices from several source ranks
 * up to 14, and the striped split (Striped Attention, in the TASP citation
 * map: token i on rank i mod n) one segment of stride n.
 * Requirements: 1 <= n <= RBA_MAX_SEGS, len[s] >= 1, sum(len) equals the
 * chunk's row count, start[s] >= 0, stride[s] >= 0 (0 is read as 1, so a
 * zero-initialised struct describes unit-stride runs), the last position
 * start[s] + (len[s] - 1) * stride[s] <= 2^31 - 1, and the segments of one
 * chunk share no position.
 */
typedef struct {
  int32_t n;
  int64_t start[RBA_MAX_SEGS];
  int64_t len[RBA_MAX_SEGS];
  int64_t stride[RBA_MAX_SEGS];
} rba_segs;

/* Attention parameters shared by a step's forward and backward. */
typedef struct {
  int32_t hq;                      /* query heads, >= 1 */
  int32_t hkv;                     /* KV heads, >= 1, divides hq */
  int32_t d;                       /* head dimension: 64 or 128 */
  float scale;                     /* softmax scale, finite and > 0 (usually 1/sqrt(d)) */
  rba_dtype dtype;                 /* Q/K/V/dO element type */
  rba_mask mask;
  const int32_t* cu_seqlens_dev;   /* DOC_CAUSAL only: device int32[n_docs+1], ascending,
                                      cu[0] = 0, global positions; document t is
                                      [cu[t], cu[t+1]).  Every position of both chunks
                                      must lie in [0, cu[n_docs]). */
  const int32_t* cu_seqlens_host;  /* DOC_CAUSAL only, optional: the same table in host
                                      memory.  When given, it is validated and used to
                                      detect empty steps without a launch. */
  int32_t n_docs;                  /* DOC_CAUSAL only: number of documents, >= 1 */
} rba_attn;

/*
 * rba_fwd_step — one ring step of the forward pass.
 *   q [sq, hq, d] (dtype), k and v [sk, hkv, d] (dtype); q_segs / kv_segs give
 *   the chunks' global positions.  Writes o_part [sq, hq, d] fp32 and
 *   lse_part [hq, sq] fp32 (natural log of the sum of exp of the scaled
 *   scores).  Rows with no allowed key get O = 0 and LSE = -inf.
 * Returns RBA_OK, RBA_STEP_EMPTY (host-side proof that no pair is allowed:
 * nothing launched, outputs untouched — the caller skips the merge), or an
 * error.  sq = 0 or sk = 0 is RBA_STEP_EMPTY.
 * dtype RBA_BF16 and RBA_F32 both support d in {64, 128}.
 */
int rba_fwd_step(const rba_attn* a,
                 const void* q, int64_t sq, const rba_segs* q_segs,
                 const void* k, const void* v, int64_t sk, const rba_segs* kv_segs,
                 float* o_part, float* lse_part, void* stream);

/*
 * rba_fwd_step_acc — rba_fwd_step whose partial is merged, in the same
 * launch, into a running result: with the step's partial (O_s, LSE_s),
 *   L = ln(e^{lse_acc} + e^{LSE_s}),
 *   o_acc = e^{lse_acc - L} o_acc + e^{LSE_s - L} O_s,   lse_acc = L
 * (the merge of rba_merge, the same arithmetic), and when o_final is
 * non-NULL the merged O is also written to it in final_dtype (RBA_BF16 or
 * RBA_F32) — the last step of a replay.  o_acc [sq, hq, d] and lse_acc
 * [hq, sq] fp32 are in/out and must already hold a result (the first step
 * of a ring goes through rba_fwd_step).  This saves the partial's round
 * trip through HBM and the merge launch.  A row to which the step shows no
 * key (LSE_s = -inf) merges as the identity: its o_acc and lse_acc are
 * neither read nor written, so a row empty on both sides keeps whatever
 * o_acc holds.  Same inputs, limits and errors as
 * rba_fwd_step; o_final must not alias o_acc.  On RBA_STEP_EMPTY nothing is
 * launched: o_acc / lse_acc are unchanged and o_final is NOT written (finish
 * with rba_merge and no partial).
 */
int rba_fwd_step_acc(const rba_attn* a,
                     const void* q, int64_t sq, const rba_segs* q_segs,
                     const void* k, const void* v, int64_t sk, const rba_segs* kv_segs,
                     float* o_acc, float* lse_acc, void* o_final, int32_t final_dtype, void* stream);

/*
 * rba_fwd_step_ws — rba_fwd_step (accumulate = 0: o, lse are the partial
 * o_part, lse_part) or rba_fwd_step_acc (accumulate = 1: o, lse are the
 * running o_acc, lse_acc, and o_final may be given) with a caller-provided
 * workspace, which lets a step whose rows with work are too few to fill the
 * GPU spread each row group's keys over several workgroups.  Defining
 * passages: the forward step above, and HSAP's sequence-aware scheduling of
 * irregular attention patterns (HSAP page, "Technical Contribution" and
 * "Methodology": device-specific work schedules for packed sequences, read
 * here at the level of one GPU's workgroups).
 *   Same arithmetic as the unsplit step: every row's keys are covered once;
 *   a split row group's items each produce a partial (O, LSE) over a run of
 *   its key tiles, and a second launch on `stream` merges them with the
 *   LSE-weighted merge of rba_merge before the result is written or merged
 *   into the running output.  Results equal the unsplit step's up to the
 *   rounding of the extra merges.
 *   workspace: device memory, 16-byte aligned, owned by the caller, at least
 *   workspace_bytes bytes; NULL (or too small for any split) = never split.
 *   Its contents on entry do not matter and are overwritten; it must not be
 *   shared with another call in flight.  rba_fwd_workspace_size gives the
 *   bytes a step would use (at most 32 MiB).
 * Same inputs, limits, errors and RBA_STEP_EMPTY behaviour as rba_fwd_step /
 * rba_fwd_step_acc; accumulate = 0 with a non-NULL o_final is
 * RBA_ERR_INVALID.  fp32 steps never split.
 */
int rba_fwd_step_ws(const rba_attn* a,
                    const void* q, int64_t sq, const rba_segs* q_segs,
                    const void* k, const void* v, int64_t sk, const rba_segs* kv_segs,
                    float* o, float* lse, int32_t accumulate, void* o_final, int32_t final_dtype,
                    void* workspace, int64_t workspace_bytes, void* stream);

/*
 * rba_fwd_step_noalloc — rba_fwd_step_ws with the workspace in a fixed
 * device array of the library instead of caller memory.  For callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the call allocates and
 * frees nothing, and calls no allocating library routine.
 *   The array is 32 MiB (the most any split plan of rba_fwd_step_ws uses;
 *   a launch that would need more takes fewer, longer items or runs
 *   unsplit, and a plan over 32 MiB would be refused with RBA_ERR_INVALID).
 *   Each device holds its own copy from the first call on it until the
 *   process ends; the first call on a device, with that device current,
 *   looks up the copy's address (hipGetSymbolAddress) and keeps it.
 *   Every call on one device shares that device's array and leaves the last
 *   split's partials in it; no part of it needs to start at zero (a split's
 *   merge reads only slots its own first launch wrote).  Calls that overlap
 *   on one device (other streams, other threads) race on the array and must
 *   be serialised by the caller.
 * Arguments, results, limits, errors and RBA_STEP_EMPTY behaviour as
 * rba_fwd_step_ws with workspace = the array; results are bit for bit those
 * of rba_fwd_step_ws given a 32 MiB workspace.  Devices 64 and above are
 * RBA_ERR_UNSUPPORTED.
 */
int rba_fwd_step_noalloc(const rba_attn* a,
                         const void* q, int64_t sq, const rba_segs* q_segs,
                         const void* k, const void* v, int64_t sk, const rba_segs* kv_segs,
                         float* o, float* lse, int32_t accumulate, void* o_final, int32_t final_dtype,
                         void* stream);

/*
 * rba_fwd_workspace_size — host-side query (reads the current device's
 * compute-unit count, launches nothing): *bytes = the workspace
 * rba_fwd_step_ws would use for this step (0 when it would not split), at
 * most 32 MiB.  Returns RBA_OK, RBA_STEP_EMPTY (*bytes = 0) or an argument
 * error as rba_fwd_step.  Document-masked steps split only with
 * cu_seqlens_host.
 */
int rba_fwd_workspace_size(const rba_attn* a, int64_t sq, const rba_segs* q_segs,
                           int64_t sk, const rba_segs* kv_segs, int64_t* bytes);

/*
 * rba_merge — LSE-weighted merge of a step's partial into the running result.
 * Defining passage: the blockwise exact attention the TASP page builds on
 * (FlashAttention and "Self-attention Does Not Need O(n^2) Memory", both in
 * the "Builds on" list of its citation map): softmax attention over a union
 * of disjoint key sets equals the partial results over each set combined
 * with weights exp(LSE_part - LSE_total); with two sets,
 *   L = ln(e^{lse_acc} + e^{lse_part}),
 *   o_acc = e^{lse_acc - L} o_acc + e^{lse_part - L} o_part,  lse_acc = L.
 *   A side with LSE = -inf has weight 0; both -inf gives (0, -inf).
 *   o_acc, o_part [sq, hq, d] fp32; lse_acc, lse_part [hq, sq] fp32.
 *   o_part and lse_part may both be NULL: then the accumulator is left as it is
 *   and only o_final is written (finalising a result that needed no merge).
 *   o_final (nullable): also write the merged O as final_dtype (RBA_BF16 rounds
 *   to nearest even, RBA_F32 copies) into o_final [sq, hq, d].
 *   o_acc may not alias o_part; o_final may not alias either.
 * d must be a multiple of 4 in [4, 1024], else RBA_ERR_UNSUPPORTED.  Every
 * (row, head) pair is merged by threads of a single wave (rba_merge_layout),
 * so the in-place update of lse_acc never races with a read of it.
 */
int rba_merge(int64_t sq, int32_t hq, int32_t d,
              float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
              void* o_final, int32_t final_dtype, void* stream);

/*
 * rba_merge_layout — host-only (no device access): the thread map rba_merge
 * launches for head dimension d.  A workgroup has *threads_per_wg threads;
 * thread t works on (row, head) pair slot t / *lanes_per_pair of the
 * workgroup's sweep and on the 16-byte vectors (t % lpp) + i * lpp,
 * i < *vecs_per_lane, of that pair (lpp = *lanes_per_pair, a power of two
 * dividing 64, so one pair's threads are lanes of one 64-lane wave).
 * Returns RBA_OK, or RBA_ERR_UNSUPPORTED for a d that rba_merge rejects.
 */
int rba_merge_layout(int32_t d, int32_t* lanes_per_pair, int32_t* vecs_per_lane, int32_t* threads_per_wg);

/*
 * rba_bwd_preprocess — delta[h, i] = sum_c dO[i, h, c] * O[i, h, c], fp32.
 * Defining passage: the backward of the attention definition above; the
 * pages' workload is training (HSAP page, "Methodology" and "Key Results":
 * training throughput on packed long sequences), whose backward pass needs,
 * per query row, this inner product of the output and its gradient.
 *   o [sq, hq, d] in o_dtype (the forward's merged output: the fp32
 *   accumulator gives delta without the output's bf16 rounding), d_o
 *   [sq, hq, d] in do_dtype (its upstream gradient); delta [hq, sq] fp32.
 *   Run once per backward pass.
 */
int rba_bwd_preprocess(int64_t sq, int32_t hq, int32_t d, int32_t o_dtype, int32_t do_dtype,
                       const void* o, const void* d_o, float* delta, void* stream);

/*
 * rba_bwd_step — one ring step of the backward pass (the gradient of
 * L = sum dO * O through this step's keys).  Defining passage: the
 * derivative of the attention definition at the top of this header, taken
 * step by step over the ring as in the forward (TASP abstract: each query
 * chunk meets every KV chunk); training is the pages' workload (HSAP page,
 * "Methodology" and "Key Results").  With P_ij = exp(s_ij - lse_i)
 * for allowed pairs (lse = the FINAL merged LSE of the forward) and
 * dS_ij = P_ij (<dO_i, v_j> - delta_i):
 *   dq_acc[i] += scale * sum_j dS_ij k_j            (accumulated, in/out)
 *   dk_step[j]  = scale * sum_{i, h in group} dS_ij q_i   (overwritten)
 *   dv_step[j]  = sum_{i, h in group} P_ij dO_i           (overwritten)
 *   q, d_o [sq, hq, d] (dtype); k, v [sk, hkv, d] (dtype); lse, delta
 *   [hq, sq] fp32; dq_acc [sq, hq, d] fp32; dk_step, dv_step [sk, hkv, d] fp32.
 * On RBA_STEP_EMPTY nothing is launched: dq_acc is unchanged and dk_step /
 * dv_step are NOT written (the step's true dK/dV are zero).  One kernel runs
 * on `stream` (after a zero fill of dk_step / dv_step when needed), holding
 * a key-stationary pass for dk_step / dv_step and a query-stationary pass
 * that adds each dq_acc row once (deterministic).  With more than one query
 * head per KV head, a dK / dV workgroup sums one or several heads of the
 * group in registers; when it does not sum the whole group, the group's
 * parts are added with fp32 atomics into the zero-filled outputs, so their
 * low bits depend on scheduling.
 * dtype RBA_BF16 only, d in {64, 128}; q, d_o, k and v must each be smaller
 * than 4 GiB, else RBA_ERR_UNSUPPORTED.
 */
int rba_bwd_step(const rba_attn* a,
                 const void* q, int64_t sq, const rba_segs* q_segs,
                 const void* k, const void* v, int64_t sk, const rba_segs* kv_segs,
                 const void* d_o, const float* lse, const float* delta,
                 float* dq_acc, float* dk_step, float* dv_step, void* stream);

/*
 * rba_bwd_step_acc — rba_bwd_step with the KV side accumulated: the step's
 * dK / dV are ADDED into dk_acc / dv_acc [sk, hkv, d] fp32 (in/out) instead
 * of overwriting per-step outputs.  In a ring, these are the gradient
 * accumulators that travel with a KV chunk back to its owner (every rank
 * whose queries meet the chunk adds its part, as the backward of the
 * attention definition sums dK_j, dV_j over all queries; TASP abstract,
 * training in HSAP methodology).  No zero fill is launched.  Same arguments,
 * layouts, limits and errors as rba_bwd_step; on RBA_STEP_EMPTY nothing is
 * launched and the accumulators are unchanged.  When a dK / dV workgroup
 * sums every query head of its group (one head per KV head, or the host's
 * choice for steps where every key tile sees the same query rows), each
 * element is read, added and written once; otherwise the additions are fp32
 * atomics (low bits depend on scheduling).
 */
int rba_bwd_step_acc(const rba_attn* a,
                     const void* q, int64_t sq, const rba_segs* q_segs,
                     const void* k, const void* v, int64_t sk, const rba_segs* kv_segs,
                     const void* d_o, const float* lse, const float* delta,
                     float* dq_acc, float* dk_acc, float* dv_acc, void* stream);

/*
 * rba_plan_step — host-only planning of a step (no device access).
 * Writes into *pairs the exact number of allowed (query row, key) pairs of
 * the step per query head (the effective work: forward 4*d flops per pair
 * and head, backward 10*d).  For DOC_CAUSAL it needs cu_seqlens_host.
 * Returns RBA_OK, RBA_STEP_EMPTY (pairs = 0) or an error.
 */
int rba_plan_step(const rba_attn* a, int64_t sq, const rba_segs* q_segs,
                  int64_t sk, const rba_segs* kv_segs, int64_t* pairs);

/*
 * rba_step_full_tiles — host-only (no device access): whether the step's
 * launches take the kernels compiled without tile classification and mask
 * code.  *fwd_full = 1 when every key tile that a forward workgroup visits
 * holds only pairs the mask allows for every row of that workgroup;
 * *bwd_full = 1 when the same holds for the dQ pass and, for the dK/dV pass,
 * every query block a workgroup of keys visits is allowed for all of its
 * keys.  These are launch choices of this library (the results are the same
 * either way); the call exists so that the decision can be checked against
 * an enumeration of the visited tiles.  The document mask and fp32 steps
 * (whose kernels always classify tiles) give 0.
 * Returns RBA_OK, or an error for invalid arguments (as rba_plan_step).
 */
int rba_step_full_tiles(const rba_attn* a, int64_t sq, const rba_segs* q_segs,
                        int64_t sk, const rba_segs* kv_segs, int32_t* fwd_full, int32_t* bwd_full);

/* Thread-local description of the last error on this thread ("" if none).
 * Valid until the next rba_* call on the same thread. */
const char* rba_last_error(void);

/* Library version string, e.g. "rba 0.1.0 gfx950". */
const char* rba_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RBA_H */
