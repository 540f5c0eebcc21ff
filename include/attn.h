/*
 * attn.h - exact attention forward, flash-decoding and backward for AMD MI355X (gfx950): the C ABI.
 *
 * What is computed
 *   For every batch entry b, head h and query row i:
 *     S_ij  = softmax_scale * sum_c Q[b,i,h,c] * K[b,j,h,c]     (j visible to i)
 *     O[b,i,h,:] = sum_j softmax_j(S_i.) * V[b,j,h,:]
 *     LSE[b,h,i] = ln sum_j exp(S_ij)                            (natural log, fp32)
 *   This is the standard attention of "LLM Lab Notes 07: Why FlashAttention Is
 *   Fast" (section 2), evaluated tile by tile with the online-softmax rescale of
 *   section 3.3 so that S never reaches device memory (sections 3.1 and 3.2).
 *   The result equals the plain definition up to floating-point rounding.
 *
 * Readings fixed by this library where the pages are silent
 *   - causal != 0 masks with bottom-right alignment: query i sees key j iff
 *     j <= i + (s_k - s_q).  With s_q == s_k this is the lower triangle; a
 *     one-row decode query sees the whole cache.
 *   - a query row that sees no key gets O = 0 and LSE = -inf.
 *   - O is rounded to the input dtype (round to nearest even); LSE is fp32.
 *   - softmax_scale is explicit (the pages use 1/sqrt(d)); any finite value,
 *     zero and negative values included, is accepted.
 *
 * Layout
 *   Q is (b, s_q, h, d); K, V are (b, s_k, h_kv, d); O is (b, s_q, h, d): the
 *   (batch, seq, heads, dim) order that flash_attn_func consumes in Lab Notes 07
 *   section 2.  h_kv == h (or 0) is plain multi-head attention; a smaller h_kv
 *   lets groups of h / h_kv consecutive query heads share one K/V head, the
 *   several "q heads" over one K tile asked about in issue #1248.  The d dimension is contiguous (stride 1).  The other three
 *   dimensions take arbitrary non-negative element strides (b, s, h order), each
 *   a multiple of 8 elements, so flattened (b, s, h*d) tensors and views are
 *   accepted without copies.  Base pointers must be 16-byte aligned.  LSE is a
 *   dense fp32 array (b, h, s_q).
 *
 * Flash-decoding (flash-attention issue #1248, "where is flash decoding second
 * stage (reduce) code?")
 *   attn_fwd_splitkv cuts the keys into num_splits contiguous ranges, split i
 *   covering keys [floor(i*s_k/n), floor((i+1)*s_k/n)), and writes for every
 *   split the partial output O_i (normalised within the split, fp32) and LSE_i.
 *   attn_combine reduces them as the issue's reply describes:
 *     LSE = log sum_i exp(LSE_i),  O = sum_i exp(LSE_i - LSE) * O_i,
 *   with max_i LSE_i subtracted before exponentiating.  attn_num_splits picks
 *   the split count from the device's compute-unit count: it splits only when
 *   b*h*(query row blocks) leaves compute units idle, as the same reply
 *   explains for the library's own heuristic.
 *
 * Ownership and threading
 *   The caller allocates every buffer (device memory) and keeps it alive until
 *   the work enqueued on `stream` has finished.  The library allocates nothing,
 *   keeps no pointer after a call returns, and enqueues kernels asynchronously
 *   on `stream` (a hipStream_t; NULL means the default stream).  Calls are
 *   thread-safe: the only state is a per-device cache of the compute-unit count
 *   and architecture, filled once (and the static buffer of attn_bwd_noalloc,
 *   described there, for callers that cannot allocate).  Buffers a call writes (O, LSE, partials,
 *   dQ, dK, dV, delta) must not overlap one another or any buffer the call
 *   reads; this is not checked, and overlapping buffers give undefined results.
 *
 * Errors
 *   Every argument is checked on the host before anything is launched.  On any
 *   error nothing is launched and no output is written; the status says why.
 *   Checks run in this order: NULL pointers, dtype, shape, head dim, layout,
 *   scale, split count, then the device.  A failed launch returns
 *   ATTN_E_LAUNCH.  Faults inside a kernel surface at the caller's next
 *   synchronisation, as for any asynchronous GPU work.
 */
#ifndef EXACT_ATTN_H
#define EXACT_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_E_NULL = -1,    /* a required pointer (or the args struct) is NULL */
  ATTN_E_DTYPE = -2,   /* dtype is not ATTN_FP16 / ATTN_BF16 */
  ATTN_E_SHAPE = -3,   /* b, h, s_q or s_k < 1, a size beyond the limits below, or
                          h_kv < 0, h_kv > h, or h not a multiple of h_kv */
  ATTN_E_HEADDIM = -4, /* d not in {16, 32, 64, 128}; inputs are never padded */
  ATTN_E_LAYOUT = -5,  /* misaligned pointer, negative stride, or a stride that is
                          not a multiple of 8 elements */
  ATTN_E_SCALE = -6,   /* softmax_scale is NaN or infinite */
  ATTN_E_SPLITS = -7,  /* num_splits outside [1, min(s_k, ATTN_MAX_SPLITS)] */
  ATTN_E_DEVICE = -8,  /* no HIP device, or the current device is not gfx950 */
  ATTN_E_LAUNCH = -9,  /* the kernel launch itself failed */
  ATTN_E_SCRATCH = -10 /* attn_bwd_noalloc: b*h*s_q exceeds ATTN_BWD_SCRATCH_ROWS */
} attn_status;

typedef enum { ATTN_FP16 = 0, ATTN_BF16 = 1 } attn_dtype;

#define ATTN_MAX_SPLITS 256
/* Size limits: b*h <= 2^24, s_q and s_k <= 2^24. */
#define ATTN_MAX_BH (1 << 24)
#define ATTN_MAX_SEQ (1 << 24)

typedef struct {
  int32_t dtype;        /* attn_dtype of Q, K, V and O */
  int32_t causal;       /* 0: every key visible; 1: bottom-right causal mask */
  int64_t b, s_q, s_k, h, d;
  const void *q;        /* device pointer, (b, s_q, h, d) */
  const void *k;        /* device pointer, (b, s_k, h, d) */
  const void *v;        /* device pointer, (b, s_k, h, d) */
  void *o;              /* device pointer, (b, s_q, h, d), written */
  float *lse;           /* device pointer, dense (b, h, s_q) fp32, written;
                           may be NULL in attn_fwd to skip it; unused by
                           attn_fwd_splitkv */
  int64_t q_stride[3];  /* element strides of Q for (b, s, h) */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];  /* unused by attn_fwd_splitkv */
  float softmax_scale;
  int64_t h_kv;         /* K/V heads: 0 means h; else h must be a multiple of h_kv
                           and query head hh reads K/V head hh / (h / h_kv) */
} attn_args;

/* Fused forward (Lab Notes 07 sections 3.1-3.3): O and LSE in one kernel. */
attn_status attn_fwd(const attn_args *args, void *stream);

/* Split count for flash-decoding on `device` (issue #1248): 1 when the
 * work-groups of one split already cover the compute units, otherwise enough
 * splits to give each compute unit about one work-group, capped by
 * ceil(s_k/64) and ATTN_MAX_SPLITS.  Work-groups per split: ceil(b*h/4) for a
 * single query row (four heads per work-group), else
 * b*h*ceil(s_q/rows_per_block) with the prefill kernel's row block.  Writes the
 * count to *n_out. */
attn_status attn_num_splits(int64_t b, int64_t h, int64_t s_q, int64_t s_k, int64_t d,
                            int device, int32_t *n_out);

/* The same heuristic for an explicit compute-unit count; touches no device. */
attn_status attn_num_splits_for(int64_t b, int64_t h, int64_t s_q, int64_t s_k,
                                int64_t d, int32_t num_cus, int32_t *n_out);

/* The heuristic for query heads sharing K/V heads (h_kv as in attn_args; 0 or h
 * gives the two functions above).  With h_kv < h, s_q <= 64 and d >= 64 the
 * library packs the g = h / h_kv query heads of a K/V head, and their s_q rows,
 * into the same work-groups (each K/V tile then serves the whole group), so a
 * split has b * h_kv * ceil(g * s_q / 256) work-groups.  Errors as above, plus
 * ATTN_E_SHAPE for an h_kv that attn_args would reject. */
attn_status attn_num_splits_kv(int64_t b, int64_t h, int64_t h_kv, int64_t s_q, int64_t s_k,
                               int64_t d, int device, int32_t *n_out);
attn_status attn_num_splits_kv_for(int64_t b, int64_t h, int64_t h_kv, int64_t s_q, int64_t s_k,
                                   int64_t d, int32_t num_cus, int32_t *n_out);

/* First stage of flash-decoding (issue #1248): per split i, the attention of
 * every query over the keys of split i only.  Writes
 *   o_part  : dense fp32 [num_splits, b, h, s_q, d], O_i normalised within split i
 *   lse_part: dense fp32 [num_splits, b, h, s_q], natural-log LSE_i
 * A row that sees no key of a split gets O_i = 0 and LSE_i = -inf.
 * args->o, args->o_stride and args->lse are ignored. */
attn_status attn_fwd_splitkv(const attn_args *args, int32_t num_splits,
                             float *o_part, float *lse_part, void *stream);

/* Second stage (issue #1248's reduce): combine num_splits partials (layouts as
 * written by attn_fwd_splitkv) into O (dtype, (b, s_q, h, d) with element strides
 * o_stride for (b, s, h), d contiguous) and LSE (dense fp32 (b, h, s_q); may be
 * NULL).  A row whose LSE_i are all -inf gets O = 0 and LSE = -inf. */
attn_status attn_combine(int32_t num_splits, int64_t b, int64_t h, int64_t s_q, int64_t d,
                         const float *o_part, const float *lse_part, int32_t dtype,
                         void *o, const int64_t o_stride[3], float *lse, void *stream);

/* Paged K/V cache.  "LLM Lab Notes 07" (section 5, "Engineering Takeaways")
 * names the paged KV cache as the standard companion of the fused kernel for
 * long contexts and gives no layout; this library takes the plainest one:
 *   - k_cache, v_cache: blocks of block_size keys, (num_blocks, block_size, h_kv,
 *     d) with element strides k_stride / v_stride for (block, slot, head), each
 *     a non-negative multiple of 8, d contiguous, base pointers 16-byte aligned;
 *   - block_table: device int32, b rows of max_blocks entries, rows
 *     block_table_stride (>= max_blocks) elements apart: key j of sequence bi is
 *     slot j % block_size of block block_table[bi][j / block_size];
 *   - seqlens_k: device int32 (b): the key count of each sequence (0 allowed);
 *     max_seqlen_k (host, >= 1) bounds every count and must not exceed
 *     max_blocks * block_size.
 * Each sequence attends over its own keys: with causal != 0 query i of sequence
 * bi sees key j iff j <= i + seqlens_k[bi] - s_q, and in attn_fwd_splitkv_paged
 * split i covers keys [floor(i*s/n), floor((i+1)*s/n)) of its own count s.  Q, O
 * and LSE are laid out as in attn_args.  block_size is a power of two in [32,
 * 2^20] and d is 64 or 128 (else ATTN_E_SHAPE / ATTN_E_HEADDIM).  The table and
 * the counts live in device memory and cannot be checked on the host: the kernel
 * clamps block ids to [0, num_blocks) and counts to [0, max_seqlen_k], so
 * malformed entries give wrong results, never an access outside the cache.
 * Every shape and pointer rule of attn_args applies otherwise. */
typedef struct {
  int32_t dtype;        /* attn_dtype of Q, the caches and O */
  int32_t causal;
  int64_t b, s_q, h, h_kv, d;   /* h_kv: 0 means h; else h must be a multiple of it */
  const void *q;        /* device pointer, (b, s_q, h, d) */
  int64_t q_stride[3];  /* element strides of Q for (b, s, h) */
  const void *k_cache;  /* device pointer, (num_blocks, block_size, h_kv, d) */
  const void *v_cache;
  int64_t k_stride[3];  /* element strides for (block, slot, head) */
  int64_t v_stride[3];
  int64_t num_blocks, block_size;
  const int32_t *block_table;   /* device pointer, (b, max_blocks), 4-byte aligned */
  int64_t block_table_stride, max_blocks;
  const int32_t *seqlens_k;     /* device pointer, (b), 4-byte aligned */
  int64_t max_seqlen_k;
  void *o;              /* device pointer, (b, s_q, h, d), written by attn_fwd_paged */
  int64_t o_stride[3];
  float *lse;           /* dense (b, h, s_q) fp32, may be NULL; attn_fwd_paged only */
  float softmax_scale;
} attn_paged_args;

/* Fused forward over a paged cache: O and LSE in one kernel (as attn_fwd). */
attn_status attn_fwd_paged(const attn_paged_args *args, void *stream);

/* First flash-decoding stage over a paged cache: partials laid out as written by
 * attn_fwd_splitkv (combine them with attn_combine); num_splits in [1,
 * min(max_seqlen_k, ATTN_MAX_SPLITS)].  args->o, o_stride and lse are ignored. */
attn_status attn_fwd_splitkv_paged(const attn_paged_args *args, int32_t num_splits,
                                   float *o_part, float *lse_part, void *stream);

/* Split count for attn_fwd_splitkv_paged: the rule of attn_num_splits_kv with
 * s_k = max_seqlen_k (the paged cache runs the same kernels and work-groups),
 * except that packed query-head groups (h_kv < h, few query rows) aim at two
 * work-groups per compute unit instead of one. */
attn_status attn_num_splits_paged(int64_t b, int64_t h, int64_t h_kv, int64_t s_q,
                                  int64_t max_seqlen_k, int64_t d, int device, int32_t *n_out);

/* Backward pass.  flash-attention issue #1335 ("2.6.3 is faster than 2.7.0 for
 * flash-attn v2 CUDA fwd/bwd") times the backward of the forward above on its
 * fp16, head-dim-16 workloads; the pages do not describe its algorithm.  What it
 * computes is the gradient of the definition at the top of this file: for an
 * upstream gradient dO of O (LSE receives no gradient), per batch entry and
 * query head, with P the forward's softmax weights,
 *   dV_j  = sum_i P_ij dO_i                      (summed over the query heads
 *   dK_j  = scale * sum_i dS_ij q_i               that share K/V head j's head)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dS_ij = P_ij (dO_i . v_j - delta_i),  delta_i = dO_i . O_i.
 * P is recomputed tile by tile from Q, K and the forward's LSE, never stored.
 * A query row that sees no key (LSE = -inf) contributes nothing and gets dQ = 0.
 * Every argument follows the rules of attn_args (shapes, h_kv, head dims,
 * alignment, strides, finite scale, gfx950 device); the tensors are:
 *   q, o, dout, dq : (b, s_q, h, d);   k, v, dk, dv : (b, s_k, h_kv, d)
 * each with its own (b, s, h) element strides.  o and lse must be the forward's
 * outputs for the same q, k, v, scale and causal flag (o in the input dtype, lse
 * as attn_fwd writes it).  dq, dk, dv are written in the input dtype, computed
 * from fp32 accumulators in a fixed order (deterministic).  delta is a caller-
 * provided workspace, dense fp32 (b, h, s_q), overwritten with delta_i.
 * The result is enqueued on `stream` as two kernels (dQ, which also writes
 * delta, then dK/dV). */
typedef struct {
  int32_t dtype;        /* attn_dtype of every tensor below except lse, delta */
  int32_t causal;
  int64_t b, s_q, s_k, h, h_kv, d;   /* h_kv: 0 means h */
  const void *q, *k, *v, *o, *dout;  /* device pointers */
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3], dout_stride[3];
  const float *lse;     /* dense (b, h, s_q) fp32, from attn_fwd */
  void *dq, *dk, *dv;   /* device pointers, written */
  int64_t dq_stride[3], dk_stride[3], dv_stride[3];
  float *delta;         /* workspace, dense (b, h, s_q) fp32, written */
  float softmax_scale;
} attn_bwd_args;

attn_status attn_bwd(const attn_bwd_args *args, void *stream);

/* attn_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * checks, kernels and results, but args->delta is ignored (it may be NULL) and
 * delta lives in a static device buffer of the library, ATTN_BWD_SCRATCH_ROWS
 * fp32 values (16 MiB) that each device holds from its first call until the
 * process ends.  The call allocates nothing; b*h*s_q must not exceed
 * ATTN_BWD_SCRATCH_ROWS (else ATTN_E_SCRATCH, checked before anything is
 * launched).  Every call on a device shares that device's buffer, which keeps
 * the last call's contents; each call rewrites all of the delta it reads before
 * reading it, so nothing needs clearing, but calls that overlap on one device
 * (other streams or threads) race on the buffer and give undefined results. */
#define ATTN_BWD_SCRATCH_ROWS (1 << 22)
attn_status attn_bwd_noalloc(const attn_bwd_args *args, void *stream);

/* Static, human-readable text for a status code. */
const char *attn_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTN_H */
