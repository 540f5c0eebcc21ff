// Internal interface between the C-ABI front end (attn_api.cpp) and the gfx950
// kernels (attn_fwd.hip, attn_decode.hip, attn_combine.hip,
// attn_bwd.hip).  Not installed; the public interface is attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

constexpr int kFP16 = 0;  // matches ATTN_FP16
constexpr int kBF16 = 1;  // matches ATTN_BF16
constexpr int kMaxSplits = 256;

// Arguments of the fused / split-KV forward kernel.  Strides are in elements,
// for the (b, s, h) dimensions; d is contiguous.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;          // fused: (b, s_q, h, d) output
  float* lse;       // fused: (b, h, s_q), may be null
  float* o_part;    // split: [n, b, h, s_q, d] fp32
  float* lse_part;  // split: [n, b, h, s_q] fp32
  int64_t qs[3], ks[3], vs[3], os[3];
  int b, h, s_q, s_k, d;
  int n_qt;         // query tiles per (b, h); filled by the launcher
  int n_splits;     // 1 for the fused kernel
  float scale_log2; // |softmax_scale| * log2(e)  (1 when zero_q)
  int neg_q;        // softmax_scale < 0: Q is negated on load
  int zero_q;       // softmax_scale == 0: Q is treated as zero
  int g;            // query heads per K/V head: query head hh reads K/V head hh / g
  // Paged K/V cache (block_table != nullptr): k and v point at the block caches,
  // ks / vs are the (block, slot, head) strides and s_k bounds every key count.
  const int* block_table;  // (b, bt_stride) block ids
  const int* seqlens_k;    // (b) key counts
  int64_t bt_stride;
  int num_blocks;
  int lbs;                 // log2(block_size)
};

struct CombineParams {
  const float* o_part;
  const float* lse_part;
  void* o;
  float* lse;
  int64_t os[3];
  int b, h, s_q, d;
  int n_splits;
};

// Arguments of the backward kernels (attn_bwd.hip).  Strides are in elements,
// for the (b, s, h) dimensions; d is contiguous.
struct BwdParams {
  const void* q;     // (b, s_q, h, d)
  const void* k;     // (b, s_k, h / g, d)
  const void* v;
  const void* o;     // forward output (b, s_q, h, d)
  const void* dout;  // upstream gradient of O (b, s_q, h, d)
  const float* lse;  // forward LSE, dense (b, h, s_q), natural log
  float* delta;      // dense (b, h, s_q): row dot of dO and O, written by the dQ kernel
  void* dq;          // (b, s_q, h, d), written
  void* dk;          // (b, s_k, h / g, d), written
  void* dv;
  int64_t qs[3], ks[3], vs[3], os[3], dos[3], dqs[3], dks[3], dvs[3];
  int b, h, s_q, s_k, d;
  int g;             // query heads per K/V head
  float scale;       // softmax scale (any finite value)
  float scale_log2;  // scale * log2(e)
};

// Compile-time tunables (overridable with -D for sweeps).
#ifndef ATTN_PREFILL_NW
#define ATTN_PREFILL_NW 8   // waves per work-group of the d >= 64 prefill kernel (32 rows each)
                            // when a head (or packed group) has more than 128 query rows
#endif
#ifndef ATTN_PREFILL_BN
#define ATTN_PREFILL_BN 32  // keys per tile of the d >= 64 prefill kernel
#endif
#ifndef ATTN_PREFILL_NBUF
#define ATTN_PREFILL_NBUF 4 // LDS ring buffers per tensor (prefetch depth + 1): 2, 4 or 8
                            // (packed decode: 2 measured 25% slower, 8 10% slower)
#endif
#ifndef ATTN_STREAM_QTILES
#define ATTN_STREAM_QTILES 2 // prefill K/V loads are nontemporal when at most this many work-groups read a tile
#endif
#ifndef ATTN_DECODE_HEADS
#define ATTN_DECODE_HEADS 4 // heads (one wave each) per work-group of the decode kernel
#endif
#ifndef ATTN_DECODE_NBUF
#define ATTN_DECODE_NBUF 3  // register buffers of wave loads in the decode kernel (2 or 3; 3 measured
                            // ~2% faster on the 32k-key decode: two batches in flight while one is used)
#endif
#ifndef ATTN_DECODE_BATCH
#define ATTN_DECODE_BATCH 8 // wave loads per tensor per batch in the decode kernel
#endif
constexpr int kPrefillNW = ATTN_PREFILL_NW;
constexpr int kPrefillBN = ATTN_PREFILL_BN;
constexpr int kPrefillNBUF = ATTN_PREFILL_NBUF;
constexpr int kStreamQTiles = ATTN_STREAM_QTILES;
constexpr int kDecodeHeads = ATTN_DECODE_HEADS;
constexpr int kDecodeBatch = ATTN_DECODE_BATCH;
#ifndef ATTN_SMALL_D_NW
#define ATTN_SMALL_D_NW 2   // waves (32 query rows each) per work-group of the d <= 32 prefill kernel
#endif

// Query heads sharing a K/V head (g > 1) with few query rows: the prefill kernel
// packs a K/V head's g * s_q query rows into its work-groups (d >= 64).
inline bool fwd_packed(int64_t g, int64_t s_q, int d) { return g > 1 && s_q <= 64 && d >= 64; }
// Work-groups per split: packed, one per (b, K/V head, block of packed rows);
// the decode kernel (s_q == 1) puts kDecodeHeads heads in one work-group; the
// prefill kernel one (b, h, query row block) per work-group.
inline int64_t fwd_groups_per_split(int64_t b, int64_t h, int64_t g, int64_t s_q, int d) {
  const int64_t bm = d >= 64 ? kPrefillNW * 32 : ATTN_SMALL_D_NW * 32;  // prefill rows per work-group
  if (fwd_packed(g, s_q, d)) return b * (h / g) * ((g * s_q + bm - 1) / bm);
  if (s_q == 1) return (b * h + kDecodeHeads - 1) / kDecodeHeads;
  return b * h * ((s_q + bm - 1) / bm);
}

// Fused / split-KV prefill kernel (s_q >= 1; used for s_q > 1), one explicit
// instantiation per (input type, causal) pair in its own object file.
template <int T_, bool CAUSAL, bool PAGED>
hipError_t launch_prefill_tc(const FwdParams& p, bool split, hipStream_t st);
extern template hipError_t launch_prefill_tc<kFP16, false, false>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_prefill_tc<kFP16, true, false>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_prefill_tc<kBF16, false, false>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_prefill_tc<kBF16, true, false>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_prefill_tc<kFP16, false, true>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_prefill_tc<kFP16, true, true>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_prefill_tc<kBF16, false, true>(const FwdParams&, bool, hipStream_t);
extern template hipError_t launch_prefill_tc<kBF16, true, true>(const FwdParams&, bool, hipStream_t);
template <bool PAGED>
inline hipError_t launch_prefill_p(const FwdParams& p, int dtype, bool causal, bool split, hipStream_t st) {
  if (dtype == kBF16)
    return causal ? launch_prefill_tc<kBF16, true, PAGED>(p, split, st) : launch_prefill_tc<kBF16, false, PAGED>(p, split, st);
  return causal ? launch_prefill_tc<kFP16, true, PAGED>(p, split, st) : launch_prefill_tc<kFP16, false, PAGED>(p, split, st);
}
inline hipError_t launch_prefill(const FwdParams& p, int dtype, bool causal, bool split, hipStream_t st) {
  return p.block_table ? launch_prefill_p<true>(p, dtype, causal, split, st)
                       : launch_prefill_p<false>(p, dtype, causal, split, st);
}
// One-row decode kernel (s_q == 1).
hipError_t launch_decode(const FwdParams& p, int dtype, bool split, hipStream_t st);
// One of the kernels above: the decode kernel for one query row unless query
// heads share K/V heads (then the packed prefill kernel reads each K/V tile once
// per group; with one query row the bottom-right causal mask hides nothing, so
// the causal flag does not matter there), the small-head kernel where it
// applies, else the prefill kernel.
// Persistent small-head forward (attn_small.hip): d <= 32 and both sequence
// lengths at most kSmallMaxSeq, fused (not split), contiguous K/V.
constexpr int kSmallMaxSeq = 256;
inline bool small_fwd_ok(const FwdParams& p) {
  return p.d <= 32 && p.s_q <= kSmallMaxSeq && p.s_k <= kSmallMaxSeq && (int64_t)p.b * p.h <= 0x7fffffff;
}
hipError_t launch_small(const FwdParams& p, int dtype, bool causal, hipStream_t st);
inline hipError_t launch_fwd(const FwdParams& p, int dtype, bool causal, bool split, hipStream_t st) {
  if (p.s_q == 1 && !fwd_packed(p.g, p.s_q, p.d)) return launch_decode(p, dtype, split, st);
  if (!split && !p.block_table && small_fwd_ok(p)) return launch_small(p, dtype, causal, st);
  return launch_prefill(p, dtype, causal, split, st);
}
hipError_t launch_combine(const CombineParams& p, int dtype, hipStream_t st);
// Backward: dQ (which also writes delta), then dK/dV, enqueued in that order on `st`.
hipError_t launch_bwd(const BwdParams& p, int dtype, bool causal, hipStream_t st);
// Device address of the backward's static delta scratch (kBwdScratchFloats fp32)
// on the current device, resolved once per device (attn_bwd.hip).
constexpr int64_t kBwdScratchFloats = int64_t(1) << 22;  // 16 MiB: b * h * s_q rows of delta
hipError_t bwd_scratch(float** out);

}  // namespace attn
