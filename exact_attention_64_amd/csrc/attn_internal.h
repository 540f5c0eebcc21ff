// Internal interface between the C-ABI front end (attn_api.cpp) and the gfx950
// kernels (attn_kernels.hip).  Not installed; the public interface is attn.h.
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

// Query rows covered by one work-group of the fused kernel for head dim d.
int fwd_rows_per_block(int d);

hipError_t launch_fwd(const FwdParams& p, int dtype, bool causal, bool split, hipStream_t st);
hipError_t launch_combine(const CombineParams& p, int dtype, hipStream_t st);

}  // namespace attn
