// Split reduction kernel for gfx950 (MI355X): flash-decoding's second stage
// (flash-attention issue #1248).
#include "attn_common.h"

namespace attn {

// ---------------------------------------------------------------------------
// Split reduction (issue #1248): one work-group per (b, h, row).
//   LSE = M + ln sum_i exp(LSE_i - M),  M = max_i LSE_i
//   O   = sum_i exp(LSE_i - LSE) * O_i
// Splits are summed in increasing order inside each of G lane groups, then the
// G group sums in increasing group order, so the result is deterministic.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int T_, int D>
__global__ __launch_bounds__(256) void combine_kernel(const CombineParams p) {
  using Tt = Ty<T_>;
  constexpr int TPS = D / 4;         // threads per split row (float4 each)
  constexpr int G = 256 / TPS;       // split rows in flight
  constexpr int PRE = 8;             // partial rows per thread loaded up front
  __shared__ float w_s[kMaxSplits];
  __shared__ float red[2][4];
  __shared__ f32x4_t acc_s[G][TPS];

  const int row = blockIdx.x;  // (b*h + head)*s_q + i
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = p.n_splits;    // <= kMaxSplits == blockDim.x
  const int64_t rows = (int64_t)p.b * p.h * p.s_q;
  const int g = tid / TPS, c4 = tid % TPS;

  // Issue the partial-output loads first; they do not depend on the weights.
  f32x4_t pre[PRE];
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const int i = g + k * G;
    pre[k] = i < n ? *(const f32x4_t*)(p.o_part + ((int64_t)i * rows + row) * D + c4 * 4)
                   : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const float x = tid < n ? p.lse_part[(int64_t)tid * rows + row] : -INFINITY;

  float mx = wave_max(x);
  if (lane == 0) red[0][wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  const float Ms = M == -INFINITY ? 0.f : M;
  float e = wave_sum(tid < n ? expf(x - Ms) : 0.f);
  if (lane == 0) red[1][wave] = e;
  __syncthreads();
  const float tot = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const bool has = M != -INFINITY && tot > 0.f;
  const float lse = has ? Ms + logf(tot) : -INFINITY;
  if (tid < n) w_s[tid] = has ? expf(x - lse) : 0.f;
  __syncthreads();

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const int i = g + k * G;
    if (i < n) acc += w_s[i] * pre[k];
  }
  for (int i = g + PRE * G; i < n; i += G)
    acc += w_s[i] * *(const f32x4_t*)(p.o_part + ((int64_t)i * rows + row) * D + c4 * 4);
  acc_s[g][c4] = acc;
  __syncthreads();
  if (tid < TPS) {
    f32x4_t a = acc_s[0][tid];
    for (int gg = 1; gg < G; ++gg) a += acc_s[gg][tid];
    const int i = row % p.s_q;
    const int bh = row / p.s_q;
    const int bb = bh / p.h, hh = bh % p.h;
    unsigned short* op = (unsigned short*)p.o + (int64_t)bb * p.os[0] + (int64_t)i * p.os[1] + (int64_t)hh * p.os[2];
    u32x2_t xo = {Tt::pack2(a[0], a[1]), Tt::pack2(a[2], a[3])};
    *(u32x2_t*)(op + tid * 4) = xo;
    if (tid == 0 && p.lse) p.lse[row] = lse;
  }
}

template <int T_>
static hipError_t launch_combine_t(const CombineParams& p, hipStream_t st) {
  const int64_t grid = (int64_t)p.b * p.h * p.s_q;
  switch (p.d) {
    case 16: hipLaunchKernelGGL((combine_kernel<T_, 16>), dim3((unsigned)grid), dim3(256), 0, st, p); break;
    case 32: hipLaunchKernelGGL((combine_kernel<T_, 32>), dim3((unsigned)grid), dim3(256), 0, st, p); break;
    case 64: hipLaunchKernelGGL((combine_kernel<T_, 64>), dim3((unsigned)grid), dim3(256), 0, st, p); break;
    default: hipLaunchKernelGGL((combine_kernel<T_, 128>), dim3((unsigned)grid), dim3(256), 0, st, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int dtype, hipStream_t st) {
  return dtype == kBF16 ? launch_combine_t<kBF16>(p, st) : launch_combine_t<kFP16>(p, st);
}

}  // namespace attn
