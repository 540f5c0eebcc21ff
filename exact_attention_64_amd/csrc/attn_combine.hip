// Split reduction kernel for gfx950 (MI355X): flash-decoding's second stage
// (flash-attention issue #1248).
#include "attn_common.h"

namespace attn {

// ---------------------------------------------------------------------------
// Split reduction (issue #1248): one work-group of CW_ waves per (b, h, row).
//   M   = max_i LSE_i
//   LSE = M + ln sum_i exp(LSE_i - M)
//   O   = sum_i exp(LSE_i - LSE) * O_i
// Every wave reduces all LSE_i itself (lane i holds LSE_i, LSE_{i+64}, ...), so
// the weights need no barrier.  Lane l of wave w owns VPL consecutive columns of
// d (column group cg = l % CW) and the splits i = w + NWC * (sg + GRP * k) (split
// group sg = l / CW); the loads of up to PRE such splits are issued before any
// of them is used.  The NWC wave sums meet once in LDS.  Sums run over splits in
// increasing order inside a lane, then over split groups in a fixed butterfly
// order, then over waves in increasing order, so the result is deterministic.
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

constexpr int kCombineWaves = 4;

template <int T_, int D>
__global__ __launch_bounds__(kCombineWaves * 64) void combine_kernel(const CombineParams p) {
  using Tt = Ty<T_>;
  constexpr int NWC = kCombineWaves;
  constexpr int VPL = D > 64 ? D / 64 : 1;     // columns per lane
  constexpr int CW = D / VPL;                   // lanes across one row of O_i
  constexpr int GRP = 64 / CW;                  // split groups per wave
  constexpr int STRIDE = NWC * GRP;             // split stride of one lane
  constexpr int PRE = 16;                       // partial rows per lane in flight
  typedef float vec_t __attribute__((ext_vector_type(VPL)));
  __shared__ vec_t acc_s[NWC][64];

  const int row = blockIdx.x;  // (b*h + head)*s_q + i
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = p.n_splits;    // <= kMaxSplits
  const int64_t rows = (int64_t)p.b * p.h * p.s_q;
  const int cg = lane % CW, sg = lane / CW;
  const int first = wave + NWC * sg;            // this lane's first split

  // First chunk of this lane's partial rows and their LSEs, then all LSEs.
  vec_t pre[PRE];
  float lpre[PRE];
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const int i = first + k * STRIDE;
    const bool in = i < n;
    pre[k] = in ? *(const vec_t*)(p.o_part + ((int64_t)i * rows + row) * D + cg * VPL) : vec_t{};
    lpre[k] = in ? p.lse_part[(int64_t)i * rows + row] : -INFINITY;
  }
  float x[kMaxSplits / 64];
#pragma unroll
  for (int c = 0; c < kMaxSplits / 64; ++c) {
    const int i = lane + 64 * c;
    x[c] = i < n ? p.lse_part[(int64_t)i * rows + row] : -INFINITY;
  }

  float mx = x[0];
#pragma unroll
  for (int c = 1; c < kMaxSplits / 64; ++c) mx = fmaxf(mx, x[c]);
  const float M = wave_max(mx);
  const float Ms = M == -INFINITY ? 0.f : M;
  float e = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxSplits / 64; ++c) e += x[c] == -INFINITY ? 0.f : expf(x[c] - Ms);
  const float tot = wave_sum(e);
  const bool has = M != -INFINITY && tot > 0.f;
  const float lse = has ? Ms + logf(tot) : -INFINITY;

  vec_t acc = {};
  if (has) {
#pragma unroll
    for (int k = 0; k < PRE; ++k)
      if (first + k * STRIDE < n) acc += expf(lpre[k] - lse) * pre[k];
    // further chunks (more than PRE * STRIDE splits): loads first, then use
    for (int i0 = first + PRE * STRIDE; i0 < n; i0 += PRE * STRIDE) {
#pragma unroll
      for (int k = 0; k < PRE; ++k) {
        const int i = i0 + k * STRIDE;
        const bool in = i < n;
        pre[k] = in ? *(const vec_t*)(p.o_part + ((int64_t)i * rows + row) * D + cg * VPL) : vec_t{};
        lpre[k] = in ? p.lse_part[(int64_t)i * rows + row] : -INFINITY;
      }
#pragma unroll
      for (int k = 0; k < PRE; ++k)
        if (i0 + k * STRIDE < n) acc += expf(lpre[k] - lse) * pre[k];
    }
  }
  // fold the split groups (lanes cg, cg + CW, ...) in a fixed order
#pragma unroll
  for (int o = CW; o < 64; o <<= 1)
#pragma unroll
    for (int v = 0; v < VPL; ++v) acc[v] += __shfl_xor(acc[v], o);
  acc_s[wave][lane] = acc;
  __syncthreads();

  if (wave == 0 && sg == 0) {
    vec_t a = acc_s[0][lane];
#pragma unroll
    for (int w = 1; w < NWC; ++w) a += acc_s[w][lane];
    const int i = row % p.s_q;
    const int bh = row / p.s_q;
    const int bb = bh / p.h, hh = bh % p.h;
    unsigned short* op = (unsigned short*)p.o + (int64_t)bb * p.os[0] + (int64_t)i * p.os[1] + (int64_t)hh * p.os[2];
    if constexpr (VPL == 2) {
      *(unsigned*)(op + cg * 2) = Tt::pack2(a[0], a[1]);
    } else {
      op[cg] = Tt::one(a[0]);
    }
    if (lane == 0 && p.lse) p.lse[row] = lse;
  }
}

template <int T_>
static hipError_t launch_combine_t(const CombineParams& p, hipStream_t st) {
  const int64_t grid = (int64_t)p.b * p.h * p.s_q;
  switch (p.d) {
    case 16: hipLaunchKernelGGL((combine_kernel<T_, 16>), dim3((unsigned)grid), dim3(kCombineWaves * 64), 0, st, p); break;
    case 32: hipLaunchKernelGGL((combine_kernel<T_, 32>), dim3((unsigned)grid), dim3(kCombineWaves * 64), 0, st, p); break;
    case 64: hipLaunchKernelGGL((combine_kernel<T_, 64>), dim3((unsigned)grid), dim3(kCombineWaves * 64), 0, st, p); break;
    default: hipLaunchKernelGGL((combine_kernel<T_, 128>), dim3((unsigned)grid), dim3(kCombineWaves * 64), 0, st, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int dtype, hipStream_t st) {
  return dtype == kBF16 ? launch_combine_t<kBF16>(p, st) : launch_combine_t<kFP16>(p, st);
}

}  // namespace attn
