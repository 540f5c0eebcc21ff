// Split reduction kernel for gfx950 (MI355X): flash-decoding's second stage
// (flash-attention issue #1248).
#include "attn_common.h"

namespace attn {

// ---------------------------------------------------------------------------
// Split reduction (issue #1248's reduce reply), per (b, h, row):
//   M   = max_i LSE_i
//   LSE = M + ln sum_i exp(LSE_i - M)
//   O   = sum_i exp(LSE_i - LSE) * O_i
// One wave per (row, slice of DC = 16 columns of O): a decode step has few rows
// (16 at b = 1, h = 16), so the reduction is spread over columns too, giving
// d / 16 waves per row and enough work-groups to issue every partial load at
// once.  Lane = sg * CW + cc: cc picks a 16-byte chunk (4 columns) of the slice,
// sg one of SG = 64 / CW split groups; the lane takes splits sg, sg + SG, ...
// (at most kMaxSplits / SG of them) and issues all their O_i and LSE_i loads
// before using any, so the kernel costs about one memory round trip.  The LSEs
// the lanes of one column chunk hold cover every split once: the maximum and
// the sum of exponentials come from one wave-wide reduction of those.  Sums run
// over a lane's splits in increasing order, then over split groups in a fixed
// butterfly order: the result is deterministic.
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

constexpr int kCombineCols = 16;  // columns of O per wave

template <int T_, int D>
__global__ __launch_bounds__(64) void combine_kernel(const CombineParams p) {
  using Tt = Ty<T_>;
  constexpr int DC = kCombineCols;              // D >= 16
  constexpr int NSL = D / DC;                   // slices (waves) per row
  constexpr int CW = DC / 4;                    // lanes across a slice
  constexpr int SG = 64 / CW;                   // split groups
  constexpr int PRE = kMaxSplits / SG;          // splits per lane, at most
  static_assert(D % DC == 0 && kMaxSplits % SG == 0, "slices and split groups must tile");

  const int row = blockIdx.x / NSL;             // (b*h + head)*s_q + i
  const int sl = blockIdx.x - row * NSL;
  const int lane = threadIdx.x;
  const int cc = lane % CW, sg = lane / CW;
  const int n = p.n_splits;                     // <= kMaxSplits
  const int64_t rows = (int64_t)p.b * p.h * p.s_q;
  const float* __restrict__ op = p.o_part + (int64_t)row * D + sl * DC + cc * 4;
  const float* __restrict__ lp = p.lse_part + row;

  f32x4_t x[PRE];
  float lw[PRE];
#pragma unroll
  for (int k = 0; k < PRE; ++k) {
    const int i = sg + SG * k;
    const bool in = i < n;
    x[k] = in ? *(const f32x4_t*)(op + (int64_t)i * rows * D) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    lw[k] = in ? lp[(int64_t)i * rows] : -INFINITY;
  }

  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < PRE; ++k) mx = fmaxf(mx, lw[k]);
  const float M = wave_max(mx);
  const float Ms = M == -INFINITY ? 0.f : M;
  float e = 0.f;
  if (cc == 0) {
#pragma unroll
    for (int k = 0; k < PRE; ++k) e += lw[k] == -INFINITY ? 0.f : expf(lw[k] - Ms);
  }
  const float tot = wave_sum(e);
  const bool has = M != -INFINITY && tot > 0.f;
  const float lse = has ? Ms + logf(tot) : -INFINITY;

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (has) {
#pragma unroll
    for (int k = 0; k < PRE; ++k)
      if (lw[k] != -INFINITY) acc += expf(lw[k] - lse) * x[k];
  }
#pragma unroll
  for (int o = CW; o < 64; o <<= 1)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] += __shfl_xor(acc[c], o);

  if (sg == 0) {
    const int i = row % p.s_q;
    const int bh = row / p.s_q;
    const int bb = bh / p.h, hh = bh % p.h;
    unsigned short* o = (unsigned short*)p.o + (int64_t)bb * p.os[0] + (int64_t)i * p.os[1] + (int64_t)hh * p.os[2] +
                        sl * DC + cc * 4;
    u32x2_t w = {Tt::pack2(acc[0], acc[1]), Tt::pack2(acc[2], acc[3])};
    *(u32x2_t*)o = w;
    if (sl == 0 && cc == 0 && p.lse) p.lse[row] = lse;
  }
}

// The same reduction for many rows (multi-token decode, many heads): one wave
// covers RPW = 256 / D whole rows, CPR = D / 4 lanes per row, each lane 4
// columns, so a split's slice of a row is one contiguous read of 4 D bytes and
// no lane idles for want of splits.  Three passes over the row's splits: the
// maximum of the LSE_i (lane c takes splits c, c + CPR, ...), the sum of
// exponentials (same lanes), then O += exp(LSE_i - LSE) * O_i over i in
// increasing order, the O_i loads issued eight at a time.  Deterministic.
template <int T_, int D>
__global__ __launch_bounds__(64) void combine_rows_kernel(const CombineParams p) {
  using Tt = Ty<T_>;
  constexpr int CPR = D / 4, RPW = 64 / CPR, CH = 8;
  const int lane = threadIdx.x, c = lane % CPR;
  const int64_t rows = (int64_t)p.b * p.h * p.s_q;
  const int64_t row = (int64_t)blockIdx.x * RPW + lane / CPR;
  const bool ok = row < rows;
  const int64_t rw = ok ? row : rows - 1;  // loads stay in bounds
  const int n = p.n_splits;                // <= kMaxSplits
  const float* __restrict__ lp = p.lse_part + rw;
  const float* __restrict__ op = p.o_part + rw * D + c * 4;

  float mx = -INFINITY;
  for (int i = c; i < n; i += CPR) mx = fmaxf(mx, lp[(int64_t)i * rows]);
#pragma unroll
  for (int o = 1; o < CPR; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const float Ms = mx == -INFINITY ? 0.f : mx;
  float e = 0.f;
  for (int i = c; i < n; i += CPR) {
    const float l = lp[(int64_t)i * rows];
    e += l == -INFINITY ? 0.f : expf(l - Ms);
  }
#pragma unroll
  for (int o = 1; o < CPR; o <<= 1) e += __shfl_xor(e, o);
  const bool has = mx != -INFINITY && e > 0.f;
  const float lse = has ? Ms + logf(e) : -INFINITY;

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (has) {
    for (int i0 = 0; i0 < n; i0 += CH) {
      f32x4_t x[CH];
      float lw[CH];
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int i = i0 + u;
        const bool in = i < n;
        x[u] = in ? *(const f32x4_t*)(op + (int64_t)i * rows * D) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        lw[u] = in ? lp[(int64_t)i * rows] : -INFINITY;
      }
#pragma unroll
      for (int u = 0; u < CH; ++u)
        if (lw[u] != -INFINITY) acc += expf(lw[u] - lse) * x[u];
    }
  }
  if (ok) {
    const int i = (int)(row % p.s_q);
    const int64_t bh = row / p.s_q;
    const int bb = (int)(bh / p.h), hh = (int)(bh % p.h);
    unsigned short* o = (unsigned short*)p.o + (int64_t)bb * p.os[0] + (int64_t)i * p.os[1] + (int64_t)hh * p.os[2] +
                        c * 4;
    u32x2_t w = {Tt::pack2(acc[0], acc[1]), Tt::pack2(acc[2], acc[3])};
    *(u32x2_t*)o = w;
    if (c == 0 && p.lse) p.lse[row] = lse;
  }
}

// Few rows (single-token decode: b * h rows): the column-sliced kernel, which
// spreads a row over d / 16 waves and its splits over the lanes; from
// kCombineRowsMin rows on, the row kernel.
constexpr int64_t kCombineRowsMin = 128;

template <int T_, int D>
static void launch_combine_d(const CombineParams& p, int64_t rows, hipStream_t st) {
  if (rows >= kCombineRowsMin) {
    constexpr int RPW = 256 / D;
    hipLaunchKernelGGL((combine_rows_kernel<T_, D>), dim3((unsigned)((rows + RPW - 1) / RPW)), dim3(64), 0, st, p);
  } else {
    hipLaunchKernelGGL((combine_kernel<T_, D>), dim3((unsigned)(rows * (D / kCombineCols))), dim3(64), 0, st, p);
  }
}

template <int T_>
static hipError_t launch_combine_t(const CombineParams& p, hipStream_t st) {
  const int64_t rows = (int64_t)p.b * p.h * p.s_q;
  switch (p.d) {
    case 16: launch_combine_d<T_, 16>(p, rows, st); break;
    case 32: launch_combine_d<T_, 32>(p, rows, st); break;
    case 64: launch_combine_d<T_, 64>(p, rows, st); break;
    default: launch_combine_d<T_, 128>(p, rows, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, int dtype, hipStream_t st) {
  return dtype == kBF16 ? launch_combine_t<kBF16>(p, st) : launch_combine_t<kFP16>(p, st);
}

}  // namespace attn
