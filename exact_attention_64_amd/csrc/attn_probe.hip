// HBM read-bandwidth probe for gfx950 (declared in include/attn_probe.h): the
// read half of a memory copy, against which the decode pass is measured.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/attn_probe.h"

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per lane

// Unit u (16 bytes) of the pattern lies at byte (u / upc) * stride + (u % upc) * 16,
// upc = chunk / 16.  Grid-stride loop with kUnroll independent loads per step.
__global__ __launch_bounds__(kThreads) void probe_read_kernel(const char* __restrict__ buf, int64_t units,
                                                             int64_t upc, int64_t stride, uint32_t* sink) {
  const int64_t nthr = (int64_t)gridDim.x * kThreads;
  int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  auto addr = [&](int64_t x) { return (const u32x4_t*)(buf + (x / upc) * stride + (x % upc) * 16); };
  for (; u + (kUnroll - 1) * nthr < units; u += kUnroll * nthr) {
    u32x4_t r[kUnroll];
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) r[i] = __builtin_nontemporal_load(addr(u + i * nthr));
#pragma unroll
    for (int i = 0; i < kUnroll; ++i) acc += r[i][0] + r[i][1] + r[i][2] + r[i][3];
  }
  for (; u < units; u += nthr) {
    const u32x4_t r = __builtin_nontemporal_load(addr(u));
    acc += r[0] + r[1] + r[2] + r[3];
  }
  // work-group sum through LDS, one word per work-group
  __shared__ uint32_t part[kThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int w = 0; w < kThreads / 64; ++w) s += part[w];
    sink[blockIdx.x] = s;
  }
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// 8 waves per work-group; operand registers ra[i], rb[j] hold random bf16 values
// (random sign, exponent and mantissa bits, magnitudes in [1/8, 2)) or the
// constant 1.0; MFMA i of a step reads
// ra[i % 8] and rb[(3 i + i / 8) % 8], so consecutive instructions change both.
template <bool RANDOM>
__global__ __launch_bounds__(512) void probe_mfma_kernel(float* out, int iters, unsigned long long* ticks) {
  const unsigned t = threadIdx.x + blockIdx.x * 512u;
  u32x4_t ra[8], rb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    unsigned h = (t * 2654435761u) ^ (i * 40503u + 12345u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h ^= h << 13; h ^= h >> 17; h ^= h << 5;
      ra[i][j] = RANDOM ? ((h & 0x81ff81ffu) | 0x3e003e00u) : 0x3f803f80u;
      h ^= h << 13; h ^= h >> 17; h ^= h << 5;
      rb[i][j] = RANDOM ? ((h & 0x81ff81ffu) | 0x3e003e00u) : 0x3f803f80u;
    }
  }
  f32x16_t acc[4] = {};
  const unsigned long long c0 = clock64(), w0 = wall_clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ra[i & 7]),
                                                           __builtin_bit_cast(bf16x8_t, rb[(3 * i + i / 8) & 7]),
                                                           acc[i & 3], 0, 0, 0);
  }
  const unsigned long long c1 = clock64(), w1 = wall_clock64();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += acc[0][i] + acc[1][i] + acc[2][i] + acc[3][i];
  out[t] = s;
  if (t == 0) {
    ticks[0] = c1 - c0;
    ticks[1] = w1 - w0;
  }
}

__global__ __launch_bounds__(64) void probe_clock_kernel(unsigned long long* out, long long wall_ticks) {
  const unsigned long long c0 = clock64(), w0 = wall_clock64();
  unsigned long long c1 = c0, w1 = w0;
  // bounded: the steady counter only moves forward, and the loop also stops
  // after 2^31 polls whatever it reads
  for (long long n = 0; n < (1ll << 31) && (long long)(w1 - w0) < wall_ticks; ++n) {
    __builtin_amdgcn_s_sleep(8);
    c1 = clock64();
    w1 = wall_clock64();
  }
  if (threadIdx.x == 0) {
    out[0] = c0;
    out[1] = c1;
    out[2] = w0;
    out[3] = w1;
  }
}

int cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) {
    (void)hipGetLastError();
    return -1;
  }
  return cus;
}

}  // namespace

extern "C" int32_t attn_probe_mfma(float* out, int32_t iters, int32_t random_operands, uint64_t* ticks, void* stream) {
  if (!out || !ticks) return -1;
  if (iters < 1) return -3;
  const int cus = cu_count();
  if (cus < 1) return -8;
  if (random_operands)
    hipLaunchKernelGGL(probe_mfma_kernel<true>, dim3((unsigned)cus), dim3(512), 0, (hipStream_t)stream, out, iters,
                       (unsigned long long*)ticks);
  else
    hipLaunchKernelGGL(probe_mfma_kernel<false>, dim3((unsigned)cus), dim3(512), 0, (hipStream_t)stream, out, iters,
                       (unsigned long long*)ticks);
  return hipGetLastError() == hipSuccess ? 0 : -9;
}

extern "C" int32_t attn_probe_clock(uint64_t* out, int64_t wall_ticks, void* stream) {
  if (!out) return -1;
  if (wall_ticks < 1 || wall_ticks > (int64_t(1) << 31)) return -3;
  hipLaunchKernelGGL(probe_clock_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, (unsigned long long*)out,
                     (long long)wall_ticks);
  return hipGetLastError() == hipSuccess ? 0 : -9;
}

extern "C" int32_t attn_probe_rates(int64_t* wall_khz, int64_t* peak_sclk_khz) {
  if (!wall_khz || !peak_sclk_khz) return -1;
  int dev = 0, w = 0, c = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&w, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
      hipDeviceGetAttribute(&c, hipDeviceAttributeClockRate, dev) != hipSuccess) {
    (void)hipGetLastError();
    return -8;
  }
  *wall_khz = w;
  *peak_sclk_khz = c;
  return 0;
}

extern "C" int32_t attn_probe_grid(int32_t grid) {
  if (grid < 0) return -3;
  if (grid > 0) return grid;
  const int cus = cu_count();
  return cus < 1 ? -8 : 4 * cus;
}

extern "C" int32_t attn_probe_read(const void* buf, int64_t bytes, int64_t chunk, int64_t stride, uint32_t* sink,
                                   int32_t grid, void* stream) {
  if (!buf || !sink) return -1;
  if (bytes < 16 || chunk < 16 || stride < chunk || bytes % 16 || chunk % 16 || stride % 16 || bytes % chunk)
    return -3;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return -5;
  const int32_t g = attn_probe_grid(grid);
  if (g < 0) return g;
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)g), dim3(kThreads), 0, (hipStream_t)stream,
                     (const char*)buf, bytes / 16, chunk / 16, stride, sink);
  return hipGetLastError() == hipSuccess ? 0 : -9;
}
