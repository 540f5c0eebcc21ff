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

}  // namespace

extern "C" int32_t attn_probe_grid(int32_t grid) {
  if (grid < 0) return -3;
  if (grid > 0) return grid;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) {
    (void)hipGetLastError();
    return -8;
  }
  return 4 * cus;
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
