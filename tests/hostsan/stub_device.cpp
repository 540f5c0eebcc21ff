// Host-only stand-in for the device side of libattn.so, so that the C-ABI front
// end (exact_attention_64_amd/csrc/attn_api.cpp) can be built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer and exercised on a machine
// without a GPU.  It answers the three HIP runtime calls the front end makes
// (one gfx950 device with 256 compute units) and, instead of launching
// kernels, records the parameters each launcher receives; stub_* accessors
// return them to the tests.  Test infrastructure only.
#include <hip/hip_runtime_api.h>

#include <cstring>
#include <string>

#include "../../exact_attention_64_amd/csrc/attn_internal.h"

namespace {
attn::FwdParams g_fwd;
attn::CombineParams g_comb;
attn::BwdParams g_bwd;
int g_kind = 0;        // 1 prefill kernel, 2 decode kernel, 3 combine, 4 backward
int g_launches = 0;
int g_dtype = -1, g_causal = -1, g_split = -1;
float g_scratch_stand_in[4];
}  // namespace

extern "C" hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
extern "C" hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* prop, int dev) {
  if (dev != 0) return hipErrorInvalidDevice;
  std::memset(prop, 0, sizeof(*prop));
  std::strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
  prop->multiProcessorCount = 256;
  return hipSuccess;
}
extern "C" hipError_t hipGetLastError() { return hipSuccess; }

namespace attn {
template <int T_, bool CAUSAL, bool PAGED>
hipError_t launch_prefill_tc(const FwdParams& p, bool split, hipStream_t) {
  g_fwd = p;
  g_kind = 1;
  g_dtype = T_;
  g_causal = CAUSAL;
  g_split = split;
  ++g_launches;
  return hipSuccess;
}
template hipError_t launch_prefill_tc<kFP16, false, false>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_prefill_tc<kFP16, true, false>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_prefill_tc<kBF16, false, false>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_prefill_tc<kBF16, true, false>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_prefill_tc<kFP16, false, true>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_prefill_tc<kFP16, true, true>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_prefill_tc<kBF16, false, true>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_prefill_tc<kBF16, true, true>(const FwdParams&, bool, hipStream_t);

hipError_t launch_decode(const FwdParams& p, int dtype, bool split, hipStream_t) {
  g_fwd = p;
  g_kind = 2;
  g_dtype = dtype;
  g_causal = -1;
  g_split = split;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_small(const FwdParams& p, int dtype, bool causal, hipStream_t) {
  g_fwd = p;
  g_kind = 5;
  g_dtype = dtype;
  g_causal = causal;
  g_split = 0;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_combine(const CombineParams& p, int dtype, hipStream_t) {
  g_comb = p;
  g_kind = 3;
  g_dtype = dtype;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_bwd(const BwdParams& p, int dtype, bool causal, hipStream_t) {
  g_bwd = p;
  g_kind = 4;
  g_dtype = dtype;
  g_causal = causal;
  ++g_launches;
  return hipSuccess;
}
hipError_t bwd_scratch(float** out) {
  *out = g_scratch_stand_in;
  return hipSuccess;
}
}  // namespace attn

extern "C" int stub_launches() { return g_launches; }
extern "C" int stub_last_kind() { return g_kind; }
extern "C" const void* stub_scratch() { return g_scratch_stand_in; }

// Field of the last launch's parameters, as a double (pointers as integers).
extern "C" double stub_field(const char* name) {
  const std::string n(name);
  if (n == "dtype") return g_dtype;
  if (n == "causal") return g_causal;
  if (n == "split") return g_split;
  if (g_kind == 1 || g_kind == 2 || g_kind == 5) {
    const attn::FwdParams& p = g_fwd;
    if (n == "b") return p.b;
    if (n == "h") return p.h;
    if (n == "s_q") return p.s_q;
    if (n == "s_k") return p.s_k;
    if (n == "d") return p.d;
    if (n == "g") return p.g;
    if (n == "n_splits") return p.n_splits;
    if (n == "scale_log2") return p.scale_log2;
    if (n == "neg_q") return p.neg_q;
    if (n == "zero_q") return p.zero_q;
    if (n == "lbs") return p.lbs;
    if (n == "num_blocks") return p.num_blocks;
    if (n == "bt_stride") return (double)p.bt_stride;
    if (n == "paged") return p.block_table != nullptr;
    if (n == "o") return (double)(uintptr_t)p.o;
    if (n == "lse") return (double)(uintptr_t)p.lse;
    if (n == "o_part") return (double)(uintptr_t)p.o_part;
    if (n == "qs1") return (double)p.qs[1];
    if (n == "ks2") return (double)p.ks[2];
  } else if (g_kind == 3) {
    const attn::CombineParams& p = g_comb;
    if (n == "n_splits") return p.n_splits;
    if (n == "d") return p.d;
    if (n == "s_q") return p.s_q;
    if (n == "os0") return (double)p.os[0];
  } else if (g_kind == 4) {
    const attn::BwdParams& p = g_bwd;
    if (n == "g") return p.g;
    if (n == "scale") return p.scale;
    if (n == "scale_log2") return p.scale_log2;
    if (n == "delta") return (double)(uintptr_t)p.delta;
    if (n == "s_k") return p.s_k;
  }
  return -12345.0;
}
