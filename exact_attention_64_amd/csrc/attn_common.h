// Device-side helpers shared by the gfx950 kernels: vector types, the per-dtype
// MFMA flavour and rounding, and cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"

namespace attn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& x) {
  static_assert(sizeof(To) == sizeof(From), "size");
  return __builtin_bit_cast(To, x);
}

// Per-dtype pieces: the MFMA flavours (32x32x16 and 16x16x32) and float -> storage
// rounding (nearest even).
template <int DT> struct Ty;
template <> struct Ty<kBF16> {
  static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8_t>(a), bitcast<bf16x8_t>(b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(a), bitcast<bf16x8_t>(b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float x, float y) {
    bf16x2_t v = {(__bf16)x, (__bf16)y};
    return bitcast<unsigned>(v);
  }
  static __device__ __forceinline__ unsigned short one(float x) { return bitcast<unsigned short>((__bf16)x); }
  static __device__ __forceinline__ void unpack2(unsigned w, float& x, float& y) {
    x = __uint_as_float(w << 16);
    y = __uint_as_float(w & 0xffff0000u);
  }
};
template <> struct Ty<kFP16> {
  static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<f16x8_t>(a), bitcast<f16x8_t>(b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8_t>(a), bitcast<f16x8_t>(b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float x, float y) {
    f16x2_t v = {(_Float16)x, (_Float16)y};
    return bitcast<unsigned>(v);
  }
  static __device__ __forceinline__ unsigned short one(float x) { return bitcast<unsigned short>((_Float16)x); }
  static __device__ __forceinline__ void unpack2(unsigned w, float& x, float& y) {
    const f16x2_t h = bitcast<f16x2_t>(w);
    x = (float)h[0];
    y = (float)h[1];
  }
};

// Work-group id -> work item, XCD-aware.  Work-groups are dispatched to the
// eight XCDs round-robin (id % 8), and each XCD has its own L2.  Item L =
// xcd * q + min(xcd, r) + id / 8 (q, r = divmod(n, 8)) gives each XCD a
// contiguous range of items, taken in order, so consecutive items (the tiles of
// one head, which read the same K/V or Q/dO rows; neighbouring heads, which share
// cache lines at small head dims) share an XCD's L2.  A bijection on [0, n) for
// every n.
__device__ __forceinline__ int xcd_item(int id, int n) {
  const int q = n / 8, r = n % 8, x = id % 8;
  return x * q + min(x, r) + id / 8;
}

// A compile-time integer, and f(IC<I>{}), ..., f(IC<N - 1>{}) unrolled.
template <int N> struct IC { static constexpr int value = N; };
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IC<I>{});
    static_for<I + 1, N>(f);
  }
}

// s_waitcnt immediate (gfx9 encoding): vmcnt(n), lgkmcnt(0), expcnt untouched.
constexpr int vmcnt_lgkm0(int n) { return (n & 0xF) | (((n >> 4) & 0x3) << 14) | (0x7 << 4); }

// Maximum of a value and its partner lane (lane ^ 32), in every lane.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Packed-pair dot products, conversions and pair sums per storage type.
template <int T_> struct Dot;
template <> struct Dot<kBF16> {
  static __device__ __forceinline__ float dot8(u32x4_t a, u32x4_t b, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2_t>(a[i]), bitcast<bf16x2_t>(b[i]), acc, false);
    return acc;
  }
  static __device__ __forceinline__ void unpack8(u32x4_t a, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(a[i] << 16);
      f[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
    }
  }
  // acc + x.lo + x.hi for a packed pair
  static __device__ __forceinline__ float sum2(unsigned x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2_t>(x), bitcast<bf16x2_t>(0x3f803f80u), acc, false);
  }
};
template <> struct Dot<kFP16> {
  static __device__ __forceinline__ float dot8(u32x4_t a, u32x4_t b, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2(bitcast<f16x2_t>(a[i]), bitcast<f16x2_t>(b[i]), acc, false);
    return acc;
  }
  static __device__ __forceinline__ void unpack8(u32x4_t a, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2_t h = bitcast<f16x2_t>(a[i]);
      f[2 * i] = (float)h[0];
      f[2 * i + 1] = (float)h[1];
    }
  }
  // acc + x.lo + x.hi for a packed pair
  static __device__ __forceinline__ float sum2(unsigned x, float acc) {
    return __builtin_amdgcn_fdot2(bitcast<f16x2_t>(x), bitcast<f16x2_t>(0x3c003c00u), acc, false);
  }
};

// One direct-to-LDS wave load: lane i copies 16 bytes from gptr to LDS byte
// address lds + 16 i (lds is wave-uniform).  Written as inline asm so that the
// compiler does not treat the LDS write as aliasing the reads of other ring
// slots or buffers and wait for every load in flight before them (it cannot
// bound the per-wave offset); the kernels order these loads with their own
// s_waitcnt vmcnt and barriers.  Loads complete in order, so the compiler's own
// vmcnt waits for other loads stay correct.  The s_nop covers the M0 -> LDS DMA
// hazard.  NT sets the nontemporal bit: a tile that no other work-group reads
// should not allocate in the caches, where it would only push other lines out
// (dirty ones at the cost of a write-back each; measured on gfx950, default-
// policy streaming reads fall to about half the rate of nontemporal ones when
// the last-level cache holds dirty lines, and run about 12% slower when clean).
template <bool NT>
__device__ __forceinline__ void lds_dma16(const void* gptr, const char* lds) {
  const unsigned m0v = (unsigned)(uintptr_t)(const LDS_AS char*)lds;
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
                 :
                 : "s"(m0v), "v"(gptr)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(m0v), "v"(gptr)
                 : "memory", "m0");
}

}  // namespace attn
