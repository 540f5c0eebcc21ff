// One-query-row (decode) split-KV kernel for gfx950 (MI355X): flash-decoding's
// first stage (flash-attention issue #1248) as a memory-streaming pass.
#include "attn_common.h"

namespace attn {

// ---------------------------------------------------------------------------
// One-query-row forward (decode), the flash-decoding first stage of issue #1248
// for s_q == 1.  The pass is bound by reading K and V once, so it runs on the
// vector ALUs with wide streaming loads and no LDS staging; matrix cores would
// idle on a single query row (the issue's reply makes the same point: decode
// speed is close to a memory copy, so spare compute does not matter).
//
// Work-group = kDecodeHeads waves; wave w streams head 4g + w (of the flattened
// b*h heads) over the whole key range of one split, so the work-group reads the
// rows of adjacent heads together: 1 KB of contiguous K (and V) per key at
// d = 128, instead of 256-byte pieces 4 KB apart.  Lane layout: a key row (D
// elements) is read by LPH = D/8 lanes, 16 bytes each, so one wave load covers
// KPI = 64/LPH consecutive keys.  Each group of LPH lanes ("slot") runs its own
// online softmax over the keys it reads; at the end the KPI slot states of the
// wave are merged by a butterfly of lane shuffles with the max-subtracted rule
// of the combine.  No LDS, no barriers.
template <int LPH>
__device__ __forceinline__ float slot_sum(float x) {
  // all-reduce over the LPH consecutive lanes of a slot (DPP within a row of 16)
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // lane ^ 1
  if (LPH >= 4) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // lane ^ 2
  if (LPH >= 8) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // half mirror
  if (LPH >= 16) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));  // mirror
  return x;
}

// Three wave-uniform 32-bit reads through the scalar data cache (read only),
// waited for together.
__device__ __forceinline__ void sload3_i32(const int* a, const int* b, const int* c, int& x, int& y, int& z) {
  asm volatile("s_load_dword %0, %3, 0x0\n\ts_load_dword %1, %4, 0x0\n\ts_load_dword %2, %5, 0x0\n\t"
               "s_waitcnt lgkmcnt(0)"
               : "=&s"(x), "=&s"(y), "=&s"(z)
               : "s"(a), "s"(b), "s"(c));
}

// PAGED: K and V are a block cache (num_blocks, block_size, h_kv, d) with
// (block, slot, head) strides; key j of batch entry bb is slot j % block_size of
// block block_table[bb][j / block_size], and the entry has seqlens_k[bb] keys.
// One batch of U * KPI <= 64 keys touches at most three blocks (block_size >= 32);
// their ids are read once per batch with scalar loads and each lane picks its
// key's block.  Ids are clamped to [0, num_blocks), key counts to [0, s_k].
template <int T_, int D, bool SPLIT, bool PAGED>
__global__ __launch_bounds__(kDecodeHeads * 64) void decode_kernel(const FwdParams p) {
  using Tt = Ty<T_>;
  using Dt = Dot<T_>;
  constexpr int LPH = D / 8;        // lanes per key row
  constexpr int KPI = 64 / LPH;     // keys per wave load (= slots per wave)
  constexpr int U = kDecodeBatch;   // wave loads per tensor in one batch
  static_assert(!PAGED || U * KPI <= 64, "a paged batch must span at most three 32-key blocks");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = lane / LPH;
  const int dc = lane % LPH;
  // 1-D grid, split fastest: work-group g covers split g % n_splits of head
  // group g / n_splits.
  const int split = blockIdx.x % p.n_splits;
  const int bh = (blockIdx.x / p.n_splits) * kDecodeHeads + wave;
  if (bh >= p.b * p.h) return;      // the whole wave; the kernel has no barriers
  const int bb = bh / p.h;
  const int hh = bh - bb * p.h;

  const int s_k = PAGED ? min(max(p.seqlens_k[bb], 0), p.s_k) : p.s_k;
  int k_lo = 0, k_hi = s_k;
  if (SPLIT) {
    k_lo = (int)(((int64_t)split * s_k) / p.n_splits);
    k_hi = (int)(((int64_t)(split + 1) * s_k) / p.n_splits);
  }
  const int ws = k_lo, we = k_hi;

  u32x4_t q = {0u, 0u, 0u, 0u};
  if (!p.zero_q) {
    q = *(const u32x4_t*)((const unsigned short*)p.q + (int64_t)bb * p.qs[0] + (int64_t)hh * p.qs[2] + dc * 8);
    if (p.neg_q) q ^= 0x80008000u;
  }
  const int hk = hh / p.g;  // K/V head of this query head
  const unsigned short* __restrict__ Kg =
      (const unsigned short*)p.k + (PAGED ? 0 : (int64_t)bb * p.ks[0]) + (int64_t)hk * p.ks[2] + dc * 8;
  const unsigned short* __restrict__ Vg =
      (const unsigned short*)p.v + (PAGED ? 0 : (int64_t)bb * p.vs[0]) + (int64_t)hk * p.vs[2] + dc * 8;
  const int64_t ksr = p.ks[1], vsr = p.vs[1];
  const int* __restrict__ tbl = PAGED ? p.block_table + (int64_t)bb * p.bt_stride : nullptr;
  const int last_blk = PAGED && we > 0 ? (we - 1) >> p.lbs : 0;  // last block with a key of this split
  const float c = p.scale_log2;

  float m = -INFINITY, l = 0.f;
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;

  // ATTN_DECODE_NBUF (three) register buffers, used in turn by a loop unrolled
  // as many times, so that the loads of the next batches are in flight while one
  // is consumed (indices stay compile-time constants and the buffers stay in
  // registers: one wave per SIMD leaves room for them).
  u32x4_t kb0[U], vb0[U], kb1[U], vb1[U];
#if ATTN_DECODE_NBUF == 3
  u32x4_t kb2[U], vb2[U];
#endif
  auto load = [&](u32x4_t (&kb)[U], u32x4_t (&vb)[U], int j0) {
    int blk[3] = {0, 0, 0};
    int kb0 = 0;
    if constexpr (PAGED) {
      kb0 = j0 >> p.lbs;
      sload3_i32(tbl + kb0, tbl + min(kb0 + 1, last_blk), tbl + min(kb0 + 2, last_blk), blk[0], blk[1], blk[2]);
#pragma unroll
      for (int i = 0; i < 3; ++i) blk[i] = min(max(blk[i], 0), p.num_blocks - 1);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * KPI + slot;
      u32x4_t xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
      if (j < we) {
        int64_t ko = (int64_t)j * ksr, vo = (int64_t)j * vsr;
        if constexpr (PAGED) {
          const int rel = j - (kb0 << p.lbs);          // [0, 3 * block_size)
          const int bi = rel >> p.lbs;
          const int64_t b = bi == 0 ? blk[0] : (bi == 1 ? blk[1] : blk[2]);
          const int r = rel & ((1 << p.lbs) - 1);
          ko = b * p.ks[0] + (int64_t)r * ksr;
          vo = b * p.vs[0] + (int64_t)r * vsr;
        }
        xk = __builtin_nontemporal_load((const u32x4_t*)(Kg + ko));
        xv = __builtin_nontemporal_load((const u32x4_t*)(Vg + vo));
      }
      kb[u] = xk;
      vb[u] = xv;
    }
  };
  auto consume = [&](const u32x4_t (&kb)[U], const u32x4_t (&vb)[U], int j0) {
    float s[U];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      s[u] = slot_sum<LPH>(Dt::dot8(q, kb[u], 0.f));
      if (j0 + u * KPI + slot >= we) s[u] = -INFINITY;
      mx = fmaxf(mx, s[u]);
    }
    const float m_new = fmaxf(m, mx * c);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pu = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u], c, -m_use));
      l += pu;
      float f[8];
      Dt::unpack8(vb[u], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = __builtin_fmaf(pu, f[e], o[e]);
    }
    m = m_new;
  };
  constexpr int STEP = U * KPI;
#if ATTN_DECODE_NBUF == 3
  // three buffers, rotated by a loop unrolled three times: while one batch is
  // consumed the next two are in flight
  if (ws < we) load(kb0, vb0, ws);
  if (ws + STEP < we) load(kb1, vb1, ws + STEP);
  for (int j0 = ws; j0 < we; j0 += 3 * STEP) {
    if (j0 + 2 * STEP < we) load(kb2, vb2, j0 + 2 * STEP);
    consume(kb0, vb0, j0);
    if (j0 + STEP >= we) break;
    if (j0 + 3 * STEP < we) load(kb0, vb0, j0 + 3 * STEP);
    consume(kb1, vb1, j0 + STEP);
    if (j0 + 2 * STEP >= we) break;
    if (j0 + 4 * STEP < we) load(kb1, vb1, j0 + 4 * STEP);
    consume(kb2, vb2, j0 + 2 * STEP);
  }
#else
  if (ws < we) load(kb0, vb0, ws);
  for (int j0 = ws; j0 < we; j0 += 2 * STEP) {
    if (j0 + STEP < we) load(kb1, vb1, j0 + STEP);
    consume(kb0, vb0, j0);
    if (j0 + STEP >= we) break;
    if (j0 + 2 * STEP < we) load(kb0, vb0, j0 + 2 * STEP);
    consume(kb1, vb1, j0 + STEP);
  }
#endif

  // Merge the KPI slot states of the wave: butterfly over the slot index
  // (partner lane = lane ^ (LPH << k)), identical states in every slot after.
#pragma unroll
  for (int sh = LPH; sh < 64; sh <<= 1) {
    const float m2 = __shfl_xor(m, sh);
    const float l2 = __shfl_xor(l, sh);
    const float M = fmaxf(m, m2);
    const float Mu = M == -INFINITY ? 0.f : M;
    const float a1 = __builtin_amdgcn_exp2f(m - Mu), a2 = __builtin_amdgcn_exp2f(m2 - Mu);
    l = a1 * l + a2 * l2;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = a1 * o[e] + a2 * __shfl_xor(o[e], sh);
    m = M;
  }
  const bool has = l > 0.f;
  const float inv = has ? 1.f / l : 0.f;
  const float lse = has ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
  if (slot == 0) {
    if (SPLIT) {
      const int64_t rowi = ((int64_t)split * p.b + bb) * p.h + hh;  // s_q == 1
      float* op = p.o_part + rowi * D + dc * 8;
      f32x4_t x0 = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
      f32x4_t x1 = {o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
      *(f32x4_t*)op = x0;
      *(f32x4_t*)(op + 4) = x1;
      if (dc == 0) p.lse_part[rowi] = lse;
    } else {
      unsigned short* op = (unsigned short*)p.o + (int64_t)bb * p.os[0] + (int64_t)hh * p.os[2] + dc * 8;
      u32x4_t x = {Tt::pack2(o[0] * inv, o[1] * inv), Tt::pack2(o[2] * inv, o[3] * inv),
                   Tt::pack2(o[4] * inv, o[5] * inv), Tt::pack2(o[6] * inv, o[7] * inv)};
      *(u32x4_t*)op = x;
      if (dc == 0 && p.lse) p.lse[(int64_t)bb * p.h + hh] = lse;
    }
  }
}

template <int T_, bool SPLIT>
static hipError_t launch_decode_t(const FwdParams& p, hipStream_t st) {
  const int64_t groups = ((int64_t)p.b * p.h + kDecodeHeads - 1) / kDecodeHeads;
  const dim3 grid((unsigned)(groups * p.n_splits));
  const dim3 block(kDecodeHeads * 64);
  if (p.block_table) {  // paged cache: d is 64 or 128 (checked on the host)
    if (p.d == 64) hipLaunchKernelGGL((decode_kernel<T_, 64, SPLIT, true>), grid, block, 0, st, p);
    else if (p.d == 128) hipLaunchKernelGGL((decode_kernel<T_, 128, SPLIT, true>), grid, block, 0, st, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  switch (p.d) {
    case 16: hipLaunchKernelGGL((decode_kernel<T_, 16, SPLIT, false>), grid, block, 0, st, p); break;
    case 32: hipLaunchKernelGGL((decode_kernel<T_, 32, SPLIT, false>), grid, block, 0, st, p); break;
    case 64: hipLaunchKernelGGL((decode_kernel<T_, 64, SPLIT, false>), grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL((decode_kernel<T_, 128, SPLIT, false>), grid, block, 0, st, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const FwdParams& p, int dtype, bool split, hipStream_t st) {
  if (dtype == kBF16) return split ? launch_decode_t<kBF16, true>(p, st) : launch_decode_t<kBF16, false>(p, st);
  return split ? launch_decode_t<kFP16, true>(p, st) : launch_decode_t<kFP16, false>(p, st);
}

}  // namespace attn
