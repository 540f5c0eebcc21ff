// Backward of exact attention for gfx950 (MI355X): dQ, dK, dV for an upstream
// gradient dO, from the forward's O and per-row LSE.
//
// flash-attention issue #1335 ("2.6.3 is faster than 2.7.0 for flash-attn v2
// CUDA fwd/bwd") times this backward on its fp16, head-dim-16 workloads without
// describing the algorithm; what it computes is the gradient of the standard
// attention of "LLM Lab Notes 07: Why FlashAttention Is Fast" (section 2), here
// evaluated tile by tile like the forward, so that neither P nor dS reaches
// device memory (sections 3.1, 3.2).  Per (batch, head), with c = scale*log2(e)
// and the forward's natural-log LSE:
//   P_ij  = exp2(c*q_i.k_j - LSE_i*log2(e))      (the forward's softmax, exactly)
//   dV_j  = sum_i P_ij dO_i
//   dP_ij = dO_i . v_j,   delta_i = dO_i . O_i
//   dS_ij = P_ij (dP_ij - delta_i)
//   dQ_i  = scale * sum_j dS_ij k_j,   dK_j = scale * sum_i dS_ij q_i
// Two kernels, both deterministic (no atomics):
//   bwd_dq_kernel    : one work-group per (b, query head, 32 to 256 query rows); it
//                      also writes delta (b, h, s_q) fp32, the row dot of dO and O,
//                      for the second kernel; K and V tiles of 32 keys stream
//                      into LDS by direct-to-LDS loads; S^T, dP^T and dS^T are
//                      formed so that each lane owns one query row (the forward's
//                      layout) and dQ^T += K^T dS^T accumulates in registers;
//   bwd_dkdv_kernel,
//   bwd_dkdv1_kernel : one work-group per (b, K/V head, 32 to 128 keys); Q and dO tiles
//                      of 32 rows (of every query head of the group) stream
//                      into LDS by direct-to-LDS loads; S, dP and dS are
//                      formed so that each lane owns
//                      one key, and dV^T += dO^T P, dK^T += Q^T dS accumulate in
//                      registers (of two partner waves at d = 128, of one wave
//                      at smaller head dims).  Query heads sharing a
//                      K/V head are summed in the same work-group, in a fixed
//                      order.
// Every product runs on v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulation;
// P and dS are rounded to the input type before they feed a product.
#include <mutex>

#include "attn_common.h"
#include "attn_tile.h"

#ifndef ATTN_BWD_SMALL_NW
#define ATTN_BWD_SMALL_NW 1  // waves per work-group of the dQ and dK/dV kernels at d <= 32 (b = 512, s = 150,
                             // d = 16: 0.305 ms with 4, 0.250 with 2, 0.240 with 1)
#endif
#ifndef ATTN_BWD_PF
#define ATTN_BWD_PF 2  // LDS operand reads in flight ahead of the d = 128 kernels' products
#endif
#ifndef ATTN_BWD_DQ_NW
#define ATTN_BWD_DQ_NW 8  // waves (32 query rows each) per work-group of the d = 128 dQ kernel
#endif

namespace attn {
namespace {

// log2-domain LSE of a row: +inf for a row that sees no key (LSE = -inf), so
// that exp2(s*c - lse2) = 0 there.
__device__ __forceinline__ float lse_log2(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// A run of N matrix products use(i, frag) whose A operands come from LDS
// (load(i)), with the reads PF products ahead of their use: the reads of
// product i + PF are issued before product i, and a scheduling barrier keeps
// them there.  Left to itself the compiler issues each read right before its
// product, which then waits out the LDS latency.
template <int I, int N, int PF> struct LdsPipe {
  template <class Load, class Use>
  static __device__ __forceinline__ void run(Load& load, Use& use, u32x4_t (&f)[PF + 1]) {
    if constexpr (I < N) {
      if constexpr (I + PF < N) f[(I + PF) % (PF + 1)] = load(I + PF);
      __builtin_amdgcn_sched_barrier(0);
      use(I, f[I % (PF + 1)]);
      LdsPipe<I + 1, N, PF>::run(load, use, f);
    }
  }
};
template <int N, int PF, class Load, class Use>
__device__ __forceinline__ void lds_pipeline(Load&& load, Use&& use) {
  u32x4_t f[PF + 1];
#pragma unroll
  for (int i = 0; i < PF && i < N; ++i) f[i] = load(i);
  LdsPipe<0, N, PF>::run(load, use, f);
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace

// ---------------------------------------------------------------------------
// dQ: one work-group = NW waves x 32 query rows of one (b, query head) (8 waves
// at d = 128, 4 at d = 64, one at d <= 32).  Per 32-key tile a wave runs three
// stages: the products S^T and dP^T (matrix core), P and dS^T (vector ALU), and
// the product dQ^T += K^T dS^T (matrix core).  With 8 waves two share each SIMD,
// and the second half of the work-group (waves 4..7) runs half a tile behind
// the first: after the barrier that ends step t it finishes tile t (P, dS^T,
// dQ^T) and then forms S^T, dP^T of tile t + 1, while the first half forms,
// finishes and multiplies tile t + 1 in that order.  So on each SIMD one wave's
// vector work overlaps the other's products instead of both waves waiting on
// the same stage.  The delay keeps three K/V tiles in LDS: the one the late
// waves finish, the current one and the one in flight.
template <int T_, int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(const BwdParams p) {
  using Tt = Ty<T_>;
  constexpr int KK = D / 16, CB = D >= 32 ? D / 32 : 1, BM = NW * 32, NTH = NW * 64;
  constexpr bool SKEW = NW == 8;
  constexpr int NB = SKEW ? 3 : 2;  // K/V tile buffers
  __shared__ __attribute__((aligned(16))) char kbuf[NB][BTile<D>::BYTES];
  __shared__ __attribute__((aligned(16))) char vbuf[NB][BTile<D>::BYTES];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool late = SKEW && wave >= NW / 2;  // wave-uniform
  const int n_qt = (p.s_q + BM - 1) / BM;
  // items (b*h, query tile) in head-major order, spread over the XCDs so that
  // the tiles of a head share one L2; causal: heaviest tiles first
  const int item = xcd_item(blockIdx.x, p.b * p.h * n_qt);
  const int bh = item / n_qt;
  const int qt_rev = item - bh * n_qt;
  const int qt = CAUSAL ? n_qt - 1 - qt_rev : qt_rev;
  const int bb = bh / p.h, hh = bh - bb * p.h, hk = hh / p.g;
  const int q0 = qt * BM;
  const int my_i = q0 + wave * 32 + l32;
  const bool row_ok = my_i < p.s_q;
  const int off = p.s_k - p.s_q;
  int k_hi = p.s_k;
  if (CAUSAL) k_hi = min(k_hi, q0 + BM - 1 + off + 1);
  const int T = k_hi > 0 ? (k_hi + 31) / 32 : 0;

  // Q and dO of this lane's row: B operands of S^T = K Q^T and dP^T = V dO^T.
  u32x4_t qf[KK], df[KK];
  float lse2 = INFINITY, dl = 0.f;
  {
    const unsigned short* Qr = (const unsigned short*)p.q + (int64_t)bb * p.qs[0] + (int64_t)my_i * p.qs[1] +
                               (int64_t)hh * p.qs[2];
    const unsigned short* Dr = (const unsigned short*)p.dout + (int64_t)bb * p.dos[0] +
                               (int64_t)my_i * p.dos[1] + (int64_t)hh * p.dos[2];
    const unsigned short* Or = (const unsigned short*)p.o + (int64_t)bb * p.os[0] + (int64_t)my_i * p.os[1] +
                               (int64_t)hh * p.os[2];
    // delta = dO . O of this lane's row: each half-wave holds half of the row's
    // columns (hi*8 + 16*kk), so the two halves meet in one lane swap
    float part = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4_t z = {0u, 0u, 0u, 0u};
      qf[kk] = row_ok ? *(const u32x4_t*)(Qr + hi * 8 + kk * 16) : z;
      df[kk] = row_ok ? *(const u32x4_t*)(Dr + hi * 8 + kk * 16) : z;
      const u32x4_t of = row_ok ? *(const u32x4_t*)(Or + hi * 8 + kk * 16) : z;
      part = Dot<T_>::dot8(df[kk], of, part);
    }
    dl = pair_sum(part);
    if (row_ok) {
      const int64_t ri = ((int64_t)bb * p.h + hh) * p.s_q + my_i;
      lse2 = lse_log2(p.lse[ri]);
      if (hi == 0) p.delta[ri] = dl;  // for the dK/dV kernel, launched after this one
    }
  }
  const float c = p.scale_log2;

  f32x16_t acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;

  const unsigned short* Kg = (const unsigned short*)p.k + (int64_t)bb * p.ks[0] + (int64_t)hk * p.ks[2];
  const unsigned short* Vg = (const unsigned short*)p.v + (int64_t)bb * p.vs[0] + (int64_t)hk * p.vs[2];
  // K and V tiles go global -> LDS by direct-to-LDS loads; rows at or past k_hi
  // re-read row k_hi - 1 (finite data, masked scores)
  // Without the skew every thread loads part of both tiles at the start of a
  // step.  With it, each half's 256 threads load one tile, spread over their
  // products: the early half K between its S^T, dP^T products, the late half V
  // between its dQ products (a wave that issues a burst of direct-to-LDS loads
  // stalls until the memory pipeline takes them).
  constexpr int NLD = SKEW ? NTH / 2 : NTH;
  const int ltid = SKEW ? tid & (NLD - 1) : tid, lwave = SKEW ? wave & (NW / 2 - 1) : wave;
  // with the skew a wave loads one of the two tiles: one set of offsets
  const TileOffs<D, NLD> ko(SKEW && late ? p.vs[1] : p.ks[1], ltid), vo(p.vs[1], ltid);
  auto load_k = [&](int t, int buf) __attribute__((always_inline)) {
    dma_tile<D, NLD>(ko, Kg, p.ks[1], t * 32, k_hi, ltid, lwave, kbuf[buf]);
  };
  auto load_v = [&](int t, int buf) __attribute__((always_inline)) {
    dma_tile<D, NLD>(SKEW ? ko : vo, Vg, p.vs[1], t * 32, k_hi, ltid, lwave, vbuf[buf]);
  };
  auto nohook = []() __attribute__((always_inline)) {};
  // S^T and dP^T of the tile in buffer buf, the two product chains interleaved
  // so that one's latency hides the other's; dP^T starts from -delta, so the
  // chain leaves dP - delta
  auto products = [&](int buf, f32x16_t& s, f32x16_t& dp, auto&& hook) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.f;
      dp[r] = -dl;
    }
    if constexpr (SKEW) {
      lds_pipeline<2 * KK, ATTN_BWD_PF>(
          [&](int i) __attribute__((always_inline)) {
            return frag_rows<D>(i % 2 == 0 ? kbuf[buf] : vbuf[buf], l32, hi, i / 2);
          },
          [&](int i, u32x4_t f) __attribute__((always_inline)) {
            if (i % 2 == 0) s = Tt::mfma(f, qf[i / 2], s);
            else dp = Tt::mfma(f, df[i / 2], dp);
            if (i == KK - 1) hook();
          });
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        s = Tt::mfma(frag_rows<D>(kbuf[buf], l32, hi, kk), qf[kk], s);
        dp = Tt::mfma(frag_rows<D>(vbuf[buf], l32, hi, kk), df[kk], dp);
      }
    }
  };
  // P and dS^T of tile t (buffer buf) for this lane's row and its 16 keys (key of
  // element r: k0 + (r/4)*8 + 4*hi + r%4), then dQ^T += K^T dS^T
  auto finish = [&](int t, int buf, const f32x16_t& s, const f32x16_t& dp, auto&& hook) __attribute__((always_inline)) {
    const int k0 = t * 32;
    // masks only where a key of the tile is past the range or (causal) after the
    // diagonal of the wave's first row; wave-uniform
    const bool edge = k0 + 32 > k_hi || (CAUSAL && k0 + 31 > q0 + wave * 32 + off);
    u32x4_t dsb[2];
    if (edge) {
#pragma unroll
      for (int t16 = 0; t16 < 2; ++t16)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int r = 8 * t16 + 2 * e + u;
            const int key = k0 + (r / 4) * 8 + hi * 4 + (r % 4);
            float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lse2));
            if (key >= k_hi || (CAUSAL && key > my_i + off)) pr = 0.f;
            x[u] = pr * dp[r];
          }
          dsb[t16][e] = Tt::pack2(x[0], x[1]);
        }
    } else {
#pragma unroll
      for (int t16 = 0; t16 < 2; ++t16)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int r = 8 * t16 + 2 * e + u;
            x[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lse2)) * dp[r];
          }
          dsb[t16][e] = Tt::pack2(x[0], x[1]);
        }
    }
    if constexpr (SKEW) {
      // consecutive products go to different accumulators
      lds_pipeline<2 * CB, ATTN_BWD_PF>(
          [&](int i) __attribute__((always_inline)) { return frag_cols<D>(kbuf[buf], lane, hi, i % CB, i / CB); },
          [&](int i, u32x4_t f) __attribute__((always_inline)) {
            acc[i % CB] = Tt::mfma(f, dsb[i / CB], acc[i % CB]);
            if (i == CB - 1) hook();
          });
    } else {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int t16 = 0; t16 < 2; ++t16)
          acc[cb] = Tt::mfma(frag_cols<D>(kbuf[buf], lane, hi, cb, t16), dsb[t16], acc[cb]);
    }
  };

  if (T > 0) {
    if (!SKEW || !late) load_k(0, 0);
    if (!SKEW || late) load_v(0, 0);
  }
  // Every load issued so far (this lane's Q, dO, O, LSE and the first tile)
  // lands here, on every path: a load still pending where the loop starts would
  // make the compiler wait inside the loop for all loads, the next tile's included.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Step t: the step's work, during which tile t + 1 is loaded (into the buffer
  // that held tile t + 1 - NB, finished before the barrier ending step t - 1);
  // after the barrier tile t + 1 is in LDS.  Both halves pass the
  // same T barriers.  The steps are unrolled over the NB buffers, so that every
  // LDS address is a per-lane register plus an immediate offset.
  f32x16_t s, dp;  // carried across the barrier by the late half
  if (!late) {
    for (int t0 = 0; t0 < T; t0 += NB)
      static_for<0, NB>([&](auto R) __attribute__((always_inline)) {
        constexpr int cur = decltype(R)::value, nxt = (cur + 1) % NB;
        const int t = t0 + cur;
        if (t < T) {
          const bool more = t + 1 < T;
          if constexpr (SKEW) {
            products(cur, s, dp, [&]() __attribute__((always_inline)) { if (more) load_k(t + 1, nxt); });
          } else {
            if (more) {
              load_k(t + 1, nxt);
              load_v(t + 1, nxt);
            }
            products(cur, s, dp, nohook);
          }
          finish(t, cur, s, dp, nohook);
          __builtin_amdgcn_s_waitcnt(0);  // the direct-to-LDS loads of tile t + 1 have landed
          __syncthreads();
        }
      });
  } else {
    for (int t0 = 0; t0 < T; t0 += NB)
      static_for<0, NB>([&](auto R) __attribute__((always_inline)) {
        constexpr int cur = decltype(R)::value, nxt = (cur + 1) % NB, prv = (cur + NB - 1) % NB;
        const int t = t0 + cur;
        if (t < T) {
          const bool more = t + 1 < T;
          auto ld = [&]() __attribute__((always_inline)) { if (more) load_v(t + 1, nxt); };
          if (t > 0) finish(t - 1, prv, s, dp, ld);
          // nothing of the next products moves above this point: their
          // accumulators reuse the registers of the finished tile's
          __builtin_amdgcn_sched_barrier(0);
          if (t == 0) products(cur, s, dp, ld);
          else products(cur, s, dp, nohook);
          __builtin_amdgcn_s_waitcnt(0);
          __syncthreads();
        }
      });
    if (T > 0) finish(T - 1, (T - 1) % NB, s, dp, nohook);
  }

  if (row_ok) {
    unsigned short* dst = (unsigned short*)p.dq + (int64_t)bb * p.dqs[0] + (int64_t)my_i * p.dqs[1] +
                          (int64_t)hh * p.dqs[2];
    store_cols<T_, D, CB>(dst, acc, hi, p.scale);
  }
}

// ---------------------------------------------------------------------------
// dK, dV for d <= 64 (single-wave form): one work-group = 4 waves x 32 keys of
// one (b, K/V head); each wave holds its keys' K and V and both accumulator sets
// (few registers at these head dims), and computes S, dP, P, dS, dV^T and dK^T
// itself, with one barrier per step.  The query rows of the g query heads that
// read the K/V head stream past in 32-row tiles.
template <int T_, int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dkdv1_kernel(const BwdParams p) {
  using Tt = Ty<T_>;
  constexpr int KK = D / 16, CB = D >= 32 ? D / 32 : 1, BK = NW * 32;
  __shared__ __attribute__((aligned(16))) char qbuf[2][BTile<D>::BYTES];
  __shared__ __attribute__((aligned(16))) char obuf[2][BTile<D>::BYTES];
  __shared__ __attribute__((aligned(16))) float lbuf[2][32];
  __shared__ __attribute__((aligned(16))) float dbuf[2][32];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h_kv = p.h / p.g;
  const int n_kt = (p.s_k + BK - 1) / BK;
  // items (b*h_kv, key block) in head-major order, spread over the XCDs so that
  // the blocks of a head share one L2; causal: low key blocks (seen by the most
  // rows) first
  const int item = xcd_item(blockIdx.x, p.b * h_kv * n_kt);
  const int bk = item / n_kt;
  const int kt = item - bk * n_kt;
  const int bb = bk / h_kv, hk = bk - bb * h_kv;
  const int k0 = kt * BK;
  const int my_j = k0 + wave * 32 + l32;
  const bool key_ok = my_j < p.s_k;
  const int off = p.s_k - p.s_q;
  // Query rows that see any key of the block: i >= k0 - off when causal.
  const int r_lo = CAUSAL ? max(0, k0 - off) : 0;
  const int qt0 = r_lo / 32;
  const int nq = r_lo < p.s_q ? (p.s_q + 31) / 32 - qt0 : 0;
  const int T = p.g * nq;

  // K and V of this lane's key: B operands of S = Q K^T and dP = dO V^T.
  u32x4_t kf[KK], vf[KK];
  {
    const int j = min(my_j, p.s_k - 1);
    const unsigned short* Kr = (const unsigned short*)p.k + (int64_t)bb * p.ks[0] + (int64_t)j * p.ks[1] +
                               (int64_t)hk * p.ks[2];
    const unsigned short* Vr = (const unsigned short*)p.v + (int64_t)bb * p.vs[0] + (int64_t)j * p.vs[1] +
                               (int64_t)hk * p.vs[2];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      kf[kk] = *(const u32x4_t*)(Kr + hi * 8 + kk * 16);
      vf[kk] = *(const u32x4_t*)(Vr + hi * 8 + kk * 16);
    }
  }
  const float c = p.scale_log2;

  f32x16_t dk[CB], dv[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[cb][r] = dv[cb][r] = 0.f;

  // Q and dO tiles go global -> LDS by direct-to-LDS loads (rows past s_q re-read
  // row s_q - 1: finite data, and their LSE is +inf, so P = 0).
  // LSE and delta of staged row tid % 32, loaded by every lane without a branch
  // (the row index is clamped) and converted only when stored, so that nothing
  // waits for these loads before the step's products.
  float lr = 0.f, dr = 0.f;
  bool row_in = false;
  const TileOffs<D, NW * 64> qo(p.qs[1], tid), oo(p.dos[1], tid);
  auto load_tile = [&](int t, int buf) __attribute__((always_inline)) {
    const int hh = hk * p.g + t / nq;
    const int q0 = (qt0 + nq - 1 - t % nq) * 32;  // last tile first
    const int row = q0 + (tid & 31);
    row_in = row < p.s_q;
    const int64_t ri = ((int64_t)bb * p.h + hh) * p.s_q + min(row, p.s_q - 1);
    lr = p.lse[ri];
    dr = p.delta[ri];
    const unsigned short* Qg = (const unsigned short*)p.q + (int64_t)bb * p.qs[0] + (int64_t)hh * p.qs[2];
    const unsigned short* Og = (const unsigned short*)p.dout + (int64_t)bb * p.dos[0] + (int64_t)hh * p.dos[2];
    dma_tile<D, NW * 64>(qo, Qg, p.qs[1], q0, p.s_q, tid, wave, qbuf[buf]);
    dma_tile<D, NW * 64>(oo, Og, p.dos[1], q0, p.s_q, tid, wave, obuf[buf]);
  };
  auto store_tile = [&](int buf) __attribute__((always_inline)) {
    if (tid < 32) {
      lbuf[buf][tid] = row_in ? lse_log2(lr) : INFINITY;
      dbuf[buf][tid] = row_in ? dr : 0.f;
    }
  };
  if (T > 0) {
    load_tile(0, 0);
    store_tile(0);
  }
  // K, V and the first tile land here, on every path (see the dQ kernel).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int t = 0; t < T; ++t) {
    const int cur = t & 1;
    const bool more = t + 1 < T;
    if (more) load_tile(t + 1, cur ^ 1);  // that buffer was last read before the barrier ending step t - 1
    const int q0 = (qt0 + nq - 1 - t % nq) * 32;  // last tile first
    const char* qb = qbuf[cur];
    const char* ob = obuf[cur];
    f32x16_t s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s = Tt::mfma(frag_rows<D>(qb, l32, hi, kk), kf[kk], s);
      dp = Tt::mfma(frag_rows<D>(ob, l32, hi, kk), vf[kk], dp);
    }
    // P and dS for this lane's key and its 16 rows (row of element r: q0 + (r/4)*8 + 4*hi + r%4).
    u32x4_t pb[2], db[2];
    const bool diag = k0 + wave * 32 + 31 > q0 + off;  // causal mask needed (wave-uniform)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4_t l4 = *(const f32x4_t*)(&lbuf[cur][r4 * 8 + hi * 4]);
      const f32x4_t d4 = *(const f32x4_t*)(&dbuf[cur][r4 * 8 + hi * 4]);
      float pr[4], ds[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * r4 + u;
        const int row = q0 + r4 * 8 + hi * 4 + u;
        float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -l4[u]));
        if (CAUSAL && diag && my_j > row + off) x = 0.f;
        pr[u] = x;
        ds[u] = x * (dp[r] - d4[u]);
      }
      // elements 8*t16 .. 8*t16 + 7 form B-operand chunk t16
      pb[r4 / 2][2 * (r4 % 2)] = Tt::pack2(pr[0], pr[1]);
      pb[r4 / 2][2 * (r4 % 2) + 1] = Tt::pack2(pr[2], pr[3]);
      db[r4 / 2][2 * (r4 % 2)] = Tt::pack2(ds[0], ds[1]);
      db[r4 / 2][2 * (r4 % 2) + 1] = Tt::pack2(ds[2], ds[3]);
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int t16 = 0; t16 < 2; ++t16) {
        dv[cb] = Tt::mfma(frag_cols<D>(ob, lane, hi, cb, t16), pb[t16], dv[cb]);
        dk[cb] = Tt::mfma(frag_cols<D>(qb, lane, hi, cb, t16), db[t16], dk[cb]);
      }
    if (more) store_tile(cur ^ 1);
    __builtin_amdgcn_s_waitcnt(0);  // the direct-to-LDS loads of tile t + 1 have landed
    __syncthreads();
  }

  if (key_ok) {
    unsigned short* dkp = (unsigned short*)p.dk + (int64_t)bb * p.dks[0] + (int64_t)my_j * p.dks[1] +
                          (int64_t)hk * p.dks[2];
    unsigned short* dvp = (unsigned short*)p.dv + (int64_t)bb * p.dvs[0] + (int64_t)my_j * p.dvs[1] +
                          (int64_t)hk * p.dvs[2];
    store_cols<T_, D, CB>(dkp, dk, hi, p.scale);
    store_cols<T_, D, CB>(dvp, dv, hi, 1.f);
  }
}

// ---------------------------------------------------------------------------
// dK, dV for d = 128 (paired form): one work-group = 8 waves over 128 keys of
// one (b, K/V head); the query rows of the g query heads that read the K/V head
// stream past in tiles of 64 rows (two 32-row halves).  The waves pair up per
// 32-key block kb (waves kb and kb + 4, which share a SIMD):
//   P-wave  (role 0): S = Q K^T, P = exp2(S*c - LSE*log2 e), hands P (fp32) to
//                     its partner through LDS, and accumulates dV^T += dO^T P;
//   dS-wave (role 1): dP - delta = dO V^T - delta, then, with the partner's P,
//                     dS = P (dP - delta), and accumulates dK^T += Q^T dS.
// So each wave holds one operand set (K or V of its keys) and one accumulator
// set, and two waves fit on a SIMD.  The dS-wave runs one tile behind: in step
// t the P-wave forms S, P and dV of tile t, while the dS-wave finishes tile
// t - 1 (dS from the P its partner left in step t - 1, then dK) and forms
// dP - delta of tile t, which it carries across the step's one barrier.
// Neither wave waits for the other inside a step, so one wave's exponentials
// or dS overlap the other's products.  LDS holds three Q tiles (t - 1 for dK,
// t, and t + 1 in flight), two dO tiles and two P buffers.
template <int T_, int D, bool CAUSAL>
__global__ __launch_bounds__(512) void bwd_dkdv_kernel(const BwdParams p) {
  using Tt = Ty<T_>;
  constexpr int KK = D / 16, CB = D >= 32 ? D / 32 : 1, BK = 128, NTH = 512, BQ = 64;
  __shared__ __attribute__((aligned(16))) char qbuf[3][2][BTile<D>::BYTES];  // [buffer][half]
  __shared__ __attribute__((aligned(16))) char obuf[2][2][BTile<D>::BYTES];
  __shared__ __attribute__((aligned(16))) float lbuf[2][BQ];
  __shared__ __attribute__((aligned(16))) float dbuf[2][BQ];  // -delta
  __shared__ __attribute__((aligned(16))) f32x4_t xbuf[2][2][4][4][64];  // [buffer][half][key block][r4][lane]: P

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = wave & 3, role = wave >> 2;
  const int h_kv = p.h / p.g;
  const int n_kt = (p.s_k + BK - 1) / BK;
  // items (b*h_kv, key block) in head-major order, spread over the XCDs so that
  // the blocks of a head share one L2; causal: low key blocks (seen by the most
  // rows) first
  const int item = xcd_item(blockIdx.x, p.b * h_kv * n_kt);
  const int bk = item / n_kt;
  const int kt = item - bk * n_kt;
  const int bb = bk / h_kv, hk = bk - bb * h_kv;
  const int k0 = kt * BK;
  const int my_j = k0 + kb * 32 + l32;
  const bool key_ok = my_j < p.s_k;
  const int off = p.s_k - p.s_q;
  // Query rows that see any key of the block: i >= k0 - off when causal.
  const int r_lo = CAUSAL ? max(0, k0 - off) : 0;
  const int qt0 = r_lo / BQ;
  const int nq = r_lo < p.s_q ? (p.s_q + BQ - 1) / BQ - qt0 : 0;
  const int T = p.g * nq;

  // This lane's key row of K (P-wave) or V (dS-wave): the B operand of
  // S = Q K^T or dP = dO V^T.
  u32x4_t opnd[KK];
  {
    const int j = min(my_j, p.s_k - 1);
    const unsigned short* R =
        role == 0 ? (const unsigned short*)p.k + (int64_t)bb * p.ks[0] + (int64_t)j * p.ks[1] + (int64_t)hk * p.ks[2]
                  : (const unsigned short*)p.v + (int64_t)bb * p.vs[0] + (int64_t)j * p.vs[1] + (int64_t)hk * p.vs[2];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) opnd[kk] = *(const u32x4_t*)(R + hi * 8 + kk * 16);
  }
  const float c = p.scale_log2;

  f32x16_t acc[CB];  // dV^T (P-wave) or dK^T (dS-wave)
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;

  // first row of tile t (tiles of a query head are walked last first)
  auto tile_q0 = [&](int t) __attribute__((always_inline)) { return (qt0 + nq - 1 - t % nq) * BQ; };
  // Q and dO tiles go global -> LDS by direct-to-LDS loads (rows past s_q re-read
  // row s_q - 1: finite data, and their LSE is +inf, so P = 0).  Wave 0 also
  // loads LSE and delta of the tile's row q0 + lane (row index clamped, no
  // branch) and converts them only when it stores them at the end of the step,
  // so that nothing waits for these loads before the step's products.
  float lr = 0.f, dr = 0.f;
  bool row_in = false;
  // The loads of tile t + 1 are spread over the products of step t: the P-waves
  // load Q between their S products, the dS-waves dO between their dP products
  // (a wave that issues a burst of direct-to-LDS loads stalls until the memory
  // pipeline takes them).  Each role's 256 threads cover a whole tile.
  constexpr int NLD = 256;
  const int ltid = tid & (NLD - 1), lwave = wave & 3;
  const TileOffs<D, NLD> qo(p.qs[1], ltid), oo(p.dos[1], ltid);
  auto load_rows = [&](int t) __attribute__((always_inline)) {  // wave 0: LSE, delta of tile t
    const int hh = hk * p.g + t / nq;
    const int row = tile_q0(t) + lane;
    row_in = row < p.s_q;
    const int64_t ri = ((int64_t)bb * p.h + hh) * p.s_q + min(row, p.s_q - 1);
    lr = p.lse[ri];
    dr = p.delta[ri];
  };
  // part j of tile t: Q (j = 0, 1) or dO (j = 2, 3), half j % 2, into qbuf[qb] / obuf[ob]
  auto load_part = [&](int t, int j, int qb, int ob) __attribute__((always_inline)) {
    const int hh = hk * p.g + t / nq;
    const int r0 = tile_q0(t) + 32 * (j % 2);
    if (j < 2) {
      const unsigned short* Qg = (const unsigned short*)p.q + (int64_t)bb * p.qs[0] + (int64_t)hh * p.qs[2];
      dma_tile<D, NLD>(qo, Qg, p.qs[1], r0, p.s_q, ltid, lwave, qbuf[qb][j % 2]);
    } else {
      const unsigned short* Og = (const unsigned short*)p.dout + (int64_t)bb * p.dos[0] + (int64_t)hh * p.dos[2];
      dma_tile<D, NLD>(oo, Og, p.dos[1], r0, p.s_q, ltid, lwave, obuf[ob][j % 2]);
    }
  };
  auto store_tile = [&](int buf) __attribute__((always_inline)) {
    if (wave == 0) {
      lbuf[buf][lane] = row_in ? lse_log2(lr) : INFINITY;
      dbuf[buf][lane] = row_in ? -dr : 0.f;  // -delta
    }
  };

  // P-wave, tile t (Q in qbuf[qc]; dO, LSE and P in slot ob = t % 2 of obuf,
  // lbuf and xbuf): S of both halves for this lane's key and its 16 rows of each
  // half (row of element r of half hf: q0 + 32*hf + (r/4)*8 + 4*hi + r%4), P into
  // xbuf, then dV^T += dO^T P.
  auto p_step = [&](int t, int qc, int ob, bool more, int qn) __attribute__((always_inline)) {
    const int q0 = tile_q0(t);
    f32x16_t sc[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[hf][r] = 0.f;
    // the two Q halves of tile t + 1 go out after products KK / 2 - 1 and 3 KK / 2 - 1
    lds_pipeline<2 * KK, ATTN_BWD_PF>(
        [&](int i) __attribute__((always_inline)) { return frag_rows<D>(qbuf[qc][i % 2], l32, hi, i / 2); },
        [&](int i, u32x4_t f) __attribute__((always_inline)) {
          sc[i % 2] = Tt::mfma(f, opnd[i / 2], sc[i % 2]);
          if (more && i % KK == KK / 2 - 1) load_part(t + 1, i / KK, qn, 0);
        });
    u32x4_t bop[2][2];  // [half][chunk]: B operand of dV^T += dO^T P
    // causal mask only where the wave's last key is after the diagonal of the
    // tile's first row; wave-uniform
    const bool diag = CAUSAL && k0 + kb * 32 + 31 > q0 + off;
    auto probs = [&](auto MASK) __attribute__((always_inline)) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4_t l4 = *(const f32x4_t*)(&lbuf[ob][32 * hf + r4 * 8 + hi * 4]);
          f32x4_t pr;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            pr[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[hf][4 * r4 + u], c, -l4[u]));
            if (decltype(MASK)::value && my_j > q0 + 32 * hf + r4 * 8 + hi * 4 + u + off) pr[u] = 0.f;
          }
          xbuf[ob][hf][kb][r4][lane] = pr;
          bop[hf][r4 / 2][2 * (r4 % 2)] = Tt::pack2(pr[0], pr[1]);
          bop[hf][r4 / 2][2 * (r4 % 2) + 1] = Tt::pack2(pr[2], pr[3]);
        }
    };
    if (diag) probs(IC<1>{});
    else probs(IC<0>{});
    // product i: half i / (2 CB), chunk (i / CB) % 2, accumulator i % CB
    lds_pipeline<4 * CB, ATTN_BWD_PF>(
        [&](int i) __attribute__((always_inline)) {
          return frag_cols<D>(obuf[ob][i / (2 * CB)], lane, hi, i % CB, (i / CB) % 2);
        },
        [&](int i, u32x4_t f) __attribute__((always_inline)) {
          acc[i % CB] = Tt::mfma(f, bop[i / (2 * CB)][(i / CB) % 2], acc[i % CB]);
        });
  };
  // dS-wave: dP - delta of a tile (dO and -delta in slot ob of obuf and dbuf), the
  // accumulators starting from -delta of their rows
  auto d_products = [&](int t, int ob, f32x16_t (&dpm)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4_t d4 = *(const f32x4_t*)(&dbuf[ob][32 * hf + r4 * 8 + hi * 4]);
#pragma unroll
        for (int u = 0; u < 4; ++u) dpm[hf][4 * r4 + u] = d4[u];
      }
    // the two dO halves of tile t + 1 go out after products KK / 2 - 1 and 3 KK / 2 - 1
    const bool more = t + 1 < T;
    lds_pipeline<2 * KK, ATTN_BWD_PF>(
        [&](int i) __attribute__((always_inline)) { return frag_rows<D>(obuf[ob][i % 2], l32, hi, i / 2); },
        [&](int i, u32x4_t f) __attribute__((always_inline)) {
          dpm[i % 2] = Tt::mfma(f, opnd[i / 2], dpm[i % 2]);
          if (more && i % KK == KK / 2 - 1) load_part(t + 1, 2 + i / KK, 0, ob ^ 1);
        });
  };
  // dS-wave: dS = P (dP - delta) of a tile (P in xbuf[xb], Q in qbuf[qc]), then
  // dK^T += Q^T dS
  auto d_finish = [&](int qc, int xb, const f32x16_t (&dpm)[2]) __attribute__((always_inline)) {
    u32x4_t bop[2][2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4_t pr = xbuf[xb][hf][kb][r4][lane];
        bop[hf][r4 / 2][2 * (r4 % 2)] = Tt::pack2(pr[0] * dpm[hf][4 * r4], pr[1] * dpm[hf][4 * r4 + 1]);
        bop[hf][r4 / 2][2 * (r4 % 2) + 1] = Tt::pack2(pr[2] * dpm[hf][4 * r4 + 2], pr[3] * dpm[hf][4 * r4 + 3]);
      }
    lds_pipeline<4 * CB, ATTN_BWD_PF>(
        [&](int i) __attribute__((always_inline)) {
          return frag_cols<D>(qbuf[qc][i / (2 * CB)], lane, hi, i % CB, (i / CB) % 2);
        },
        [&](int i, u32x4_t f) __attribute__((always_inline)) {
          acc[i % CB] = Tt::mfma(f, bop[i / (2 * CB)][(i / CB) % 2], acc[i % CB]);
        });
  };

  if (T > 0) {
    if (wave == 0) load_rows(0);
#pragma unroll
    for (int j = 0; j < 2; ++j) load_part(0, 2 * role + j, 0, 0);
    store_tile(0);
  }
  // K or V and the first tile land here, on every path (see the dQ kernel).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Step t: the step's work, during which tile t + 1 is loaded (Q into the
  // buffer that held tile t - 2, dO into the one that held t - 1: both finished
  // before the barrier ending step t - 1) and wave 0 stores LSE and delta of
  // tile t + 1; after the barrier tile t + 1 is in LDS.  Both roles pass the same
  // T barriers.  The steps are unrolled over the period of the buffer rings (3
  // Q buffers, 2 of the rest), so that every LDS address is a per-lane register
  // plus an immediate offset.
  if (role == 0) {
    for (int t0 = 0; t0 < T; t0 += 6)
      static_for<0, 6>([&](auto R) __attribute__((always_inline)) {
        constexpr int r = decltype(R)::value, qc = r % 3, ob = r % 2;
        const int t = t0 + r;
        if (t < T) {
          const bool more = t + 1 < T;
          if (more && wave == 0) load_rows(t + 1);
          p_step(t, qc, ob, more, (r + 1) % 3);
          if (more) store_tile(ob ^ 1);
          __builtin_amdgcn_s_waitcnt(0);  // the direct-to-LDS loads of tile t + 1 have landed
          __syncthreads();
        }
      });
  } else {
    f32x16_t dpm[2];  // dP - delta of the last tile formed, carried across the barrier
    for (int t0 = 0; t0 < T; t0 += 6)
      static_for<0, 6>([&](auto R) __attribute__((always_inline)) {
        constexpr int r = decltype(R)::value, ob = r % 2;
        const int t = t0 + r;
        if (t < T) {
          if (t > 0) d_finish((r + 2) % 3, ob ^ 1, dpm);  // tile t - 1
          // nothing of the next products moves above this point: their
          // accumulators reuse the registers of the finished tile's
          __builtin_amdgcn_sched_barrier(0);
          d_products(t, ob, dpm);
          __builtin_amdgcn_s_waitcnt(0);
          __syncthreads();
        }
      });
    if (T > 0) d_finish((T - 1) % 3, (T - 1) & 1, dpm);
  }

  if (key_ok) {
    unsigned short* dst =
        role == 0 ? (unsigned short*)p.dv + (int64_t)bb * p.dvs[0] + (int64_t)my_j * p.dvs[1] + (int64_t)hk * p.dvs[2]
                  : (unsigned short*)p.dk + (int64_t)bb * p.dks[0] + (int64_t)my_j * p.dks[1] + (int64_t)hk * p.dks[2];
    store_cols<T_, D, CB>(dst, acc, hi, role == 0 ? 1.f : p.scale);
  }
}

// ---------------------------------------------------------------------------
// Launchers: the dQ kernel (which also writes delta), then the dK/dV kernel
// (which reads it), in order on one stream.

template <int T_, int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdParams& p, hipStream_t st) {
  // d = 128: 8 waves (256 rows) share each K/V tile (measured 3-6% faster on the
  // 16k causal backward than 4); smaller head dims keep 4 (8 measured 2% slower at d = 16)
  constexpr int NWQ = D == 128 ? ATTN_BWD_DQ_NW : (D <= 32 ? ATTN_BWD_SMALL_NW : 4);
  const int64_t g_dq = (int64_t)p.b * p.h * ((p.s_q + NWQ * 32 - 1) / (NWQ * 32));
  hipLaunchKernelGGL((bwd_dq_kernel<T_, D, CAUSAL, NWQ>), dim3((unsigned)g_dq), dim3(NWQ * 64), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t g_kv = (int64_t)p.b * (p.h / p.g) * ((p.s_k + 127) / 128);
  // d = 128: paired waves (a single wave would need both operand and both
  // accumulator sets, more than 256 registers); d <= 64: single-wave form
  if constexpr (D == 128) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<T_, D, CAUSAL>), dim3((unsigned)g_kv), dim3(512), 0, st, p);
  } else {
    constexpr int NWK = D <= 32 ? ATTN_BWD_SMALL_NW : 4;
    const int64_t g1 = (int64_t)p.b * (p.h / p.g) * ((p.s_k + NWK * 32 - 1) / (NWK * 32));
    hipLaunchKernelGGL((bwd_dkdv1_kernel<T_, D, CAUSAL, NWK>), dim3((unsigned)g1), dim3(NWK * 64), 0, st, p);
  }
  return hipGetLastError();
}

template <int T_, bool CAUSAL>
static hipError_t launch_bwd_c(const BwdParams& p, hipStream_t st) {
  switch (p.d) {
    case 16: return launch_bwd_t<T_, 16, CAUSAL>(p, st);
    case 32: return launch_bwd_t<T_, 32, CAUSAL>(p, st);
    case 64: return launch_bwd_t<T_, 64, CAUSAL>(p, st);
    default: return launch_bwd_t<T_, 128, CAUSAL>(p, st);
  }
}

// Static delta buffer of attn_bwd_noalloc (for callers that cannot allocate):
// one copy per device, held until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, once per device with that device current, and only that
// address is handed to the kernels.
static __device__ __align__(256) float scratch[kBwdScratchFloats];

hipError_t bwd_scratch(float** out) {
  static std::mutex mu;
  static float* addr[64] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(ptr);
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_bwd(const BwdParams& p, int dtype, bool causal, hipStream_t st) {
  if (dtype == kBF16) return causal ? launch_bwd_c<kBF16, true>(p, st) : launch_bwd_c<kBF16, false>(p, st);
  return causal ? launch_bwd_c<kFP16, true>(p, st) : launch_bwd_c<kFP16, false>(p, st);
}

}  // namespace attn
