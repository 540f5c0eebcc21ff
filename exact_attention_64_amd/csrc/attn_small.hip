// Fused forward for small heads (d = 16, 32) over short sequences (s_q, s_k <=
// 256) on gfx950 (MI355X): persistent work-groups that stream (batch, head)
// items through two LDS buffers.
//
// At these sizes an item (one head of one batch entry: Q, K and V of at most
// 256 rows of 32 or 64 bytes) is a few KB and its arithmetic is a few
// microseconds of one wave, so a work-group per item spends most of its life
// waiting for its first loads.  Here a work-group loops over a sequence of items
// (as many work-groups as fit on the chip at once) and loads its next item
// into the second buffer with direct-to-LDS loads while it computes the
// current one from the first: one barrier per item, and the memory latency is
// paid once per work-group instead of once per item.
//
// Per item, wave w owns query rows 32w .. 32w + 31 and each lane one row (the
// layout of S^T = K Q^T on the 32x32x16 product, as in the backward's dQ
// kernel).  The whole key range of the item is in LDS, so the softmax of
// "LLM Lab Notes 07: Why FlashAttention Is Fast" (section 2) is taken exactly
// in two passes over the key tiles: the row maximum of the scores, then
// P = exp2((s - max) * scale * log2 e), the row sum and O^T += V^T P^T.  The
// second pass forms S^T again instead of keeping it in registers: the matrix
// core has time to spare at these head dims, and the registers saved keep more
// waves resident.  O = O / sum, LSE = max + ln(sum).  (fp16 at d = 16 takes one
// pass against tile 0's maximum first and the two passes only where a row sum
// shows a later score far above it.)
#include <mutex>

#include "attn_common.h"
#include "attn_internal.h"
#include "attn_tile.h"

namespace attn {

template <int T_, int D, bool CAUSAL, int NT>
__global__ __launch_bounds__(512) void small_kernel(const FwdParams p, int n_items) {
  using Tt = Ty<T_>;
  constexpr int KK = D / 16, NCH = D / 8, TB = BTile<D>::BYTES;
  constexpr int LPT = TB / 1024;  // 1 KB wave loads per 32-row tile (1 at d = 16, 2 at d = 32)
  extern __shared__ __attribute__((aligned(16))) char smem[];

  // NT key tiles (s_k > 32 (NT - 1)); one 32-row query block per wave
  const int nqb = blockDim.x / 64;
  const int slots = nqb + 2 * NT;  // 32-row tiles per item buffer: Q blocks, K tiles, V tiles
  // fp16 at D = 16: NT tiles of ones after the two item buffers (see `vsrc`
  // below), 128 bytes further on than a tile boundary so that the half-waves
  // reading ones and those reading V in one transposed read use different banks.
  // (bf16 keeps 8 bits of P: its row sum is taken from P before the rounding,
  // which keeps the log-sum-exp within 1e-3 when a few keys dominate.)
  constexpr bool ONES_ROWS = D == 16 && T_ == kFP16;
  char* const ones_lds = smem + 2 * slots * TB + 128;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int off = p.s_k - p.s_q;
  // c = |scale| * log2 e (1 at scale 0); a negative scale is folded into Q by
  // flipping its sign bits, a zero scale by zeroing it (then every score is 0)
  const float c = p.scale_log2;
  const unsigned qneg = p.neg_q ? 0x80008000u : 0u;
  const unsigned qkeep = p.zero_q ? 0u : 0xffffffffu;

  // Loads.  Wave load u of a tile fills its 16-byte slots 64 u + lane: row
  // (64 u + lane) / NCH of the tile, physical chunk lane % NCH, which receives
  // the logical chunk the swizzle maps there.  A lane's element offset from the
  // tile's first row is fixed per tensor and computed once; rows at or past the
  // end (the last tile only) re-read the last row (finite data: masked keys still
  // meet V in the product).
  int orow[LPT], ocol[LPT];
#pragma unroll
  for (int u = 0; u < LPT; ++u) {
    orow[u] = (64 * u + lane) / NCH;
    ocol[u] = ((lane % NCH) ^ BTile<D>::sw(orow[u])) * 8;
  }
  int64_t qo[LPT], ko[LPT], vo[LPT];
#pragma unroll
  for (int u = 0; u < LPT; ++u) {
    qo[u] = (int64_t)orow[u] * p.qs[1] + ocol[u];
    ko[u] = (int64_t)orow[u] * p.ks[1] + ocol[u];
    vo[u] = (int64_t)orow[u] * p.vs[1] + ocol[u];
  }
  auto tile = [&](const unsigned short* G, int64_t rs, const int64_t (&o)[LPT], int row0, int n, char* dst)
      __attribute__((always_inline)) {
    if (row0 + 32 <= n) {  // wave-uniform
#pragma unroll
      for (int u = 0; u < LPT; ++u) lds_dma16<false>(G + (int64_t)row0 * rs + o[u], dst + u * 1024);
    } else {
#pragma unroll
      for (int u = 0; u < LPT; ++u)
        lds_dma16<false>(G + (int64_t)min(row0 + orow[u], n - 1) * rs + ocol[u], dst + u * 1024);
    }
  };
  // wave w loads its own Q block and K, V tiles w, w + nqb, ...
  auto load_item = [&](int item, int buf) __attribute__((always_inline)) {
    const int bb = item / p.h, hh = item - bb * p.h, hk = hh / p.g;
    char* base = smem + buf * slots * TB;
    const unsigned short* Qg = (const unsigned short*)p.q + (int64_t)bb * p.qs[0] + (int64_t)hh * p.qs[2];
    const unsigned short* Kg = (const unsigned short*)p.k + (int64_t)bb * p.ks[0] + (int64_t)hk * p.ks[2];
    const unsigned short* Vg = (const unsigned short*)p.v + (int64_t)bb * p.vs[0] + (int64_t)hk * p.vs[2];
    tile(Qg, p.qs[1], qo, 32 * wave, p.s_q, base + wave * TB);
    for (int j = wave; j < NT; j += nqb) {
      tile(Kg, p.ks[1], ko, 32 * j, p.s_k, base + (nqb + j) * TB);
      tile(Vg, p.vs[1], vo, 32 * j, p.s_k, base + (nqb + NT + j) * TB);
    }
  };

  // This wave's rows of item `item` from buffer buf.
  auto compute = [&](int item, int buf) __attribute__((always_inline)) {
    const int bb = item / p.h, hh = item - bb * p.h;
    const char* base = smem + buf * slots * TB;
    const char* kt0 = base + nqb * TB;
    const char* vt0 = base + (nqb + NT) * TB;
    // At d = 16 rows 16..31 of the P V product's A operand (V^T) would repeat
    // rows 0..15; with ONES_ROWS the half-waves that supply them read tiles of
    // ones instead, so those accumulator rows come out as the row sum of the
    // rounded P.
    const char* vsrc = ONES_ROWS && (lane & 16) ? ones_lds : vt0;
    const int i = 32 * wave + l32;  // this lane's row
    u32x4_t qf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qf[kk] = frag_rows<D>(base + wave * TB, l32, hi, kk);
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[kk][e] = (qf[kk][e] & qkeep) ^ qneg;
    }
    // S^T of key tile j; element r is key 32 j + (r/4)*8 + 4 hi + r%4.  Formed
    // once per pass: the matrix core has time to spare, registers do not.
    auto scores = [&](int j) __attribute__((always_inline)) {
      f32x16_t sj;
      if (!CAUSAL && j == NT - 1) {
        // without the causal mask only the last key tile can hold keys past s_k
        // (as s_k > 32 (NT - 1)); its product starts from -inf there instead of 0
#pragma unroll
        for (int r = 0; r < 16; ++r) sj[r] = 32 * j + (r / 4) * 8 + 4 * hi + (r % 4) < p.s_k ? 0.f : -INFINITY;
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) sj[r] = 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) sj = Tt::mfma(frag_rows<D>(kt0 + j * TB, l32, hi, kk), qf[kk], sj);
      return sj;
    };
    // tiles the wave's rows can see: all, or (causal) up to its last row's
    // diagonal; with the causal mask, masks where a tile runs past s_k or past
    // the diagonal of the wave's first row (all wave-uniform)
    int nk = p.s_k;
    if (CAUSAL) nk = min(nk, 32 * wave + 31 + off + 1);
    auto live = [&](int j) __attribute__((always_inline)) { return !CAUSAL || 32 * j < nk; };
    auto edge = [&](int j) __attribute__((always_inline)) {
      return CAUSAL && (32 * j + 31 > 32 * wave + off || 32 * j + 32 > p.s_k);
    };
    auto visible = [&](int j, int r) __attribute__((always_inline)) {
      const int key = 32 * j + (r / 4) * 8 + 4 * hi + (r % 4);
      return key < p.s_k && (!CAUSAL || key <= i + off);
    };
    float m, mc, l;
    f32x16_t acc[1];
    if constexpr (ONES_ROWS) {
      // fp16 at d = 16: one pass against a reference from tile 0 (any reference
      // gives the same quotient, section 3.3: a common factor of O and the sum
      // cancels), the two-pass form as fallback.  A row that sees any key sees key
      // 0 (causal visibility is a prefix), so a row whose reference is -inf sees
      // nothing.  Against tile 0's maximum every P of a row is at most its sum l
      // (the largest at least 1): l <= 2^20 keeps every rounded P finite.
      // Otherwise (or l NaN) the wave takes the row maximum over all tiles,
      // against which every P is at most 1, and repeats the pass.
      auto tile_max = [&](int j, const f32x16_t& sj, float mm) __attribute__((always_inline)) {
        if (edge(j)) {
#pragma unroll
          for (int r = 0; r < 16; ++r) mm = fmaxf(mm, visible(j, r) ? sj[r] : -INFINITY);
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) mm = fmaxf(mm, sj[r]);
        }
        return mm;
      };
      // P = exp2(s c - mc), 0 where masked, rounded to fp16, O^T += V^T P^T; the
      // row sum of the rounded P comes from the ones rows.  S0: tile 0's scores
      // are already formed, in s0.
      auto pass = [&](auto S0, float mc_, const f32x16_t& s0) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[0][r] = 0.f;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          if (!live(j)) continue;
          const bool eg = edge(j);
          const f32x16_t sj = decltype(S0)::value && j == 0 ? s0 : scores(j);
          u32x4_t pb[2];
#pragma unroll
          for (int t16 = 0; t16 < 2; ++t16)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float x[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const int r = 8 * t16 + 2 * e + u;
                x[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(sj[r], c, -mc_));
                if (eg && !visible(j, r)) x[u] = 0.f;
              }
              pb[t16][e] = Tt::pack2(x[0], x[1]);
            }
#pragma unroll
          for (int t16 = 0; t16 < 2; ++t16)
            acc[0] = Tt::mfma(frag_cols<D>(vsrc + j * TB, lane, hi, 0, t16), pb[t16], acc[0]);
          // the next tile's V^T reads stay after this tile's products (registers)
          __builtin_amdgcn_sched_barrier(0);
        }
        return acc[0][8];
      };
      f32x16_t s0;
      m = -INFINITY;
      if (live(0)) {
        s0 = scores(0);
        m = pair_max(tile_max(0, s0, m));
      }
      mc = m == -INFINITY ? 0.f : m * c;
      l = pass(IC<1>{}, mc, s0);
      if (__builtin_amdgcn_ballot_w64(!(l <= 0x1p20f)) != 0) {
#pragma unroll
        for (int j = 1; j < NT; ++j)
          if (live(j)) m = tile_max(j, scores(j), m);
        m = pair_max(m);
        mc = m == -INFINITY ? 0.f : m * c;
        l = pass(IC<0>{}, mc, s0);
      }
    } else {
      // the row maximum over visible keys (the two half-waves hold the two halves
      // of each tile's keys for the same rows)
      m = -INFINITY;
  #pragma unroll
      for (int j = 0; j < NT; ++j) {
        if (!live(j)) continue;
        const f32x16_t sj = scores(j);
        if (edge(j)) {
  #pragma unroll
          for (int r = 0; r < 16; ++r) m = fmaxf(m, visible(j, r) ? sj[r] : -INFINITY);
        } else {
  #pragma unroll
          for (int r = 0; r < 16; ++r) m = fmaxf(m, sj[r]);
        }
      }
      m = pair_max(m);
      mc = m == -INFINITY ? 0.f : m * c;

      // P (0 where masked), its row sum, O^T += V^T P^T with P rounded to the
      // input type.  fp16: the row sum of the rounded P comes from the matrix core,
      // from the ones rows or else a product with an A operand of ones (fp16 keeps
      // 11 bits of P; bf16 sums P in fp32 on the vector ALU)
      constexpr bool SUM_MFMA = T_ == kFP16 && !ONES_ROWS;
      const u32x4_t ones = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
      f32x16_t sum;
  #pragma unroll
      for (int r = 0; r < 16; ++r) acc[0][r] = sum[r] = 0.f;
      l = 0.f;
  #pragma unroll
      for (int j = 0; j < NT; ++j) {
        if (!live(j)) continue;
        const bool eg = edge(j);
        const f32x16_t sj = scores(j);
        u32x4_t pb[2];
  #pragma unroll
        for (int t16 = 0; t16 < 2; ++t16)
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            float x[2];
  #pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int r = 8 * t16 + 2 * e + u;
              x[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(sj[r], c, -mc));
              if (eg && !visible(j, r)) x[u] = 0.f;
              if (T_ != kFP16) l += x[u];
            }
            pb[t16][e] = Tt::pack2(x[0], x[1]);
          }
  #pragma unroll
        for (int t16 = 0; t16 < 2; ++t16) {
          acc[0] = Tt::mfma(frag_cols<D>(vsrc + j * TB, lane, hi, 0, t16), pb[t16], acc[0]);
          if (SUM_MFMA) sum = Tt::mfma(ones, pb[t16], sum);
        }
        // the next tile's V^T reads stay after this tile's products (registers)
        __builtin_amdgcn_sched_barrier(0);
      }
      l = ONES_ROWS ? acc[0][8] : (SUM_MFMA ? sum[0] : pair_sum(l));
    }

    if (i < p.s_q) {
      const bool any = l > 0.f;
      unsigned short* dst = (unsigned short*)p.o + (int64_t)bb * p.os[0] + (int64_t)i * p.os[1] +
                            (int64_t)hh * p.os[2];
      store_cols<T_, D, 1>(dst, acc, hi, any ? __builtin_amdgcn_rcpf(l) : 0.f);
      if (p.lse && hi == 0)
        p.lse[((int64_t)bb * p.h + hh) * p.s_q + i] = any ? (mc + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
    }
  };

  // Items in head-major order, one contiguous range per XCD (work-group g runs on
  // XCD g % 8), the XCD's work-groups interleaved over it: at d <= 32 a row of
  // K or V is 32 or 64 bytes, so neighbouring heads share cache lines, and they
  // are worked on at the same time through the same L2.
  const int xcd = blockIdx.x % 8, m = blockIdx.x / 8;
  const int per = n_items / 8, extra = n_items % 8;
  const int lo = xcd * per + min(xcd, extra), hi_item = lo + per + (xcd < extra ? 1 : 0);
  const int step = (int)(gridDim.x / 8) + (xcd < (int)(gridDim.x % 8) ? 1 : 0);  // work-groups on this XCD
  int item = lo + m;
  if (item < hi_item) load_item(item, 0);
  if constexpr (ONES_ROWS) {
    for (int x = tid; x < NT * TB / 16; x += blockDim.x)
      *(u32x4_t*)(ones_lds + 16 * x) = u32x4_t{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
  }
  // the first item lands here, on every path
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // Iteration k: the loads of the next item go to buffer (k + 1) % 2, last read
  // before the barrier ending iteration k - 1; after this iteration's barrier
  // they have landed.  Every wave of a work-group passes the same barriers (its
  // item sequence is uniform).
  // The item's O stores (and LSE stores) are each wave's last vector memory
  // operations of the iteration, and those complete in issue order: waiting
  // until no more than NST of them are in flight waits for the next item's
  // loads without waiting for this item's stores to reach memory.  Every wave
  // has a valid row (lane 0 of the last wave at least), so it issues them all.
  constexpr int NST = D / 8;  // 8-byte O stores per lane (4 columns each, half of a lane pair's 8)
  for (int k = 0; item < hi_item; ++k, item += step) {
    const int buf = k & 1;
    const int nxt = item + step;
    if (nxt < hi_item) load_item(nxt, buf ^ 1);
    compute(item, buf);
    if (p.lse) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(NST + 1));
    else __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(NST));
    __syncthreads();
  }
}

namespace {

// Work-groups of one launch: as many as are resident at once (the occupancy of
// the instantiation at its block size and LDS, times the compute units), at
// most one per item.  Cached per (device, waves per work-group, key tiles).
template <int T_, int D, bool CAUSAL, int NT>
hipError_t launch_small_nt(const FwdParams& p, hipStream_t st) {
  const int nqb = (p.s_q + 31) / 32;
  const int block = 64 * nqb;
  const size_t lds = (2 * (size_t)(nqb + 2 * NT) + (D == 16 && T_ == kFP16 ? NT : 0)) * BTile<D>::BYTES +
                     (D == 16 && T_ == kFP16 ? 128 : 0);
  static std::mutex mu;
  static int cached[64][9] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int resident;
  {
    std::lock_guard<std::mutex> lk(mu);
    resident = cached[dev][nqb];
    if (resident == 0) {
      int cus = 0, occ = 0;
      e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess) return e;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, small_kernel<T_, D, CAUSAL, NT>, block, lds);
      if (e != hipSuccess) return e;
      resident = cached[dev][nqb] = (occ > 0 ? occ : 1) * (cus > 0 ? cus : 1);
    }
  }
  const int64_t n_items = (int64_t)p.b * p.h;
  const int grid = (int)(n_items < resident ? n_items : resident);
  hipLaunchKernelGGL((small_kernel<T_, D, CAUSAL, NT>), dim3(grid), dim3(block), lds, st, p, (int)n_items);
  return hipGetLastError();
}

template <int T_, int D, bool CAUSAL>
hipError_t launch_small_t(const FwdParams& p, hipStream_t st) {
  switch ((p.s_k + 31) / 32) {
    case 1: return launch_small_nt<T_, D, CAUSAL, 1>(p, st);
    case 2: return launch_small_nt<T_, D, CAUSAL, 2>(p, st);
    case 3: return launch_small_nt<T_, D, CAUSAL, 3>(p, st);
    case 4: return launch_small_nt<T_, D, CAUSAL, 4>(p, st);
    case 5: return launch_small_nt<T_, D, CAUSAL, 5>(p, st);
    case 6: return launch_small_nt<T_, D, CAUSAL, 6>(p, st);
    case 7: return launch_small_nt<T_, D, CAUSAL, 7>(p, st);
    default: return launch_small_nt<T_, D, CAUSAL, 8>(p, st);
  }
}

}  // namespace

hipError_t launch_small(const FwdParams& p, int dtype, bool causal, hipStream_t st) {
  if (dtype == kBF16) {
    if (p.d == 16) return causal ? launch_small_t<kBF16, 16, true>(p, st) : launch_small_t<kBF16, 16, false>(p, st);
    return causal ? launch_small_t<kBF16, 32, true>(p, st) : launch_small_t<kBF16, 32, false>(p, st);
  }
  if (p.d == 16) return causal ? launch_small_t<kFP16, 16, true>(p, st) : launch_small_t<kFP16, 16, false>(p, st);
  return causal ? launch_small_t<kFP16, 32, true>(p, st) : launch_small_t<kFP16, 32, false>(p, st);
}

}  // namespace attn
