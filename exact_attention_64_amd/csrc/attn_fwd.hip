// Fused exact attention forward (prefill) kernel for gfx950 (MI355X).
//
// The fused kernel follows "LLM Lab Notes 07: Why FlashAttention Is Fast":
// the score matrix is produced one tile at a time and never stored (section 3.1,
// tiling), K/V tiles pass through on-chip LDS and only O and LSE are written back
// (section 3.2, IO-awareness), and the running row maximum rescales the partial
// output whenever it grows, which keeps the result exact (section 3.3, online
// softmax).  The split-KV variant and the combine kernel implement the two stages
// of flash-decoding discussed in flash-attention issue #1248 ("where is flash
// decoding second stage (reduce) code?").
//
// Data flow of the fused kernel (one work-group = NW waves, 64*RB... rows each):
//   Q fragment   : registers, loaded once, in the B-operand layout of
//                  v_mfma_f32_32x32x16_{bf16,f16}.
//   K, V tiles   : BN keys x D, global -> registers -> LDS, double-buffered.
//   S^T = K Q^T  : MFMA, so each lane owns one query row and 16 of every 32 keys
//                  and the row maximum needs one permlane32 swap.
//   P            : exp2 of the scaled scores minus the running maximum (log2(e)
//                  folded into the scale), rounded to the input type.
//   O^T += V^T P^T : MFMA; V^T fragments come from ds_read_b64_tr_b16.
#include "attn_common.h"

namespace attn {

// ---------------------------------------------------------------------------
// LDS tile layouts.  A tile holds BN rows (keys) of D elements; a row is NCH
// 16-byte chunks.  Chunks are XOR-swizzled per row so that the two read
// patterns below touch all 64 LDS banks without conflicts:
//  K: ds_read_b128, 16 consecutive lanes read one chunk column of 16 rows;
//  V: ds_read_b64_tr_b16, a half-wave reads 64 bytes of each of 4 rows.
template <int D> struct Swz {
  static constexpr int NCH = D / 8;
  static __device__ __forceinline__ int k(int row) {
    return (row / (16 / NCH)) % NCH;
  }
  static __device__ __forceinline__ int v(int row) {
    return NCH == 16 ? 4 * (row % 4) : (NCH == 8 ? 4 * ((row / 2) % 2) : 0);
  }
};

// ---------------------------------------------------------------------------
// Fused forward kernel.
//   T_ : kBF16 / kFP16.  D: head dim.  NW: waves per work-group.
//   RB : 32-row blocks per wave.  BN: keys per tile.  SPLIT: write fp32
//   per-split partials (flash-decoding first stage) instead of O / LSE.
template <int T_, int D, int NW, int RB, int BN, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(NW * 64, 1) void fwd_kernel(const FwdParams p) {
  using Tt = Ty<T_>;
  constexpr int NCH = D / 8;               // 16-byte chunks per row
  constexpr int KK = D / 16;               // k-steps of the S^T MFMA
  constexpr int NB = BN / 32;              // 32-key blocks per tile
  constexpr int CB = D >= 32 ? D / 32 : 1; // 32-row (d) blocks of O^T
  constexpr int BM = NW * RB * 32;         // query rows per work-group
  constexpr int NT = NW * 64;
  constexpr int TILE_BYTES = BN * D * 2;
  constexpr int CPT = (BN * NCH + NT - 1) / NT;  // staged chunks per thread per tensor

  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;  // which half of the wave

  // ---- work-group -> (q tile, batch*head, split); heaviest causal tiles first
  const int per_qt = p.b * p.h * p.n_splits;
  const int qt_rev = blockIdx.x / per_qt;
  const int rem = blockIdx.x - qt_rev * per_qt;
  const int bh = rem / p.n_splits;
  const int split = rem - bh * p.n_splits;
  const int qt = CAUSAL ? (p.n_qt - 1 - qt_rev) : qt_rev;
  const int bb = bh / p.h;
  const int hh = bh - bb * p.h;
  const int q0 = qt * BM;
  const int off = p.s_k - p.s_q;  // bottom-right causal offset

  int k_lo = 0, k_hi = p.s_k;
  if (SPLIT) {
    k_lo = (int)(((int64_t)split * p.s_k) / p.n_splits);
    k_hi = (int)(((int64_t)(split + 1) * p.s_k) / p.n_splits);
  }
  if (CAUSAL) k_hi = min(k_hi, q0 + BM + off);
  const int ntiles = k_hi > k_lo ? (k_hi - k_lo + BN - 1) / BN : 0;

  const unsigned short* __restrict__ Qg = (const unsigned short*)p.q + (int64_t)bb * p.qs[0] + (int64_t)hh * p.qs[2];
  const unsigned short* __restrict__ Kg = (const unsigned short*)p.k + (int64_t)bb * p.ks[0] + (int64_t)hh * p.ks[2];
  const unsigned short* __restrict__ Vg = (const unsigned short*)p.v + (int64_t)bb * p.vs[0] + (int64_t)hh * p.vs[2];

  const int qw0 = q0 + wave * RB * 32;  // first query row of this wave

  // ---- Q fragments (B operand of S^T = K Q^T): row qw0 + rb*32 + l32, d = hi*8 + 16*kk
  u32x4_t qf[RB][KK];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int i = qw0 + rb * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (i < p.s_q && !p.zero_q) {
        x = *(const u32x4_t*)(Qg + (int64_t)i * p.qs[1] + hi * 8 + kk * 16);
        if (p.neg_q) x ^= 0x80008000u;
      }
      qf[rb][kk] = x;
    }
  }

  f32x16_t o[CB][RB];
  float m[RB], l[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[cb][rb][r] = 0.f;
  }
  const float c = p.scale_log2;

  // ---- staging: chunk f of a tile -> row f / NCH, chunk f % NCH
  u32x4_t stk[CPT], stv[CPT];
  auto stage_load = [&](int t) {
    const int k0 = k_lo + t * BN;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int f = tid + i * NT;
      u32x4_t xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
      if (f < BN * NCH) {
        const int row = f / NCH, ch = f % NCH;
        const int key = k0 + row;
        if (key < k_hi) {
          xk = *(const u32x4_t*)(Kg + (int64_t)key * p.ks[1] + ch * 8);
          xv = *(const u32x4_t*)(Vg + (int64_t)key * p.vs[1] + ch * 8);
        }
      }
      stk[i] = xk;
      stv[i] = xv;
    }
  };
  auto stage_store = [&](int buf) {
    char* kb = smem + buf * 2 * TILE_BYTES;
    char* vb = kb + TILE_BYTES;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int f = tid + i * NT;
      if (f < BN * NCH) {
        const int row = f / NCH, ch = f % NCH;
        *(u32x4_t*)(kb + row * D * 2 + 16 * (ch ^ Swz<D>::k(row))) = stk[i];
        *(u32x4_t*)(vb + row * D * 2 + 16 * (ch ^ Swz<D>::v(row))) = stv[i];
      }
    }
  };

  const bool wave_live = qw0 < p.s_q;
  const int wave_last_key = qw0 + RB * 32 - 1 + off;  // causal visibility of the wave's last row

  if (ntiles > 0) {
    stage_load(0);
    stage_store(0);
    __syncthreads();
  }
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) stage_load(t + 1);
    const int k0 = k_lo + t * BN;
    const bool skip = !wave_live || (CAUSAL && k0 > wave_last_key);
    if (!skip) {
      const char* kb = smem + (t & 1) * 2 * TILE_BYTES;
      const char* vb = kb + TILE_BYTES;
      // S^T = K Q^T
      f32x16_t s[NB][RB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[nb][rb][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int row = nb * 32 + l32;
          const int ch = hi + 2 * kk;
          const u32x4_t kf = *(const u32x4_t*)(kb + row * D * 2 + 16 * (ch ^ Swz<D>::k(row)));
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) s[nb][rb] = Tt::mfma(kf, qf[rb][kk], s[nb][rb]);
        }
      }
      // masks: keys past the range end, and (causal) keys after the diagonal
      const bool need_mask = (k0 + BN > k_hi) || (CAUSAL && k0 + BN - 1 > qw0 + off);
      if (need_mask) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int i = qw0 + rb * 32 + l32;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + nb * 32 + (r / 4) * 8 + hi * 4 + (r % 4);
              const bool bad = key >= k_hi || (CAUSAL && key > i + off);
              if (bad) s[nb][rb][r] = -INFINITY;
            }
        }
      }
      // online softmax, base 2, log2(e) folded into c
      u32x4_t pf[RB][BN / 16];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float mx = -INFINITY;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[nb][rb][r]);
        mx = pair_max(mx);
        const float m_new = fmaxf(m[rb], mx * c);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m[rb] - m_use);
        float lsum = 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[nb][rb][r], c, -m_use));
            s[nb][rb][r] = pv;
            lsum += pv;
          }
        l[rb] = l[rb] * alpha + lsum;
        m[rb] = m_new;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[cb][rb][r] *= alpha;
#pragma unroll
        for (int t16 = 0; t16 < BN / 16; ++t16) {
          u32x4_t x;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[e] = Tt::pack2(s[t16 / 2][rb][8 * (t16 % 2) + 2 * e], s[t16 / 2][rb][8 * (t16 % 2) + 2 * e + 1]);
          pf[rb][t16] = x;
        }
      }
      // O^T += V^T P^T.  A-operand lane layout: d row cb*32 + l32, keys
      // 16*t16 + 4*hi + {0..3} and 16*t16 + 8 + 4*hi + {0..3}; each half comes
      // from one transposed LDS read in which lane x of a 16-lane group fetches
      // 4 columns of key row (x / 4).
      const int g16 = (lane >> 4) & 1;      // column half within the 32-wide block
      const int xr = (lane & 15) >> 2;      // key row within the group of 4
      const int xq = lane & 3;              // 4-column quad
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        int col = cb * 32 + g16 * 16 + xq * 4;
        if (D < 32) col &= (D - 1);         // D=16: the upper 16 rows of O^T are unused
        const int ch = col / 8, half = (col % 8) / 4;
#pragma unroll
        for (int t16 = 0; t16 < BN / 16; ++t16) {
          u32x4_t vf;
#pragma unroll
          for (int rd = 0; rd < 2; ++rd) {
            const int row = 16 * t16 + 8 * rd + 4 * hi + xr;
            const char* a = vb + row * D * 2 + 16 * (ch ^ Swz<D>::v(row)) + 8 * half;
            const s16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4_t*)(a));
            const u32x2_t yy = bitcast<u32x2_t>(y);
            vf[2 * rd] = yy[0];
            vf[2 * rd + 1] = yy[1];
          }
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) o[cb][rb] = Tt::mfma(vf, pf[rb][t16], o[cb][rb]);
        }
      }
    }
    if (t + 1 < ntiles) stage_store((t + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int i = qw0 + rb * 32 + l32;
    const float lt = pair_sum(l[rb]);
    const bool has = lt > 0.f;
    const float inv = has ? 1.f / lt : 0.f;
    const float lse = has ? (m[rb] + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
    if (i < p.s_q) {
      if (SPLIT) {
        const int64_t rowi = (((int64_t)split * p.b + bb) * p.h + hh) * p.s_q + i;
        float* op = p.o_part + rowi * D;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int col = cb * 32 + r4 * 8 + hi * 4;
            if (col < D) {
              f32x4_t x = {o[cb][rb][4 * r4] * inv, o[cb][rb][4 * r4 + 1] * inv,
                           o[cb][rb][4 * r4 + 2] * inv, o[cb][rb][4 * r4 + 3] * inv};
              *(f32x4_t*)(op + col) = x;
            }
          }
        if (hi == 0) p.lse_part[rowi] = lse;
      } else {
        unsigned short* op = (unsigned short*)p.o + (int64_t)bb * p.os[0] + (int64_t)i * p.os[1] + (int64_t)hh * p.os[2];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int col = cb * 32 + r4 * 8 + hi * 4;
            if (col < D) {
              u32x2_t x = {Tt::pack2(o[cb][rb][4 * r4] * inv, o[cb][rb][4 * r4 + 1] * inv),
                           Tt::pack2(o[cb][rb][4 * r4 + 2] * inv, o[cb][rb][4 * r4 + 3] * inv)};
              *(u32x2_t*)(op + col) = x;
            }
          }
        if (hi == 0 && p.lse) p.lse[((int64_t)bb * p.h + hh) * p.s_q + i] = lse;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Software-pipelined fused forward for d in {64, 128} (the long-sequence path).
//
// Four waves, each owning 64 query rows (two 32-row MFMA blocks, so every K/V
// fragment read from LDS feeds two MFMAs).  One wave per SIMD: the matrix core
// and the vector ALU are kept busy by the same wave, so iteration t issues three
// independent streams of work that the scheduler can interleave:
//   MFMA  S_{t+1} = K_{t+1} Q^T          (scores of the next tile)
//   VALU  P_t = exp2(S_t * c - m)        (softmax of the current tile)
//   MFMA  O  += V_{t-1}^T P_{t-1}^T      (output of the previous tile)
// K_{t+2} and V_t stream global -> LDS with direct-to-LDS loads while this runs
// (two buffers each; one barrier per tile).
//
// The output is rescaled lazily: the reference maximum m of a row only moves when
// a tile's maximum exceeds it by more than TAU (log2 units), so P stays below
// 2^TAU and O/l are rescaled on a handful of tiles instead of every tile.  O and l
// always share the same reference, so O/l is the same exact softmax (only the
// rounding differs), as the online-softmax argument of Lab Notes 07 section 3.3
// requires.  When the reference moves it moves to the row maximum itself, so a
// row whose largest score sits in its first visible tile gets weight exactly 1 on
// that key.
template <int T_, int D, int BN, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(256, 1) void fwdp_kernel(const FwdParams p) {
  using Tt = Ty<T_>;
  constexpr int NW = 4, RB = 2;
  constexpr int NCH = D / 8, KK = D / 16, NB = BN / 32, CB = D / 32, BM = NW * RB * 32;
  constexpr int NT16 = BN / 16;
  constexpr int TILE = BN * D * 2;
  constexpr int WLOADS = TILE / (1024 * NW);  // 1 KB wave loads per tensor per wave
  static_assert(WLOADS >= 1 && TILE % (1024 * NW) == 0, "a tile must split into 1 KB wave loads");
  constexpr float TAU = 8.f;

  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];
  char* const kbuf0 = smem;
  char* const kbuf1 = smem + TILE;
  char* const vbuf0 = smem + 2 * TILE;
  char* const vbuf1 = smem + 3 * TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int per_qt = p.b * p.h * p.n_splits;
  const int qt_rev = blockIdx.x / per_qt;
  const int rem = blockIdx.x - qt_rev * per_qt;
  const int bh = rem / p.n_splits;
  const int split = rem - bh * p.n_splits;
  const int qt = CAUSAL ? (p.n_qt - 1 - qt_rev) : qt_rev;
  const int bb = bh / p.h;
  const int hh = bh - bb * p.h;
  const int q0 = qt * BM;
  const int off = p.s_k - p.s_q;

  int k_lo = 0, k_hi = p.s_k;
  if (SPLIT) {
    k_lo = (int)(((int64_t)split * p.s_k) / p.n_splits);
    k_hi = (int)(((int64_t)(split + 1) * p.s_k) / p.n_splits);
  }
  if (CAUSAL) k_hi = min(k_hi, q0 + BM + off);
  const int T = k_hi > k_lo ? (k_hi - k_lo + BN - 1) / BN : 0;

  const unsigned short* __restrict__ Qg = (const unsigned short*)p.q + (int64_t)bb * p.qs[0] + (int64_t)hh * p.qs[2];
  const unsigned short* __restrict__ Kg = (const unsigned short*)p.k + (int64_t)bb * p.ks[0] + (int64_t)hh * p.ks[2];
  const unsigned short* __restrict__ Vg = (const unsigned short*)p.v + (int64_t)bb * p.vs[0] + (int64_t)hh * p.vs[2];
  const int64_t ksr = p.ks[1], vsr = p.vs[1];

  const int qw0 = q0 + wave * RB * 32;
  u32x4_t qf[RB][KK];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int i = qw0 + rb * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (i < p.s_q && !p.zero_q) {
        x = *(const u32x4_t*)(Qg + (int64_t)i * p.qs[1] + hi * 8 + kk * 16);
        if (p.neg_q) x ^= 0x80008000u;
      }
      qf[rb][kk] = x;
    }
  }

  f32x16_t o[CB][RB];
  float m[RB], l[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[cb][rb][r] = 0.f;
  }
  const float c = p.scale_log2;

  // global -> LDS, 16 bytes per lane; slot (row, physical chunk) receives the
  // logical chunk that the swizzle maps there.  Rows past the range end re-read
  // the last valid key (finite data; those scores are masked).
  auto stage = [&](const unsigned short* __restrict__ G, int64_t gs, int tile, char* buf, bool isv) {
    const int k0 = k_lo + tile * BN;
#pragma unroll
    for (int i = 0; i < WLOADS; ++i) {
      const int blk = wave * WLOADS + i;
      const int slot = blk * 64 + lane;
      const int row = slot / NCH, pc = slot % NCH;
      const int ch = pc ^ (isv ? Swz<D>::v(row) : Swz<D>::k(row));
      const int key = min(k0 + row, k_hi - 1);
      __builtin_amdgcn_global_load_lds((const void*)(G + (int64_t)key * gs + ch * 8),
                                       (LDS_AS void*)(buf + blk * 1024), 16, 0, 0);
    }
  };

  // S^T (+)= K Q^T over the d-steps [kk0, kk1); kk0 == 0 starts from zero.
  auto qk = [&](const char* kb, f32x16_t (&s)[NB][RB], int kk0, int kk1) {
    if (kk0 == 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[nb][rb][r] = 0.f;
    }
#pragma unroll
    for (int kk = kk0; kk < kk1; ++kk) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int row = nb * 32 + l32;
        const int ch = hi + 2 * kk;
        const u32x4_t kf = *(const u32x4_t*)(kb + row * D * 2 + 16 * (ch ^ Swz<D>::k(row)));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[nb][rb] = Tt::mfma(kf, qf[rb][kk], s[nb][rb]);
      }
    }
  };

  const int g16 = (lane >> 4) & 1, xr = (lane & 15) >> 2, xq = lane & 3;
  auto pv = [&](const char* vb, const u32x4_t (&pf)[RB][NT16]) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int col = cb * 32 + g16 * 16 + xq * 4;
      const int ch = col / 8, half = (col % 8) / 4;
#pragma unroll
      for (int t16 = 0; t16 < NT16; ++t16) {
        u32x4_t vf;
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
          const int row = 16 * t16 + 8 * rd + 4 * hi + xr;
          const char* a = vb + row * D * 2 + 16 * (ch ^ Swz<D>::v(row)) + 8 * half;
          const u32x2_t yy = bitcast<u32x2_t>(__builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4_t*)(a)));
          vf[2 * rd] = yy[0];
          vf[2 * rd + 1] = yy[1];
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[cb][rb] = Tt::mfma(vf, pf[rb][t16], o[cb][rb]);
      }
    }
  };

  // -inf for keys past the range end and (causal) keys after a row's diagonal.
  auto mask_tile = [&](f32x16_t (&s)[NB][RB], int k0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int i = qw0 + rb * 32 + l32;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + nb * 32 + (r / 4) * 8 + hi * 4 + (r % 4);
          if (key >= k_hi || (CAUSAL && key > i + off)) s[nb][rb][r] = -INFINITY;
        }
    }
  };

  // Move the reference maximum of every row of the wave to max(m, tile max) and
  // multiply O and l by alpha = 2^(m_old - m_new).  A P tile computed with the
  // old reference and not yet multiplied into O is multiplied by alpha as well
  // (one extra rounding to fp16/bf16 of that tile, on the few tiles where the
  // reference moves).
  auto new_ref = [&](const float (&mt)[RB], float (&alpha)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float m_new = fmaxf(m[rb], mt[rb]);
      alpha[rb] = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[rb] - m_new);
      m[rb] = m_new;
      l[rb] *= alpha[rb];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[cb][rb][r] *= alpha[rb];
    }
  };
  auto scale_p = [&](u32x4_t (&pf)[RB][NT16], const float (&alpha)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int t16 = 0; t16 < NT16; ++t16)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned w = pf[rb][t16][e];
          float a, b;
          Tt::unpack2(w, a, b);
          pf[rb][t16][e] = Tt::pack2(a * alpha[rb], b * alpha[rb]);
        }
  };

  auto expo = [&](const f32x16_t (&s)[NB][RB], u32x4_t (&pf)[RB][NT16]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float m_use = m[rb] == -INFINITY ? 0.f : m[rb];
      float lsum = 0.f;
#pragma unroll
      for (int t16 = 0; t16 < NT16; ++t16) {
        u32x4_t x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r0 = 8 * (t16 % 2) + 2 * e;
          const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t16 / 2][rb][r0], c, -m_use));
          const float b = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t16 / 2][rb][r0 + 1], c, -m_use));
          lsum += a + b;
          x[e] = Tt::pack2(a, b);
        }
        pf[rb][t16] = x;
      }
      l[rb] += lsum;
    }
  };

  f32x16_t sA[NB][RB], sB[NB][RB];
  u32x4_t pA[RB][NT16], pB[RB][NT16];

  if (T > 0) {
    stage(Kg, ksr, 0, kbuf0, false);
    if (T > 1) stage(Kg, ksr, 1, kbuf1, false);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    qk(kbuf0, sA, 0, KK);
  }

  // One tile step, the same straight-line code for every tile: tiles a wave's rows
  // cannot see are masked rather than skipped (the wave would only wait at the
  // barrier otherwise), so apart from the mask on diagonal / range-end tiles and
  // the rare reference move there is no branch, and the MFMA streams (second half
  // of S_{t+1}, O += P_{t-1} V_{t-1}) interleave with the softmax VALU work.
  auto iter = [&](int t, bool first, f32x16_t (&s_cur)[NB][RB], f32x16_t (&s_nxt)[NB][RB],
                  u32x4_t (&p_prev)[RB][NT16], u32x4_t (&p_cur)[RB][NT16],
                  char* kb_free, const char* kb_next, char* vb_free, const char* vb_prev) {
    if (t + 2 < T) stage(Kg, ksr, t + 2, kb_free, false);
    stage(Vg, vsr, t, vb_free, true);
    const int k0 = k_lo + t * BN;
    if ((k0 + BN > k_hi) || (CAUSAL && k0 + BN - 1 > qw0 + off)) mask_tile(s_cur, k0);
    qk(kb_next, s_nxt, 0, KK / 2);
    float mt[RB];
    bool need = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = -INFINITY;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[nb][rb][r]);
      mt[rb] = pair_max(mx) * c;
      need |= mt[rb] > m[rb] + TAU;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      float alpha[RB];
      new_ref(mt, alpha);
      if (!first) scale_p(p_prev, alpha);
    }
    qk(kb_next, s_nxt, KK / 2, KK);
    expo(s_cur, p_cur);
    if (!first) pv(vb_prev, p_prev);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  if (T > 0) iter(0, true, sA, sB, pB, pA, kbuf0, kbuf1, vbuf0, vbuf1);
  int t = 1;
  for (; t + 1 < T; t += 2) {
    iter(t, false, sB, sA, pA, pB, kbuf1, kbuf0, vbuf1, vbuf0);
    iter(t + 1, false, sA, sB, pB, pA, kbuf0, kbuf1, vbuf0, vbuf1);
  }
  if (t < T) iter(t, false, sB, sA, pA, pB, kbuf1, kbuf0, vbuf1, vbuf0);
  if (T >= 1) {
    if ((T - 1) & 1) pv(vbuf1, pB);
    else pv(vbuf0, pA);
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int i = qw0 + rb * 32 + l32;
    const float lt = pair_sum(l[rb]);
    const bool has = lt > 0.f;
    const float inv = has ? 1.f / lt : 0.f;
    const float lse = has ? (m[rb] + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
    if (i < p.s_q) {
      if (SPLIT) {
        const int64_t rowi = (((int64_t)split * p.b + bb) * p.h + hh) * p.s_q + i;
        float* op = p.o_part + rowi * D;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int col = cb * 32 + r4 * 8 + hi * 4;
            f32x4_t x = {o[cb][rb][4 * r4] * inv, o[cb][rb][4 * r4 + 1] * inv,
                         o[cb][rb][4 * r4 + 2] * inv, o[cb][rb][4 * r4 + 3] * inv};
            *(f32x4_t*)(op + col) = x;
          }
        if (hi == 0) p.lse_part[rowi] = lse;
      } else {
        unsigned short* op = (unsigned short*)p.o + (int64_t)bb * p.os[0] + (int64_t)i * p.os[1] + (int64_t)hh * p.os[2];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int col = cb * 32 + r4 * 8 + hi * 4;
            u32x2_t x = {Tt::pack2(o[cb][rb][4 * r4] * inv, o[cb][rb][4 * r4 + 1] * inv),
                         Tt::pack2(o[cb][rb][4 * r4 + 2] * inv, o[cb][rb][4 * r4 + 3] * inv)};
            *(u32x2_t*)(op + col) = x;
          }
        if (hi == 0 && p.lse) p.lse[((int64_t)bb * p.h + hh) * p.s_q + i] = lse;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers

template <int T_, int D, int NW, int RB, int BN, bool CAUSAL, bool SPLIT>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t st) {
  constexpr int BM = NW * RB * 32;
  FwdParams q = p;
  q.n_qt = (p.s_q + BM - 1) / BM;
  const int64_t grid = (int64_t)q.n_qt * p.b * p.h * p.n_splits;
  hipLaunchKernelGGL((fwd_kernel<T_, D, NW, RB, BN, CAUSAL, SPLIT>), dim3((unsigned)grid), dim3(NW * 64), 0, st, q);
  return hipGetLastError();
}

template <int T_, int D, int BN, bool CAUSAL, bool SPLIT>
static hipError_t launch_fwdp_t(const FwdParams& p, hipStream_t st) {
  constexpr int BM = 4 * 2 * 32;
  FwdParams q = p;
  q.n_qt = (p.s_q + BM - 1) / BM;
  const int64_t grid = (int64_t)q.n_qt * p.b * p.h * p.n_splits;
  hipLaunchKernelGGL((fwdp_kernel<T_, D, BN, CAUSAL, SPLIT>), dim3((unsigned)grid), dim3(256), 0, st, q);
  return hipGetLastError();
}

template <int T_, int D, bool CAUSAL, bool SPLIT>
static hipError_t launch_fwd_d(const FwdParams& p, hipStream_t st) {
  if constexpr (D >= 64) return launch_fwdp_t<T_, D, kPrefillBN, CAUSAL, SPLIT>(p, st);
  else return launch_fwd_t<T_, D, 4, 1, 32, CAUSAL, SPLIT>(p, st);
}

template <int T_, bool CAUSAL, bool SPLIT>
static hipError_t launch_fwd_c(const FwdParams& p, hipStream_t st) {
  switch (p.d) {
    case 16: return launch_fwd_d<T_, 16, CAUSAL, SPLIT>(p, st);
    case 32: return launch_fwd_d<T_, 32, CAUSAL, SPLIT>(p, st);
    case 64: return launch_fwd_d<T_, 64, CAUSAL, SPLIT>(p, st);
    default: return launch_fwd_d<T_, 128, CAUSAL, SPLIT>(p, st);
  }
}

template <int T_>
static hipError_t launch_fwd_dt(const FwdParams& p, bool causal, bool split, hipStream_t st) {
  if (causal) return split ? launch_fwd_c<T_, true, true>(p, st) : launch_fwd_c<T_, true, false>(p, st);
  return split ? launch_fwd_c<T_, false, true>(p, st) : launch_fwd_c<T_, false, false>(p, st);
}

hipError_t launch_prefill(const FwdParams& p, int dtype, bool causal, bool split, hipStream_t st) {
  return dtype == kBF16 ? launch_fwd_dt<kBF16>(p, causal, split, st)
                        : launch_fwd_dt<kFP16>(p, causal, split, st);
}

}  // namespace attn
