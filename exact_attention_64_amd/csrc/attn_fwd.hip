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
// Data flow (one work-group = NW waves of 32 query rows each):
//   Q fragment   : registers, loaded once, in the B-operand layout of the
//                  products: v_mfma_f32_16x16x32_{bf16,f16} at d >= 64 (two
//                  16-row blocks per wave), v_mfma_f32_32x32x16 at d <= 32.
//   K, V tiles   : 32 keys x D, global -> LDS with direct-to-LDS loads into a
//                  ring of four slots per tensor, shared by the NW waves.
//   S^T = K Q^T  : MFMA, so each lane owns query rows (two at d >= 64, 8 of
//                  every 32 keys each; one at d <= 32, 16 keys) and a row
//                  maximum is a reduction over 4 (or 2) lanes.
//   P            : exp2 of the scaled scores minus the row's reference (log2(e)
//                  folded into the scale), rounded to the input type.
//   O^T += V^T P^T : MFMA; V^T fragments come from ds_read_b64_tr_b16.
#include <type_traits>

#include "attn_common.h"

namespace attn {

// ---------------------------------------------------------------------------
// LDS tile layouts.  A tile holds BN rows (keys) of D elements; a row is NCH
// 16-byte chunks.  Chunks are XOR-swizzled per row so that the two read
// patterns below touch all 64 LDS banks without conflicts:
//  K: ds_read_b128, 16 consecutive lanes read one chunk column of 16 rows;
//  V: ds_read_b64_tr_b16, a half-wave reads 32 bytes (d >= 64) or 64 bytes
//     (d <= 32) of each of 8 or 4 rows.
template <int D> struct Swz {
  static constexpr int NCH = D / 8;
  static __device__ __forceinline__ int k(int row) {
    return (row / (16 / NCH)) % NCH;
  }
  static __device__ __forceinline__ int v(int row) {
    if constexpr (D == 128) return 2 * (row % 8);
    else if constexpr (D == 64) return 2 * ((row / 2) % 4);
    else return 0;
  }
};

// ---------------------------------------------------------------------------
// Software-pipelined fused forward (every head dim; NW = 8 waves for d >= 64,
// 4 for d <= 32).
//
// NW waves share each K/V tile; every wave owns 32 query rows, so a wave needs
// at most 256 registers and two waves share each SIMD, one hiding the other's
// LDS and load latency.  The K and V tiles stream global -> LDS with
// direct-to-LDS loads through a ring of NBUF buffers per tensor, NBUF - 1 tiles
// ahead of their use, so a step waits only for loads issued NBUF - 1 steps
// earlier.  Step t:
//   1. issues the loads of K_{t+NBUF} and V_{t+NBUF-2};
//   2. reads the transposed V_{t-1} fragments (ds_read_b64_tr_b16) and issues
//      O += V_{t-1}^T P_{t-1}^T on the matrix core;
//   3. reads the K_{t+1} fragments and issues S_{t+1} = K_{t+1} Q^T, while the
//      vector ALU turns S_t into P_t = exp2(S_t * c - m);
//   4. waits for K_{t+2} and V_t, and passes one barrier.
// Q stays in registers for the whole key loop.
//
// Softmax bookkeeping per row: a reference m, the sum l of exp2(s*c - m) and O
// accumulated against the same m, so O/l is the exact softmax (Lab Notes 07,
// section 3.3: rescaling by the running maximum keeps the result exact).  The
// common step computes P against the current m without taking a maximum at all;
// only when a row has no reference yet, or a lane's partial row sum exceeds PMAX
// (2^15 for fp16, whose P must stay below its largest finite value 65504 once
// rounded; 2^64 for bf16), does a rare step take the tile's row maxima, move m up
// to them, multiply O and l by 2^(m_old - m_new) and recompute the tile.  So every
// rounded P stays finite, m never falls below the running maximum by more than
// log2(PMAX), and no exponent overflows; rows whose scores fall far below m only
// lose terms that are negligible against the row's maximum.

// PACK (query heads sharing a K/V head, few query rows): a work-group covers one
// (batch, K/V head) and its g * s_q query rows, row r being query head
// hk * g + r / s_q at position r % s_q, so every K/V tile serves the whole group.
// NT: K/V tiles are read with the nontemporal bit (few work-groups read each tile).
// One wave-uniform 32-bit read through the scalar data cache (read only).  The
// compiler would issue a block-table read as a vector load (the DMA helper's
// memory clobber keeps it from proving the table unchanged), and waiting for
// that load would mean waiting for every K/V load in flight before it.
__device__ __forceinline__ int sload_i32(const int* ptr) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr));
  return v;
}

// PAGED: K and V are a block cache, (num_blocks, block_size, h_kv, d) with
// strides (block, slot, head); key j of batch entry bb is slot j % block_size of
// block block_table[bb][j / block_size], and the entry has seqlens_k[bb] keys.
// Block ids and key counts come from device memory, which the host cannot check:
// they are clamped to [0, num_blocks) and [0, s_k], so no access leaves the
// cache.  block_size is a power of two >= BN, so a tile touches at most two blocks.
template <int T_, int D, int BN, int NW, int NBUF, bool PACK, bool NT, bool PAGED, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(D >= 64 ? 2 : 4, D >= 64 ? 2 : 4)))
void fwdp_kernel(const FwdParams p) {
  using Tt = Ty<T_>;
  static_assert(BN == 32, "one 32-key tile per step");
  // M16 (d >= 64): 16x16x32 products.  A wave's 32 query rows are RB = 2 blocks
  // of 16 (lane l owns rows l % 16 and 16 + l % 16), a key tile NB = 2 blocks of
  // 16 for S^T, KK products of 32 head columns each, O^T in CB = d / 16 blocks
  // of 16 head columns, and one P operand of all 32 keys per row block.  Per
  // flop these products move a fifth less accumulator and operand data through
  // the registers than 32x32x16 ones, and under the package power limit the
  // register-only softmax step ran 8% faster on them (2.15 against 1.92 GHz).
  // Otherwise (d <= 32) 32x32x16 products, one 32-row block, 16 keys per lane;
  // CB: 32-row blocks of O^T (at d = 16 one block, whose upper 16 rows repeat
  // the lower ones and are not stored).
  // Packed groups on 4 waves (at most 64 rows: a few query heads of a few
  // positions) take one 16-row block per wave (WR = 16 rows), so that the rows
  // spread over more waves and SIMDs instead of filling one wave.
  constexpr bool M16 = D >= 64;
  constexpr int RB = M16 ? (PACK && NW == 4 ? 1 : 2) : 1, NB = M16 ? 2 : 1;
  constexpr int WR = M16 ? 16 * RB : 32;  // query rows per wave
  constexpr int NCH = D / 8, KK = M16 ? D / 32 : D / 16, BM = NW * WR;
  constexpr int CB = M16 ? D / 16 : (D >= 32 ? D / 32 : 1);
  constexpr int NT16 = M16 ? 1 : BN / 16;
  using Acc = typename std::conditional<M16, f32x4_t, f32x16_t>::type;
  constexpr int NE = M16 ? 4 : 16;  // accumulator elements per lane
  constexpr int TILE = BN * D * 2;
  constexpr int NLOAD = TILE / 1024;            // 1 KB wave loads per tensor per tile
  constexpr int NLW = NLOAD < NW ? NLOAD : NW;  // waves that take part in the loads
  constexpr int WL = NLOAD / NLW;               // loads per taking-part wave
  static_assert(NLOAD >= 1 && NLOAD % NLW == 0, "a tile must split into 1 KB wave loads");
  static_assert(NBUF == 2 || NBUF == 4 || NBUF == 8, "the step loop is unrolled by NBUF");
  constexpr int P = NBUF - 1;                   // prefetch distance in tiles
  constexpr int PAIR = 2 * WL;                  // loads of one (K, V) pair per wave
  // Bound on a lane's partial row sum of P before a rebase is forced.  Every P of
  // the lane is at most that sum, and P is rounded to the input type before the
  // P V product: fp16's largest finite value is 65504, so its bound is 2^15; bf16
  // has fp32's exponent range, where 2^64 keeps rebases rare.
  constexpr float PMAX = T_ == kFP16 ? 0x1p15f : 0x1p64f;

  // QLDS: Q reaches its registers through LDS, loaded by the same direct-to-LDS
  // loads as K and V and issued just before them, so that one memory round trip
  // brings Q and the first tiles (loaded into registers, Q would be waited for
  // on its own first).  Used where the extra NW * TILE bytes of LDS cost no
  // occupancy: the 8-wave launch (one work-group per compute unit) and d = 16.
  constexpr bool QLDS = NW == 8 || D == 16;
  static_assert(!QLDS || WR == 32, "Q through LDS fills 32 rows per wave");
  __shared__ __attribute__((aligned(1024))) char kbuf[NBUF][TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf[NBUF][TILE];
  __shared__ __attribute__((aligned(1024))) char qbuf[QLDS ? NW : 1][QLDS ? TILE : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int l16 = lane & 15, g4 = lane >> 4;  // M16 lane position: column, 4-lane group

  const int nh = PACK ? p.h / p.g : p.h;  // heads indexed by the grid
  // Work items.  Causal: query tiles in order of decreasing work across all heads
  // (tile-major: the heaviest tiles of every head first).  Otherwise head-major
  // (head, split, query tile) and spread over the XCDs so that the tiles of a
  // head, and neighbouring heads, share one L2 (at d = 16 a key row is 32 bytes
  // and neighbouring heads share cache lines: b = 512, s = 150, h = 16 measured
  // 140 -> 111 us; the tile-major order measured ~1% faster on the 16k causal
  // prefill).
  int rem, qt_rev;
  if constexpr (CAUSAL) {
    const int per_qt = p.b * nh * p.n_splits;
    qt_rev = blockIdx.x / per_qt;
    rem = blockIdx.x - qt_rev * per_qt;
  } else {
    const int item = xcd_item(blockIdx.x, p.n_qt * p.b * nh * p.n_splits);
    rem = item / p.n_qt;
    qt_rev = item - rem * p.n_qt;
  }
  const int bh = rem / p.n_splits;
  const int split = rem - bh * p.n_splits;
  const int qt = CAUSAL ? (p.n_qt - 1 - qt_rev) : qt_rev;
  const int bb = bh / nh;
  const int hg = bh - bb * nh;
  const int hk = PACK ? hg : hg / p.g;   // K/V head of the work-group
  const int q0 = qt * BM;
  // keys of this batch entry: its own count when paged, else s_k
  const int s_k = PAGED ? min(max(p.seqlens_k[bb], 0), p.s_k) : p.s_k;
  const int off = s_k - p.s_q;
  // This lane's rows: query head my_h, position my_i (both uniform per
  // work-group unless packed).  Position bounds for the masking decisions are
  // exact for one head's contiguous rows and conservative when packed.
  int my_i[RB], my_h[RB];
  bool row_ok[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int rw = q0 + wave * WR + (M16 ? 16 * rb + l16 : l32);
    row_ok[rb] = rw < (PACK ? p.g * p.s_q : p.s_q);
    my_i[rb] = PACK ? rw % p.s_q : rw;
    my_h[rb] = PACK ? hk * p.g + rw / p.s_q : hg;
  }
  const int pos_wg_lo = PACK ? 0 : q0;
  const int pos_wg_hi = PACK ? p.s_q - 1 : q0 + BM - 1;
  const int pos_wave_lo = PACK ? 0 : q0 + wave * WR;
  // A wave with no rows at all only loads its share of each tile: packed
  // work-groups often have such waves (6 heads x 1 row fill one wave of eight),
  // and so does the last query tile of a head whose length is not a multiple of
  // the work-group's rows (s_q = 150 over 128-row work-groups: three of four).
  const bool live = q0 + wave * WR < (PACK ? p.g * p.s_q : p.s_q);

  int k_lo = 0, k_hi = s_k;
  if (SPLIT) {
    k_lo = (int)(((int64_t)split * s_k) / p.n_splits);
    k_hi = (int)(((int64_t)(split + 1) * s_k) / p.n_splits);
  }
  if (CAUSAL) k_hi = min(k_hi, pos_wg_hi + off + 1);
  const int T = k_hi > k_lo ? (k_hi - k_lo + BN - 1) / BN : 0;

  const unsigned short* __restrict__ Kg = (const unsigned short*)p.k + (PAGED ? 0 : (int64_t)bb * p.ks[0]) + (int64_t)hk * p.ks[2];
  const unsigned short* __restrict__ Vg = (const unsigned short*)p.v + (PAGED ? 0 : (int64_t)bb * p.vs[0]) + (int64_t)hk * p.vs[2];
  const int* __restrict__ tbl = PAGED ? p.block_table + (int64_t)bb * p.bt_stride : nullptr;
  const int64_t ksr = p.ks[1], vsr = p.vs[1];

  // Q fragments (B operand of S^T = K Q^T): this lane's row of block rb, d =
  // 32 kk + 8 g4 (M16) or 16 kk + 8 hi.  Rows past the end are zero; a negative
  // scale is folded in by negating Q, a zero scale by zeroing it.
  u32x4_t qf[RB][KK];
  auto fix_q = [&](u32x4_t x, int rb) {
    if (!row_ok[rb] || p.zero_q) return u32x4_t{0u, 0u, 0u, 0u};
    return p.neg_q ? (x ^ 0x80008000u) : x;
  };
  auto q_chunk = [&](int kk) { return M16 ? 4 * kk + g4 : hi + 2 * kk; };  // 16-byte chunk of d
  if constexpr (QLDS) {
    // This wave's 32 rows into qbuf[wave], chunks swizzled as in a K tile; rows
    // past the end re-read the last row (zeroed once in registers).
    const int rows = PACK ? p.g * p.s_q : p.s_q;
#pragma unroll
    for (int i = 0; i < TILE / 1024; ++i) {
      const int slot = i * 64 + lane;
      const int row = slot / NCH, pc = slot % NCH;
      const int rw_ = min(q0 + wave * 32 + row, rows - 1);
      const int pos = PACK ? rw_ % p.s_q : rw_;
      const int head = PACK ? hk * p.g + rw_ / p.s_q : hg;
      const unsigned short* src = (const unsigned short*)p.q + (int64_t)bb * p.qs[0] + (int64_t)pos * p.qs[1] +
                                  (int64_t)head * p.qs[2] + (pc ^ Swz<D>::k(row)) * 8;
      lds_dma16<false>((const void*)src, qbuf[wave] + i * 1024);
    }
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const unsigned short* __restrict__ Qr = (const unsigned short*)p.q + (int64_t)bb * p.qs[0] +
                                              (int64_t)my_i[rb] * p.qs[1] + (int64_t)my_h[rb] * p.qs[2];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        u32x4_t x = {0u, 0u, 0u, 0u};
        if (row_ok[rb] && !p.zero_q) x = *(const u32x4_t*)(Qr + 8 * q_chunk(kk));
        qf[rb][kk] = fix_q(x, rb);
      }
    }
    // Wait for Q here, on every path: a load still pending where the key loop
    // starts would make the compiler wait for all loads (vmcnt(0)) inside it.
    __builtin_amdgcn_s_waitcnt(0);
  }

  Acc o[CB][RB];
  float m[RB], l[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < NE; ++r) o[cb][rb][r] = 0.f;
  }
  const float c = p.scale_log2;

  // ---- global -> LDS staging, 16 bytes per lane, by the first NLW waves.
  // Slot (row, physical chunk) receives the logical chunk the swizzle maps
  // there.  Per-lane row offsets are computed once; a tile adds its key
  // offset.  Rows past the range end (only in the last tile) re-read the last
  // valid key: finite data, masked scores.
  const bool loader = wave < NLW;
  int64_t koff[WL], voff[WL];
#pragma unroll
  for (int i = 0; i < WL; ++i) {
    const int slot = (wave * WL + i) * 64 + lane;
    const int row = (slot / NCH) % BN, pc = slot % NCH;
    koff[i] = (int64_t)row * ksr + (pc ^ Swz<D>::k(row)) * 8;
    voff[i] = (int64_t)row * vsr + (pc ^ Swz<D>::v(row)) * 8;
  }
  // `full`: the caller knows the tile lies inside the key range.
  auto stage = [&](const unsigned short* __restrict__ G, int64_t gs, const int64_t (&goff)[WL],
                   bool isv, int tile, char* buf, bool full) {
    if (NLW < NW && !loader) return;
    const int k0 = k_lo + tile * BN;
    if constexpr (PAGED) {
      // Block of the tile's first key and, when the tile runs past that block
      // and keys there are in range, the next one (both wave-uniform loads).
      const int bsz = 1 << p.lbs;
      const int kb0 = k0 >> p.lbs;
      const int r0 = k0 - (kb0 << p.lbs);
      const int blk0 = min(max(sload_i32(tbl + kb0), 0), p.num_blocks - 1);
      int blk1 = blk0;
      if (r0 + BN > bsz && ((kb0 + 1) << p.lbs) < k_hi) blk1 = min(max(sload_i32(tbl + kb0 + 1), 0), p.num_blocks - 1);
      const int64_t bstride = isv ? p.vs[0] : p.ks[0];
      const bool whole = full || k0 + BN <= k_hi;
#pragma unroll
      for (int i = 0; i < WL; ++i) {
        const int slot = (wave * WL + i) * 64 + lane;
        const int row = slot / NCH, pc = slot % NCH;
        const int key = whole ? k0 + row : min(k0 + row, k_hi - 1);  // past the end: re-read the last key
        const int rel = key - (kb0 << p.lbs);                         // [0, 2 * block_size)
        const bool second = rel >= bsz;
        const int64_t blk = second ? blk1 : blk0;
        const int ch = pc ^ (isv ? Swz<D>::v(row) : Swz<D>::k(row));
        lds_dma16<NT>((const void*)(G + blk * bstride + (int64_t)(second ? rel - bsz : rel) * gs + ch * 8),
                      buf + (wave * WL + i) * 1024);
      }
      return;
    }
    if (full || k0 + BN <= k_hi) {
      const unsigned short* __restrict__ Gt = G + (int64_t)k0 * gs;
#pragma unroll
      for (int i = 0; i < WL; ++i)
        lds_dma16<NT>((const void*)(Gt + goff[i]), buf + (wave * WL + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < WL; ++i) {
        const int slot = (wave * WL + i) * 64 + lane;
        const int row = slot / NCH, pc = slot % NCH;
        const int key = min(k0 + row, k_hi - 1);
        const int ch = pc ^ (isv ? Swz<D>::v(row) : Swz<D>::k(row));
        lds_dma16<NT>((const void*)(G + (int64_t)key * gs + ch * 8), buf + (wave * WL + i) * 1024);
      }
    }
  };

  // LDS -> registers: K fragments (A operand of S^T = K Q^T) of one tile, and
  // V^T fragments (A operand of O^T += V^T P^T).
  // M16: K block kb, product kk: key row 16 kb + l16, d chunk 4 kk + g4.  V^T
  // block cb: head column 16 cb + l16 and the 8 keys of K slots 8 g4 .. 8 g4 + 7
  // of the P V product, keys 4 g4 + {0..3} and 16 + 4 g4 + {0..3} (the keys the
  // lane's S^T elements hold, so the P operand is the exponentiated S^T packed
  // in place); each half from one transposed read in which lane x of a 16-lane
  // group fetches 4 columns of key row x / 4 and receives column x of the 4 rows.
  // Otherwise: K row l32, d chunk hi + 2 kk; V^T head column cb*32 + l32, keys
  // 16*t16 + 4*hi + {0..3} and 16*t16 + 8 + 4*hi + {0..3}.
  const int g16 = (lane >> 4) & 1, xr = (lane & 15) >> 2, xq = lane & 3;
  auto read_k = [&](const char* kb, u32x4_t (&kf)[KK][NB]) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int row = M16 ? 16 * b + l16 : l32;
        const int ch = M16 ? 4 * kk + g4 : hi + 2 * kk;
        kf[kk][b] = *(const u32x4_t*)(kb + row * D * 2 + 16 * (ch ^ Swz<D>::k(row)));
      }
  };
  auto read_v = [&](const char* vb, u32x4_t (&vf)[CB][NT16]) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int col = M16 ? 16 * cb + 4 * xq : (cb * 32 + g16 * 16 + xq * 4) & (D >= 32 ? 0x7fffffff : D - 1);
      const int ch = col / 8, half = (col % 8) / 4;
#pragma unroll
      for (int t16 = 0; t16 < NT16; ++t16)
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
          const int row = M16 ? 16 * rd + 4 * g4 + xr : 16 * t16 + 8 * rd + 4 * hi + xr;
          const char* a = vb + row * D * 2 + 16 * (ch ^ Swz<D>::v(row)) + 8 * half;
          const u32x2_t yy = bitcast<u32x2_t>(__builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4_t*)(a)));
          vf[cb][t16][2 * rd] = yy[0];
          vf[cb][t16][2 * rd + 1] = yy[1];
        }
    }
  };
  // (M16: the four S^T blocks' products interleaved, so that no product waits
  // on the one just issued)
  auto qk = [&](const u32x4_t (&kf)[KK][NB], Acc (&s)[NB][RB]) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < NE; ++r) s[b][rb][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          if constexpr (M16) s[b][rb] = Tt::mfma16(kf[kk][b], qf[rb][kk], s[b][rb]);
          else s[b][rb] = Tt::mfma(kf[kk][b], qf[rb][kk], s[b][rb]);
        }
  };
  auto pv = [&](const u32x4_t (&vf)[CB][NT16], const u32x4_t (&pf)[RB][NT16]) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int t16 = 0; t16 < NT16; ++t16) {
          if constexpr (M16) o[cb][rb] = Tt::mfma16(vf[cb][t16], pf[rb][t16], o[cb][rb]);
          else o[cb][rb] = Tt::mfma(vf[cb][t16], pf[rb][t16], o[cb][rb]);
        }
  };
  // key of S^T element r of key block b
  auto key_of = [&](int k0, int b, int r) {
    return M16 ? k0 + 16 * b + 4 * g4 + r : k0 + (r / 4) * 8 + hi * 4 + (r % 4);
  };

  // -inf for keys past the range end and (causal) keys after a row's diagonal.
  auto mask_tile = [&](Acc (&s)[NB][RB], int k0) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < NE; ++r) {
          const int key = key_of(k0, b, r);
          if (key >= k_hi || (CAUSAL && key > my_i[rb] + off)) s[b][rb][r] = -INFINITY;
        }
  };

  // P = exp2(S * c - m) rounded to the input type; ls: this lane's sums per row.
  // M16: the P operand of row block rb holds the lane's 8 keys in K-slot order,
  // key block 0's four then key block 1's.
  auto expo = [&](const Acc (&s)[NB][RB], u32x4_t (&pf)[RB][NT16], float (&ls)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float m_use = m[rb] == -INFINITY ? 0.f : m[rb];
      float lsum = 0.f;
#pragma unroll
      for (int t16 = 0; t16 < NT16; ++t16) {
        u32x4_t x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sa = M16 ? s[e / 2][rb][2 * (e % 2)] : s[0][rb][8 * t16 + 2 * e];
          const float sb = M16 ? s[e / 2][rb][2 * (e % 2) + 1] : s[0][rb][8 * t16 + 2 * e + 1];
          const float a = __builtin_amdgcn_exp2f(__builtin_fmaf(sa, c, -m_use));
          const float b = __builtin_amdgcn_exp2f(__builtin_fmaf(sb, c, -m_use));
          x[e] = Tt::pack2(a, b);
          lsum += a + b;
        }
        pf[rb][t16] = x;
      }
      ls[rb] = lsum;
    }
  };

  // the maximum over the lanes that hold one row (4 at M16, 2 otherwise)
  auto row_max = [&](float x) {
    if constexpr (M16) x = fmaxf(x, __shfl_xor(x, 16));
    return pair_max(x);
  };
  auto row_sum = [&](float x) {
    if constexpr (M16) x += __shfl_xor(x, 16);
    return pair_sum(x);
  };

  // Rare step: move each row's reference to max(m, tile max), rescale O and l,
  // and recompute this tile's P against the new reference.
  auto rebase = [&](const Acc (&s)[NB][RB], u32x4_t (&pf)[RB][NT16], float (&ls)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < NE; ++r) mx = fmaxf(mx, s[b][rb][r]);
      const float m_new = fmaxf(m[rb], row_max(mx) * c);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[rb] - m_new);
      m[rb] = m_new;
      l[rb] *= alpha;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < NE; ++r) o[cb][rb][r] *= alpha;
    }
    expo(s, pf, ls);
  };

  Acc sA[NB][RB], sB[NB][RB];
  u32x4_t pA[RB][NT16], pB[RB][NT16];

  // Prologue: K_0 and K_1, then the (K_{j+2}, V_j) pairs j < NBUF - 2, so that
  // step t always finds the pairs up to t + NBUF - 3 issued.  `full`: every
  // prologue load was issued, so the wait counts below are exact (otherwise
  // the prologue waits for everything).
  const bool full = T > P;
  if (T > 0) {
    stage(Kg, ksr, koff, false, 0, kbuf[0], false);
    if (T > 1) stage(Kg, ksr, koff, false, 1, kbuf[1], false);
#pragma unroll
    for (int j = 0; j + 2 <= P; ++j) {
      if (j + 2 < T) stage(Kg, ksr, koff, false, j + 2, kbuf[(j + 2) % NBUF], false);
      if (j < T) stage(Vg, vsr, voff, true, j, vbuf[j % NBUF], false);
    }
  }
  asm volatile("" ::: "memory");
  // K_0 (and Q, issued before it) landed; a wave that loads no K/V has only Q
  // in flight.
  if (full && (NLW == NW || loader)) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0(WL + (P - 1) * PAIR));
  else __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if constexpr (QLDS) {
    const char* qb = qbuf[wave];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = M16 ? 16 * rb + l16 : l32;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qf[rb][kk] = fix_q(*(const u32x4_t*)(qb + row * D * 2 + 16 * (q_chunk(kk) ^ Swz<D>::k(row))), rb);
    }
  }
  if (T > 0 && live) {
    u32x4_t kf[KK][NB];
    read_k(kbuf[0], kf);
    qk(kf, sA);
  }
  // K_1 has landed, and every wave has read K_0 (step 0 loads over it).
  asm volatile("" ::: "memory");
  if (full) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0((P - 1) * PAIR));
  else __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // Step t.  Buffers: K_t's slot takes K_{t+NBUF}; K_{t+1} is read; V_{t-2}'s
  // slot takes V_{t+NBUF-2}; V_{t-1} is read.  At the end, the loads of
  // K_{t+2} and V_t (issued NBUF - 1 steps earlier) must have landed; later
  // pairs may still be in flight.
  // HC: what the caller knows at compile time.  0: nothing; 1: tile t + 1
  // exists, which keeps the product/softmax block of the step free of branches
  // (the scheduler cannot interleave across them); 2: interior step, where
  // moreover both loads exist and lie inside the key range and tile t needs no
  // mask, so the whole step is straight-line code apart from the rare rebase.
  auto iter = [&](auto HC, int t, bool first, Acc (&s)[NB][RB], Acc (&s_next)[NB][RB],
                  u32x4_t (&p_prev)[RB][NT16], u32x4_t (&p_cur)[RB][NT16],
                  char* kb_w, const char* kb_r, char* vb_w, const char* vb_r) __attribute__((always_inline)) {
    constexpr int hc = decltype(HC)::value;
    if (hc == 2 || t + P + 1 < T) stage(Kg, ksr, koff, false, t + P + 1, kb_w, hc == 2);
    if (hc == 2 || t + P - 1 < T) stage(Vg, vsr, voff, true, t + P - 1, vb_w, hc == 2);
    const bool has_next = hc >= 1 || t + 1 < T;
    const int k0 = k_lo + t * BN;
    const bool need_mask = hc != 2 && ((k0 + BN > k_hi) || (CAUSAL && k0 + BN - 1 > pos_wave_lo + off));
    if (live) {
      u32x4_t kf[KK][NB], vf[CB][NT16];
      if (!first) read_v(vb_r, vf);
      if (need_mask) mask_tile(s, k0);
      __builtin_amdgcn_sched_barrier(0);
      float ls[RB];
      if (!first) pv(vf, p_prev);
      // M16: the P V products issue as one group, ahead of the K reads,
      // exponentials and score products that the scheduler interleaves (left
      // free to mix all of them it took 4-5% more cycles on the 16k causal
      // prefill)
      if constexpr (M16) __builtin_amdgcn_sched_barrier(0);
      if (has_next) read_k(kb_r, kf);
      expo(s, p_cur, ls);
      if (has_next) qk(kf, s_next);
      __builtin_amdgcn_sched_barrier(0);
      bool bad = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) bad = bad || m[rb] == -INFINITY || !(ls[rb] <= PMAX);
      if (__builtin_amdgcn_ballot_w64(bad) != 0) rebase(s, p_cur, ls);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) l[rb] += ls[rb];
    }
    asm volatile("" ::: "memory");
    if (hc == 2 || t + P + 1 < T) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0((P - 1) * PAIR));
    else __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // One step with r = t % NBUF known at compile time, so every LDS address is
  // an immediate offset.
  auto step = [&](auto HC, int t, auto RC) __attribute__((always_inline)) {
    constexpr int r = decltype(RC)::value;
    char* kb_w = kbuf[r];
    const char* kb_r = kbuf[(r + 1) % NBUF];
    char* vb_w = vbuf[(r + NBUF - 2) % NBUF];
    const char* vb_r = vbuf[(r + NBUF - 1) % NBUF];
    if constexpr (r % 2 == 1) iter(HC, t, false, sB, sA, pA, pB, kb_w, kb_r, vb_w, vb_r);
    else iter(HC, t, false, sA, sB, pB, pA, kb_w, kb_r, vb_w, vb_r);
  };
  // The key loop.  Interior steps first: t + P + 1 < n_full (every load a full
  // tile) and, when causal, tile t entirely at or below the diagonal of the
  // work-group's first row.  Then steps that all have a next tile, then the
  // last (up to NBUF) steps, which know nothing at compile time.
  const int n_full = (k_hi - k_lo) / BN;
  int t_clean = n_full - P - 1;
  if (CAUSAL) t_clean = min(t_clean, (pos_wg_lo + off - k_lo + 1) / BN);
  if (T > 0) iter(IC<0>{}, 0, true, sA, sB, pB, pA, kbuf[0], kbuf[1], vbuf[NBUF - 2], vbuf[NBUF - 1]);
  int t = 1;
  for (; t + NBUF <= t_clean; t += NBUF)
    static_for<0, NBUF>([&](auto I) __attribute__((always_inline)) {
      step(IC<2>{}, t + I.value, IC<(I.value + 1) % NBUF>{});
    });
  for (; t + NBUF < T; t += NBUF)
    static_for<0, NBUF>([&](auto I) __attribute__((always_inline)) {
      step(IC<1>{}, t + I.value, IC<(I.value + 1) % NBUF>{});
    });
  static_for<0, NBUF>([&](auto I) __attribute__((always_inline)) {
    if (t + I.value < T) step(IC<0>{}, t + I.value, IC<(I.value + 1) % NBUF>{});
  });
  if (T >= 1 && live) {
    u32x4_t vf[CB][NT16];
    read_v(vbuf[(T - 1) % NBUF], vf);
    if ((T - 1) & 1) pv(vf, pB);
    else pv(vf, pA);
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2.  Element r of O^T
  // block cb is head column 16 cb + 4 g4 + r (M16) or cb*32 + (r/4)*8 + 4 hi +
  // r%4.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int i = my_i[rb], hh = my_h[rb];
    const float lt = row_sum(l[rb]);
    const bool has = lt > 0.f;
    const float inv = has ? 1.f / lt : 0.f;
    const float lse = has ? (m[rb] + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
    const bool lse_lane = M16 ? g4 == 0 : hi == 0;
    if (row_ok[rb]) {
      if (SPLIT) {
        const int64_t rowi = (((int64_t)split * p.b + bb) * p.h + hh) * p.s_q + i;
        float* op = p.o_part + rowi * D;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int r4 = 0; r4 < NE / 4; ++r4) {
            const int col = M16 ? 16 * cb + 4 * g4 : cb * 32 + r4 * 8 + hi * 4;
            if (col >= D) continue;
            f32x4_t x = {o[cb][rb][4 * r4] * inv, o[cb][rb][4 * r4 + 1] * inv,
                         o[cb][rb][4 * r4 + 2] * inv, o[cb][rb][4 * r4 + 3] * inv};
            *(f32x4_t*)(op + col) = x;
          }
        if (lse_lane) p.lse_part[rowi] = lse;
      } else {
        unsigned short* op = (unsigned short*)p.o + (int64_t)bb * p.os[0] + (int64_t)i * p.os[1] + (int64_t)hh * p.os[2];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int r4 = 0; r4 < NE / 4; ++r4) {
            const int col = M16 ? 16 * cb + 4 * g4 : cb * 32 + r4 * 8 + hi * 4;
            if (col >= D) continue;
            u32x2_t x = {Tt::pack2(o[cb][rb][4 * r4] * inv, o[cb][rb][4 * r4 + 1] * inv),
                         Tt::pack2(o[cb][rb][4 * r4 + 2] * inv, o[cb][rb][4 * r4 + 3] * inv)};
            *(u32x2_t*)(op + col) = x;
          }
        if (lse_lane && p.lse) p.lse[((int64_t)bb * p.h + hh) * p.s_q + i] = lse;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers

// Ring depth: 8 slots at d = 16 (1 KB tiles: a short head's whole K/V is in
// flight after the prologue, and 8 work-groups still share a compute unit), else
// kPrefillNBUF.
template <int T_, int D, int NW, bool PACK, bool NT, bool PAGED, bool CAUSAL, bool SPLIT>
static hipError_t launch_fwdp_t(const FwdParams& p, hipStream_t st) {
  constexpr int BM = NW * (D >= 64 && PACK && NW == 4 ? 16 : 32);  // the kernel's rows per work-group
  constexpr int NBUF = D == 16 ? 8 : kPrefillNBUF;
  FwdParams q = p;
  const int64_t rows = PACK ? (int64_t)p.g * p.s_q : p.s_q;
  const int64_t nh = PACK ? p.h / p.g : p.h;
  q.n_qt = (int)((rows + BM - 1) / BM);
  const int64_t grid = (int64_t)q.n_qt * p.b * nh * p.n_splits;
  hipLaunchKernelGGL((fwdp_kernel<T_, D, kPrefillBN, NW, NBUF, PACK, NT, PAGED, CAUSAL, SPLIT>),
                     dim3((unsigned)grid), dim3(NW * 64), 0, st, q);
  return hipGetLastError();
}

// Launch shape at d >= 64 from the rows one head (or packed group) brings:
//  - at most 128 (decode and short chunks; 64 for packed groups, whose 4-wave
//    work-groups take 16 rows per wave): 4 waves, so two work-groups share a
//    compute unit and twice as many key streams are in flight (measured 1.66x
//    faster than 8 waves on b = 8, h = 48, s_q = 4, 4096 keys);
//  - otherwise 8 waves (256 rows) sharing each K/V tile.
// K/V loads are nontemporal when at most kStreamQTiles work-groups read each
// tile.  (At d <= 32 a key row is 32 or 64 bytes and shares its cache lines with
// the neighbouring heads that other work-groups read; reading those
// nontemporally measured slower, b = 512, s = 150, h = 16, d = 16.)
template <int T_, int D, bool PACK, bool PAGED, bool CAUSAL, bool SPLIT>
static hipError_t launch_fwd_rows(const FwdParams& p, hipStream_t st) {
  const int64_t rows = PACK ? (int64_t)p.g * p.s_q : p.s_q;
  if (rows <= 4 * (PACK ? 16 : 32)) return launch_fwdp_t<T_, D, 4, PACK, true, PAGED, CAUSAL, SPLIT>(p, st);
  if ((rows + kPrefillNW * 32 - 1) / (kPrefillNW * 32) <= kStreamQTiles)
    return launch_fwdp_t<T_, D, kPrefillNW, PACK, true, PAGED, CAUSAL, SPLIT>(p, st);
  return launch_fwdp_t<T_, D, kPrefillNW, PACK, false, PAGED, CAUSAL, SPLIT>(p, st);
}

template <int T_, int D, bool PAGED, bool CAUSAL, bool SPLIT>
static hipError_t launch_fwd_d(const FwdParams& p, hipStream_t st) {
  // d <= 32: ATTN_SMALL_D_NW = 2 waves (64 query rows) per work-group and up to
  // four waves per SIMD (a work-group there has few steps and its start-up
  // latency dominates, so more, smaller work-groups win: b = 512, s = 150,
  // h = 16 measured 103.6 us with 2 waves, 110 with 4, 115 with 1); the paged
  // cache is served at d >= 64 only (the host rejects the rest)
  if constexpr (D >= 64) {
    return fwd_packed(p.g, p.s_q, D) ? launch_fwd_rows<T_, D, true, PAGED, CAUSAL, SPLIT>(p, st)
                                     : launch_fwd_rows<T_, D, false, PAGED, CAUSAL, SPLIT>(p, st);
  } else if constexpr (!PAGED) {
    return launch_fwdp_t<T_, D, ATTN_SMALL_D_NW, false, false, false, CAUSAL, SPLIT>(p, st);
  } else {
    return hipErrorInvalidValue;
  }
}

template <int T_, bool CAUSAL, bool PAGED, bool SPLIT>
static hipError_t launch_fwd_c(const FwdParams& p, hipStream_t st) {
  switch (p.d) {
    case 16: return launch_fwd_d<T_, 16, PAGED, CAUSAL, SPLIT>(p, st);
    case 32: return launch_fwd_d<T_, 32, PAGED, CAUSAL, SPLIT>(p, st);
    case 64: return launch_fwd_d<T_, 64, PAGED, CAUSAL, SPLIT>(p, st);
    default: return launch_fwd_d<T_, 128, PAGED, CAUSAL, SPLIT>(p, st);
  }
}

template <int T_, bool CAUSAL, bool PAGED>
hipError_t launch_prefill_tc(const FwdParams& p, bool split, hipStream_t st) {
  return split ? launch_fwd_c<T_, CAUSAL, PAGED, true>(p, st) : launch_fwd_c<T_, CAUSAL, PAGED, false>(p, st);
}

// The library compiles this file once per (input type, causal, paged) triple,
// selected by ATTN_FWD_DTYPE, ATTN_FWD_CAUSAL and ATTN_FWD_PAGED, so the kernel
// sets build in parallel; launch_prefill (attn_internal.h) picks among them.
#if !defined(ATTN_FWD_DTYPE) || !defined(ATTN_FWD_CAUSAL) || !defined(ATTN_FWD_PAGED)
#error "compile with -DATTN_FWD_DTYPE=<0|1> -DATTN_FWD_CAUSAL=<0|1> -DATTN_FWD_PAGED=<0|1>"
#endif
template hipError_t launch_prefill_tc<ATTN_FWD_DTYPE, (ATTN_FWD_CAUSAL != 0), (ATTN_FWD_PAGED != 0)>(
    const FwdParams&, bool, hipStream_t);

}  // namespace attn
