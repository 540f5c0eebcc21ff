// C-ABI front end: argument validation, the split-count heuristic, per-device
// capability cache and kernel dispatch.  Every check runs on the host before
// any launch; on error nothing is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/attn.h"
#include "attn_internal.h"

static_assert(attn::kBwdScratchFloats == ATTN_BWD_SCRATCH_ROWS, "the scratch size is part of the ABI");

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool strides_ok(const int64_t s[3]) {
  for (int i = 0; i < 3; ++i)
    if (s[i] < 0 || (s[i] % 8) != 0) return false;
  return true;
}

bool headdim_ok(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

attn_status check_shape(int64_t b, int64_t h, int64_t s_q, int64_t s_k) {
  if (b < 1 || h < 1 || s_q < 1 || s_k < 1) return ATTN_E_SHAPE;
  if (s_q > ATTN_MAX_SEQ || s_k > ATTN_MAX_SEQ) return ATTN_E_SHAPE;
  if (b > ATTN_MAX_BH || h > ATTN_MAX_BH || b * h > ATTN_MAX_BH) return ATTN_E_SHAPE;
  return ATTN_OK;
}

// Common checks of attn_args.  need_o: O and its strides are used.
attn_status check_args(const attn_args* a, bool need_o) {
  if (!a) return ATTN_E_NULL;
  if (!a->q || !a->k || !a->v || (need_o && !a->o)) return ATTN_E_NULL;
  if (a->dtype != ATTN_FP16 && a->dtype != ATTN_BF16) return ATTN_E_DTYPE;
  attn_status st = check_shape(a->b, a->h, a->s_q, a->s_k);
  if (st != ATTN_OK) return st;
  if (a->h_kv < 0 || a->h_kv > a->h || (a->h_kv > 0 && a->h % a->h_kv != 0)) return ATTN_E_SHAPE;
  if (!headdim_ok(a->d)) return ATTN_E_HEADDIM;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v)) return ATTN_E_LAYOUT;
  if (!strides_ok(a->q_stride) || !strides_ok(a->k_stride) || !strides_ok(a->v_stride)) return ATTN_E_LAYOUT;
  if (need_o && (!aligned16(a->o) || !strides_ok(a->o_stride))) return ATTN_E_LAYOUT;
  if (need_o && a->lse && !aligned4(a->lse)) return ATTN_E_LAYOUT;
  if (!std::isfinite(a->softmax_scale)) return ATTN_E_SCALE;
  return ATTN_OK;
}

struct DevInfo {
  bool filled = false;
  bool gfx950 = false;
  int cus = 0;
};
std::mutex g_mu;
DevInfo g_dev[64];

attn_status device_info(int dev, DevInfo* out) {
  if (dev < 0 || dev >= 64) return ATTN_E_DEVICE;
  std::lock_guard<std::mutex> lk(g_mu);
  DevInfo& d = g_dev[dev];
  if (!d.filled) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_E_DEVICE;
    d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.filled = true;
  }
  *out = d;
  return ATTN_OK;
}

attn_status current_device_ok() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return ATTN_E_DEVICE;
  }
  DevInfo info;
  attn_status st = device_info(dev, &info);
  if (st != ATTN_OK) return st;
  return info.gfx950 ? ATTN_OK : ATTN_E_DEVICE;
}

void fill_params(const attn_args* a, attn::FwdParams* p) {
  std::memset(p, 0, sizeof(*p));
  p->q = a->q;
  p->k = a->k;
  p->v = a->v;
  p->o = a->o;
  p->lse = a->lse;
  for (int i = 0; i < 3; ++i) {
    p->qs[i] = a->q_stride[i];
    p->ks[i] = a->k_stride[i];
    p->vs[i] = a->v_stride[i];
    p->os[i] = a->o_stride[i];
  }
  p->b = (int)a->b;
  p->h = (int)a->h;
  p->s_q = (int)a->s_q;
  p->s_k = (int)a->s_k;
  p->d = (int)a->d;
  p->n_splits = 1;
  p->g = a->h_kv > 0 ? (int)(a->h / a->h_kv) : 1;
  const float s = a->softmax_scale;
  // The kernels work in base 2 with log2(e) folded into the scale.  A negative
  // scale is applied by negating Q on load; a zero scale by zeroing Q (then every
  // score is exactly 0, as the definition requires).
  p->zero_q = s == 0.f;
  p->neg_q = s < 0.f;
  p->scale_log2 = s == 0.f ? 1.f : std::fabs(s) * 1.4426950408889634f;
}

int64_t group_of(const attn_args* a) { return a->h_kv > 0 ? a->h / a->h_kv : 1; }

// Checks of attn_paged_args (same order as check_args).  need_o: O is written.
attn_status check_paged(const attn_paged_args* a, bool need_o) {
  if (!a) return ATTN_E_NULL;
  if (!a->q || !a->k_cache || !a->v_cache || !a->block_table || !a->seqlens_k || (need_o && !a->o))
    return ATTN_E_NULL;
  if (a->dtype != ATTN_FP16 && a->dtype != ATTN_BF16) return ATTN_E_DTYPE;
  attn_status st = check_shape(a->b, a->h, a->s_q, a->max_seqlen_k);
  if (st != ATTN_OK) return st;
  if (a->h_kv < 0 || a->h_kv > a->h || (a->h_kv > 0 && a->h % a->h_kv != 0)) return ATTN_E_SHAPE;
  const int64_t bsz = a->block_size;
  if (bsz < 32 || bsz > (1 << 20) || (bsz & (bsz - 1)) != 0) return ATTN_E_SHAPE;
  if (a->num_blocks < 1 || a->num_blocks > 0x7fffffff || a->max_blocks < 1 ||
      a->block_table_stride < a->max_blocks || a->max_blocks > ATTN_MAX_SEQ ||
      a->max_seqlen_k > a->max_blocks * bsz)
    return ATTN_E_SHAPE;
  if (a->d != 64 && a->d != 128) return ATTN_E_HEADDIM;
  if (!aligned16(a->q) || !aligned16(a->k_cache) || !aligned16(a->v_cache) ||
      !aligned4(a->block_table) || !aligned4(a->seqlens_k))
    return ATTN_E_LAYOUT;
  if (!strides_ok(a->q_stride) || !strides_ok(a->k_stride) || !strides_ok(a->v_stride)) return ATTN_E_LAYOUT;
  if (need_o && (!aligned16(a->o) || !strides_ok(a->o_stride))) return ATTN_E_LAYOUT;
  if (need_o && a->lse && !aligned4(a->lse)) return ATTN_E_LAYOUT;
  if (!std::isfinite(a->softmax_scale)) return ATTN_E_SCALE;
  return ATTN_OK;
}

void fill_paged_params(const attn_paged_args* a, attn::FwdParams* p) {
  std::memset(p, 0, sizeof(*p));
  p->q = a->q;
  p->k = a->k_cache;
  p->v = a->v_cache;
  p->o = a->o;
  p->lse = a->lse;
  for (int i = 0; i < 3; ++i) {
    p->qs[i] = a->q_stride[i];
    p->ks[i] = a->k_stride[i];
    p->vs[i] = a->v_stride[i];
    p->os[i] = a->o_stride[i];
  }
  p->b = (int)a->b;
  p->h = (int)a->h;
  p->s_q = (int)a->s_q;
  p->s_k = (int)a->max_seqlen_k;
  p->d = (int)a->d;
  p->n_splits = 1;
  p->g = a->h_kv > 0 ? (int)(a->h / a->h_kv) : 1;
  const float s = a->softmax_scale;
  p->zero_q = s == 0.f;
  p->neg_q = s < 0.f;
  p->scale_log2 = s == 0.f ? 1.f : std::fabs(s) * 1.4426950408889634f;
  p->block_table = a->block_table;
  p->seqlens_k = a->seqlens_k;
  p->bt_stride = a->block_table_stride;
  p->num_blocks = (int)a->num_blocks;
  int lbs = 0;
  while ((int64_t(1) << lbs) < a->block_size) ++lbs;
  p->lbs = lbs;
}

bool paged_grid_ok(const attn_paged_args* a, int64_t n_splits) {
  const int64_t g = a->h_kv > 0 ? a->h / a->h_kv : 1;
  return attn::fwd_groups_per_split(a->b, a->h, g, a->s_q, (int)a->d) * n_splits <= 0x7fffffff;
}

// One split per compute unit's worth of missing work (see attn.h): `work` is the
// number of work-groups of one split.
int64_t splits_for_work(int64_t work, int64_t s_k, int64_t num_cus) {
  int64_t n = 1;
  if (work < num_cus) {
    // About one work-group per compute unit (measured best for the one-row
    // decode kernel: fewer, longer key streams), each split keeping >= 64 keys.
    n = ceil_div(num_cus, work);
    n = n < ceil_div(s_k, 64) ? n : ceil_div(s_k, 64);
    n = n < ATTN_MAX_SPLITS ? n : ATTN_MAX_SPLITS;
    n = n < 1 ? 1 : n;
  }
  return n;
}

bool grid_ok(const attn_args* a, int64_t n_splits) {
  const int64_t grid = attn::fwd_groups_per_split(a->b, a->h, group_of(a), a->s_q, (int)a->d) * n_splits;
  return grid <= 0x7fffffff;
}

}  // namespace

extern "C" {

const char* attn_status_str(int32_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_E_NULL: return "a required pointer is NULL";
    case ATTN_E_DTYPE: return "dtype must be ATTN_FP16 or ATTN_BF16";
    case ATTN_E_SHAPE: return "b, h, s_q and s_k must be >= 1 and within the size limits";
    case ATTN_E_HEADDIM: return "head dim must be 16, 32, 64 or 128";
    case ATTN_E_LAYOUT: return "pointers must be 16-byte aligned and strides non-negative multiples of 8 elements";
    case ATTN_E_SCALE: return "softmax_scale must be finite";
    case ATTN_E_SPLITS: return "num_splits must be in [1, min(s_k, ATTN_MAX_SPLITS)]";
    case ATTN_E_DEVICE: return "no usable gfx950 device";
    case ATTN_E_LAUNCH: return "kernel launch failed";
    case ATTN_E_SCRATCH: return "the problem needs more than the library's static scratch (b*h*s_q > ATTN_BWD_SCRATCH_ROWS)";
    default: return "unknown status";
  }
}

attn_status attn_fwd(const attn_args* a, void* stream) {
  attn_status st = check_args(a, true);
  if (st != ATTN_OK) return st;
  if (!grid_ok(a, 1)) return ATTN_E_SHAPE;
  st = current_device_ok();
  if (st != ATTN_OK) return st;
  attn::FwdParams p;
  fill_params(a, &p);
  hipError_t e = attn::launch_fwd(p, a->dtype, a->causal != 0, false, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

attn_status attn_num_splits_kv_for(int64_t b, int64_t h, int64_t h_kv, int64_t s_q, int64_t s_k,
                                   int64_t d, int32_t num_cus, int32_t* n_out) {
  if (!n_out) return ATTN_E_NULL;
  attn_status st = check_shape(b, h, s_q, s_k);
  if (st != ATTN_OK) return st;
  if (h_kv < 0 || h_kv > h || (h_kv > 0 && h % h_kv != 0)) return ATTN_E_SHAPE;
  if (!headdim_ok(d)) return ATTN_E_HEADDIM;
  if (num_cus < 1) return ATTN_E_DEVICE;
  // Parallel work without splitting: work-groups per split (one per (b, h, query
  // row block), per group of heads for a single query row, or per (b, K/V head)
  // when query heads sharing a K/V head are packed).
  const int64_t g = h_kv > 0 ? h / h_kv : 1;
  const int64_t work = attn::fwd_groups_per_split(b, h, g, s_q, (int)d);
  *n_out = (int32_t)splits_for_work(work, s_k, num_cus);
  return ATTN_OK;
}

attn_status attn_num_splits_for(int64_t b, int64_t h, int64_t s_q, int64_t s_k, int64_t d,
                                int32_t num_cus, int32_t* n_out) {
  return attn_num_splits_kv_for(b, h, h, s_q, s_k, d, num_cus, n_out);
}

attn_status attn_num_splits_kv(int64_t b, int64_t h, int64_t h_kv, int64_t s_q, int64_t s_k, int64_t d,
                               int device, int32_t* n_out) {
  if (!n_out) return ATTN_E_NULL;
  attn_status st = check_shape(b, h, s_q, s_k);
  if (st != ATTN_OK) return st;
  if (!headdim_ok(d)) return ATTN_E_HEADDIM;
  DevInfo info;
  st = device_info(device, &info);
  if (st != ATTN_OK) return st;
  if (!info.gfx950) return ATTN_E_DEVICE;
  return attn_num_splits_kv_for(b, h, h_kv, s_q, s_k, d, info.cus, n_out);
}

attn_status attn_num_splits(int64_t b, int64_t h, int64_t s_q, int64_t s_k, int64_t d, int device,
                            int32_t* n_out) {
  return attn_num_splits_kv(b, h, h, s_q, s_k, d, device, n_out);
}

attn_status attn_fwd_splitkv(const attn_args* a, int32_t num_splits, float* o_part, float* lse_part,
                             void* stream) {
  attn_status st = check_args(a, false);
  if (st == ATTN_OK && (!o_part || !lse_part)) st = ATTN_E_NULL;
  if (st != ATTN_OK) return st;
  if (!aligned16(o_part) || !aligned4(lse_part)) return ATTN_E_LAYOUT;
  const int64_t max_n = a->s_k < ATTN_MAX_SPLITS ? a->s_k : ATTN_MAX_SPLITS;
  if (num_splits < 1 || num_splits > max_n) return ATTN_E_SPLITS;
  if (!grid_ok(a, num_splits)) return ATTN_E_SHAPE;
  st = current_device_ok();
  if (st != ATTN_OK) return st;
  attn::FwdParams p;
  fill_params(a, &p);
  p.o = nullptr;
  p.lse = nullptr;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.n_splits = num_splits;
  hipError_t e = attn::launch_fwd(p, a->dtype, a->causal != 0, true, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

attn_status attn_fwd_paged(const attn_paged_args* a, void* stream) {
  attn_status st = check_paged(a, true);
  if (st != ATTN_OK) return st;
  if (!paged_grid_ok(a, 1)) return ATTN_E_SHAPE;
  st = current_device_ok();
  if (st != ATTN_OK) return st;
  attn::FwdParams p;
  fill_paged_params(a, &p);
  hipError_t e = attn::launch_fwd(p, a->dtype, a->causal != 0, false, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

attn_status attn_fwd_splitkv_paged(const attn_paged_args* a, int32_t num_splits, float* o_part,
                                   float* lse_part, void* stream) {
  attn_status st = check_paged(a, false);
  if (st == ATTN_OK && (!o_part || !lse_part)) st = ATTN_E_NULL;
  if (st != ATTN_OK) return st;
  if (!aligned16(o_part) || !aligned4(lse_part)) return ATTN_E_LAYOUT;
  const int64_t max_n = a->max_seqlen_k < ATTN_MAX_SPLITS ? a->max_seqlen_k : ATTN_MAX_SPLITS;
  if (num_splits < 1 || num_splits > max_n) return ATTN_E_SPLITS;
  if (!paged_grid_ok(a, num_splits)) return ATTN_E_SHAPE;
  st = current_device_ok();
  if (st != ATTN_OK) return st;
  attn::FwdParams p;
  fill_paged_params(a, &p);
  p.o = nullptr;
  p.lse = nullptr;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.n_splits = num_splits;
  hipError_t e = attn::launch_fwd(p, a->dtype, a->causal != 0, true, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

attn_status attn_num_splits_paged(int64_t b, int64_t h, int64_t h_kv, int64_t s_q, int64_t max_seqlen_k,
                                  int64_t d, int device, int32_t* n_out) {
  if (!n_out) return ATTN_E_NULL;
  attn_status st = check_shape(b, h, s_q, max_seqlen_k);
  if (st != ATTN_OK) return st;
  if (h_kv < 0 || h_kv > h || (h_kv > 0 && h % h_kv != 0)) return ATTN_E_SHAPE;
  if (d != 64 && d != 128) return ATTN_E_HEADDIM;
  DevInfo info;
  st = device_info(device, &info);
  if (st != ATTN_OK) return st;
  if (!info.gfx950 || info.cus < 1) return ATTN_E_DEVICE;
  const int64_t g = h_kv > 0 ? h / h_kv : 1;
  // Packed groups over a paged cache: two work-groups per compute unit, since the
  // block ids each tile needs are scalar loads in the key stream's critical path
  // (b = 8, h = 48, h_kv = 8, 4096 keys in 64-key blocks: 8 splits ran 8-11%
  // faster than 4, for 1 and 4 query rows).
  const int64_t cus = attn::fwd_packed(g, s_q, (int)d) ? 2 * (int64_t)info.cus : info.cus;
  *n_out = (int32_t)splits_for_work(attn::fwd_groups_per_split(b, h, g, s_q, (int)d), max_seqlen_k, cus);
  return ATTN_OK;
}

}  // extern "C"

namespace {

// Checks and launch shared by attn_bwd (delta from the caller) and
// attn_bwd_noalloc (delta in the library's static scratch): `delta` is the
// buffer the kernels use; nullptr means the static one.
attn_status bwd_run(const attn_bwd_args* a, float* delta, void* stream) {
  if (!a) return ATTN_E_NULL;
  if (!a->q || !a->k || !a->v || !a->o || !a->dout || !a->lse || !a->dq || !a->dk || !a->dv) return ATTN_E_NULL;
  if (a->dtype != ATTN_FP16 && a->dtype != ATTN_BF16) return ATTN_E_DTYPE;
  attn_status st = check_shape(a->b, a->h, a->s_q, a->s_k);
  if (st != ATTN_OK) return st;
  if (a->h_kv < 0 || a->h_kv > a->h || (a->h_kv > 0 && a->h % a->h_kv != 0)) return ATTN_E_SHAPE;
  const int64_t g = a->h_kv > 0 ? a->h / a->h_kv : 1;
  if (!headdim_ok(a->d)) return ATTN_E_HEADDIM;
  // grids: delta (d/8 lanes per (b, row, head), 256 per work-group), dQ (64 to
  // 256 query rows per work-group), dK/dV (64 or 128 keys); every one must fit a
  // 32-bit grid dimension (checked with the smallest blocks, 64)
  if (ceil_div(a->b * a->s_q * a->h * (a->d / 8), 256) > 0x7fffffff ||
      a->b * a->h * ceil_div(a->s_q, 64) > 0x7fffffff || a->b * (a->h / g) * ceil_div(a->s_k, 64) > 0x7fffffff)
    return ATTN_E_SHAPE;
  const void* t16[] = {a->q, a->k, a->v, a->o, a->dout, a->dq, a->dk, a->dv};
  for (const void* t : t16)
    if (!aligned16(t)) return ATTN_E_LAYOUT;
  if (!aligned4(a->lse) || (delta && !aligned4(delta))) return ATTN_E_LAYOUT;
  const int64_t* strides[] = {a->q_stride, a->k_stride, a->v_stride, a->o_stride,
                              a->dout_stride, a->dq_stride, a->dk_stride, a->dv_stride};
  for (const int64_t* s : strides)
    if (!strides_ok(s)) return ATTN_E_LAYOUT;
  if (!std::isfinite(a->softmax_scale)) return ATTN_E_SCALE;
  if (!delta && a->b * a->h * a->s_q > attn::kBwdScratchFloats) return ATTN_E_SCRATCH;
  st = current_device_ok();
  if (st != ATTN_OK) return st;
  if (!delta && attn::bwd_scratch(&delta) != hipSuccess) {
    (void)hipGetLastError();
    return ATTN_E_DEVICE;
  }
  attn::BwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.o = a->o;
  p.dout = a->dout;
  p.lse = a->lse;
  p.delta = delta;
  p.dq = a->dq;
  p.dk = a->dk;
  p.dv = a->dv;
  for (int i = 0; i < 3; ++i) {
    p.qs[i] = a->q_stride[i];
    p.ks[i] = a->k_stride[i];
    p.vs[i] = a->v_stride[i];
    p.os[i] = a->o_stride[i];
    p.dos[i] = a->dout_stride[i];
    p.dqs[i] = a->dq_stride[i];
    p.dks[i] = a->dk_stride[i];
    p.dvs[i] = a->dv_stride[i];
  }
  p.b = (int)a->b;
  p.h = (int)a->h;
  p.s_q = (int)a->s_q;
  p.s_k = (int)a->s_k;
  p.d = (int)a->d;
  p.g = (int)g;
  // base 2 inside the kernels: P = exp2(scale*log2(e) * q.k - LSE*log2(e));
  // the sign of the scale stays in it (the forward's LSE already carries it)
  p.scale = a->softmax_scale;
  p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
  hipError_t e = attn::launch_bwd(p, a->dtype, a->causal != 0, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

}  // namespace

extern "C" {

attn_status attn_bwd(const attn_bwd_args* a, void* stream) {
  if (a && !a->delta) return ATTN_E_NULL;
  return bwd_run(a, a ? a->delta : nullptr, stream);
}

attn_status attn_bwd_noalloc(const attn_bwd_args* a, void* stream) { return bwd_run(a, nullptr, stream); }

attn_status attn_combine(int32_t num_splits, int64_t b, int64_t h, int64_t s_q, int64_t d,
                         const float* o_part, const float* lse_part, int32_t dtype, void* o,
                         const int64_t o_stride[3], float* lse, void* stream) {
  if (!o_part || !lse_part || !o || !o_stride) return ATTN_E_NULL;
  if (dtype != ATTN_FP16 && dtype != ATTN_BF16) return ATTN_E_DTYPE;
  attn_status st = check_shape(b, h, s_q, 1);
  if (st != ATTN_OK) return st;
  if (b * h * s_q > 0x7fffffff) return ATTN_E_SHAPE;
  if (!headdim_ok(d)) return ATTN_E_HEADDIM;
  if (b * h * s_q * (d / 16) > 0x7fffffff) return ATTN_E_SHAPE;  // one wave per 16 columns of a row
  if (!aligned16(o_part) || !aligned4(lse_part) || !aligned16(o) || !strides_ok(o_stride) ||
      (lse && !aligned4(lse)))
    return ATTN_E_LAYOUT;
  if (num_splits < 1 || num_splits > ATTN_MAX_SPLITS) return ATTN_E_SPLITS;
  st = current_device_ok();
  if (st != ATTN_OK) return st;
  attn::CombineParams p;
  std::memset(&p, 0, sizeof(p));
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.o = o;
  p.lse = lse;
  for (int i = 0; i < 3; ++i) p.os[i] = o_stride[i];
  p.b = (int)b;
  p.h = (int)h;
  p.s_q = (int)s_q;
  p.d = (int)d;
  p.n_splits = num_splits;
  hipError_t e = attn::launch_combine(p, dtype, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

}  // extern "C"
