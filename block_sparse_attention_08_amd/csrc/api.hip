// Host side of the C ABI declared in include/sparse_attn.h: argument
// validation, buffer sizes, and one launch per call on the caller's stream.
// No allocation, no synchronisation, no state.
#include <math.h>
#include <stdint.h>

#include "../../include/sparse_attn.h"
#include "launch.h"

#define SA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

sa_status check_desc(const sa_desc* d, sa::Shape* s) {
  if (!d) return SA_ERR_NULL;
  if (d->batch < 1 || d->heads_q < 1 || d->heads_kv < 1 || d->seq_len < 1 || d->head_dim < 1 ||
      d->block < 1)
    return SA_ERR_SHAPE;
  if (d->heads_q % d->heads_kv != 0) return SA_ERR_SHAPE;
  if (d->dtype != SA_DTYPE_F32 && d->dtype != SA_DTYPE_BF16) return SA_ERR_DTYPE;
  if (d->select_mode != SA_SELECT_ALPHA && d->select_mode != SA_SELECT_DENSITY) return SA_ERR_PARAM;
  if (d->select_mode == SA_SELECT_ALPHA && !(d->alpha > 0.0 && d->alpha <= 1.0)) return SA_ERR_PARAM;
  if (d->select_mode == SA_SELECT_DENSITY && !(d->density > 0.0 && d->density <= 1.0))
    return SA_ERR_PARAM;
  if ((d->causal != 0 && d->causal != 1) || (d->approx != 0 && d->approx != 1)) return SA_ERR_PARAM;
  if (isnan(d->scale) || isinf(d->scale)) return SA_ERR_PARAM;
  if (d->head_dim != 64 && d->head_dim != 128) return SA_ERR_UNSUPPORTED;
  if (d->block != 64 && d->block != 128) return SA_ERR_UNSUPPORTED;
  // in 64 bits: seq_len + block - 1 overflows an int near INT32_MAX
  const int64_t M64 = ((int64_t)d->seq_len + d->block - 1) / d->block;
  if (M64 > sa::kMaxBlocks) return SA_ERR_UNSUPPORTED;
  const int M = (int)M64;
  if ((int64_t)d->batch * d->heads_q > 65535) return SA_ERR_UNSUPPORTED;   // grid z of the score pass
  // every workgroup count and per-row index of the kernels is a 32-bit int
  const int64_t items = (int64_t)d->batch * (d->heads_q + 2 * (int64_t)d->heads_kv) * M;
  if (items > INT32_MAX / 2) return SA_ERR_SHAPE;
  if (s) {
    s->B = d->batch;
    s->Hq = d->heads_q;
    s->Hkv = d->heads_kv;
    s->N = d->seq_len;
    s->D = d->head_dim;
    s->block = d->block;
    s->M = M;
    s->dtype = d->dtype;
  }
  return SA_OK;
}

float resolve_scale(const sa_desc* d) {
  return d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)d->head_dim);
}

sa_status from_hip(hipError_t e) { return e == hipSuccess ? SA_OK : SA_ERR_HIP; }

sa::SelectParams select_params(const sa_desc* d) {
  sa::SelectParams p;
  p.scale = resolve_scale(d);
  p.mode = d->select_mode;
  p.alpha = (float)d->alpha;
  p.density = d->density;
  p.causal = d->causal;
  p.force_diag = d->causal && d->approx;
  return p;
}

}  // namespace

SA_EXPORT int32_t sparse_attn_abi_version(void) { return SPARSE_ATTN_ABI_VERSION; }

SA_EXPORT const char* sparse_attn_status_string(sa_status st) {
  switch (st) {
    case SA_OK: return "ok";
    case SA_ERR_NULL: return "a required pointer is NULL";
    case SA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case SA_ERR_DTYPE: return "unknown dtype";
    case SA_ERR_PARAM: return "alpha, density, select_mode, scale or a flag is out of range";
    case SA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case SA_ERR_UNSUPPORTED: return "unsupported head_dim, block or number of blocks";
    case SA_ERR_HIP: return "the HIP runtime reported an error";
    case SA_ERR_SCRATCH: return "the problem needs more scratch than the library's fixed array holds";
  }
  return "unknown status";
}

SA_EXPORT sa_status sparse_attn_buffer_sizes(const sa_desc* desc, sa_sizes* sizes) {
  sa::Shape s;
  const sa_status st = check_desc(desc, &s);
  if (st != SA_OK) return st;
  if (!sizes) return SA_ERR_NULL;
  const size_t f = sizeof(float);
  sizes->q_bar = (size_t)s.B * s.Hq * s.M * s.D * f;
  sizes->k_bar = (size_t)s.B * s.Hkv * s.M * s.D * f;
  sizes->v_sum = desc->approx ? sizes->k_bar : 0;
  sizes->tail = (desc->approx && desc->dtype == SA_DTYPE_BF16) ? 2 * (size_t)s.B * s.Hkv * s.M * s.D * 2 : 0;
  sizes->blk_idx = (size_t)s.B * s.Hq * s.M * s.M * sizeof(int32_t);
  sizes->blk_cnt = (size_t)s.B * s.Hq * s.M * sizeof(int32_t);
  return SA_OK;
}

SA_EXPORT sa_status sparse_attn_block_pool(const sa_desc* desc, const void* q, const void* k,
                                           const void* v, float* q_bar, float* k_bar,
                                           float* v_sum, void* tail, void* stream) {
  sa::Shape s;
  const sa_status st = check_desc(desc, &s);
  if (st != SA_OK) return st;
  const bool need_tail = desc->approx && desc->dtype == SA_DTYPE_BF16;
  if (!q || !k || !q_bar || !k_bar) return SA_ERR_NULL;
  if (desc->approx && (!v || !v_sum)) return SA_ERR_NULL;
  if (need_tail && !tail) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_bar) || !aligned16(k_bar)) return SA_ERR_ALIGN;
  if (desc->approx && (!aligned16(v) || !aligned16(v_sum))) return SA_ERR_ALIGN;
  if (need_tail && !aligned16(tail)) return SA_ERR_ALIGN;
  return from_hip(sa::launch_pool(s, q, k, desc->approx ? v : nullptr, q_bar, k_bar,
                                  desc->approx ? v_sum : nullptr, need_tail ? tail : nullptr,
                                  (hipStream_t)stream));
}

SA_EXPORT sa_status sparse_attn_select(const sa_desc* desc, const float* q_bar, const float* k_bar,
                                       int32_t* blk_idx, int32_t* blk_cnt, void* stream) {
  sa::Shape s;
  const sa_status st = check_desc(desc, &s);
  if (st != SA_OK) return st;
  if (!q_bar || !k_bar || !blk_idx || !blk_cnt) return SA_ERR_NULL;
  if (!aligned16(q_bar) || !aligned16(k_bar) || !aligned16(blk_idx) || !aligned16(blk_cnt))
    return SA_ERR_ALIGN;
  return from_hip(sa::launch_select(s, select_params(desc), q_bar, k_bar, blk_idx, blk_cnt,
                                    (hipStream_t)stream));
}

SA_EXPORT sa_status sparse_attn_route(const sa_desc* desc, const void* q, const void* k, const void* v,
                                      float* q_bar, float* k_bar, float* v_sum, void* tail,
                                      int32_t* blk_idx, int32_t* blk_cnt, void* stream) {
  sa::Shape s;
  const sa_status st = check_desc(desc, &s);
  if (st != SA_OK) return st;
  const bool need_tail = desc->approx && desc->dtype == SA_DTYPE_BF16;
  if (!q || !k || !q_bar || !k_bar || !blk_idx || !blk_cnt) return SA_ERR_NULL;
  if (desc->approx && (!v || !v_sum)) return SA_ERR_NULL;
  if (need_tail && !tail) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_bar) || !aligned16(k_bar) || !aligned16(blk_idx) ||
      !aligned16(blk_cnt))
    return SA_ERR_ALIGN;
  if (desc->approx && (!aligned16(v) || !aligned16(v_sum))) return SA_ERR_ALIGN;
  if (need_tail && !aligned16(tail)) return SA_ERR_ALIGN;
  return from_hip(sa::launch_route_fused(s, select_params(desc), q, k, desc->approx ? v : nullptr, q_bar,
                                         k_bar, desc->approx ? v_sum : nullptr, need_tail ? tail : nullptr,
                                         blk_idx, blk_cnt, (hipStream_t)stream));
}

namespace {

sa_status fwd_impl(const sa_desc* desc, const void* q, const void* k, const void* v, const float* k_bar,
                   const float* v_sum, const void* tail, const int32_t* blk_idx, const int32_t* blk_cnt,
                   void* out, float* lse, void* stream) {
  sa::Shape s;
  const sa_status st = check_desc(desc, &s);
  if (st != SA_OK) return st;
  const bool f32_tail = desc->approx && desc->dtype == SA_DTYPE_F32;
  const bool bf16_tail = desc->approx && desc->dtype == SA_DTYPE_BF16;
  if (!q || !k || !v || !blk_idx || !blk_cnt || !out) return SA_ERR_NULL;
  if (f32_tail && (!k_bar || !v_sum)) return SA_ERR_NULL;
  if (bf16_tail && !tail) return SA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(blk_idx) ||
      !aligned16(blk_cnt))
    return SA_ERR_ALIGN;
  if (f32_tail && (!aligned16(k_bar) || !aligned16(v_sum))) return SA_ERR_ALIGN;
  if (bf16_tail && !aligned16(tail)) return SA_ERR_ALIGN;
  if (lse && !aligned16(lse)) return SA_ERR_ALIGN;
  sa::FwdParams p;
  p.scale = resolve_scale(desc);
  p.causal = desc->causal;
  p.approx = desc->approx;
  p.lse = lse;
  return from_hip(sa::launch_fwd(s, p, q, k, v, f32_tail ? k_bar : nullptr, f32_tail ? v_sum : nullptr,
                                 bf16_tail ? tail : nullptr, blk_idx, blk_cnt, out,
                                 (hipStream_t)stream));
}

}  // namespace

SA_EXPORT sa_status sparse_attn_fwd(const sa_desc* desc, const void* q, const void* k, const void* v,
                                    const float* k_bar, const float* v_sum, const void* tail,
                                    const int32_t* blk_idx, const int32_t* blk_cnt, void* out,
                                    void* stream) {
  return fwd_impl(desc, q, k, v, k_bar, v_sum, tail, blk_idx, blk_cnt, out, nullptr, stream);
}

SA_EXPORT sa_status sparse_attn_check_lists(const sa_desc* desc, const int32_t* blk_idx,
                                            const int32_t* blk_cnt, uint32_t* result, void* stream) {
  sa::Shape s;
  const sa_status st = check_desc(desc, &s);
  if (st != SA_OK) return st;
  if (!blk_idx || !blk_cnt || !result) return SA_ERR_NULL;
  if (!aligned16(blk_idx) || !aligned16(blk_cnt) || !aligned16(result)) return SA_ERR_ALIGN;
  return from_hip(sa::launch_check_lists(s, desc->causal, desc->approx, blk_idx, blk_cnt, result,
                                         (hipStream_t)stream));
}

SA_EXPORT sa_status sparse_attn_bwd_buffer_sizes(const sa_desc* desc, sa_bwd_sizes* sizes) {
  sa::Shape s;
  const sa_status st = check_desc(desc, &s);
  if (st != SA_OK) return st;
  if (!sizes) return SA_ERR_NULL;
  const sa::BwdSizes z = sa::bwd_sizes(s, desc->approx);
  sizes->lse = z.lse;
  sizes->delta = z.delta;
  sizes->sel_bits = z.sel_bits;
  sizes->col_idx = z.col_idx;
  sizes->col_cnt = z.col_cnt;
  sizes->dk_bar = z.dk_bar;
  sizes->dv_bar = z.dv_bar;
  return SA_OK;
}

SA_EXPORT sa_status sparse_attn_bwd(const sa_desc* desc, const void* q, const void* k, const void* v,
                                    const void* tail, const int32_t* blk_idx, const int32_t* blk_cnt,
                                    const void* out, const float* lse, const void* dout, float* delta,
                                    uint32_t* sel_bits, int32_t* col_idx, int32_t* col_cnt, float* dk_bar,
                                    float* dv_bar, void* dq, void* dk, void* dv, void* stream) {
  sa::Shape s;
  const sa_status st = check_desc(desc, &s);
  if (st != SA_OK) return st;
  if (desc->dtype != SA_DTYPE_BF16) return SA_ERR_UNSUPPORTED;
  const bool ap = desc->approx != 0;
  if (!q || !k || !v || !blk_idx || !blk_cnt || !out || !lse || !dout || !delta || !sel_bits || !col_idx ||
      !col_cnt || !dq || !dk || !dv)
    return SA_ERR_NULL;
  if (ap && (!tail || !dk_bar || !dv_bar)) return SA_ERR_NULL;
  const void* al[] = {q, k, v, blk_idx, blk_cnt, out, lse, dout, delta, sel_bits, col_idx, col_cnt, dq, dk, dv};
  for (const void* p : al)
    if (!aligned16(p)) return SA_ERR_ALIGN;
  if (ap && (!aligned16(tail) || !aligned16(dk_bar) || !aligned16(dv_bar))) return SA_ERR_ALIGN;
  sa::BwdParams p;
  p.scale = resolve_scale(desc);
  p.causal = desc->causal;
  p.approx = desc->approx;
  sa::BwdPtrs x;
  x.q = q;
  x.k = k;
  x.v = v;
  x.tail = ap ? tail : nullptr;
  x.out = out;
  x.dout = dout;
  x.blk_idx = blk_idx;
  x.blk_cnt = blk_cnt;
  x.lse = lse;
  x.delta = delta;
  x.sel_bits = sel_bits;
  x.col_idx = col_idx;
  x.col_cnt = col_cnt;
  x.dk_bar = ap ? dk_bar : nullptr;
  x.dv_bar = ap ? dv_bar : nullptr;
  x.dq = dq;
  x.dk = dk;
  x.dv = dv;
  return from_hip(sa::launch_bwd(s, p, x, (hipStream_t)stream));
}

SA_EXPORT sa_status sparse_attn_fwd_lse(const sa_desc* desc, const void* q, const void* k, const void* v,
                                        const float* k_bar, const float* v_sum, const void* tail,
                                        const int32_t* blk_idx, const int32_t* blk_cnt, void* out,
                                        float* lse, void* stream) {
  if (!lse) return SA_ERR_NULL;
  return fwd_impl(desc, q, k, v, k_bar, v_sum, tail, blk_idx, blk_cnt, out, lse, stream);
}
