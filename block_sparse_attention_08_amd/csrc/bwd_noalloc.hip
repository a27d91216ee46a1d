// sparse_attn_bwd_noalloc: the backward of sparse_attn_bwd with its scratch
// (delta, sel_bits, col_idx, col_cnt and the pooled partial sums) held in a
// fixed array of device memory owned by the library, for callers that cannot
// allocate (code under HIP graph capture, serving loops that forbid
// hipMalloc).  Same kernels and launches as sparse_attn_bwd; nothing here
// allocates or frees.
//
// The array lives for the life of the process on every device that has run
// this entry point.  Every call on one device shares that device's copy, and
// calls overlapping on one device (on different streams) race on it; calls
// on one stream are ordered and safe.  No part of the scratch needs initial
// contents: every kernel of the backward writes what it later reads.
#include <mutex>

#include "../../include/sparse_attn.h"
#include "launch.h"

#define SA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = (size_t)SPARSE_ATTN_BWD_NOALLOC_SCRATCH_BYTES;
constexpr size_t kAlign = 256;
constexpr int kMaxDevices = 64;

// The device array.  In host code `scratch` names a host-side stand-in, not
// device memory: only the per-device address from hipGetSymbolAddress below
// is ever handed to a kernel or a copy.
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Device address of `scratch` on the current device, looked up once per
// device; nullptr if the runtime refuses.
void* scratch_ptr(int dev) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

SA_EXPORT sa_status sparse_attn_bwd_noalloc_scratch(const sa_desc* desc, size_t* need, size_t* cap) {
  sa_bwd_sizes z;
  const sa_status st = sparse_attn_bwd_buffer_sizes(desc, &z);
  if (st != SA_OK) return st;
  if (!need || !cap) return SA_ERR_NULL;
  *need = round_up(z.delta) + round_up(z.sel_bits) + round_up(z.col_idx) + round_up(z.col_cnt) +
          round_up(z.dk_bar) + round_up(z.dv_bar);
  *cap = kScratchBytes;
  return SA_OK;
}

SA_EXPORT sa_status sparse_attn_bwd_noalloc(const sa_desc* desc, const void* q, const void* k,
                                            const void* v, const void* tail, const int32_t* blk_idx,
                                            const int32_t* blk_cnt, const void* out, const float* lse,
                                            const void* dout, void* dq, void* dk, void* dv,
                                            void* stream) {
  sa_bwd_sizes z;
  sa_status st = sparse_attn_bwd_buffer_sizes(desc, &z);
  if (st != SA_OK) return st;
  // the caller's arguments first, as sparse_attn_bwd checks them, so that no
  // device call is made for a call that cannot run
  if (desc->dtype != SA_DTYPE_BF16) return SA_ERR_UNSUPPORTED;
  const void* args[] = {q, k, v, blk_idx, blk_cnt, out, lse, dout, dq, dk, dv};
  for (const void* p : args) {
    if (!p) return SA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(p) & 15u) return SA_ERR_ALIGN;
  }
  if (desc->approx && !tail) return SA_ERR_NULL;
  if (desc->approx && (reinterpret_cast<uintptr_t>(tail) & 15u)) return SA_ERR_ALIGN;
  size_t need = 0, cap = 0;
  st = sparse_attn_bwd_noalloc_scratch(desc, &need, &cap);
  if (st != SA_OK) return st;
  if (need > cap) return SA_ERR_SCRATCH;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SA_ERR_HIP;
  char* base = static_cast<char*>(scratch_ptr(dev));
  if (!base) return SA_ERR_HIP;
  // carve the scratch in the order of sa_bwd_sizes, each piece 256-aligned
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = bytes ? base + off : nullptr;
    off += round_up(bytes);
    return p;
  };
  float* delta = reinterpret_cast<float*>(take(z.delta));
  uint32_t* sel_bits = reinterpret_cast<uint32_t*>(take(z.sel_bits));
  int32_t* col_idx = reinterpret_cast<int32_t*>(take(z.col_idx));
  int32_t* col_cnt = reinterpret_cast<int32_t*>(take(z.col_cnt));
  float* dk_bar = reinterpret_cast<float*>(take(z.dk_bar));
  float* dv_bar = reinterpret_cast<float*>(take(z.dv_bar));
  return sparse_attn_bwd(desc, q, k, v, tail, blk_idx, blk_cnt, out, lse, dout, delta, sel_bits, col_idx,
                         col_cnt, dk_bar, dv_bar, dq, dk, dv, stream);
}
