// Stage 1: block pooling.
//
// One sweep over Q, K (and V when the 0th-order tail is on) that writes, per
// contiguous block of `block` tokens, the mean query, the mean key and the
// value sum (PISA explainer, section "how candidate blocks are narrowed":
// per-block Q/K representatives and V sums; FlashPrefill summary 2(a):
// average-pooled keys).  The last block may be short; means divide by the
// number of real tokens in it.
//
// HBM-bound: every input byte is read once with 16-byte loads that are
// coalesced along a row, all loads of a workgroup are issued before any
// arithmetic, and only M*d floats per head are written.
#include "route_common.h"

namespace sa {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
  __shared__ float red[PoolRed<T, D>::kFloats];
  pool_item<T, D>(a, blockIdx.x, threadIdx.x, red);
}

template <typename T, int D>
hipError_t run(const PoolArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((pool_kernel<T, D>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

PoolArgs make_pool_args(const Shape& s, const void* q, const void* k, const void* v, float* q_bar,
                        float* k_bar, float* v_sum, void* tail) {
  PoolArgs a{};
  a.src[0] = q;
  a.src[1] = k;
  a.src[2] = v;
  a.dst[0] = q_bar;
  a.dst[1] = k_bar;
  a.dst[2] = v_sum;
  a.items[0] = s.B * s.Hq * s.M;
  a.items[1] = s.B * s.Hkv * s.M;
  a.items[2] = (v && v_sum) ? s.B * s.Hkv * s.M : 0;
  if (tail && v && v_sum) {
    a.tail[1] = static_cast<uint16_t*>(tail);
    a.tail[2] = static_cast<uint16_t*>(tail) + (size_t)s.B * s.Hkv * s.M * s.D;
  }
  a.is_mean[0] = 1;
  a.is_mean[1] = 1;
  a.is_mean[2] = 0;
  a.N = s.N;
  a.M = s.M;
  a.block = s.block;
  return a;
}

hipError_t launch_pool(const Shape& s, const void* q, const void* k, const void* v,
                       float* q_bar, float* k_bar, float* v_sum, void* tail, hipStream_t st) {
  const PoolArgs a = make_pool_args(s, q, k, v, q_bar, k_bar, v_sum, tail);
  const int grid = a.items[0] + a.items[1] + a.items[2];
  if (s.dtype == 1) {
    return s.D == 128 ? run<uint16_t, 128>(a, grid, st) : run<uint16_t, 64>(a, grid, st);
  }
  return s.D == 128 ? run<float, 128>(a, grid, st) : run<float, 64>(a, grid, st);
}

}  // namespace sa
