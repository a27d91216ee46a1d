// Stages 1 and 2 in one launch: block pooling, then block scoring,
// selection and compaction, with one grid-wide barrier in between (the
// scores of a head need the pooled keys of all its blocks).
//
// The routing stages compute what pool.hip and select.hip compute, with the
// same per-item code (pooled block representatives: PISA explainer, section
// "how candidate blocks are narrowed"; FlashPrefill summary 2(a)-(c): pooled
// scores, alpha * max threshold, index lists); fusing them is FlashPrefill's
// pattern-discovery step without a second launch.  The kernel is launched
// cooperatively with as many workgroups as fit on the device at once: phase
// 1 strides over the pooling items (each workgroup of NW waves works on NW/4
// items at a time, 256 threads each), phase 2 over the 16-block strips of the
// scoring/selection.
//
// On this device the barrier is the expensive part: the pooled vectors
// written under one XCD's L2 must be written back and the other XCDs' L2
// lines dropped before any strip is scored, which is what a kernel boundary
// does too.  The separate two-launch path measured faster; this entry point
// is kept for callers that want a single launch.
#include <hip/hip_cooperative_groups.h>

#include "route_common.h"

namespace sa {
namespace {

template <typename T, int D, int NW, int MAXCH>
__global__ __launch_bounds__(64 * NW) void route_fused_kernel(PoolArgs pa, RouteArgs ra) {
  constexpr int NSUB = NW / 4;   // 256-thread pooling groups per workgroup
  constexpr int kPoolBytes = NSUB * PoolRed<T, D>::kFloats * 4;
  constexpr int kRouteBytes = RouteLds<MAXCH>::kWords * 4;
  constexpr int kBytes = kPoolBytes > kRouteBytes ? kPoolBytes : kRouteBytes;
  __shared__ __attribute__((aligned(16))) char lds[kBytes];

  // ---- phase 1: pooling; every workgroup runs the same number of rounds,
  // and every wave passes one barrier inside a round and one after it
  const int sub = threadIdx.x >> 8;
  float* red = reinterpret_cast<float*>(lds) + sub * PoolRed<T, D>::kFloats;
  const int n_pool = pa.items[0] + pa.items[1] + pa.items[2];
  const int per_round = gridDim.x * NSUB;
  const int rounds = (n_pool + per_round - 1) / per_round;
  for (int r = 0; r < rounds; ++r) {
    const int item = r * per_round + blockIdx.x * NSUB + sub;
    if (item < n_pool)
      pool_item<T, D>(pa, item, threadIdx.x & 255, red);
    else
      __syncthreads();   // the barrier inside pool_item
    __syncthreads();     // `red` is rewritten next round
  }

  // pooled vectors of every head written and visible device-wide
  cooperative_groups::this_grid().sync();

  // ---- phase 2: scores, selection, compaction per strip
  uint32_t* S = reinterpret_cast<uint32_t*>(lds);
  for (int item = blockIdx.x; item < ra.total; item += gridDim.x) {
    route_item<D, NW, MAXCH>(ra, item, S);
    __syncthreads();     // S is rewritten by the next strip
  }
}

template <typename T, int D, int NW, int MAXCH>
hipError_t run_fused(const PoolArgs& pa, const RouteArgs& ra, hipStream_t st) {
  const void* kern = reinterpret_cast<const void*>(&route_fused_kernel<T, D, NW, MAXCH>);
  int per_cu = 0, dev = 0, cus = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * NW, 0);
  if (e != hipSuccess) return e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  const int n_pool = pa.items[0] + pa.items[1] + pa.items[2];
  const int want = max((n_pool + NW / 4 - 1) / (NW / 4), ra.total);
  const int grid = min(per_cu * cus, want);
  PoolArgs p = pa;
  RouteArgs r = ra;
  void* args[] = {&p, &r};
  e = hipLaunchCooperativeKernel(kern, dim3(grid), dim3(64 * NW), args, 0, st);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

// Same workgroup shapes as the separate scoring kernel.
template <typename T, int D>
hipError_t dispatch_fused(const PoolArgs& pa, const RouteArgs& ra, hipStream_t st) {
  if (ra.M <= 128) return run_fused<T, D, 16, 2>(pa, ra, st);
  if (ra.M <= 512) return run_fused<T, D, 8, 8>(pa, ra, st);
  return run_fused<T, D, 16, 32>(pa, ra, st);
}

}  // namespace

hipError_t launch_route_fused(const Shape& s, const SelectParams& p, const void* q, const void* k,
                              const void* v, float* q_bar, float* k_bar, float* v_sum, void* tail,
                              int32_t* blk_idx, int32_t* blk_cnt, hipStream_t st) {
  const PoolArgs pa = make_pool_args(s, q, k, v, q_bar, k_bar, v_sum, tail);
  const RouteArgs ra = make_route_args(s, p, q_bar, k_bar, blk_idx, blk_cnt);
  if (s.dtype == 1)
    return s.D == 128 ? dispatch_fused<uint16_t, 128>(pa, ra, st) : dispatch_fused<uint16_t, 64>(pa, ra, st);
  return s.D == 128 ? dispatch_fused<float, 128>(pa, ra, st) : dispatch_fused<float, 64>(pa, ra, st);
}

}  // namespace sa
