// Stage 2: pooled block scores, selection and compaction, in one kernel.
//
// Scores: s_IJ = scale * qbar_I . kbar_J for every eligible key block J
// (FlashPrefill summary 2(a)/2(b): one score per pair of blocks, from pooled
// vectors -- an (N/b)^2 matrix, never the N^2/b token-level one).  The
// matrix never leaves the chip: a workgroup of NW waves takes a strip of 16
// query blocks of one head.
//
//   product   float32 matrix cores (v_mfma_f32_16x16x4f32): the waves split
//             the strip's eligible key blocks into NW contiguous ranges of
//             16-column tiles; the strip's Qbar rows are the A operand
//             (registers, loaded once), Kbar rows of the tile the B operand,
//             read straight from L2 with the next tile's loads in flight
//             during the current tile's products.  Scaled scores go to LDS
//             as order-preserving integer keys (0 = not eligible).
//   select    one wave per row, 64 columns per register: the row's keys from
//             LDS, then
//               alpha mode:   threshold alpha * max_J s_IJ (FlashPrefill
//                             summary 2(b)): one wave max-reduction, no sort,
//                             no sum; keep s_IJ >= threshold (non-positive
//                             max: threshold = max, only the arg-max kept);
//               density mode: top-k with k = ceil(density * |E_I|) (PISA
//                             explainer, documented call with density=0.15):
//                             the k-th largest key by a bitwise radix select
//                             (32 counting passes of ballots, no sort), equal
//                             scores taken in ascending J.
//   compact   ballot + prefix popcount straight into the row's block list
//             (FlashPrefill summary 2(c): index lists for jumping to the
//             selected blocks).
#include "route_common.h"

namespace sa {
namespace {

template <int D, int NW, int MAXCH>
__global__ __launch_bounds__(64 * NW) void route_kernel(RouteArgs a) {
  __shared__ uint32_t S[RouteLds<MAXCH>::kWords];
  const int item = xcd_local_item(blockIdx.x, a.total);
  if (item < 0) return;
  route_item<D, NW, MAXCH>(a, item, S);
}

template <int D, int NW, int MAXCH>
hipError_t run_route(const RouteArgs& r, hipStream_t st) {
  const int grid = 8 * ((r.total + 7) / 8);
  hipLaunchKernelGGL((route_kernel<D, NW, MAXCH>), dim3(grid), dim3(64 * NW), 0, st, r);
  return hipGetLastError();
}

// LDS holds the strip's keys: 8 KB (M <= 128), 33 KB (M <= 512), 66 KB
// (M <= 1024), 131 KB (M <= 2048).  Sixteen waves (one per row of the strip
// in the select phase) where that fills the CU; eight for 129..1024 blocks,
// where several 8-wave workgroups per CU overlap one another's load latency,
// products and selection (measured faster than fewer 16-wave ones: at 1024
// blocks two 8-wave workgroups per CU take 107 us against 131 us for one
// 16-wave workgroup with the 2048-block layout).
template <int D>
hipError_t dispatch_route(const RouteArgs& r, hipStream_t st) {
  if (r.M <= 128) return run_route<D, 16, 2>(r, st);
  if (r.M <= 512) return run_route<D, 8, 8>(r, st);
  if (r.M <= 1024) return run_route<D, 8, 16>(r, st);
  return run_route<D, 16, 32>(r, st);
}

}  // namespace

RouteArgs make_route_args(const Shape& s, const SelectParams& p, const float* q_bar,
                          const float* k_bar, int32_t* blk_idx, int32_t* blk_cnt) {
  RouteArgs r{};
  r.q_bar = q_bar;
  r.k_bar = k_bar;
  r.idx = blk_idx;
  r.cnt = blk_cnt;
  r.Hq = s.Hq;
  r.Hkv = s.Hkv;
  r.M = s.M;
  r.total = s.B * s.Hq * ((s.M + kRows - 1) / kRows);
  r.scale = p.scale;
  r.mode = p.mode;
  r.alpha = p.alpha;
  r.density = p.density;
  r.causal = p.causal;
  r.force_diag = p.force_diag;
  return r;
}

hipError_t launch_select(const Shape& s, const SelectParams& p, const float* q_bar,
                         const float* k_bar, int32_t* blk_idx, int32_t* blk_cnt, hipStream_t st) {
  const RouteArgs r = make_route_args(s, p, q_bar, k_bar, blk_idx, blk_cnt);
  return s.D == 128 ? dispatch_route<128>(r, st) : dispatch_route<64>(r, st);
}

}  // namespace sa
