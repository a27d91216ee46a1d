// Device-side validation of block lists (sparse_attn_check_lists): every row
// of blk_idx / blk_cnt is checked against the layout the attention kernels
// rely on -- 1 <= count <= |E_I|, entries in [0, M), strictly ascending,
// eligible (J <= I when causal), and with causal attention and the tail on
// the diagonal block present (its pooled key would hold later tokens; FlashPrefill
// summary 2(c) index lists, PISA explainer routing table).  Results go to a
// three-word device record: OR of the violation flags, the number of bad
// rows, the lowest bad row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sparse_attn.h"
#include "device_common.h"
#include "launch.h"

namespace sa {
namespace {

struct CheckArgs {
  const int32_t* idx;
  const int32_t* cnt;
  uint32_t* res;   // [flags, bad rows, first bad row]
  int M, rows, causal, need_diag;
};

__global__ __launch_bounds__(64) void clear_result_kernel(uint32_t* res) {
  if (threadIdx.x == 0) {
    res[0] = 0u;
    res[1] = 0u;
    res[2] = 0xFFFFFFFFu;
  }
}

// One wave per row (b, h, I); four rows per workgroup.
__global__ __launch_bounds__(256) void check_lists_kernel(CheckArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int lane = threadIdx.x & 63;
  const int I = row % a.M;
  const int E = a.causal ? I + 1 : a.M;
  const int n = a.cnt[row];
  uint32_t flags = 0u;
  if (n < 1 || n > E) flags |= SA_LIST_COUNT;
  const int len = n < 0 ? 0 : (n > a.M ? a.M : n);   // entries that exist in the row
  const int32_t* list = a.idx + (size_t)row * a.M;
  bool diag = false;
  for (int e0 = 0; e0 < len; e0 += 64) {
    const int e = e0 + lane;
    if (e < len) {
      const int J = list[e];
      if (J < 0 || J >= a.M) flags |= SA_LIST_RANGE;
      else if (a.causal && J > I) flags |= SA_LIST_INELIGIBLE;
      if (e > 0 && J <= list[e - 1]) flags |= SA_LIST_ORDER;
      if (J == I) diag = true;
    }
  }
  if (a.need_diag && !__any(diag)) flags |= SA_LIST_NO_DIAGONAL;
  // OR across the wave
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) flags |= (uint32_t)__shfl_xor((int)flags, o, 64);
  if (lane == 0 && flags) {
    atomicOr(&a.res[0], flags);
    atomicAdd(&a.res[1], 1u);
    atomicMin(&a.res[2], (uint32_t)row);
  }
}

}  // namespace

hipError_t launch_check_lists(const Shape& s, int causal, int approx, const int32_t* blk_idx,
                              const int32_t* blk_cnt, uint32_t* result, hipStream_t st) {
  CheckArgs a{};
  a.idx = blk_idx;
  a.cnt = blk_cnt;
  a.res = result;
  a.M = s.M;
  a.rows = s.B * s.Hq * s.M;
  a.causal = causal;
  a.need_diag = causal && approx;
  hipLaunchKernelGGL(clear_result_kernel, dim3(1), dim3(64), 0, st, result);
  hipLaunchKernelGGL(check_lists_kernel, dim3((a.rows + 3) / 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace sa
