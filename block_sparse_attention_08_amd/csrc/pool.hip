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
#include "device_common.h"
#include "launch.h"

namespace sa {
namespace {

struct PoolArgs {
  const void* src[3];
  float* dst[3];
  uint16_t* tail[3];  // bf16 copies: [1] block means of k, [2] block means of v
  int items[3];   // B * heads * M for q, k, v (v: 0 when not pooled)
  int is_mean[3];
  int N, M, block;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
  constexpr int VEC = 16 / sizeof(T);      // elements per 16-byte load
  constexpr int LPR = D / VEC;             // lanes covering one row
  constexpr int RPP = 256 / LPR;           // rows per pass of the workgroup
  constexpr int MAXP = 128 / RPP;          // passes for the largest block
  __shared__ float red[RPP][D];

  int item = blockIdx.x;
  int which = 0;
  while (which < 2 && item >= a.items[which]) {
    item -= a.items[which];
    ++which;
  }
  const int bh = item / a.M;
  const int J = item - bh * a.M;
  const int t0 = J * a.block;
  const int n = min(a.block, a.N - t0);
  const T* base = static_cast<const T*>(a.src[which]) + ((size_t)bh * a.N + t0) * D;

  const int t = threadIdx.x;
  const int c = t % LPR;
  const int r0 = t / LPR;

  u32x4 buf[MAXP];
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    const int r = r0 + p * RPP;
    if (p * RPP < a.block && r < n)
      buf[p] = *reinterpret_cast<const u32x4*>(base + (size_t)r * D + c * VEC);
    else
      buf[p] = u32x4{0u, 0u, 0u, 0u};
  }

  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    const uint32_t w[4] = {buf[p][0], buf[p][1], buf[p][2], buf[p][3]};
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(w[e] << 16);
        acc[2 * e + 1] += __uint_as_float(w[e] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(w[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[r0][c * VEC + e] = acc[e];
  __syncthreads();

  if (t < D) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RPP; ++r) s += red[r][t];
    if (a.is_mean[which]) s = s / (float)n;
    a.dst[which][(size_t)item * D + t] = s;
    // bf16 tail operands: the pseudo-key (mean k) and its value (mean v)
    if (a.tail[which])
      a.tail[which][(size_t)item * D + t] =
          (uint16_t)f32_to_bf16_bits(a.is_mean[which] ? s : s / (float)n);
  }
}

template <typename T, int D>
hipError_t run(const PoolArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((pool_kernel<T, D>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const Shape& s, const void* q, const void* k, const void* v,
                       float* q_bar, float* k_bar, float* v_sum, void* tail, hipStream_t st) {
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
  const int grid = a.items[0] + a.items[1] + a.items[2];
  if (s.dtype == 1) {
    return s.D == 128 ? run<uint16_t, 128>(a, grid, st) : run<uint16_t, 64>(a, grid, st);
  }
  return s.D == 128 ? run<float, 128>(a, grid, st) : run<float, 64>(a, grid, st);
}

}  // namespace sa
