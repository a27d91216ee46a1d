// Stage 2: pooled block scores, selection and compaction.
//
// Scores: s_IJ = scale * qbar_I . kbar_J for every eligible key block J
// (FlashPrefill summary 2(a)/2(b): a score per pair of blocks from pooled
// vectors; the M x M score matrix lives only in LDS, never in HBM).  They are
// computed in float32 with the fp32 matrix cores (v_mfma_f32_16x16x4f32):
// a workgroup owns a strip of 16 query-block rows and its four waves sweep
// the 16-column tiles of K-bar.
//
// Selection (per row, one wave per row):
//   alpha mode   -- FlashPrefill summary 2(b): threshold alpha * max_J s_IJ
//                   from one wave max-reduction, no sort, no running sum;
//   density mode -- top-k with k = ceil(density*|E_I|) (PISA explainer,
//                   documented call with density=0.15): the k-th largest
//                   score is found by a bitwise radix select over
//                   order-preserving integer keys (32 counting passes with
//                   ballots, no sort); equal scores are taken in ascending J.
// Compaction: ballot + prefix popcount writes the kept block indices in
// ascending order (FlashPrefill summary 2(c): index lists for jumping
// straight to the selected blocks).
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace sa {
namespace {

constexpr int kRows = 16;  // query-block rows per workgroup

struct SelArgs {
  const float* q_bar;
  const float* k_bar;
  int32_t* idx;
  int32_t* cnt;
  int Hq, Hkv, M, tiles, ld;
  float scale;
  int mode;
  float alpha;
  double density;
  int causal;
  int force_diag;
};

// k = ceil(density * E - 1e-9) clamped to [1, E], in double without
// contraction so it matches the same expression evaluated on any host.
__device__ __noinline__ int topk_count(double density, int E) {
#pragma clang fp contract(off)
  const double x = density * (double)E - 1e-9;
  int k = (int)ceil(x);
  return k < 1 ? 1 : (k > E ? E : k);
}

template <int D>
__global__ __launch_bounds__(256) void select_kernel(SelArgs a) {
  extern __shared__ float srow[];  // [kRows][ld]
  const int tile = blockIdx.x % a.tiles;
  const int bh = blockIdx.x / a.tiles;
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int I0 = tile * kRows;
  const float* qb = a.q_bar + (size_t)bh * a.M * D;
  const float* kb = a.k_bar + (size_t)(b * a.Hkv + g) * a.M * D;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  constexpr int KV = D / 16;  // float4 loads per lane per operand

  // ---- scores: C[i][j] = sum_k A[i][k] B[k][j] with A = qbar rows, B = kbar^T.
  // Lane group lg supplies the k-range [lg*D/4, (lg+1)*D/4) one element per step.
  f32x4 qa[KV];
  {
    const int qi = I0 + lr;
#pragma unroll
    for (int v = 0; v < KV; ++v)
      qa[v] = qi < a.M ? *reinterpret_cast<const f32x4*>(qb + (size_t)qi * D + lg * (D / 4) + 4 * v)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int Jend = a.causal ? min(a.M, I0 + kRows) : a.M;
  for (int J0 = w * 16; J0 < Jend; J0 += 64) {
    const int kj = J0 + lr;
    f32x4 kv[KV];
#pragma unroll
    for (int v = 0; v < KV; ++v)
      kv[v] = kj < a.M ? *reinterpret_cast<const f32x4*>(kb + (size_t)kj * D + lg * (D / 4) + 4 * v)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < KV; ++v) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[v][e], kv[v][e], acc, 0, 0, 0);
    }
    // 16x16 accumulator: lane holds column lr, rows 4*lg + r.
    if (kj < a.M) {
#pragma unroll
      for (int r = 0; r < 4; ++r) srow[(4 * lg + r) * a.ld + kj] = acc[r] * a.scale;
    }
  }
  __syncthreads();

  // ---- selection + compaction, one wave per row.
  for (int rr = w; rr < kRows; rr += 4) {
    const int I = I0 + rr;
    if (I >= a.M) break;
    const int E = a.causal ? I + 1 : a.M;
    const float* row = srow + rr * a.ld;
    int32_t* out = a.idx + ((size_t)bh * a.M + I) * a.M;
    const bool diag = a.force_diag != 0;
    int count = 0;
    if (a.mode == 0) {
      float m = -INFINITY;
      for (int J = lane; J < E; J += 64) m = fmaxf(m, row[J]);
      m = wave_max(m);
      const float t = m > 0.f ? a.alpha * m : m;
      for (int J0 = 0; J0 < E; J0 += 64) {
        const int J = J0 + lane;
        const bool p = J < E && (row[J] >= t || (diag && J == I));
        const uint64_t bal = __ballot(p);
        if (p) out[count + lanes_below(bal)] = J;
        count += __popcll(bal);
      }
    } else {
      const int k = topk_count(a.density, E);
      // Largest key T with #{J : key_J >= T} >= k, one bit at a time.
      uint32_t prefix = 0;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = prefix | (1u << bit);
        int c = 0;
        for (int J0 = 0; J0 < E; J0 += 64) {
          const int J = J0 + lane;
          c += __popcll(__ballot(J < E && order_key(row[J]) >= cand));
        }
        if (c >= k) prefix = cand;
      }
      int greater = 0;
      for (int J0 = 0; J0 < E; J0 += 64) {
        const int J = J0 + lane;
        greater += __popcll(__ballot(J < E && order_key(row[J]) > prefix));
      }
      const int need = k - greater;  // keys equal to T to keep, lowest J first
      int ties = 0;
      for (int J0 = 0; J0 < E; J0 += 64) {
        const int J = J0 + lane;
        const uint32_t key = J < E ? order_key(row[J]) : 0u;
        const bool gt = J < E && key > prefix;
        const bool eq = J < E && key == prefix;
        const uint64_t beq = __ballot(eq);
        const bool p = gt || (eq && ties + lanes_below(beq) < need) || (diag && J == I && J < E);
        ties += __popcll(beq);
        const uint64_t bal = __ballot(p);
        if (p) out[count + lanes_below(bal)] = J;
        count += __popcll(bal);
      }
    }
    if (lane == 0) a.cnt[(size_t)bh * a.M + I] = count;
  }
}

template <int D>
hipError_t run(const SelArgs& a, int grid, hipStream_t st) {
  const size_t lds = (size_t)kRows * a.ld * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_kernel<D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((select_kernel<D>), dim3(grid), dim3(256), lds, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const Shape& s, const SelectParams& p, const float* q_bar,
                         const float* k_bar, int32_t* blk_idx, int32_t* blk_cnt, hipStream_t st) {
  SelArgs a{};
  a.q_bar = q_bar;
  a.k_bar = k_bar;
  a.idx = blk_idx;
  a.cnt = blk_cnt;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.M = s.M;
  a.tiles = (s.M + kRows - 1) / kRows;
  a.ld = s.M + 4;
  a.scale = p.scale;
  a.mode = p.mode;
  a.alpha = p.alpha;
  a.density = p.density;
  a.causal = p.causal;
  a.force_diag = p.force_diag;
  const int grid = s.B * s.Hq * a.tiles;
  return s.D == 128 ? run<128>(a, grid, st) : run<64>(a, grid, st);
}

}  // namespace sa
