// Stage 2: pooled block scores, selection and compaction.
//
// Scores: s_IJ = scale * qbar_I . kbar_J for every eligible key block J
// (FlashPrefill summary 2(a)/2(b): one score per pair of blocks, from pooled
// vectors -- an (N/b)^2 matrix, never the N^2/b token-level one).
//
// Two kernels:
//   score_kernel   -- per head, a float32 matrix-core product Qbar Kbar^T
//                     (v_mfma_f32_16x16x4f32) over 64 x 64 output tiles: a
//                     workgroup holds 16 Qbar rows per wave in registers and
//                     one 64-row Kbar tile in LDS.  For causal attention the
//                     tiles above the diagonal exit at once.  The scaled
//                     scores are stored, as float bits, in the caller's
//                     block-list buffer (it has M*M 32-bit slots per head).
//   compact_kernel -- one wave per row: loads the row's eligible scores into
//                     registers, decides the kept set, and overwrites the
//                     row in place with the ascending kept indices.
//                       alpha mode:   threshold alpha * max_J s_IJ from one
//                                     wave max-reduction, no sort, no sum
//                                     (FlashPrefill summary 2(b)); keep
//                                     s_IJ >= threshold (non-positive max:
//                                     threshold = max, only arg-max kept);
//                       density mode: top-k with k = ceil(density * |E_I|)
//                                     (PISA explainer, documented call with
//                                     density=0.15): the k-th largest score
//                                     by a bitwise radix select over
//                                     order-preserving integer keys (32
//                                     counting passes of ballots, no sort),
//                                     equal scores taken in ascending J.
//                     Compaction: ballot + prefix popcount (FlashPrefill
//                     summary 2(c): index lists for jumping straight to the
//                     selected blocks).
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace sa {
namespace {

constexpr int kTile = 64;    // output tile edge of the score product

struct ScoreArgs {
  const float* q_bar;
  const float* k_bar;
  float* scores;     // [B, Hq, M, M] (the block-list buffer)
  int Hq, Hkv, M;
  float scale;
  int causal;
};

// grid: x = column tile, y = row tile, z = batch * head
template <int D>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  constexpr int CH = D / 4;            // 16-byte chunks per Kbar row
  constexpr int KV = D / 16;           // chunks per lane group
  __shared__ __attribute__((aligned(16))) float Ks[kTile * D];

  const int J0 = blockIdx.x * kTile;
  const int R0 = blockIdx.y * kTile;
  if (a.causal && J0 > R0 + kTile - 1) return;     // wholly above the diagonal
  const int bh = blockIdx.z;
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const int I0 = R0 + 16 * w;                       // this wave's first row
  const float* qb = a.q_bar + (size_t)bh * a.M * D;
  const float* kb = a.k_bar + (size_t)(b * a.Hkv + g) * a.M * D;
  float* srow = a.scores + (size_t)bh * a.M * a.M;

  // stage Kbar rows J0.. into LDS, 16-byte chunks XOR-swizzled by (row & 15)
#pragma unroll
  for (int i = 0; i < kTile * CH / 256; ++i) {
    const int u = t + 256 * i;
    const int r = u / CH, c = u % CH;
    const f32x4 x = J0 + r < a.M ? *reinterpret_cast<const f32x4*>(kb + (size_t)(J0 + r) * D + 4 * c)
                                 : f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(Ks + r * D + 4 * (c ^ (r & 15))) = x;
  }
  // A operand: row I0 + lr, k = lg*(D/4) + 4v + e at step (v, e).
  f32x4 qa[KV];
  {
    const int qi = I0 + lr;
#pragma unroll
    for (int v = 0; v < KV; ++v)
      qa[v] = qi < a.M ? *reinterpret_cast<const f32x4*>(qb + (size_t)qi * D + lg * (D / 4) + 4 * v)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();
#pragma unroll
  for (int sub = 0; sub < kTile / 16; ++sub) {
    const int r = 16 * sub + lr;                    // Kbar tile row = output column
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const f32x4 kv = *reinterpret_cast<const f32x4*>(Ks + r * D + 4 * ((lg * KV + v) ^ (r & 15)));
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[v][e], kv[e], acc, 0, 0, 0);
    }
    // 16x16 accumulator: lane holds column J0 + r, rows I0 + 4*lg + q
    const int J = J0 + r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int I = I0 + 4 * lg + q;
      if (I < a.M && J < a.M) srow[(size_t)I * a.M + J] = acc[q] * a.scale;
    }
  }
}

struct CompactArgs {
  int32_t* idx;       // in: scores as float bits; out: kept indices
  int32_t* cnt;       // out: counts
  int rows, M;
  int mode;
  float alpha;
  double density;
  int causal, force_diag;
};

// inverse of order_key
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// k = ceil(density * E - 1e-9) clamped to [1, E], in double without
// contraction so it matches the same expression evaluated on any host.
__device__ __noinline__ int topk_count(double density, int E) {
#pragma clang fp contract(off)
  const double x = density * (double)E - 1e-9;
  int k = (int)ceil(x);
  return k < 1 ? 1 : (k > E ? E : k);
}

template <int MAXCH>
__global__ __launch_bounds__(256) void compact_kernel(CompactArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int I = row % a.M;
  const int E = a.causal ? I + 1 : a.M;
  const int nch = (E + 63) >> 6;
  int32_t* out = a.idx + (size_t)row * a.M;
  const bool diag = a.force_diag != 0;

  // the row's eligible scores as order-preserving keys (0 = not eligible)
  uint32_t key[MAXCH];
#pragma unroll
  for (int c = 0; c < MAXCH; ++c) {
    const int J = 64 * c + lane;
    key[c] = (c < nch && J < E) ? order_key(__int_as_float(out[J])) : 0u;
  }

  uint32_t T;       // keep key > T, and key == T for the first `need` of them
  int need;
  if (a.mode == 0) {
    uint32_t mk = 0u;
#pragma unroll
    for (int ch = 0; ch < MAXCH; ++ch) mk = max(mk, key[ch]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mk = max(mk, (uint32_t)__shfl_xor((int)mk, o, 64));
    const float m = key_value(mk);
    T = order_key(m > 0.f ? a.alpha * m : m);
    need = 1 << 30;       // keep key >= T: every score equal to the threshold too
  } else {
    const int k = topk_count(a.density, E);
    // largest T with #{J : key_J >= T} >= k, one bit at a time
    uint32_t prefix = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = prefix | (1u << bit);
      int c = 0;
#pragma unroll
      for (int ch = 0; ch < MAXCH; ++ch)
        if (ch < nch) c += __popcll(__ballot(key[ch] >= cand));
      if (c >= k) prefix = cand;
    }
    int greater = 0;
#pragma unroll
    for (int ch = 0; ch < MAXCH; ++ch)
      if (ch < nch) greater += __popcll(__ballot(key[ch] > prefix));
    T = prefix;
    need = k - greater;
  }

  int count = 0, ties = 0;
#pragma unroll
  for (int ch = 0; ch < MAXCH; ++ch) {
    if (ch < nch) {
      const int J = 64 * ch + lane;
      const bool eq = key[ch] == T && J < E;
      const uint64_t beq = __ballot(eq);
      const bool p = key[ch] > T || (eq && ties + lanes_below(beq) < need) || (diag && J == I);
      ties += __popcll(beq);
      const uint64_t bal = __ballot(p);
      if (p) out[count + lanes_below(bal)] = J;
      count += __popcll(bal);
    }
  }
  if (lane == 0) a.cnt[row] = count;
}

template <int D>
hipError_t run_scores(const ScoreArgs& s, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((score_kernel<D>), dim3(grid), dim3(256), 0, st, s);
  return hipGetLastError();
}

template <int MAXCH>
hipError_t run_compact(const CompactArgs& c, hipStream_t st) {
  hipLaunchKernelGGL((compact_kernel<MAXCH>), dim3((c.rows + 3) / 4), dim3(256), 0, st, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const Shape& s, const SelectParams& p, const float* q_bar,
                         const float* k_bar, int32_t* blk_idx, int32_t* blk_cnt, hipStream_t st) {
  ScoreArgs sa{};
  sa.q_bar = q_bar;
  sa.k_bar = k_bar;
  sa.scores = reinterpret_cast<float*>(blk_idx);
  sa.Hq = s.Hq;
  sa.Hkv = s.Hkv;
  sa.M = s.M;
  sa.scale = p.scale;
  sa.causal = p.causal;
  const int tiles = (s.M + kTile - 1) / kTile;
  const dim3 grid(tiles, tiles, s.B * s.Hq);
  hipError_t e = s.D == 128 ? run_scores<128>(sa, grid, st) : run_scores<64>(sa, grid, st);
  if (e != hipSuccess) return e;

  CompactArgs ca{};
  ca.idx = blk_idx;
  ca.cnt = blk_cnt;
  ca.rows = s.B * s.Hq * s.M;
  ca.M = s.M;
  ca.mode = p.mode;
  ca.alpha = p.alpha;
  ca.density = p.density;
  ca.causal = p.causal;
  ca.force_diag = p.force_diag;
  if (s.M <= 128) return run_compact<2>(ca, st);
  if (s.M <= 512) return run_compact<8>(ca, st);
  return run_compact<32>(ca, st);
}

}  // namespace sa
