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
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace sa {
namespace {

constexpr int kRows = 16;     // query blocks per workgroup (one 16x16 product row tile)

struct RouteArgs {
  const float* q_bar;
  const float* k_bar;
  int32_t* idx;      // [B, Hq, M, M]: row capacity M, first cnt entries written
  int32_t* cnt;      // [B, Hq, M]
  int Hq, Hkv, M, total;
  float scale;
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

// NW waves; MAXCH: 64-column chunks per row (M <= 64 * MAXCH).
template <int D, int NW, int MAXCH>
__global__ __launch_bounds__(64 * NW) void route_kernel(RouteArgs a) {
  constexpr int NV = D / 16;               // f32x4 operand chunks per lane and tile
  constexpr int LDW = 64 * MAXCH + 4;      // words per key row; +4 keeps the 16x16 stores conflict-free
  __shared__ uint32_t S[kRows * LDW];

  const int item = xcd_local_item(blockIdx.x, a.total);
  if (item < 0) return;
  const int strips = (a.M + kRows - 1) / kRows;
  const int bh = item / strips;
  const int I0 = kRows * (strips - 1 - item % strips);    // longest causal strips first
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int g = h / (a.Hq / a.Hkv);

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int lr = lane & 15;
  const int lg = lane >> 4;

  // eligible columns [0, Jmax) of the strip, as T tiles of 16; wave w owns
  // tiles [t0, t0 + nt)
  const int Jmax = a.causal ? min(a.M, I0 + kRows) : a.M;
  const int T = (Jmax + 15) >> 4;
  const int TW = (T + NW - 1) / NW;
  const int t0 = w * TW;
  const int nt = max(0, min(T, t0 + TW) - t0);

  const float* qb = a.q_bar + (size_t)bh * a.M * D;
  const float* kb = a.k_bar + (size_t)(b * a.Hkv + g) * a.M * D;

  // ---- scores: A = Qbar row I0 + lr, k = 16v + 4lg + e at step (v, e);
  //      B = Kbar row 16t + lr at the same k (the four lane groups read 64
  //      contiguous bytes of a row per load); the 16x16 result of tile t has
  //      row 4lg + q, column 16t + lr in lane (lr, lg), register q
  if (nt > 0) {
    f32x4 qa[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v)
      qa[v] = *reinterpret_cast<const f32x4*>(qb + (size_t)min(I0 + lr, a.M - 1) * D + 16 * v + 4 * lg);
    auto load_tile = [&](f32x4 (&dst)[NV], int tile) {
      const float* src = kb + (size_t)min(16 * tile + lr, a.M - 1) * D + 4 * lg;
#pragma unroll
      for (int v = 0; v < NV; ++v) dst[v] = *reinterpret_cast<const f32x4*>(src + 16 * v);
    };
    auto score_tile = [&](const f32x4 (&kv)[NV], int tile) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[v][e], kv[v][e], acc, 0, 0, 0);
      const int J = 16 * tile + lr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int I = I0 + 4 * lg + q;
        const bool ok = I < a.M && J < a.M && (!a.causal || J <= I);
        S[(4 * lg + q) * LDW + J] = ok ? order_key(acc[q] * a.scale) : 0u;
      }
    };
    f32x4 k0[NV], k1[NV];
    load_tile(k0, t0);
    for (int i = 0; i < nt; i += 2) {
      if (i + 1 < nt) load_tile(k1, t0 + i + 1);
      score_tile(k0, t0 + i);
      if (i + 1 < nt) {
        if (i + 2 < nt) load_tile(k0, t0 + i + 2);
        score_tile(k1, t0 + i + 1);
      }
    }
  }
  __syncthreads();

  // ---- one wave per row: select and compact
  const bool diag = a.force_diag != 0;
  for (int rr = w; rr < kRows; rr += NW) {
    const int I = I0 + rr;
    if (I >= a.M) break;
    const int E = a.causal ? I + 1 : a.M;
    const int nch = (E + 63) >> 6;
    const int row = bh * a.M + I;
    int32_t* out = a.idx + (size_t)row * a.M;

    uint32_t key[MAXCH];
#pragma unroll
    for (int c = 0; c < MAXCH; ++c) {
      const int J = 64 * c + lane;
      key[c] = (c < nch && J < E) ? S[rr * LDW + J] : 0u;
    }

    uint32_t T_;      // keep key > T_, and key == T_ for the first `need` of them
    int need;
    if (a.mode == 0) {
      uint32_t mk = 0u;
#pragma unroll
      for (int ch = 0; ch < MAXCH; ++ch) mk = max(mk, key[ch]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) mk = max(mk, (uint32_t)__shfl_xor((int)mk, o, 64));
      const float m = key_value(mk);
      T_ = order_key(m > 0.f ? a.alpha * m : m);
      need = 1 << 30;     // every score equal to the threshold is kept
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
      T_ = prefix;
      need = k - greater;
    }

    int count = 0, ties = 0;
#pragma unroll
    for (int ch = 0; ch < MAXCH; ++ch) {
      if (ch < nch) {
        const int J = 64 * ch + lane;
        const bool eq = key[ch] == T_ && J < E;
        const uint64_t beq = __ballot(eq);
        const bool p = key[ch] > T_ || (eq && ties + lanes_below(beq) < need) || (diag && J == I);
        ties += __popcll(beq);
        const uint64_t bal = __ballot(p);
        if (p) out[count + lanes_below(bal)] = J;
        count += __popcll(bal);
      }
    }
    if (lane == 0) a.cnt[row] = count;
  }
}

template <int D, int NW, int MAXCH>
hipError_t run_route(const RouteArgs& r, hipStream_t st) {
  const int grid = 8 * ((r.total + 7) / 8);
  hipLaunchKernelGGL((route_kernel<D, NW, MAXCH>), dim3(grid), dim3(64 * NW), 0, st, r);
  return hipGetLastError();
}

// LDS holds the strip's keys: 8 KB (M <= 128), 33 KB (M <= 512), 131 KB
// (M <= 2048).  Sixteen waves (one per row of the strip in the select phase)
// where that fills the CU; eight for 129..512 blocks, where two 16-wave
// workgroups per CU measured slower than four 8-wave ones.
template <int D>
hipError_t dispatch_route(const RouteArgs& r, hipStream_t st) {
  if (r.M <= 128) return run_route<D, 16, 2>(r, st);
  if (r.M <= 512) return run_route<D, 8, 8>(r, st);
  return run_route<D, 16, 32>(r, st);
}

}  // namespace

hipError_t launch_select(const Shape& s, const SelectParams& p, const float* q_bar,
                         const float* k_bar, int32_t* blk_idx, int32_t* blk_cnt, hipStream_t st) {
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
  return s.D == 128 ? dispatch_route<128>(r, st) : dispatch_route<64>(r, st);
}

}  // namespace sa
