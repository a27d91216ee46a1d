// Device code shared by the routing kernels (block pooling, block scoring +
// selection) and their fused single-launch form: the per-item bodies and
// their arguments.  Included by pool.hip, select.hip and route_fused.hip.
#pragma once

#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace sa {

struct PoolArgs {
  const void* src[3];
  float* dst[3];
  uint16_t* tail[3];  // bf16 copies: [1] block means of k, [2] block means of v
  int items[3];   // B * heads * M for q, k, v (v: 0 when not pooled)
  int is_mean[3];
  int N, M, block;
};

PoolArgs make_pool_args(const Shape& s, const void* q, const void* k, const void* v, float* q_bar,
                        float* k_bar, float* v_sum, void* tail);

// LDS floats of the pooling reduction of one 256-thread item
template <typename T, int D>
struct PoolRed {
  static constexpr int kFloats = (256 / (D / (16 / (int)sizeof(T)))) * D;
};

// One pooling item (tensor, batch*head, block) by 256 threads t = 0..255:
// all loads first, then a reduction through `red` (PoolRed<T, D> floats).
// The caller's workgroup passes one barrier inside; `red` may be reused only
// after another barrier.
template <typename T, int D>
__device__ __forceinline__ void pool_item(const PoolArgs& a, int item, int t, float* red_) {
  constexpr int VEC = 16 / sizeof(T);      // elements per 16-byte load
  constexpr int LPR = D / VEC;             // lanes covering one row
  constexpr int RPP = 256 / LPR;           // rows per pass of the workgroup
  constexpr int MAXP = 128 / RPP;          // passes for the largest block
  float (*red)[D] = reinterpret_cast<float (*)[D]>(red_);

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
static __device__ __noinline__ int topk_count(double density, int E) {
#pragma clang fp contract(off)
  const double x = density * (double)E - 1e-9;
  int k = (int)ceil(x);
  return k < 1 ? 1 : (k > E ? E : k);
}

// LDS words of a strip's score keys; +4 per row keeps the 16x16 stores
// conflict-free.
template <int MAXCH>
struct RouteLds {
  static constexpr int kLdw = 64 * MAXCH + 4;
  static constexpr int kWords = kRows * kLdw;
};

// One strip of 16 query blocks of one head (route item `item`), by a
// workgroup of NW waves; MAXCH: 64-column chunks per row (M <= 64 * MAXCH).
// S: RouteLds<MAXCH>::kWords words of LDS.  Every thread passes one barrier.
template <int D, int NW, int MAXCH>
__device__ __forceinline__ void route_item(const RouteArgs& a, int item, uint32_t* S) {
  constexpr int NV = D / 16;               // f32x4 operand chunks per lane and tile
  constexpr int LDW = RouteLds<MAXCH>::kLdw;
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
      // threshold mode keeps a few blocks of a long row: one ballot skips a
      // chunk with no key at or above the threshold (it has no tie to count
      // either); top-k rows keep a share of every chunk, so they skip nothing
      if (ch < nch && (a.mode != 0 || __ballot(key[ch] >= T_ || (diag && 64 * ch + lane == I)))) {
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

RouteArgs make_route_args(const Shape& s, const SelectParams& p, const float* q_bar,
                          const float* k_bar, int32_t* blk_idx, int32_t* blk_cnt);

}  // namespace sa
