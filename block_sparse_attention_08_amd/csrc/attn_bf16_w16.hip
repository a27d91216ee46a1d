// Stage 3 for bf16 inputs, 16 query rows per wave: block-sparse flash
// attention on the gfx950 matrix cores with v_mfma_f32_16x16x32_bf16.
//
// Computes exactly what attn_bf16.hip computes (exact softmax over the
// listed key blocks, FlashPrefill summary 2(c) index-driven tiles; the
// 0th-order tail of unlisted eligible blocks as pseudo-keys with weight n_J,
// PISA explainer routing table; one running max / sum, FlashAttention
// tutorial section 2).  The difference is the work split: a workgroup of
// block/16 waves, each owning 16 query rows, so one K tile and one V tile in
// LDS (32 KB) feed four waves of a 64-row block -- four workgroups, sixteen
// waves per CU -- where the 32-row layout fits only eight.
//
// Per 64-key tile and wave:
//   S^T = K Q^T: 4 key groups x d/32 steps of 16x16x32 (K from LDS as A,
//       the wave's Q rows in registers as B).  Lane l holds query row l%16,
//       keys 16t + 4*(l/16) + r of key group t: a row's 64 scores sit in
//       the four lanes l%16 + 16g, combined with two permlane swaps; on
//       tiles without masks each finished key group is folded into the row
//       max beside the products of the next.
//   P = exp2(S * scale * log2 e - m), packed to bf16: the registers of key
//       groups 2c and 2c+1 are directly the B operand of PV step c.
//   O^T += V^T P^T: d/16 tiles x 2 steps; V^T gathered from the row-major V
//       tile with ds_read_b64_tr_b16.
// K/V tiles move HBM -> LDS with buffer loads straight into LDS (range-
// checked: rows past the last key read zero), XOR-swizzled per row (K:
// chunk ^ (row & 15), V: chunk ^ 2*(row & 7) for d = 128) so the operand
// reads are free of bank conflicts.  One K and one V buffer, two barriers per
// tile (the next K tile loads during softmax and PV, the next V tile during
// the next S).  Serves 64-row query blocks only.
#include <math.h>

#include "attn_common.h"
#include "device_common.h"
#include "launch.h"

namespace sa {
namespace {

struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* tail_k;
  const uint16_t* tail_v;
  const int32_t* idx;
  const int32_t* cnt;
  uint16_t* out;
  float* lse;
  int Hq, Hkv, N, M, G, total;
  float scale_log2;
  int causal, approx;
};

template <int D, int BLK>
struct Cfg {
  static constexpr int NW = BLK / 16;         // waves
  static constexpr int NT = 64 * NW;          // threads
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int NI = KT * CPR / NT;    // 16-byte DMA loads per thread per tile
  static constexpr int NKS = D / 32;          // 32-wide d steps of S
  static constexpr int NOT = D / 16;          // 16-wide d tiles of O
  static constexpr int ROWB = D * 2;          // bytes per LDS row
  static constexpr int RPK = 1024 / ROWB;     // rows filled by one 1 KB DMA instruction
  static_assert(NI >= 1 && (NW * RPK) % 16 == 0, "per-lane DMA offsets must repeat every instruction");
};

template <int D>
__device__ __forceinline__ int k_chunk(int r, int c) { return c ^ (r & (D == 128 ? 15 : 7)); }
template <int D>
__device__ __forceinline__ int v_chunk(int r, int c) { return c ^ (D == 128 ? 2 * (r & 7) : 2 * (r & 3)); }

// Byte offset in the tile of the 16-byte chunk this lane copies with every
// DMA instruction (instruction i adds i*NW KB: whole rows, and the swizzle
// repeats every 16 rows).
template <int D, int BLK, bool IS_V>
__device__ __forceinline__ int dma_lane_off(int w, int lane) {
  using C = Cfg<D, BLK>;
  const int P = w * 64 + lane;
  const int r = P / C::CPR, pc = P % C::CPR;
  const int c = IS_V ? v_chunk<D>(r, pc) : k_chunk<D>(r, pc);
  return r * C::ROWB + c * 16;
}

template <int D, int BLK>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, int tile_off, char* lds, int w,
                                         int lane_off) {
  using C = Cfg<D, BLK>;
#pragma unroll
  for (int i = 0; i < C::NI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (i * C::NW + w) * 1024), 16,
                                             tile_off + i * C::NW * 1024 + lane_off, 0, 0, 0);
}

// Gather: like dma_tile, but instruction i reads this lane's chunk of the
// row at byte offset ro[i] (per-lane rows, e.g. the pooled rows of a tail
// tile).
template <int D, int BLK>
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t rs, const int (&ro)[Cfg<D, BLK>::NI], int col,
                                         char* lds, int w) {
  using C = Cfg<D, BLK>;
#pragma unroll
  for (int i = 0; i < C::NI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (i * C::NW + w) * 1024), 16, ro[i] + col, 0, 0,
                                             0);
}

// value of a query row over its four lanes (l%16 + 16g)
__device__ __forceinline__ float row_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D, int BLK>
__global__ __launch_bounds__(4 * BLK, 4) void attn_w16_kernel(Args a) {
  using C = Cfg<D, BLK>;
  static_assert(BLK == KT, "one 64-key tile per block");
  constexpr int TB = KT * D * 2;   // bytes of one K or V tile
  __shared__ __attribute__((aligned(1024))) char Ks[TB];
  __shared__ __attribute__((aligned(1024))) char Vs[TB];
  // tail only: selection bitmap, then the ascending list of the eligible
  // blocks that are not listed (the pooled rows the tail tiles gather)
  __shared__ uint32_t selbits[kMaxBlocks / 32];
  __shared__ uint16_t tail_rows[kMaxBlocks];

  const int item = xcd_local_item(blockIdx.x, a.total);
  if (item < 0) return;
  const int hg = item % a.G;
  int rest = item / a.G;
  const int I = a.M - 1 - rest % a.M;
  rest /= a.M;
  const int g = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int h = g * a.G + hg;
  const int bh = b * a.Hq + h;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lr = lane & 15;   // query row inside the wave
  const int lg = lane >> 4;   // lane group: keys 4*lg .. 4*lg+3 of every key group

  const int q_tok = I * BLK + 16 * w + lr;
  const bool q_ok = q_tok < a.N;

  // Q fragment (B operand of S^T): row q_tok, d = 32*s + 8*lg + e
  bf16x8 qf[C::NKS];
  {
    const uint16_t* qrow = a.q + ((size_t)bh * a.N + (q_ok ? q_tok : 0)) * D;
#pragma unroll
    for (int s = 0; s < C::NKS; ++s) {
      const u32x4 x = q_ok ? *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * lg) : u32x4{0u, 0u, 0u, 0u};
      qf[s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const int n_sel = scalar_view(a.cnt)[(size_t)bh * a.M + I];
  const const_i32* list = scalar_view(a.idx + ((size_t)bh * a.M + I) * a.M);
  const int Jend = a.causal ? I + 1 : a.M;
  const int n_exact = n_sel;
  // every listed block is eligible, so Jend - n_sel eligible blocks remain
  const int n_rest = a.approx ? Jend - n_sel : 0;
  const int n_tiles = n_exact + (n_rest + KT - 1) / KT;
  const int last_n = a.N - (a.M - 1) * BLK;
  // tail logits carry log2(n_J): log2(BLK) for every block but a short last
  // one, whose row (the largest index, so the last tail row) gets the
  // difference added to its score
  const float log2_blk = __log2f((float)BLK);
  const float last_fix = (__log2f((float)last_n) - log2_blk) / a.scale_log2;

  if (a.approx) {
    for (int i = t; i < kMaxBlocks / 32; i += C::NT) selbits[i] = 0u;
    __syncthreads();
    for (int e = t; e < n_sel; e += C::NT) {
      const int J = list[e];
      atomicOr(&selbits[J >> 5], 1u << (J & 31));
    }
    __syncthreads();
    if (w == 0) {   // ballot compaction of the unlisted eligible blocks
      int base = 0;
      for (int J0 = 0; J0 < Jend; J0 += 64) {
        const int J = J0 + lane;
        const int Jc = J < Jend ? J : 0;   // keeps the bitmap read in range
        const bool rest_J = J < Jend && !((selbits[Jc >> 5] >> (Jc & 31)) & 1u);
        const uint64_t bal = __ballot(rest_J);
        if (rest_J) tail_rows[base + lanes_below(bal)] = (uint16_t)J;
        base += __popcll(bal);
      }
    }
    __syncthreads();
  }

  const int head_bytes = a.N * C::ROWB;
  const size_t pp_off = (size_t)(b * a.Hkv + g) * a.M * D;
  const __amdgpu_buffer_rsrc_t krs = head_rsrc(a.k + (size_t)(b * a.Hkv + g) * a.N * D, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(a.v + (size_t)(b * a.Hkv + g) * a.N * D, head_bytes);
  const __amdgpu_buffer_rsrc_t tkrs = head_rsrc(a.approx ? a.tail_k + pp_off : a.k, a.M * C::ROWB);
  const __amdgpu_buffer_rsrc_t tvrs = head_rsrc(a.approx ? a.tail_v + pp_off : a.v, a.M * C::ROWB);
  const int koff = dma_lane_off<D, BLK, false>(w, lane);
  const int voff = dma_lane_off<D, BLK, true>(w, lane);
  // tail gathers: the row this lane copies with DMA instruction i of a tile
  // is row0 + i * NW * RPK; its chunk offset inside the row is fixed
  const int row0 = (w * 64 + lane) / C::CPR;
  const int kcol = koff - row0 * C::ROWB;
  const int vcol = voff - row0 * C::ROWB;

  // LDS operand addresses (tile-invariant): K rows 16t + lr, chunk 4s + lg;
  // V transpose-read source rows 4*lg + (lr >> 2) (+32c, +16 half), columns
  // 16nt + 4*(lr & 3)
  int kbase[C::NKS];
#pragma unroll
  for (int s = 0; s < C::NKS; ++s) kbase[s] = lr * C::ROWB + k_chunk<D>(lr, 4 * s + lg) * 16;
  int vbase[C::NOT];
  {
    const int jr = 4 * lg + (lr >> 2);
#pragma unroll
    for (int nt = 0; nt < C::NOT; ++nt) {
      const int n = 16 * nt + 4 * (lr & 3);
      vbase[nt] = jr * C::ROWB + v_chunk<D>(jr, n >> 3) * 16 + (n & 7) * 2;
    }
  }

  // first key of exact tile e (one 64-key tile per listed block); tail
  // tiles are numbered from 0 and gather KT pooled rows each
  auto tile_key0 = [&](int e) -> int { return e < n_exact ? list[e] * BLK : e - n_exact; };
  // tail tile tt: byte offsets (row index from tail_rows, 0 for the padding
  // of the last tile, masked later) of this lane's rows
  auto tail_offs = [&](int tt, int (&ro)[C::NI]) {
#pragma unroll
    for (int i = 0; i < C::NI; ++i) {
      const int r = KT * tt + row0 + i * C::NW * C::RPK;
      ro[i] = (r < n_rest ? (int)tail_rows[r] : 0) * C::ROWB;
    }
  };
  auto issue_k = [&](int e, int key0) {
    if (e < n_exact) {
      dma_tile<D, BLK>(krs, key0 * C::ROWB, Ks, w, koff);
    } else {
      int ro[C::NI];
      tail_offs(key0, ro);
      dma_rows<D, BLK>(tkrs, ro, kcol, Ks, w);
    }
  };
  auto issue_v = [&](int e, int key0) {
    if (e < n_exact) {
      dma_tile<D, BLK>(vrs, key0 * C::ROWB, Vs, w, voff);
    } else {
      int ro[C::NI];
      tail_offs(key0, ro);
      dma_rows<D, BLK>(tvrs, ro, vcol, Vs, w);
    }
  };

  f32x4 o[C::NOT];
#pragma unroll
  for (int i = 0; i < C::NOT; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;   // running reference max (scaled log2 domain)
  float l = 0.f;         // this lane's partial row sum
  const float c = a.scale_log2;

  // One tile: S, masks, online softmax, PV.  MODE says which masks the tile
  // needs (a separate copy of the body per mode keeps the unmasked tiles free
  // of mask code and of the register copies a conditional mask would cause).
  // One K and one V buffer, two barriers: K e+1 loads during the softmax and
  // PV of tile e, V e+1 during S of tile e+1.
  auto step = [&](int e, int key0, int key1, auto mode) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode)::value;
    constexpr bool FOLD = MODE == kModePlain || MODE == kModeTail;   // tiles without masks

    // ---- S^T = K Q^T (K operands read three steps ahead).  Tiles without
    // masks fold each finished key group into the row max two products into
    // the next group, beside the products (pinned there by scheduling
    // barriers).
    f32x4 s[4];
    float mx = -INFINITY;
    // the matrix phases (S, PV) run at raised wave priority: a wave that is
    // issuing products keeps the matrix core fed while the other waves of
    // the SIMD fill the gaps with their softmax arithmetic
    __builtin_amdgcn_s_setprio(1);
    {
      constexpr int NSTEP = 4 * C::NKS;
      constexpr int KD = 3;
      bf16x8 kr[KD];
#pragma unroll
      for (int i = 0; i < KD; ++i)
        kr[i] = *reinterpret_cast<const bf16x8*>(Ks + kbase[i % C::NKS] + 16 * (i / C::NKS) * C::ROWB);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NSTEP; ++st) {
        const int tg = st / C::NKS, ks = st % C::NKS;
        const bf16x8 ka = kr[st % KD];
        if (st + KD < NSTEP) {
          const int n2 = st + KD;
          kr[st % KD] = *reinterpret_cast<const bf16x8*>(Ks + kbase[n2 % C::NKS] + 16 * (n2 / C::NKS) * C::ROWB);
        }
        s[tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[ks], s[tg], 0, 0, 0);
        if constexpr (FOLD) {
          if (tg > 0 && ks == (C::NKS > 2 ? 2 : C::NKS - 1)) {
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[tg - 1][r]);
            asm volatile("" ::"v"(mx));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (FOLD) {
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[3][r]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    wait_vm();
    __syncthreads();               // K buffer free, V tile e landed in every wave
    if (e + 1 < n_tiles) issue_k(e + 1, key1);

    // ---- masks: register r of key group tg holds key key0 + 16*tg + 4*lg + r
    if constexpr (MODE == kModeTailLast) {
      // last tail tile: padding rows masked; a short last block's row (the
      // last real row when listed here) gets its multiplicity fix
      const int lim = n_rest - KT * key0 - 4 * lg;
      const int fix_kr = (last_n != BLK && tail_rows[n_rest - 1] == a.M - 1) ? lim - 1 : -1;
#pragma unroll
      for (int tg = 0; tg < 4; ++tg)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kr = 16 * tg + r;            // row - KT*tt - 4*lg
          s[tg][r] = kr < lim ? (kr == fix_kr ? s[tg][r] + last_fix : s[tg][r]) : -INFINITY;
        }
    } else if constexpr (MODE == kModeEdge) {
      int lim = a.N - key0;
      if (a.causal) lim = min(lim, q_tok - key0 + 1);
      lim -= 4 * lg;
#pragma unroll
      for (int tg = 0; tg < 4; ++tg)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[tg][r] = 16 * tg + r < lim ? s[tg][r] : -INFINITY;
    }

    // ---- online softmax
    if constexpr (!FOLD) {
#pragma unroll
      for (int tg = 0; tg < 4; ++tg)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[tg][r]);
    }
    mx = row_max4(mx);
    // tail rows: + log2(n_J) (a uniform offset; a short last block's
    // difference is already in its score)
    const float lb = MODE >= kModeTail ? log2_blk : 0.f;
    const float mxs = fmaf(mx, c, lb);
    const bool grow = mxs > m + 8.f;
    if (__ballot(grow)) {
      const float m_new = grow ? mxs : m;
      const float corr = __builtin_amdgcn_exp2f(m - m_new);
      l *= corr;
#pragma unroll
      for (int nt = 0; nt < C::NOT; ++nt) o[nt] *= corr;
      m = m_new;
    }
    const float mb = (m == -INFINITY ? 0.f : m) - lb;
    // P of register pair 2tg + hp (key group tg, registers 2hp, 2hp+1) in wd;
    // PV step cc (keys 32cc .. 32cc+31) takes slots 4cc .. 4cc+3
    uint32_t wd[8];
    float lsum = 0.f;
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
#pragma unroll
      for (int hp = 0; hp < 2; ++hp) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[tg][2 * hp], c, -mb));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[tg][2 * hp + 1], c, -mb));
        wd[2 * tg + hp] = pack2(p0, p1);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd[2 * tg + hp]), kOnes, lsum, false);
      }
    }
    const bf16x8 pk0 = __builtin_bit_cast(bf16x8, u32x4{wd[0], wd[1], wd[2], wd[3]});

    // ---- O^T += V^T P^T (V operands four ahead).  The d/16 products of
    // keys 0..31 each carry a share of the exponentials of keys 32..63, so
    // the matrix core and the vector ALU work side by side in this wave.
    {
      constexpr int NPV = 2 * C::NOT;
      constexpr int VD = 4;
      constexpr int EPS = 8 / C::NOT;   // elements of keys 32..63 per product
      static_assert(EPS * C::NOT == 8, "exponential split");
      auto vop = [&](int j) -> bf16x8 {
        const int nt = j % C::NOT, cc = j / C::NOT;
        const char* p = Vs + vbase[nt] + (32 * cc) * C::ROWB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 16 * C::ROWB));
        return __builtin_bit_cast(
            bf16x8, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      };
      bf16x8 vr[VD];
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int j = 0; j < VD; ++j) vr[j] = vop(j);
      float pe = 0.f;
#pragma unroll
      for (int j = 0; j < C::NOT; ++j) {
        const bf16x8 va = vr[j % VD];
        vr[j % VD] = vop(j + VD);
        o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pk0, o[j], 0, 0, 0);
#pragma unroll
        for (int u = 0; u < EPS; ++u) {
          const int q = j * EPS + u;   // element q: key group 2 + q/4, register q%4
          const float p = __builtin_amdgcn_exp2f(fmaf(s[2 + (q >> 2)][q & 3], c, -mb));
          if (q & 1) {
            wd[4 + (q >> 1)] = pack2(pe, p);
            lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd[4 + (q >> 1)]), kOnes, lsum, false);
            // empty volatile statements keep each value's computation in
            // this step (plain arithmetic would be sunk to its first use)
            asm volatile("" ::"v"(wd[4 + (q >> 1)]));
          } else {
            pe = p;
            asm volatile("" ::"v"(pe));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      const bf16x8 pk1 = __builtin_bit_cast(bf16x8, u32x4{wd[4], wd[5], wd[6], wd[7]});
#pragma unroll
      for (int j = C::NOT; j < NPV; ++j) {
        const bf16x8 va = vr[j % VD];
        if (j + VD < NPV) vr[j % VD] = vop(j + VD);
        o[j - C::NOT] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pk1, o[j - C::NOT], 0, 0, 0);
      }
    }
    l += lsum;

    __builtin_amdgcn_s_setprio(0);
    wait_vm();
    __syncthreads();   // V buffer free, K tile e+1 landed in every wave
    if (e + 1 < n_tiles) issue_v(e + 1, key1);
  };

  int key0 = tile_key0(0);
  issue_k(0, key0);
  issue_v(0, key0);
  wait_vm();
  __syncthreads();

  // Only the ragged last block (J = M-1) and the causal diagonal (J = I)
  // need the edge mask; either is the largest index a list may hold, so in
  // an ascending list it can only be the last entry.
  int n_plain = n_exact;
  if (n_exact > 0) {
    const int J = list[n_exact - 1];
    if ((J + 1) * BLK > a.N || (a.causal && J >= I)) n_plain = n_exact - 1;
  }
  int e = 0;
  for (; e < n_plain; ++e) {
    const int key1 = e + 1 < n_tiles ? tile_key0(e + 1) : 0;
    step(e, key0, key1, ModeC<kModePlain>{});
    key0 = key1;
  }
  for (; e < n_exact; ++e) {
    const int key1 = e + 1 < n_tiles ? tile_key0(e + 1) : 0;
    step(e, key0, key1, ModeC<kModeEdge>{});
    key0 = key1;
  }
  for (; e < n_tiles - 1; ++e) {
    const int key1 = tile_key0(e + 1);
    step(e, key0, key1, ModeC<kModeTail>{});
    key0 = key1;
  }
  if (e < n_tiles) step(e, key0, 0, ModeC<kModeTailLast>{});

  // ---- epilogue: O / l in bf16.  Register r of d-tile nt holds row lr,
  // d = 16*nt + 4*lg + r; the wave's 16 rows leave through its quarter of
  // the free K buffer (staged row store).
  const float lt = row_sum4(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  // log of the denominator: sum_a exp(z_a) = lt * 2^m
  if (a.lse && q_ok && lg == 0) a.lse[(size_t)bh * a.N + q_tok] = __logf(lt) + m * 0.69314718055994531f;
  char* stage = Ks + w * 16 * C::ROWB;
#pragma unroll
  for (int nt = 0; nt < C::NOT; ++nt) {
    const int ch = 2 * nt + (lg >> 1);          // 16-byte chunk of the row
    const u32x2 x = {pack2(o[nt][0] * inv, o[nt][1] * inv), pack2(o[nt][2] * inv, o[nt][3] * inv)};
    *reinterpret_cast<u32x2*>(stage + lr * C::ROWB + stage_slot<D>(lr, ch) * 16 + 8 * (lg & 1)) = x;
  }
  const int tok0 = I * BLK + 16 * w;            // the wave's first query token
  store_staged_rows<D, 16>(stage, a.out + ((size_t)bh * a.N + tok0) * D, a.N - tok0, lane);
}

// 64-row blocks: four 4-wave workgroups per CU (32 KB of tile buffers each).
template <int D>
hipError_t run(const Args& a, hipStream_t st) {
  const int grid = 8 * ((a.total + 7) / 8);
  hipLaunchKernelGGL((attn_w16_kernel<D, 64>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_w16(const Shape& s, const FwdParams& p, const void* q, const void* k,
                          const void* v, const void* tail, const int32_t* blk_idx,
                          const int32_t* blk_cnt, void* out, hipStream_t st) {
  Args a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  if (p.approx) {
    a.tail_k = static_cast<const uint16_t*>(tail);
    a.tail_v = a.tail_k + (size_t)s.B * s.Hkv * s.M * s.D;
  }
  a.idx = blk_idx;
  a.cnt = blk_cnt;
  a.out = static_cast<uint16_t*>(out);
  a.lse = p.lse;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.N = s.N;
  a.M = s.M;
  a.G = s.Hq / s.Hkv;
  a.total = s.B * s.Hq * s.M;
  a.scale_log2 = p.scale * 1.4426950408889634f;
  a.causal = p.causal;
  a.approx = p.approx;
  if (s.block != 64) return hipErrorInvalidValue;
  return s.D == 128 ? run<128>(a, st) : run<64>(a, st);
}

}  // namespace sa
