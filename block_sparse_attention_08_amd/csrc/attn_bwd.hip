// Gradients of stage 3 (bf16 inputs): dq, dk, dv of the block-sparse
// attention with the 0th-order tail, for the selection the forward used.
//
// PISA explainer, "minimal documented usage": the 0th-order variant is the
// one meant for training, so gradients flow through the exact blocks and
// through the pooled pseudo-keys of the tail; the block selection is held
// fixed (it passes no gradient).  With P_ia the softmax weight of key a
// (token j of a listed block, or pooled block J with multiplicity n_J:
// P = n_J exp(z - L)), u_a its value (v_j, or the bf16 block mean of v) and
// dO the output gradient:
//     dz_ia = P_ia (dO_i . u_a - D_i),   D_i = dO_i . o_i
//     dq_i  = scale sum_a dz_ia key_a
//     dk_j  = scale sum_i dz_ij q_i,  dv_j = sum_i P_ij dO_i      (exact)
//     dkbar_J = scale sum_i dz_iJ q_i, dubar_J = sum_i P_iJ dO_i (pooled)
// and the block means spread dkbar_J / n_J and dubar_J / n_J over the
// tokens of block J.  The forward's log-denominator L_i (written by
// sparse_attn_fwd_lse) gives P without a running max: exp2(z log2 e - L log2 e).
//
// Kernels (one launch each, in order):
//   bwd_delta   D_i = dO_i . o_i and -L_i log2 e (float32)
//   bwd_bitmap  the selection as bits, one row per (batch, query head, block)
//   bwd_cols    per (batch, KV group, key block J): the (query head, query
//               block) pairs that list J, ascending (the transposed lists)
//   bwd_dq      per 64 query rows of a query block, like the forward: its
//               listed blocks, then its unlisted eligible pooled rows
//               (gathered), tile by tile: S^T = K Q^T, dP^T = V dO^T, dS^T,
//               dQ^T += K^T dS^T
//   bwd_dtail   per KV group, 64 pooled rows and one of 16 ranges of query
//               blocks: every query block of the range whose tail holds
//               them: S = Q Kbar^T, dP = dO Vbar^T, dVbar^T += dO^T P,
//               dKbar^T += Q^T dS (float32 partial sums per range)
//   bwd_dkv     per 64 keys of a key block: the pairs of its transposed
//               list, tile by tile, dV^T += dO^T P, dK^T += Q^T dS; adds the
//               pooled gradients of its block (the 16 partial sums) / n_J
//               and writes dk, dv
// All products are v_mfma_f32_16x16x32_bf16 with 16 rows (queries, keys or
// pooled rows) per wave held in registers and 64-row tiles of the other
// operand in LDS (HBM -> LDS by buffer loads into LDS).  One XOR swizzle of
// the 16-byte chunks serves both LDS read patterns (row fragments with
// ds_read_b128, transposed fragments with ds_read_b64_tr_b16).
#include <math.h>

#include "attn_common.h"
#include "device_common.h"
#include "launch.h"

namespace sa {
namespace {

constexpr int BT = 64;   // rows per LDS tile (keys, queries or pooled rows)
constexpr int kTailChunks = 16;   // query-block ranges of the pooled-gradient pass
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct BC {
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int ROWB = D * 2;         // bytes per row
  static constexpr int RPK = 1024 / ROWB;    // rows per 1 KB DMA instruction
  static constexpr int NKS = D / 32;         // 32-wide d steps
  static constexpr int NOT = D / 16;         // 16-wide d tiles
  static constexpr int TB = BT * ROWB;       // bytes of one tile
};

// Chunk c of row r sits at chunk swz(r, c): rows 0..15 of one chunk column
// land on 16 different chunks (row fragments), and rows 0..7 (8..15) of two
// adjacent chunk columns on 16 different chunks (transposed fragments).
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  return c ^ ((((r & 7) << 1) | ((r >> 3) & 1)) & (BC<D>::CPR - 1));
}

// ---- tile DMA: instruction i of wave w fills LDS bytes [(i*NW + w) KB, +1 KB)
// = rows (i*NW + w)*RPK + lane/CPR; the row step per instruction is a
// multiple of 16, so the swizzled column of a lane is the same for every i.
template <int D, int NW>
struct Dma {
  static constexpr int NI = BT * BC<D>::CPR / (64 * NW);
  static_assert(NI >= 1 && (NW * BC<D>::RPK) % 16 == 0, "tile DMA layout");
  __device__ static int row0(int w, int lane) { return w * BC<D>::RPK + lane / BC<D>::CPR; }
  __device__ static int col(int w, int lane) { return swz<D>(row0(w, lane), lane % BC<D>::CPR) * 16; }
  // BT consecutive rows from byte `off` of the resource
  __device__ static void tile(__amdgpu_buffer_rsrc_t rs, int off, char* lds, int w, int voff) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (i * NW + w) * 1024), 16,
                                               off + i * NW * 1024 + voff, 0, 0, 0);
  }
  // rows at per-lane byte offsets ro[i]
  __device__ static void rows(__amdgpu_buffer_rsrc_t rs, const int (&ro)[NI], int col, char* lds, int w) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (i * NW + w) * 1024), 16, ro[i] + col, 0, 0,
                                               0);
  }
};

// LDS offsets of this lane's fragments (tile-invariant): row fragments
// (rows lr, chunk 4s + lg) and transposed fragments (rows 4*lg + lr/4 of a
// 16-row half, columns 16*nt + 4*(lr & 3)).
template <int D>
struct Frag {
  int rb[BC<D>::NKS];
  int tb[BC<D>::NOT];
  __device__ Frag(int lr, int lg) {
#pragma unroll
    for (int s = 0; s < BC<D>::NKS; ++s) rb[s] = lr * BC<D>::ROWB + swz<D>(lr, 4 * s + lg) * 16;
    const int jr = 4 * lg + (lr >> 2);
#pragma unroll
    for (int nt = 0; nt < BC<D>::NOT; ++nt) {
      const int n = 16 * nt + 4 * (lr & 3);
      tb[nt] = jr * BC<D>::ROWB + swz<D>(jr, n >> 3) * 16 + (n & 7) * 2;
    }
  }
};

// LDS fragments are read this many products ahead of the product that uses
// them, through a ring of registers.
constexpr int kRing = 6;

// Two row products, interleaved step by step:
//   acc0[tg] = T0_rows(16tg..16tg+15) . R0^T,  acc1[tg] = T1_rows(..) . R1^T
// lane (lr, lg), register r = tile row 16tg + 4lg + r against register row
// lr.  A scheduling barrier after each product keeps the program order: the
// read kRing steps ahead is issued before each product, so the products run
// back to back while the later reads are in flight, and products on one
// accumulator are eight steps apart.
template <int D>
__device__ __forceinline__ void gemm_rows2(f32x4 (&acc0)[4], const char* t0, const bf16x8 (&r0)[BC<D>::NKS],
                                           f32x4 (&acc1)[4], const char* t1, const bf16x8 (&r1)[BC<D>::NKS],
                                           const Frag<D>& f) {
  constexpr int NS = 2 * 4 * BC<D>::NKS;     // tiles x row groups x d steps
  // step i: tile i & 1, row group (i >> 1) % 4, d step (i >> 1) / 4
  auto frag = [&](int i) -> bf16x8 {
    const char* t = (i & 1) ? t1 : t0;
    return *reinterpret_cast<const bf16x8*>(t + f.rb[(i >> 1) / 4] + 16 * ((i >> 1) % 4) * BC<D>::ROWB);
  };
#pragma unroll
  for (int tg = 0; tg < 4; ++tg) {
    acc0[tg] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[tg] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 ring[kRing];
#pragma unroll
  for (int i = 0; i < kRing; ++i) ring[i] = frag(i);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const bf16x8 a = ring[i % kRing];
    if (i + kRing < NS) ring[i % kRing] = frag(i + kRing);
    const int tg = (i >> 1) % 4, st = (i >> 1) / 4;
    if (i & 1)
      acc1[tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, r1[st], acc1[tg], 0, 0, 0);
    else
      acc0[tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, r0[st], acc0[tg], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Transposed fragment of d-tile nt, tile rows 32cc .. 32cc + 31.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, const Frag<D>& f, int nt, int cc) {
  const char* p = tile + f.tb[nt] + 32 * cc * BC<D>::ROWB;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 16 * BC<D>::ROWB));
  return __builtin_bit_cast(
      bf16x8, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// Two transposed products, interleaved step by step:
//   acc0[nt] += T0^T(d-tile nt) . X0,  acc1[nt] += T1^T(d-tile nt) . X1,
// X packed from a gemm_rows-shaped array (x[cc]: tile rows of row groups 2cc
// and 2cc+1).  Read ring and scheduling as in gemm_rows2; products on one
// accumulator are 2 * (d tiles) steps apart.
template <int D>
__device__ __forceinline__ void gemm_tr2(f32x4 (&acc0)[BC<D>::NOT], const char* t0, const bf16x8 (&x0)[2],
                                         f32x4 (&acc1)[BC<D>::NOT], const char* t1, const bf16x8 (&x1)[2],
                                         const Frag<D>& f) {
  constexpr int NOT = BC<D>::NOT;
  constexpr int NS = 2 * 2 * NOT;            // tiles x halves x d tiles
  // step i: tile i & 1, d tile (i >> 1) % NOT, half (i >> 1) / NOT
  auto frag = [&](int i) -> bf16x8 { return tr_frag<D>((i & 1) ? t1 : t0, f, (i >> 1) % NOT, (i >> 1) / NOT); };
  bf16x8 ring[kRing];
#pragma unroll
  for (int i = 0; i < kRing; ++i) ring[i] = frag(i);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const bf16x8 a = ring[i % kRing];
    if (i + kRing < NS) ring[i % kRing] = frag(i + kRing);
    const int nt = (i >> 1) % NOT, cc = (i >> 1) / NOT;
    if (i & 1)
      acc1[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, x1[cc], acc1[nt], 0, 0, 0);
    else
      acc0[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, x0[cc], acc0[nt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// acc[tg] = T_rows(16tg..16tg+15) . R^T: lane (lr, lg), register r = tile row
// 16tg + 4lg + r against register row lr.
template <int D>
__device__ __forceinline__ void gemm_rows(f32x4 (&acc)[4], const char* tile, const Frag<D>& f,
                                          const bf16x8 (&rg)[BC<D>::NKS]) {
#pragma unroll
  for (int tg = 0; tg < 4; ++tg) acc[tg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < BC<D>::NKS; ++s)
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(tile + f.rb[s] + 16 * tg * BC<D>::ROWB);
      acc[tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, rg[s], acc[tg], 0, 0, 0);
    }
}

// acc[nt] += T^T(d-tile nt) . X, X packed from a gemm_rows-shaped array
// (pk[cc]: tile rows of row groups 2cc and 2cc+1).
template <int D>
__device__ __forceinline__ void gemm_tr(f32x4 (&acc)[BC<D>::NOT], const char* tile, const Frag<D>& f,
                                        const bf16x8 (&pk)[2]) {
#pragma unroll
  for (int nt = 0; nt < BC<D>::NOT; ++nt)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const char* p = tile + f.tb[nt] + 32 * cc * BC<D>::ROWB;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 16 * BC<D>::ROWB));
      const bf16x8 a = __builtin_bit_cast(
          bf16x8, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pk[cc], acc[nt], 0, 0, 0);
    }
}

__device__ __forceinline__ void pack_rows(const f32x4 (&x)[4], bf16x8 (&pk)[2]) {
  uint32_t wd[8];
#pragma unroll
  for (int tg = 0; tg < 4; ++tg) {
    wd[2 * tg] = pack2(x[tg][0], x[tg][1]);
    wd[2 * tg + 1] = pack2(x[tg][2], x[tg][3]);
  }
#pragma unroll
  for (int cc = 0; cc < 2; ++cc)
    pk[cc] = __builtin_bit_cast(bf16x8, u32x4{wd[4 * cc], wd[4 * cc + 1], wd[4 * cc + 2], wd[4 * cc + 3]});
}

// one bf16 row fragment per 32-wide d step: row `row` (zeros if !ok)
template <int D>
__device__ __forceinline__ void load_row(bf16x8 (&dst)[BC<D>::NKS], const uint16_t* rowp, bool ok, int lg) {
#pragma unroll
  for (int s = 0; s < BC<D>::NKS; ++s) {
    const u32x4 x = ok ? *reinterpret_cast<const u32x4*>(rowp + 32 * s + 8 * lg) : u32x4{0u, 0u, 0u, 0u};
    dst[s] = __builtin_bit_cast(bf16x8, x);
  }
}

struct BwdArgs {
  const uint16_t *q, *k, *v, *out, *dout;
  const uint16_t *tail_k, *tail_v;   // bf16 block means of k and v
  const int32_t *idx, *cnt;
  const float* lse;
  float* delta;
  uint32_t* bits;      // [B, Hq, M, W]
  int32_t *col_idx, *col_cnt;   // [B, Hkv, M, G*M], [B, Hkv, M]
  float *dk_bar, *dv_bar;       // [B, Hkv, M, D]
  uint16_t *dq, *dk, *dv;
  int B, Hq, Hkv, N, M, G, W, block;
  float scale, scale_log2;
  int causal, approx;
};

// ---------------------------------------------------------------- D_i
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;                  // lanes per row (16 bytes each)
  const long row = ((long)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int c = threadIdx.x % LPR;
  const long rows = (long)a.B * a.Hq * a.N;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 o = *reinterpret_cast<const u32x4*>(a.out + row * D + 8 * c);
    const u32x4 g = *reinterpret_cast<const u32x4*>(a.dout + row * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(bf16_bits_to_f32(o[e] & 0xFFFFu), bf16_bits_to_f32(g[e] & 0xFFFFu), acc);
      acc = fmaf(bf16_bits_to_f32(o[e] >> 16), bf16_bits_to_f32(g[e] >> 16), acc);
    }
  }
#pragma unroll
  for (int o = LPR / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, LPR);
  if (row < rows && c == 0) {
    a.delta[row] = acc;
    // minus the log-denominator in log2 units: the exponent of P is then
    // one fused multiply-add of the score
    a.delta[rows + row] = -a.lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------- bitmap
__global__ __launch_bounds__(64) void bwd_bitmap_kernel(BwdArgs a) {
  __shared__ uint32_t bits[kMaxBlocks / 32];
  const long row = blockIdx.x;                 // (b * Hq + h) * M + I
  for (int i = threadIdx.x; i < a.W; i += 64) bits[i] = 0u;
  __syncthreads();
  const int n = a.cnt[row];
  const int32_t* list = a.idx + row * a.M;
  for (int e = threadIdx.x; e < n; e += 64) {
    const int J = list[e];
    atomicOr(&bits[J >> 5], 1u << (J & 31));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < a.W; i += 64) a.bits[row * a.W + i] = bits[i];
}

// ------------------------------------------------------- transposed lists
// One wave per (b, g, 32 key blocks): pair x = h_local * M + I in ascending
// order; its bitmap word holds the 32 key blocks' bits.
__global__ __launch_bounds__(64) void bwd_cols_kernel(BwdArgs a) {
  const int lane = threadIdx.x;
  const int wi = blockIdx.x % a.W;
  const int grp = blockIdx.x / a.W;           // b * Hkv + g
  const int b = grp / a.Hkv, g = grp - (grp / a.Hkv) * a.Hkv;
  const int GM = a.G * a.M;
  int count[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) count[j] = 0;
  for (int x0 = 0; x0 < GM; x0 += 64) {
    const int x = x0 + lane;
    uint32_t word = 0u;
    if (x < GM) {
      const int hl = x / a.M, I = x - hl * a.M;
      word = a.bits[(((long)b * a.Hq + g * a.G + hl) * a.M + I) * a.W + wi];
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int J = 32 * wi + j;
      if (J >= a.M) break;
      const bool in = (word >> j) & 1u;
      const uint64_t bal = __ballot(in);
      if (in) a.col_idx[((long)grp * a.M + J) * GM + count[j] + lanes_below(bal)] = x;
      count[j] += __popcll(bal);
    }
  }
  if (lane < 32 && 32 * wi + lane < a.M) {
    int c = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) c = lane == j ? count[j] : c;
    a.col_cnt[(long)grp * a.M + 32 * wi + lane] = c;
  }
}

// ---------------------------------------------------------------- dq
// Workgroup per 64 query rows (four waves): a 128-row block is split over two
// workgroups, adjacent in the item order so they share its K/V tiles in L2.
template <int D, int BLK>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int NW = 4;
  constexpr int PARTS = BLK / 64;              // 64-row parts of a block
  constexpr int NT = 64 * NW;
  constexpr int SUB = BLK / BT;                // 64-key tiles per block
  using C = BC<D>;
  using DM = Dma<D, NW>;
  __shared__ __attribute__((aligned(1024))) char Kt[C::TB];
  __shared__ __attribute__((aligned(1024))) char Vt[C::TB];
  __shared__ uint32_t selbits[kMaxBlocks / 32];
  __shared__ uint16_t tail_rows[kMaxBlocks];

  const int total = a.B * a.Hq * a.M * PARTS;
  const int item = xcd_local_item(blockIdx.x, total);
  if (item < 0) return;
  const int part = item % PARTS;
  const int hg = (item / PARTS) % a.G;
  int rest = item / PARTS / a.G;
  const int I = a.M - 1 - rest % a.M;
  rest /= a.M;
  const int g = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int h = g * a.G + hg;
  const int bh = b * a.Hq + h;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int q_tok = I * BLK + 64 * part + 16 * w + lr;
  const bool q_ok = q_tok < a.N;
  const size_t qrow = (size_t)bh * a.N + (q_ok ? q_tok : 0);

  bf16x8 qf[C::NKS], gf[C::NKS];
  load_row<D>(qf, a.q + qrow * D, q_ok, lg);
  load_row<D>(gf, a.dout + qrow * D, q_ok, lg);
  const float nLc = q_ok ? a.delta[(size_t)a.B * a.Hq * a.N + qrow] : -INFINITY;   // P = 0 on padding rows
  const float Dd = q_ok ? a.delta[qrow] : 0.f;

  const int n_sel = scalar_view(a.cnt)[(size_t)bh * a.M + I];
  const const_i32* list = scalar_view(a.idx + ((size_t)bh * a.M + I) * a.M);
  const int Jend = a.causal ? I + 1 : a.M;
  const int last_n = a.N - (a.M - 1) * BLK;
  const int n_rest = a.approx ? Jend - n_sel : 0;
  const int n_tt = (n_rest + BT - 1) / BT;
  int edge = 0;   // the last listed block needs the edge mask (ragged end / diagonal)
  if (n_sel > 0) {
    const int J = list[n_sel - 1];
    edge = ((J + 1) * BLK > a.N || (a.causal && J >= I)) ? 1 : 0;
  }
  const int n_exact = SUB * n_sel;
  const int n_plain = n_exact - SUB * edge;
  const int n_tiles = n_exact + n_tt;
  const float log2_blk = __log2f((float)BLK);
  const float last_fix = (__log2f((float)last_n) - log2_blk) / a.scale_log2;

  if (a.approx) {
    for (int i = t; i < kMaxBlocks / 32; i += NT) selbits[i] = 0u;
    __syncthreads();
    for (int e = t; e < n_sel; e += NT) {
      const int J = list[e];
      atomicOr(&selbits[J >> 5], 1u << (J & 31));
    }
    __syncthreads();
    if (w == 0) {
      int base = 0;
      for (int J0 = 0; J0 < Jend; J0 += 64) {
        const int J = J0 + lane;
        const int Jc = J < Jend ? J : 0;
        const bool rest_J = J < Jend && !((selbits[Jc >> 5] >> (Jc & 31)) & 1u);
        const uint64_t bal = __ballot(rest_J);
        if (rest_J) tail_rows[base + lanes_below(bal)] = (uint16_t)J;
        base += __popcll(bal);
      }
    }
    __syncthreads();
  }

  const int head_bytes = a.N * C::ROWB;
  const size_t kv_off = (size_t)(b * a.Hkv + g) * a.N * D;
  const size_t pp_off = (size_t)(b * a.Hkv + g) * a.M * D;
  const __amdgpu_buffer_rsrc_t krs = head_rsrc(a.k + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(a.v + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t tkrs = head_rsrc(a.approx ? a.tail_k + pp_off : a.k, a.M * C::ROWB);
  const __amdgpu_buffer_rsrc_t tvrs = head_rsrc(a.approx ? a.tail_v + pp_off : a.v, a.M * C::ROWB);
  const int row0 = DM::row0(w, lane);
  const int col = DM::col(w, lane);
  const int voff = row0 * C::ROWB + col;
  const Frag<D> fr(lr, lg);

  // tile e: exact (key = first token) or tail (key = tail tile index)
  auto tile_key = [&](int e) -> int {
    return e < n_exact ? list[e / SUB] * BLK + (e % SUB) * BT : e - n_exact;
  };
  auto issue = [&](int e, int key, bool is_v) {
    char* dst = is_v ? Vt : Kt;
    if (e < n_exact) {
      DM::tile(is_v ? vrs : krs, key * C::ROWB, dst, w, voff);
    } else {
      int ro[DM::NI];
#pragma unroll
      for (int i = 0; i < DM::NI; ++i) {
        const int r = BT * key + row0 + i * NW * C::RPK;
        ro[i] = (r < n_rest ? (int)tail_rows[r] : 0) * C::ROWB;
      }
      DM::rows(is_v ? tvrs : tkrs, ro, col, dst, w);
    }
  };

  f32x4 dq[C::NOT];
#pragma unroll
  for (int i = 0; i < C::NOT; ++i) dq[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float c = a.scale_log2;

  int key = n_tiles > 0 ? tile_key(0) : 0;
  if (n_tiles > 0) {
    issue(0, key, false);
    issue(0, key, true);
  }
  wait_vm();
  __syncthreads();
  for (int e = 0; e < n_tiles; ++e) {
    f32x4 s[4], dp[4];
    __builtin_amdgcn_s_setprio(1);
    gemm_rows<D>(s, Kt, fr, qf);
    gemm_rows<D>(dp, Vt, fr, gf);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();                           // V tile free
    const int key1 = e + 1 < n_tiles ? tile_key(e + 1) : 0;
    if (e + 1 < n_tiles) issue(e + 1, key1, true);

    // masks: register r of row group tg holds key key + 16*tg + 4*lg + r
    float lb = 0.f;
    if (e >= n_exact) {
      lb = log2_blk;
      if (e == n_tiles - 1) {                  // padding rows, short last block
        const int lim = n_rest - BT * key - 4 * lg;
        const int fix_kr = (last_n != BLK && tail_rows[n_rest - 1] == a.M - 1) ? lim - 1 : -1;
#pragma unroll
        for (int tg = 0; tg < 4; ++tg)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int kr = 16 * tg + r;
            s[tg][r] = kr < lim ? (kr == fix_kr ? s[tg][r] + last_fix : s[tg][r]) : -INFINITY;
          }
      }
    } else if (e >= n_plain) {                 // ragged end / causal diagonal
      int lim = a.N - key;
      if (a.causal) lim = min(lim, q_tok - key + 1);
      lim -= 4 * lg;
#pragma unroll
      for (int tg = 0; tg < 4; ++tg)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[tg][r] = 16 * tg + r < lim ? s[tg][r] : -INFINITY;
    }
    // P = exp2(z log2 e + lb - L log2 e), dS = P (dP - D)
    const float off = lb + nLc;
#pragma unroll
    for (int tg = 0; tg < 4; ++tg)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[tg][r], c, off));
        s[tg][r] = p * (dp[tg][r] - Dd);
      }
    bf16x8 pk[2];
    pack_rows(s, pk);
    __builtin_amdgcn_s_setprio(1);
    gemm_tr<D>(dq, Kt, fr, pk);                // dQ^T += K^T dS^T
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();                           // K tile free
    if (e + 1 < n_tiles) issue(e + 1, key1, false);
    wait_vm();
    __syncthreads();
    key = key1;
  }

  // dq straight from the fragments: a staged store would take this pass
  // (128 registers at four waves per SIMD) past its register budget
  if (q_ok) {
    uint16_t* orow = a.dq + qrow * D;
#pragma unroll
    for (int nt = 0; nt < C::NOT; ++nt) {
      const u32x2 x = {pack2(dq[nt][0] * a.scale, dq[nt][1] * a.scale),
                       pack2(dq[nt][2] * a.scale, dq[nt][3] * a.scale)};
      *reinterpret_cast<u32x2*>(orow + 16 * nt + 4 * lg) = x;
    }
  }
}

// dq for 128-row blocks: two 16-row groups per wave, so every K, V and K^T
// fragment read from LDS feeds the products of both groups (half the LDS
// operand bytes per product of the one-group form above; −13% on the dq
// pass at 128K).  Workgroup = one query block, four waves of 32 rows, two
// workgroups per CU (234 registers).  Same arithmetic, in the same order, as
// the one-group form: the gradients are bit-identical.
template <int D>
__device__ __forceinline__ void gemm_rows_g2(f32x4 (&acc)[2][4], const char* tile, const Frag<D>& f,
                                             const bf16x8 (&rg)[2][BC<D>::NKS]) {
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) acc[g][tg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < BC<D>::NKS; ++s)
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(tile + f.rb[s] + 16 * tg * BC<D>::ROWB);
#pragma unroll
      for (int g = 0; g < 2; ++g) acc[g][tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, rg[g][s], acc[g][tg], 0, 0, 0);
    }
}

template <int D>
__device__ __forceinline__ void gemm_tr_g2(f32x4 (&acc)[2][BC<D>::NOT], const char* tile, const Frag<D>& f,
                                           const bf16x8 (&pk)[2][2]) {
#pragma unroll
  for (int nt = 0; nt < BC<D>::NOT; ++nt)
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const bf16x8 a = tr_frag<D>(tile, f, nt, cc);
#pragma unroll
      for (int g = 0; g < 2; ++g) acc[g][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pk[g][cc], acc[g][nt], 0, 0, 0);
    }
}

template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq2_kernel(BwdArgs a) {
  constexpr int BLK = 128;
  constexpr int NW = 4;
  constexpr int NT = 64 * NW;
  constexpr int SUB = BLK / BT;                // 64-key tiles per block
  using C = BC<D>;
  using DM = Dma<D, NW>;
  __shared__ __attribute__((aligned(1024))) char Kt[C::TB];
  __shared__ __attribute__((aligned(1024))) char Vt[C::TB];
  __shared__ uint32_t selbits[kMaxBlocks / 32];
  __shared__ uint16_t tail_rows[kMaxBlocks];

  const int total = a.B * a.Hq * a.M;
  const int item = xcd_local_item(blockIdx.x, total);
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
  const int lr = lane & 15, lg = lane >> 4;
  // row group rg: query row I*BLK + 32w + 16rg + lr
  int q_tok[2];
  bf16x8 qf[2][C::NKS], gf[2][C::NKS];
  float nLc[2], Dd[2];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    q_tok[rg] = I * BLK + 32 * w + 16 * rg + lr;
    const bool ok = q_tok[rg] < a.N;
    const size_t qrow = (size_t)bh * a.N + (ok ? q_tok[rg] : 0);
    load_row<D>(qf[rg], a.q + qrow * D, ok, lg);
    load_row<D>(gf[rg], a.dout + qrow * D, ok, lg);
    nLc[rg] = ok ? a.delta[(size_t)a.B * a.Hq * a.N + qrow] : -INFINITY;   // P = 0 on padding rows
    Dd[rg] = ok ? a.delta[qrow] : 0.f;
  }

  const int n_sel = scalar_view(a.cnt)[(size_t)bh * a.M + I];
  const const_i32* list = scalar_view(a.idx + ((size_t)bh * a.M + I) * a.M);
  const int Jend = a.causal ? I + 1 : a.M;
  const int last_n = a.N - (a.M - 1) * BLK;
  const int n_rest = a.approx ? Jend - n_sel : 0;
  const int n_tt = (n_rest + BT - 1) / BT;
  int edge = 0;
  if (n_sel > 0) {
    const int J = list[n_sel - 1];
    edge = ((J + 1) * BLK > a.N || (a.causal && J >= I)) ? 1 : 0;
  }
  const int n_exact = SUB * n_sel;
  const int n_plain = n_exact - SUB * edge;
  const int n_tiles = n_exact + n_tt;
  const float log2_blk = __log2f((float)BLK);
  const float last_fix = (__log2f((float)last_n) - log2_blk) / a.scale_log2;

  if (a.approx) {
    for (int i = t; i < kMaxBlocks / 32; i += NT) selbits[i] = 0u;
    __syncthreads();
    for (int e = t; e < n_sel; e += NT) {
      const int J = list[e];
      atomicOr(&selbits[J >> 5], 1u << (J & 31));
    }
    __syncthreads();
    if (w == 0) {
      int base = 0;
      for (int J0 = 0; J0 < Jend; J0 += 64) {
        const int J = J0 + lane;
        const int Jc = J < Jend ? J : 0;
        const bool rest_J = J < Jend && !((selbits[Jc >> 5] >> (Jc & 31)) & 1u);
        const uint64_t bal = __ballot(rest_J);
        if (rest_J) tail_rows[base + lanes_below(bal)] = (uint16_t)J;
        base += __popcll(bal);
      }
    }
    __syncthreads();
  }

  const int head_bytes = a.N * C::ROWB;
  const size_t kv_off = (size_t)(b * a.Hkv + g) * a.N * D;
  const size_t pp_off = (size_t)(b * a.Hkv + g) * a.M * D;
  const __amdgpu_buffer_rsrc_t krs = head_rsrc(a.k + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(a.v + kv_off, head_bytes);
  const __amdgpu_buffer_rsrc_t tkrs = head_rsrc(a.approx ? a.tail_k + pp_off : a.k, a.M * C::ROWB);
  const __amdgpu_buffer_rsrc_t tvrs = head_rsrc(a.approx ? a.tail_v + pp_off : a.v, a.M * C::ROWB);
  const int row0 = DM::row0(w, lane);
  const int col = DM::col(w, lane);
  const int voff = row0 * C::ROWB + col;
  const Frag<D> fr(lr, lg);

  auto tile_key = [&](int e) -> int {
    return e < n_exact ? list[e / SUB] * BLK + (e % SUB) * BT : e - n_exact;
  };
  auto issue = [&](int e, int key, bool is_v) {
    char* dst = is_v ? Vt : Kt;
    if (e < n_exact) {
      DM::tile(is_v ? vrs : krs, key * C::ROWB, dst, w, voff);
    } else {
      int ro[DM::NI];
#pragma unroll
      for (int i = 0; i < DM::NI; ++i) {
        const int r = BT * key + row0 + i * NW * C::RPK;
        ro[i] = (r < n_rest ? (int)tail_rows[r] : 0) * C::ROWB;
      }
      DM::rows(is_v ? tvrs : tkrs, ro, col, dst, w);
    }
  };

  f32x4 dq[2][C::NOT];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg)
#pragma unroll
    for (int i = 0; i < C::NOT; ++i) dq[rg][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float c = a.scale_log2;

  int key = n_tiles > 0 ? tile_key(0) : 0;
  if (n_tiles > 0) {
    issue(0, key, false);
    issue(0, key, true);
  }
  wait_vm();
  __syncthreads();
  for (int e = 0; e < n_tiles; ++e) {
    f32x4 s[2][4], dp[2][4];
    __builtin_amdgcn_s_setprio(1);
    gemm_rows_g2<D>(s, Kt, fr, qf);
    gemm_rows_g2<D>(dp, Vt, fr, gf);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();                           // V tile free
    const int key1 = e + 1 < n_tiles ? tile_key(e + 1) : 0;
    if (e + 1 < n_tiles) issue(e + 1, key1, true);

    float lb = 0.f;
    if (e >= n_exact) {
      lb = log2_blk;
      if (e == n_tiles - 1) {
        const int lim = n_rest - BT * key - 4 * lg;
        const int fix_kr = (last_n != BLK && tail_rows[n_rest - 1] == a.M - 1) ? lim - 1 : -1;
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
#pragma unroll
          for (int tg = 0; tg < 4; ++tg)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int kr = 16 * tg + r;
              s[rg][tg][r] = kr < lim ? (kr == fix_kr ? s[rg][tg][r] + last_fix : s[rg][tg][r]) : -INFINITY;
            }
      }
    } else if (e >= n_plain) {
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) {
        int lim = a.N - key;
        if (a.causal) lim = min(lim, q_tok[rg] - key + 1);
        lim -= 4 * lg;
#pragma unroll
        for (int tg = 0; tg < 4; ++tg)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[rg][tg][r] = 16 * tg + r < lim ? s[rg][tg][r] : -INFINITY;
      }
    }
    bf16x8 pk[2][2];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const float off = lb + nLc[rg];
#pragma unroll
      for (int tg = 0; tg < 4; ++tg)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[rg][tg][r], c, off));
          s[rg][tg][r] = p * (dp[rg][tg][r] - Dd[rg]);
        }
      pack_rows(s[rg], pk[rg]);
    }
    __builtin_amdgcn_s_setprio(1);
    gemm_tr_g2<D>(dq, Kt, fr, pk);             // dQ^T += K^T dS^T
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();                           // K tile free
    if (e + 1 < n_tiles) issue(e + 1, key1, false);
    wait_vm();
    __syncthreads();
    key = key1;
  }

#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    if (q_tok[rg] < a.N) {
      uint16_t* orow = a.dq + ((size_t)bh * a.N + q_tok[rg]) * D;
#pragma unroll
      for (int nt = 0; nt < C::NOT; ++nt) {
        const u32x2 x = {pack2(dq[rg][nt][0] * a.scale, dq[rg][nt][1] * a.scale),
                         pack2(dq[rg][nt][2] * a.scale, dq[rg][nt][3] * a.scale)};
        *reinterpret_cast<u32x2*>(orow + 16 * nt + 4 * lg) = x;
      }
    }
  }
}

// --------------------------------------------------- dk/dv and pooled grads
// Shared body: NW waves, 16 register rows each (keys or pooled rows); loops
// over 64-row query tiles handed out by `next`.  POOLED: register rows are
// pooled rows with per-lane log2 weight `lw` (-inf: not in this query
// block's tail); otherwise key tokens with the causal mask on the diagonal.
template <int D, int NW, bool POOLED>
struct KvAcc {
  f32x4 dk[BC<D>::NOT];
  f32x4 dv[BC<D>::NOT];
};

template <int D, int NW, bool POOLED>
__device__ __forceinline__ void kv_tile(const BwdArgs& a, KvAcc<D, NW, POOLED>& acc, const char* Qt, const char* Ot,
                                        const float* nLt, const float* Dt, const Frag<D>& fr,
                                        const bf16x8 (&kf)[BC<D>::NKS], const bf16x8 (&vf)[BC<D>::NKS],
                                        int lg, float lw, bool diag, int diag_lim) {
  f32x4 s[4], dp[4];
  // matrix phases at raised wave priority (the other waves of the SIMD fill
  // the gaps with their vector work)
  __builtin_amdgcn_s_setprio(1);
  // dk/dv: the products read their LDS operands through the read-ahead
  // ring (two waves per SIMD leave LDS latency exposed otherwise; 6% faster
  // at 128K).  The pooled pass (three waves per SIMD) and the dq pass (four)
  // measured faster with the compiler's own schedule, which needs fewer
  // registers.
  constexpr bool RING = !POOLED;
  if constexpr (RING) {
    gemm_rows2<D>(s, Qt, kf, dp, Ot, vf, fr);   // S = Q K^T, dP = dO V^T (rows: queries)
  } else {
    gemm_rows<D>(s, Qt, fr, kf);
    gemm_rows<D>(dp, Ot, fr, vf);
  }
  __builtin_amdgcn_s_setprio(0);
  const float c = a.scale_log2;
  // causal diagonal (a tile of the key block's own query block, the same
  // for the whole workgroup): query row 16tg + 4lg + r sees the key only at
  // or after it
  if (!POOLED && diag) {
#pragma unroll
    for (int tg = 0; tg < 4; ++tg)
#pragma unroll
      for (int r = 0; r < 4; ++r) s[tg][r] = 16 * tg + 4 * lg + r >= diag_lim ? s[tg][r] : -INFINITY;
  }
#pragma unroll
  for (int tg = 0; tg < 4; ++tg) {
    const f32x4 nL = *reinterpret_cast<const f32x4*>(nLt + 16 * tg + 4 * lg);
    const f32x4 Dv = *reinterpret_cast<const f32x4*>(Dt + 16 * tg + 4 * lg);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[tg][r], c, POOLED ? lw + nL[r] : nL[r]));
      s[tg][r] = p;
      dp[tg][r] = p * (dp[tg][r] - Dv[r]);
    }
  }
  bf16x8 pk[2], dk_[2];
  pack_rows(s, pk);
  pack_rows(dp, dk_);
  __builtin_amdgcn_s_setprio(1);
  if constexpr (RING) {
    gemm_tr2<D>(acc.dv, Ot, pk, acc.dk, Qt, dk_, fr);   // dV^T += dO^T P, dK^T += Q^T dS
  } else {
    gemm_tr<D>(acc.dv, Ot, fr, pk);
    gemm_tr<D>(acc.dk, Qt, fr, dk_);
  }
  __builtin_amdgcn_s_setprio(0);
}

// Query tile (rows q0.. of head bh) into Qt/Ot, the -L log2 e and D values
// of its rows into Lt/Dt, all by loads into LDS (waves 0 and 1 move the 64
// floats).  Rows past the end of the sequence read zeros: Q and dO rows of
// zero make P dO, dP and D zero there, so such rows add nothing.
template <int D, int NW>
__device__ __forceinline__ void issue_query_tile(const BwdArgs& a, int bh, int q0, char* Qt, char* Ot, float* Lt,
                                                 float* Dt, int w, int voff) {
  using DM = Dma<D, NW>;
  const int head_bytes = a.N * BC<D>::ROWB;
  DM::tile(head_rsrc(a.q + (size_t)bh * a.N * D, head_bytes), q0 * BC<D>::ROWB, Qt, w, voff);
  DM::tile(head_rsrc(a.dout + (size_t)bh * a.N * D, head_bytes), q0 * BC<D>::ROWB, Ot, w, voff);
  if (w < 2) {
    const long rows = (long)a.B * a.Hq * a.N;
    const float* src = (w == 0 ? a.delta + rows : a.delta) + (size_t)bh * a.N;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, a.N * 4, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(w == 0 ? Lt : Dt), 4, q0 * 4 + (threadIdx.x & 63) * 4, 0, 0,
                                             0);
  }
}

// Workgroup per 64 keys (four waves): a 128-row block is split over two
// workgroups, adjacent in the item order so they share its query tiles in L2
// (two independent workgroups per CU hide each other's barriers).
template <int D, int BLK>
__global__ __launch_bounds__(256, 2) void bwd_dkv_kernel(BwdArgs a) {
  constexpr int NW = 4;
  constexpr int PARTS = BLK / 64;              // 64-key parts of a block
  constexpr int SUB = BLK / BT;
  using C = BC<D>;
  using DM = Dma<D, NW>;
  // double-buffered query tiles (Q, dO, and the -L log2 e, D of their rows), each
  // buffer a separate LDS object named statically in the unrolled loop
  __shared__ __attribute__((aligned(1024))) char Q0[C::TB];
  __shared__ __attribute__((aligned(1024))) char Q1[C::TB];
  __shared__ __attribute__((aligned(1024))) char O0[C::TB];
  __shared__ __attribute__((aligned(1024))) char O1[C::TB];
  __shared__ __attribute__((aligned(16))) float L0[BT];
  __shared__ __attribute__((aligned(16))) float L1[BT];
  __shared__ __attribute__((aligned(16))) float D0[BT];
  __shared__ __attribute__((aligned(16))) float D1[BT];

  const int total = a.B * a.Hkv * a.M * PARTS;
  const int item = xcd_local_item(blockIdx.x, total);
  if (item < 0) return;
  const int part = item % PARTS;
  const int blk = item / PARTS;
  const int grp = blk / a.M;                   // b * Hkv + g
  const int J = blk - grp * a.M;
  const int b = grp / a.Hkv;
  const int g = grp - b * a.Hkv;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int k_tok = J * BLK + 64 * part + 16 * w + lr;
  const bool k_ok = k_tok < a.N;
  const size_t krow = (size_t)grp * a.N + (k_ok ? k_tok : 0);
  bf16x8 kf[C::NKS], vf[C::NKS];
  load_row<D>(kf, a.k + krow * D, k_ok, lg);
  load_row<D>(vf, a.v + krow * D, k_ok, lg);

  const int voff = DM::row0(w, lane) * C::ROWB + DM::col(w, lane);
  const Frag<D> fr(lr, lg);
  KvAcc<D, NW, false> acc;
#pragma unroll
  for (int i = 0; i < C::NOT; ++i) {
    acc.dk[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc.dv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int GM = a.G * a.M;
  const int n_col = scalar_view(a.col_cnt)[(size_t)grp * a.M + J];
  const const_i32* cl = scalar_view(a.col_idx + ((size_t)grp * a.M + J) * GM);
  // tile t: sub-tile t % SUB of the query block of list entry t / SUB (a
  // sub-tile past the end of the sequence has no valid rows: L = +inf there,
  // so it adds nothing)
  const int n_t = n_col * SUB;
  auto tile_of = [&](int tt, int& bh, int& q0, int& I) {
    const int x = cl[tt / SUB];
    const int hl = x / a.M;
    I = x - hl * a.M;
    bh = b * a.Hq + g * a.G + hl;
    q0 = I * BLK + BT * (tt % SUB);
  };

  int bh0 = 0, q00 = 0, I0 = 0;
  if (n_t > 0) {
    tile_of(0, bh0, q00, I0);
    issue_query_tile<D, NW>(a, bh0, q00, Q0, O0, L0, D0, w, voff);
  }
  wait_vm();
  __syncthreads();
  // one tile: Qc/Oc/Lc/Dc hold tile tt; tile tt+1 goes to Qn/On/Ln/Dn
  auto step = [&](int tt, const char* Qc, const char* Oc, const float* Lc, const float* Dc, char* Qn, char* On,
                  float* Ln, float* Dn) __attribute__((always_inline)) {
    int bh1 = 0, q01 = 0, I1 = 0;
    if (tt + 1 < n_t) {
      tile_of(tt + 1, bh1, q01, I1);
      issue_query_tile<D, NW>(a, bh1, q01, Qn, On, Ln, Dn, w, voff);
    }
    // causal diagonal: row r of the tile (token q0 + r) sees key k_tok iff
    // r >= k_tok - q0
    kv_tile<D, NW, false>(a, acc, Qc, Oc, Lc, Dc, fr, kf, vf, lg, 0.f, a.causal && I0 == J, k_tok - q00);
    wait_vm();
    __syncthreads();
    bh0 = bh1;
    q00 = q01;
    I0 = I1;
  };
  for (int tt = 0; tt < n_t; tt += 2) {
    step(tt, Q0, O0, L0, D0, Q1, O1, L1, D1);
    if (tt + 1 < n_t) step(tt + 1, Q1, O1, L1, D1, Q0, O0, L0, D0);
  }

  // Gradients of this block's pooled key and mean value: the sum of the
  // pooled pass's partials, one component per thread (t < 2D), into the
  // query buffer Q0 (free: the loop ended with a barrier).
  const float* pooled = reinterpret_cast<const float*>(Q0);
  if (a.approx) {
    static_assert(64 * NW >= 2 * D && 2 * D * 4 <= C::TB, "pooled-gradient reduction layout");
    if (t < 2 * D) {
      const size_t pstride = (size_t)a.B * a.Hkv * a.M * D;   // between chunks' partial sums
      const float* src = (t < D ? a.dk_bar : a.dv_bar) + ((size_t)grp * a.M + J) * D + (t % D);
      float sum = 0.f;
#pragma unroll
      for (int c = 0; c < kTailChunks; ++c) sum += src[c * pstride];
      reinterpret_cast<float*>(Q0)[t] = sum;
    }
    __syncthreads();
  }
  // dk, dv of the wave's 16 keys (row lr, d = 16*nt + 4*lg + r) through its
  // quarters of the free Q1 and O1 buffers (staged row store; Q0 holds the
  // pooled sums)
  {
    const float n = (float)min(BLK, a.N - J * BLK);
    char* sk = Q1 + w * 16 * C::ROWB;
    char* sv = O1 + w * 16 * C::ROWB;
#pragma unroll
    for (int nt = 0; nt < C::NOT; ++nt) {
      const int d0 = 16 * nt + 4 * lg;
      f32x4 x = acc.dk[nt] * a.scale, y = acc.dv[nt];
      if (a.approx) {   // spread evenly over the block's tokens
        x += *reinterpret_cast<const f32x4*>(pooled + d0) / n;
        y += *reinterpret_cast<const f32x4*>(pooled + D + d0) / n;
      }
      const int off = lr * C::ROWB + stage_slot<D>(lr, 2 * nt + (lg >> 1)) * 16 + 8 * (lg & 1);
      *reinterpret_cast<u32x2*>(sk + off) = u32x2{pack2(x[0], x[1]), pack2(x[2], x[3])};
      *reinterpret_cast<u32x2*>(sv + off) = u32x2{pack2(y[0], y[1]), pack2(y[2], y[3])};
    }
    const int tok0 = J * BLK + 64 * part + 16 * w;   // the wave's first key token
    const size_t obase = ((size_t)grp * a.N + tok0) * D;
    store_staged_rows<D, 16>(sk, a.dk + obase, a.N - tok0, lane);
    store_staged_rows<D, 16>(sv, a.dv + obase, a.N - tok0, lane);
  }
}

// Pooled gradients: workgroup per (b, g, 64 pooled rows, chunk), four
// waves.  The chunk's (query head, query block) pairs are taken 256 at a
// time: each thread tests one pair against the selection bitmap (is any of
// the 64 pooled rows in that query block's tail?) and the pairs that pass
// are compacted in ascending order into LDS with the 64-bit mask of rows in
// the tail.  Their query tiles then stream through double-buffered LDS like
// the dk/dv pass: the next tile loads while the current one is used.
template <int D, int BLK>
__global__ __launch_bounds__(256, 2) void bwd_dtail_kernel(BwdArgs a) {
  constexpr int NW = 4;
  constexpr int SUB = BLK / BT;
  constexpr int WIN = 64 * NW;                 // pairs tested per window
  using C = BC<D>;
  using DM = Dma<D, NW>;
  __shared__ __attribute__((aligned(1024))) char Q0[C::TB];
  __shared__ __attribute__((aligned(1024))) char Q1[C::TB];
  __shared__ __attribute__((aligned(1024))) char O0[C::TB];
  __shared__ __attribute__((aligned(1024))) char O1[C::TB];
  __shared__ __attribute__((aligned(16))) float L0[BT];
  __shared__ __attribute__((aligned(16))) float L1[BT];
  __shared__ __attribute__((aligned(16))) float D0[BT];
  __shared__ __attribute__((aligned(16))) float D1[BT];
  __shared__ int xs[WIN];                      // passing pairs x = hl * M + I
  __shared__ uint64_t xmask[WIN];              // their rows in the tail (bit j: row 64pt + j)
  __shared__ int wcnt[NW];

  const int tiles = (a.M + BT - 1) / BT;
  const int chunk = blockIdx.x % kTailChunks;
  const int grp = blockIdx.x / kTailChunks / tiles;   // b * Hkv + g
  const int pt = blockIdx.x / kTailChunks - grp * tiles;
  const int b = grp / a.Hkv;
  const int g = grp - b * a.Hkv;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int Jl = BT * pt + 16 * w + lr;        // this lane's pooled row
  const bool j_ok = Jl < a.M;
  const size_t prow = (size_t)grp * a.M + (j_ok ? Jl : 0);
  bf16x8 kf[C::NKS], vf[C::NKS];
  load_row<D>(kf, a.tail_k + prow * D, j_ok, lg);
  load_row<D>(vf, a.tail_v + prow * D, j_ok, lg);
  const int nJ = Jl == a.M - 1 ? a.N - (a.M - 1) * a.block : a.block;
  const float lw_in = __log2f((float)nJ);

  const int voff = DM::row0(w, lane) * C::ROWB + DM::col(w, lane);
  const Frag<D> fr(lr, lg);
  KvAcc<D, NW, true> acc;
#pragma unroll
  for (int i = 0; i < C::NOT; ++i) {
    acc.dk[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc.dv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // this workgroup's share of the (query head, query block) pairs x =
  // hl * M + I
  const int GM = a.G * a.M;
  const int per = (GM + kTailChunks - 1) / kTailChunks;
  const int x1 = min(GM, (chunk + 1) * per);
  for (int xw = chunk * per; xw < x1; xw += WIN) {
    // ---- test and compact: pooled row 64pt + j is in the tail of (bh, I)
    // when it is eligible (below M, and at most I when causal) and not
    // listed; words 2pt and 2pt + 1 of the bitmap row hold those 64 rows
    uint64_t m = 0;
    const int x = xw + t;
    if (x < x1) {
      const int hl = x / a.M, I = x - hl * a.M;
      const int bh = b * a.Hq + g * a.G + hl;
      const uint32_t* row = a.bits + ((size_t)bh * a.M + I) * a.W;
      const uint32_t lo = row[2 * pt];
      const uint32_t hi = 2 * pt + 1 < a.W ? row[2 * pt + 1] : 0xFFFFFFFFu;
      const int lim = min(a.M, a.causal ? I + 1 : a.M) - BT * pt;
      const uint64_t valid = lim >= 64 ? ~0ull : (lim <= 0 ? 0ull : (1ull << lim) - 1ull);
      m = ~(((uint64_t)hi << 32) | lo) & valid;
    }
    const uint64_t bal = __ballot(m != 0);
    if (lane == 0) wcnt[w] = __popcll(bal);
    __syncthreads();
    int base = 0, n = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      base += i < w ? wcnt[i] : 0;
      n += wcnt[i];
    }
    if (m != 0) {
      const int pos = base + lanes_below(bal);
      xs[pos] = x;
      xmask[pos] = m;
    }
    __syncthreads();

    // ---- the passing pairs' query tiles (SUB per query block), pipelined
    const int n_t = n * SUB;
    // tile tt: head row bh, first query row q0, this lane's log2 weight
    auto tile_of = [&](int tt, int& bh, int& q0, float& lw) {
      const int e = tt / SUB;
      const int xe = xs[e];
      const int hl = xe / a.M, I = xe - hl * a.M;
      bh = b * a.Hq + g * a.G + hl;
      q0 = I * a.block + BT * (tt % SUB);
      lw = ((xmask[e] >> (16 * w + lr)) & 1ull) ? lw_in : -INFINITY;
    };
    int bh0 = 0, q00 = 0;
    float lw0 = 0.f;
    if (n_t > 0) {
      tile_of(0, bh0, q00, lw0);
      issue_query_tile<D, NW>(a, bh0, q00, Q0, O0, L0, D0, w, voff);
    }
    wait_vm();
    __syncthreads();
    auto step = [&](int tt, const char* Qc, const char* Oc, const float* Lc, const float* Dc, char* Qn, char* On,
                    float* Ln, float* Dn) __attribute__((always_inline)) {
      int bh1 = 0, q01 = 0;
      float lw1 = 0.f;
      if (tt + 1 < n_t) {
        tile_of(tt + 1, bh1, q01, lw1);
        issue_query_tile<D, NW>(a, bh1, q01, Qn, On, Ln, Dn, w, voff);
      }
      // a sub-tile past the end of the sequence (the last block's second
      // half) has no rows: skipped
      if (q00 < a.N) kv_tile<D, NW, true>(a, acc, Qc, Oc, Lc, Dc, fr, kf, vf, lg, lw0, false, 0);
      wait_vm();
      __syncthreads();
      bh0 = bh1;
      q00 = q01;
      lw0 = lw1;
    };
    for (int tt = 0; tt < n_t; tt += 2) {
      step(tt, Q0, O0, L0, D0, Q1, O1, L1, D1);
      if (tt + 1 < n_t) step(tt + 1, Q1, O1, L1, D1, Q0, O0, L0, D0);
    }
  }
  if (j_ok) {   // this chunk's partial sums
    const size_t part = (size_t)chunk * a.B * a.Hkv * a.M + prow;
    float* kb = a.dk_bar + part * D;
    float* vb = a.dv_bar + part * D;
#pragma unroll
    for (int nt = 0; nt < C::NOT; ++nt) {
      const int d0 = 16 * nt + 4 * lg;
      *reinterpret_cast<f32x4*>(kb + d0) = acc.dk[nt] * a.scale;
      *reinterpret_cast<f32x4*>(vb + d0) = acc.dv[nt];
    }
  }
}

template <int D, int BLK>
hipError_t run_bwd(const BwdArgs& a, hipStream_t st) {
  const long rows = (long)a.B * a.Hq * a.N;
  hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((rows * (D / 8) + 255) / 256)), dim3(256), 0, st, a);
  hipLaunchKernelGGL(bwd_bitmap_kernel, dim3(a.B * a.Hq * a.M), dim3(64), 0, st, a);
  hipLaunchKernelGGL(bwd_cols_kernel, dim3(a.B * a.Hkv * a.W), dim3(64), 0, st, a);
  if constexpr (BLK == 128) {
    const int nq = a.B * a.Hq * a.M;
    hipLaunchKernelGGL((bwd_dq2_kernel<D>), dim3(8 * ((nq + 7) / 8)), dim3(256), 0, st, a);
  } else {
    const int nq = a.B * a.Hq * a.M * (BLK / 64);
    hipLaunchKernelGGL((bwd_dq_kernel<D, BLK>), dim3(8 * ((nq + 7) / 8)), dim3(256), 0, st, a);
  }
  if (a.approx) {
    const int tiles = (a.M + BT - 1) / BT;
    hipLaunchKernelGGL((bwd_dtail_kernel<D, BLK>), dim3(a.B * a.Hkv * tiles * kTailChunks), dim3(256), 0, st,
                       a);
  }
  const int nk = a.B * a.Hkv * a.M * (BLK / 64);
  hipLaunchKernelGGL((bwd_dkv_kernel<D, BLK>), dim3(8 * ((nk + 7) / 8)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

BwdSizes bwd_sizes(const Shape& s, int approx) {
  BwdSizes z{};
  const size_t W = (size_t)(s.M + 31) / 32;
  z.lse = (size_t)s.B * s.Hq * s.N * sizeof(float);
  z.delta = 2 * z.lse;   // D, then -L log2 e
  z.sel_bits = (size_t)s.B * s.Hq * s.M * W * sizeof(uint32_t);
  z.col_idx = (size_t)s.B * s.Hq * s.M * s.M * sizeof(int32_t);
  z.col_cnt = (size_t)s.B * s.Hkv * s.M * sizeof(int32_t);
  z.dk_bar = approx ? (size_t)kTailChunks * s.B * s.Hkv * s.M * s.D * sizeof(float) : 0;
  z.dv_bar = z.dk_bar;
  return z;
}

hipError_t launch_bwd(const Shape& s, const BwdParams& p, const BwdPtrs& x, hipStream_t st) {
  BwdArgs a{};
  a.q = static_cast<const uint16_t*>(x.q);
  a.k = static_cast<const uint16_t*>(x.k);
  a.v = static_cast<const uint16_t*>(x.v);
  a.out = static_cast<const uint16_t*>(x.out);
  a.dout = static_cast<const uint16_t*>(x.dout);
  if (p.approx) {
    a.tail_k = static_cast<const uint16_t*>(x.tail);
    a.tail_v = a.tail_k + (size_t)s.B * s.Hkv * s.M * s.D;
  }
  a.idx = x.blk_idx;
  a.cnt = x.blk_cnt;
  a.lse = x.lse;
  a.delta = x.delta;
  a.bits = x.sel_bits;
  a.col_idx = x.col_idx;
  a.col_cnt = x.col_cnt;
  a.dk_bar = x.dk_bar;
  a.dv_bar = x.dv_bar;
  a.dq = static_cast<uint16_t*>(x.dq);
  a.dk = static_cast<uint16_t*>(x.dk);
  a.dv = static_cast<uint16_t*>(x.dv);
  a.B = s.B;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.N = s.N;
  a.M = s.M;
  a.G = s.Hq / s.Hkv;
  a.W = (s.M + 31) / 32;
  a.block = s.block;
  a.scale = p.scale;
  a.scale_log2 = p.scale * kLog2e;
  a.causal = p.causal;
  a.approx = p.approx;
  if (s.D == 128) return s.block == 128 ? run_bwd<128, 128>(a, st) : run_bwd<128, 64>(a, st);
  return s.block == 128 ? run_bwd<64, 128>(a, st) : run_bwd<64, 64>(a, st);
}

}  // namespace sa
