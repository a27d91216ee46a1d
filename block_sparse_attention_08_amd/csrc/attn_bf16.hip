// Stage 3 for bf16 inputs: block-sparse flash attention on the gfx950 matrix
// cores, with the 0th-order tail.
//
// What is computed (per query token i of query block I, head h):
//   exact part  -- softmax over the tokens of the listed key blocks J
//                  (index-driven: the K/V tile address is base + J*block*d,
//                  FlashPrefill summary 2(c)), causal mask j <= i inside the
//                  diagonal block, keys past N masked;
//   tail        -- with approx=1 every eligible unlisted block J is one
//                  pseudo-key kbar_J with weight n_J in the normaliser and the
//                  value sum SigmaV_J in the numerator (PISA explainer,
//                  routing table and "why softmax survives"), evaluated as
//                  logit + ln n_J with value SigmaV_J / n_J;
//   both are folded into one running max / sum (FlashAttention tutorial,
//   section 2, online softmax), answer o / l.
//
// Mapping: one workgroup per (batch, head, query block) with block/32 waves;
// wave w owns 32 query rows.  Per key tile (one block of `block` keys, or
// `block` pooled rows for the tail):
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16; A = K tile rows read from LDS,
//                 B = the wave's Q rows (registers for the whole kernel).
//                 The accumulator holds one query row per lane (lanes l and
//                 l+32 share row l%32, 16 keys each), so the row max needs
//                 one cross-lane exchange and the softmax state is per lane.
//   P = exp2(S*scale*log2e - m), packed to bf16 in place: these registers are
//                 directly the B operand of the next product.
//   O^T += V^T P^T  A = V^T fragments gathered from the row-major V tile with
//                 the LDS transpose read (ds_read_b64_tr_b16).
// The running max is only moved (and O, l rescaled) when a row's max grows
// by more than 8 in log2 units, so p <= 256 and most tiles skip the rescale.
//
// K/V tiles travel HBM -> LDS with buffer_load_dwordx4 ... lds (no
// registers), through buffer resources whose range check returns zero past
// the last key.  Each wave instruction fills 1 KB of LDS contiguously, so
// every lane picks the global 16-byte chunk that belongs at its LDS slot:
// the LDS tiles are row-major with 16-byte chunks XOR-swizzled by row, which
// keeps the MFMA operand reads free of bank conflicts without padding.
// This kernel serves 128-row query blocks (64-row blocks go to the 16-row-
// per-wave kernel): K and V are double-buffered and the loop is software-
// pipelined -- S of tile e+1 sits next to the softmax of tile e, one barrier
// per tile.  Tail tiles take the same path:
// KT pooled rows of the bf16 block means of k and v that the pool pass
// wrote once per head.
// Workgroups are ordered so that each XCD receives a contiguous range of
// (kv head, query block) items, with the query heads of one KV group
// adjacent, so K/V blocks shared by neighbouring items stay in one L2.
#include <math.h>

#include "attn_common.h"
#include "device_common.h"
#include "launch.h"

namespace sa {

hipError_t launch_fwd_f32(const Shape& s, const FwdParams& p, const void* q, const void* k,
                          const void* v, const float* k_bar, const float* v_sum,
                          const int32_t* blk_idx, const int32_t* blk_cnt, void* out,
                          hipStream_t st);
hipError_t launch_fwd_w16(const Shape& s, const FwdParams& p, const void* q, const void* k,
                          const void* v, const void* tail, const int32_t* blk_idx,
                          const int32_t* blk_cnt, void* out, hipStream_t st);

namespace {

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* tail_k;   // [B, Hkv, M, D] bf16 block means of k
  const uint16_t* tail_v;   // [B, Hkv, M, D] bf16 block means of v
  const int32_t* idx;
  const int32_t* cnt;
  uint16_t* out;
  int Hq, Hkv, N, M, G, total;
  float scale_log2;  // scale * log2(e)
  int causal, approx;
};

template <int D, int BLK>
struct Cfg {
  static constexpr int NW = BLK / 32;         // waves
  static constexpr int NT = 64 * NW;          // threads
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int NI = KT * CPR / NT;    // 16-byte loads per thread per tile
  static constexpr int NKS = D / 16;          // 16-wide d steps of S
  static constexpr int NOT = D / 32;          // 32-wide d tiles of O
  static constexpr int ROWB = D * 2;          // bytes per LDS row
  static constexpr int SUB = BLK / KT;        // tiles per key block
  static_assert(NI >= 1, "tile smaller than the workgroup");
};

// LDS swizzles of the 16-byte chunks of a tile row (free of bank conflicts
// for the MFMA operand reads whether the LDS serves 128 or 256 bytes a clock):
// K rows: chunk ^ (row & 15) (d = 128) or chunk ^ (row & 7) (d = 64);
// V rows: chunk ^ {0, 4, 10, 14}[row & 3] (d = 128) or chunk ^ 2*(row & 3).
template <int D>
__device__ __forceinline__ int k_chunk(int r, int c) { return c ^ (r & (D == 128 ? 15 : 7)); }
template <int D>
__device__ __forceinline__ int v_chunk(int r, int c) {
  return D == 128 ? c ^ (((r & 3) << 2) | (r & 2)) : c ^ ((r & 3) << 1);
}

// Combine a value of lane l with lane l ^ 32 (the two halves of a wave hold
// the two halves of a query row): one v_permlane32_swap, no LDS traffic.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}



// Byte offset, inside a KT x D tile, of the global 16-byte chunk this lane
// copies with direct load i: instruction i of wave w fills LDS chunks
// (i*NW + w)*64 + lane, so rows advance by whole KB per instruction and the
// lane's swizzle repeats with period NVAR in i (the swizzle period in rows
// over the rows per KB, divided by the waves).  Instruction i reads
// lane_off[i % NVAR] + i*NW*1024.
template <int D, int BLK>
struct DmaCfg {
  static constexpr int ROWS_PER_KB = 1024 / (2 * D);
  static constexpr int PERIOD = D == 128 ? 16 : 8;            // K swizzle period in rows
  static constexpr int STEP = Cfg<D, BLK>::NW * ROWS_PER_KB;  // rows per instruction step
  static constexpr int NVAR = STEP % PERIOD == 0 ? 1 : PERIOD / STEP;
};

template <int D, int BLK, bool IS_V>
__device__ __forceinline__ int dma_lane_off(int i, int w, int lane) {
  using C = Cfg<D, BLK>;
  const int P = (i * C::NW + w) * 64 + lane;
  const int r = P / C::CPR, pc = P % C::CPR;
  const int c = IS_V ? v_chunk<D>(r, pc) : k_chunk<D>(r, pc);
  return (r - i * C::NW * DmaCfg<D, BLK>::ROWS_PER_KB) * C::ROWB + c * 16;
}


// Direct HBM -> LDS load of one exact K or V tile: KT rows starting at byte
// `tile_off` of the head.
template <int D, int BLK>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, int tile_off, char* lds, int w,
                                         const int (&lane_off)[DmaCfg<D, BLK>::NVAR]) {
  using C = Cfg<D, BLK>;
#pragma unroll
  for (int i = 0; i < C::NI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (i * C::NW + w) * 1024), 16,
                                             lane_off[i % DmaCfg<D, BLK>::NVAR],
                                             tile_off + i * C::NW * 1024, 0, 0);
}

template <int D, int BLK>
struct State {
  f32x16 o[Cfg<D, BLK>::NOT];
  float m;   // running reference max (log2 domain, scaled)
  float l;   // this lane's partial row sum
};

// Register r of the S^T accumulator s[js] holds key key0 + 32*js + 8*(r/4)
// + 4*hh + (r%4) of the tile; kr(js, r) is that key minus key0 + 4*hh.
__device__ __forceinline__ constexpr int kr_of(int js, int r) { return 32 * js + 8 * (r >> 2) + (r & 3); }

// Exact tile at the end of the sequence or on the causal diagonal: keys with
// kr >= lim are masked.
__device__ __forceinline__ void mask_exact(f32x16 (&s)[2], int lim) {
#pragma unroll
  for (int js = 0; js < 2; ++js)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[js][r] = kr_of(js, r) < lim ? s[js][r] : -INFINITY;
}

// Tail tile (pooled rows): rows past the eligible range or in the selected
// set are masked; the others get the logit offset log2(n_J)/(scale*log2 e)
// so that exp2 of the scaled logit is n_J * exp(q.kbar_J): the pseudo-key's
// multiplicity.  `word` holds the selection bits of the 32 rows from
// key0 + 32*js, shifted by 4*hh.
__device__ __forceinline__ void mask_tail(f32x16 (&s)[2], int lim, uint32_t w0, uint32_t w1,
                                          int last_kr, float bias, float bias_last) {
#pragma unroll
  for (int js = 0; js < 2; ++js) {
    const uint32_t word = js ? w1 : w0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = kr_of(js, r);
      const bool on = kr < lim && !((word >> (kr - 32 * js)) & 1u);
      s[js][r] = on ? s[js][r] + (kr == last_kr ? bias_last : bias) : -INFINITY;
    }
  }
}

// V^T operand of PV step (nt, kc): two LDS transpose reads.
template <int D, int BLK>
__device__ __forceinline__ bf16x8 v_operand(const char* Vs, const int (&vbase)[Cfg<D, BLK>::NOT], int nt, int kc) {
  using C = Cfg<D, BLK>;
  const char* p = Vs + vbase[nt] + (16 * kc) * C::ROWB;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * C::ROWB));
  return __builtin_bit_cast(
      bf16x8, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// K operand of S step (js, ks).
template <int D, int BLK>
__device__ __forceinline__ bf16x8 k_operand(const char* Ks, const int (&kbase)[Cfg<D, BLK>::NKS], int step) {
  using C = Cfg<D, BLK>;
  const int js = step / C::NKS, ks = step % C::NKS;
  return *reinterpret_cast<const bf16x8*>(Ks + kbase[ks] + 32 * js * C::ROWB);
}

// Online softmax, part 1, for one 64-key tile (S^T accumulators s[0], s[1],
// already masked): running max with lazy rescale of O and l.  Returns the
// reference max (0 while no key has been seen) for the exponentials.
template <int D, int BLK>
__device__ __forceinline__ float softmax_max(State<D, BLK>& st, const f32x16 (&s)[2], float c) {
  using C = Cfg<D, BLK>;
  float mx = -INFINITY;
#pragma unroll
  for (int js = 0; js < 2; ++js)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[js][r]);
  mx = half_max(mx);
  const float mxs = mx * c;
  const bool grow = mxs > st.m + 8.f;
  if (__ballot(grow)) {
    const float m_new = grow ? mxs : st.m;
    const float corr = __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= corr;
#pragma unroll
    for (int nt = 0; nt < C::NOT; ++nt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[nt][r] *= corr;
    }
    st.m = m_new;
  }
  return st.m == -INFINITY ? 0.f : st.m;
}

// S^T = K Q^T for one 64-key tile held in LDS (K operands read 3 ahead).
template <int D, int BLK>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[2], const char* Ks, const int (&kbase)[Cfg<D, BLK>::NKS],
                                        const bf16x8 (&qf)[Cfg<D, BLK>::NKS]) {
  using C = Cfg<D, BLK>;
  constexpr int NSTEP = 2 * C::NKS;
  constexpr int KD = 3;
  s[0] = f32x16{};
  s[1] = f32x16{};
  bf16x8 kr[KD];
#pragma unroll
  for (int i = 0; i < KD; ++i) kr[i] = k_operand<D, BLK>(Ks, kbase, i);
#pragma unroll
  for (int step = 0; step < NSTEP; ++step) {
    const bf16x8 ka = kr[step % KD];
    if (step + KD < NSTEP) kr[step % KD] = k_operand<D, BLK>(Ks, kbase, step + KD);
    s[step / C::NKS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[step % C::NKS], s[step / C::NKS], 0, 0, 0);
  }
}

// Pipelined tile step: S^T of the next tile (one MFMA per step) interleaved
// with the exponentials of this tile, then O^T += V^T P^T.  LDS operands are
// read ahead through small register rings (K three steps ahead; the first V
// operands during the last S steps, then four ahead), and a scheduling
// barrier between steps keeps the compiler from regrouping the
// exponentials ahead of the products, so the matrix cores and the vector
// ALUs work side by side.
template <int D, int BLK>
__device__ __forceinline__ void pipe_step(State<D, BLK>& st, const f32x16 (&s)[2], f32x16 (&s_next)[2],
                                          const char* Ks_next, const char* Vs,
                                          const int (&kbase)[Cfg<D, BLK>::NKS],
                                          const int (&vbase)[Cfg<D, BLK>::NOT],
                                          const bf16x8 (&qf)[Cfg<D, BLK>::NKS], float c, float mb) {
  using C = Cfg<D, BLK>;
  constexpr int NSTEP = 2 * C::NKS;          // S MFMAs of one 64-key tile
  constexpr int PER = 16 / NSTEP;            // element pairs per step (1, or 2 for d = 64)
  static_assert(PER * NSTEP == 16, "16 element pairs (32 scores) per lane and tile");
  constexpr int KD = 3;                      // K operand ring depth
  constexpr int VD = 4;                      // V operand ring depth
  constexpr int NPV = 4 * C::NOT;            // PV MFMAs of one tile
  uint32_t wd[16];
  float lsum = 0.f;
  s_next[0] = f32x16{};
  s_next[1] = f32x16{};
  bf16x8 kr[KD];
#pragma unroll
  for (int i = 0; i < KD; ++i) kr[i] = k_operand<D, BLK>(Ks_next, kbase, i);
  bf16x8 vr[VD];
#pragma unroll
  for (int step = 0; step < NSTEP; ++step) {
    const int js = step / C::NKS, ks = step % C::NKS;
    const bf16x8 ka = kr[step % KD];
    if (step + KD < NSTEP) kr[step % KD] = k_operand<D, BLK>(Ks_next, kbase, step + KD);
    const int vi = step - (NSTEP - VD);      // start the V operands in the last steps
    if (vi >= 0) vr[vi] = v_operand<D, BLK>(Vs, vbase, vi / 4, vi % 4);
    s_next[js] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s_next[js], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = step * PER + u;          // element pair 0..15
      const int ej = q >> 3, r0 = 2 * (q & 7);
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[ej][r0], c, -mb));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[ej][r0 + 1], c, -mb));
      wd[q] = pack2(p0, p1);
      lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd[q]), kOnes, lsum, false);
      // an empty volatile statement using the packed pair: keeps its
      // computation inside this step (pure arithmetic would otherwise be
      // moved past the scheduling barrier)
      asm volatile("" ::"v"(wd[q]));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  st.l += lsum;
  // pair q = 8*ej + (r0/2) holds keys of sub-tile ej, registers r0, r0+1;
  // PV step kc = 2*ej + h2 takes registers 8*h2 .. 8*h2 + 7 of sub-tile ej
  bf16x8 pk[4];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    const int base = 8 * (kc >> 1) + 4 * (kc & 1);
    pk[kc] = __builtin_bit_cast(bf16x8, u32x4{wd[base], wd[base + 1], wd[base + 2], wd[base + 3]});
  }
#pragma unroll
  for (int j = 0; j < NPV; ++j) {
    const bf16x8 va = vr[j % VD];
    if (j + VD < NPV) vr[j % VD] = v_operand<D, BLK>(Vs, vbase, (j + VD) / 4, (j + VD) % 4);
    st.o[j / 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pk[j % 4], st.o[j / 4], 0, 0, 0);
  }
}

template <int D, int BLK>
__global__ __launch_bounds__(2 * BLK, 2) void attn_bf16_kernel(FwdArgs a) {
  using C = Cfg<D, BLK>;
  static_assert(BLK == 128, "64-row query blocks use the 16-row-per-wave kernel");
  // Double-buffered K and V tiles: tile e uses buffers K[e & 1], V[e & 1].
  // Four separate LDS objects, each named statically in every unrolled tile
  // step: the compiler can then tell that the transposed V reads of one
  // buffer do not overlap the tile loads in flight into the other, and does
  // not make the reads wait for those loads.
  __shared__ __attribute__((aligned(1024))) char K0[KT * D * 2];
  __shared__ __attribute__((aligned(1024))) char K1[KT * D * 2];
  __shared__ __attribute__((aligned(1024))) char V0[KT * D * 2];
  __shared__ __attribute__((aligned(1024))) char V1[KT * D * 2];
  // one spare word: the tail mask reads the word after the tile's first
  __shared__ uint32_t selbits[kMaxBlocks / 32 + 1];

  const int item = xcd_local_item(blockIdx.x, a.total);
  if (item < 0) return;
  // item -> (b, g, I descending, head inside the group)
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
  const int lq = lane & 31;   // query row inside the wave / MFMA column
  const int hh = lane >> 5;   // lane half

  const int q_tok = I * BLK + 32 * w + lq;
  const bool q_ok = q_tok < a.N;

  // Q fragment (B operand of S^T): row q_tok, d = 16*ks + 8*hh + e.
  bf16x8 qf[C::NKS];
  {
    const uint16_t* qrow = a.q + ((size_t)bh * a.N + (q_ok ? q_tok : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      const u32x4 x = q_ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * hh)
                           : u32x4{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const int n_sel = scalar_view(a.cnt)[(size_t)bh * a.M + I];
  const const_i32* list = scalar_view(a.idx + ((size_t)bh * a.M + I) * a.M);
  const int Jend = a.causal ? I + 1 : a.M;
  const int n_exact = n_sel * C::SUB;
  const int n_tiles = n_exact + (a.approx ? (Jend + KT - 1) / KT : 0);
  const int last_n = a.N - (a.M - 1) * BLK;
  // tail logit offsets: log2(n_J) / (scale * log2 e)
  const float bias_blk = __log2f((float)BLK) / a.scale_log2;
  const float bias_last = __log2f((float)last_n) / a.scale_log2;

  if (a.approx) {
    for (int i = t; i < kMaxBlocks / 32 + 1; i += C::NT) selbits[i] = 0u;
    __syncthreads();
    for (int e = t; e < n_sel; e += C::NT) {
      const int J = list[e];
      atomicOr(&selbits[J >> 5], 1u << (J & 31));
    }
  }

  const int head_bytes = a.N * C::ROWB;
  const __amdgpu_buffer_rsrc_t krs = head_rsrc(a.k + (size_t)(b * a.Hkv + g) * a.N * D, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(a.v + (size_t)(b * a.Hkv + g) * a.N * D, head_bytes);
  const size_t pp_off = (size_t)(b * a.Hkv + g) * a.M * D;
  const __amdgpu_buffer_rsrc_t tkrs = head_rsrc(a.approx ? a.tail_k + pp_off : a.k, a.M * C::ROWB);
  const __amdgpu_buffer_rsrc_t tvrs = head_rsrc(a.approx ? a.tail_v + pp_off : a.v, a.M * C::ROWB);

  // LDS byte offsets of this lane's K operand rows (per 16-wide d step) and
  // V transpose-read bases (per 32-wide d tile); tile-invariant.
  int kbase[C::NKS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) kbase[ks] = lq * C::ROWB + k_chunk<D>(lq, 2 * ks + hh) * 16;
  int vbase[C::NOT];
  {
    const int i16 = lane & 15, grp = lane >> 4;
    const int jr = 4 * (grp >> 1) + (i16 >> 2);          // row inside a 16-key step
#pragma unroll
    for (int nt = 0; nt < C::NOT; ++nt) {
      const int n = 32 * nt + 16 * (grp & 1) + 4 * (i16 & 3);
      vbase[nt] = jr * C::ROWB + v_chunk<D>(jr, n >> 3) * 16 + (n & 7) * 2;
    }
  }

  // first key (token index, or pooled row for tail tiles) of tile e
  auto tile_key0 = [&](int e) -> int {
    if (e < n_exact) return list[e / C::SUB] * BLK + (e % C::SUB) * KT;
    return (e - n_exact) * KT;
  };
  int koff[DmaCfg<D, BLK>::NVAR], voff[DmaCfg<D, BLK>::NVAR];
#pragma unroll
  for (int i = 0; i < DmaCfg<D, BLK>::NVAR; ++i) {
    koff[i] = dma_lane_off<D, BLK, false>(i, w, lane);
    voff[i] = dma_lane_off<D, BLK, true>(i, w, lane);
  }
  // exact tiles: KT keys of the head; tail tiles: KT pooled rows (bf16 block
  // means of k and of v from the pool pass), both straight into LDS
  auto issue_k = [&](int e, int key0, char* dst) {
    dma_tile<D, BLK>(e < n_exact ? krs : tkrs, key0 * C::ROWB, dst, w, koff);
  };
  auto issue_v = [&](int e, int key0, char* dst) {
    dma_tile<D, BLK>(e < n_exact ? vrs : tvrs, key0 * C::ROWB, dst, w, voff);
  };

  State<D, BLK> st;
#pragma unroll
  for (int i = 0; i < C::NOT; ++i) st.o[i] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
  const float c = a.scale_log2;

  // mask tile e in place (tail tiles: selection bits, eligibility and the
  // multiplicity offset; exact tiles: end of sequence and causal diagonal)
  auto mask_tile = [&](f32x16 (&sv)[2], int e, int key0) {
    if (e >= n_exact) {
      const uint32_t w0 = selbits[key0 >> 5] >> (4 * hh);
      const uint32_t w1 = selbits[(key0 >> 5) + 1] >> (4 * hh);
      mask_tail(sv, Jend - key0 - 4 * hh, w0, w1, a.M - 1 - key0 - 4 * hh, bias_blk, bias_last);
    } else if (key0 + KT > a.N || (a.causal && key0 + KT > I * BLK)) {
      int lim = a.N - key0;
      if (a.causal) lim = min(lim, q_tok - key0 + 1);
      mask_exact(sv, lim - 4 * hh);
    }
  };

  // Pipeline: while the softmax of tile e runs on the vector ALUs, the
  // matrix cores compute S of tile e+1; K e+2 and V e+1 load meanwhile.
  // One barrier per tile: it retires tile e's buffers and publishes the
  // loads issued during it.
  int key0 = tile_key0(0);
  int key1 = n_tiles > 1 ? tile_key0(1) : 0;
  issue_k(0, key0, K0);
  issue_v(0, key0, V0);
  if (n_tiles > 1) issue_k(1, key1, K1);
  wait_vm();
  __syncthreads();
  f32x16 s[2];
  qk_tile<D, BLK>(s, K0, kbase, qf);

  // one tile step; Kn holds tile e+1 (read now) and receives tile e+2, Vc
  // holds tile e, Vn receives tile e+1
  auto step = [&](int e, const char* Kn, char* Kc, const char* Vc, char* Vn) __attribute__((always_inline)) {
    const int key2 = e + 2 < n_tiles ? tile_key0(e + 2) : 0;
    if (e + 1 < n_tiles) issue_v(e + 1, key1, Vn);
    if (e + 2 < n_tiles) issue_k(e + 2, key2, Kc);
    mask_tile(s, e, key0);
    const float mb = softmax_max<D, BLK>(st, s, c);
    // S of tile e+1 (on the last tile this reads a retired buffer and the
    // result is dropped) interleaved with the softmax of tile e
    f32x16 s_next[2];
    pipe_step<D, BLK>(st, s, s_next, Kn, Vc, kbase, vbase, qf, c, mb);
    wait_vm();
    __syncthreads();
#pragma unroll
    for (int js = 0; js < 2; ++js) s[js] = s_next[js];
    key0 = key1;
    key1 = key2;
  };
  for (int e = 0; e < n_tiles; e += 2) {
    step(e, K1, K0, V0, V1);
    if (e + 1 < n_tiles) step(e + 1, K0, K1, V1, V0);
  }

  // ---- epilogue: O / l, bf16, row q_tok; register r of d-tile nt holds
  // d = 32*nt + 8*(r/4) + 4*hh + (r%4).
  const float lt = half_sum(st.l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (q_ok) {
    uint16_t* orow = a.out + ((size_t)bh * a.N + q_tok) * D;
#pragma unroll
    for (int nt = 0; nt < C::NOT; ++nt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * nt + 8 * q4 + 4 * hh;
        const u32x2 x = {pack2(st.o[nt][4 * q4] * inv, st.o[nt][4 * q4 + 1] * inv),
                         pack2(st.o[nt][4 * q4 + 2] * inv, st.o[nt][4 * q4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d0) = x;
      }
    }
  }
}

template <int D, int BLK>
hipError_t run(const FwdArgs& a, hipStream_t st) {
  const int grid = 8 * ((a.total + 7) / 8);
  hipLaunchKernelGGL((attn_bf16_kernel<D, BLK>), dim3(grid), dim3(2 * BLK), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const Shape& s, const FwdParams& p, const void* q, const void* k,
                      const void* v, const float* k_bar, const float* v_sum, const void* tail,
                      const int32_t* blk_idx, const int32_t* blk_cnt, void* out, hipStream_t st) {
  if (s.dtype == 0)
    return launch_fwd_f32(s, p, q, k, v, k_bar, v_sum, blk_idx, blk_cnt, out, st);
  // 64-row query blocks: 16 rows per wave (four waves share one K/V tile)
  if (s.block == 64) return launch_fwd_w16(s, p, q, k, v, tail, blk_idx, blk_cnt, out, st);
  FwdArgs a{};
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
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.N = s.N;
  a.M = s.M;
  a.G = s.Hq / s.Hkv;
  a.total = s.B * s.Hq * s.M;
  a.scale_log2 = p.scale * 1.4426950408889634f;
  a.causal = p.causal;
  a.approx = p.approx;
  return s.D == 128 ? run<128, 128>(a, st) : run<64, 128>(a, st);
}

}  // namespace sa
