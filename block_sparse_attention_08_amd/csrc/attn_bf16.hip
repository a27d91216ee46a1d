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
// wave w owns 32 query rows.  Keys are visited in tiles of KT = block/2 keys
// (two tiles per listed block; a tail tile is KT pooled rows).  Per tile:
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16; A = K tile rows read from LDS,
//                 B = the wave's Q rows (registers for the whole kernel).
//                 The accumulator holds one query row per lane (lanes l and
//                 l+32 share row l%32, 16 keys each per 32-key group), so the
//                 row max needs one cross-lane exchange and the softmax state
//                 is per lane.
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
// keeps the MFMA operand reads free of bank conflicts without padding.  Tail
// tiles gather their pooled rows (bf16 block means of k and v, written once
// per head by the pool pass) by per-lane row offsets from the list of
// unlisted eligible blocks, built in LDS at the start.
//
// K and V are double-buffered and the loop is software-pipelined: S of tile
// e+1 sits next to the exponentials of tile e, and the row max of tile e+1
// next to the PV products of tile e; one barrier per tile.  Tiles that need
// masks (the ragged last block, the causal diagonal, the partly filled last
// tail tile) are visited last, in a loop of their own, so the main loop
// carries no mask code; the order of the tiles does not change the softmax.
// 128-row blocks: four waves, 64-key tiles, 64 KB of tile buffers, two
// workgroups per CU.  64-row blocks with at least kPipelinedMinBlocks64
// blocks per row: two waves over 32-key tiles (32 KB of tile buffers, four
// workgroups per CU); measured against the 16-row-per-wave kernel on the
// image workload's inputs: 10% slower at 192 blocks, even at 384, 17% faster
// at 512 and 27% at 640, where the double-buffered tiles hide K/V fetches
// that no longer hit in the caches.
// Workgroups are ordered so that each XCD receives a contiguous range of
// (kv head, query block) items, with the query heads of one KV group
// adjacent, so K/V blocks shared by neighbouring items stay in one L2.
#include <math.h>

#include <type_traits>

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

// 64-row blocks per row from which the pipelined two-wave kernel is used
constexpr int kPipelinedMinBlocks64 = 384;

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* tail_k;   // [B, Hkv, M, D] bf16 block means of k
  const uint16_t* tail_v;   // [B, Hkv, M, D] bf16 block means of v
  const int32_t* idx;
  const int32_t* cnt;
  uint16_t* out;
  float* lse;
  int Hq, Hkv, N, M, G, total;
  float scale_log2;  // scale * log2(e)
  int causal, approx;
};

template <int D, int BLK>
struct Cfg {
  static constexpr int NW = BLK / 32;         // waves
  static constexpr int NT = 64 * NW;          // threads
  static constexpr int T = BLK / 2;           // keys per tile (two tiles per block)
  static constexpr int NJS = T / 32;          // 32-key groups of S^T per tile
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int NI = T * CPR / NT;     // 16-byte DMA loads per thread per tile
  static constexpr int NKS = D / 16;          // 16-wide d steps of S
  static constexpr int NOT = D / 32;          // 32-wide d tiles of O
  static constexpr int ROWB = D * 2;          // bytes per LDS row
  static constexpr int RPK = 1024 / ROWB;     // rows filled by one 1 KB DMA instruction
  static constexpr int TB = T * ROWB;         // bytes of one K or V tile
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

// DMA lane layout: instruction i of wave w fills LDS chunks (i*NW + w)*64 +
// lane of the tile, i.e. row r_i = (i*NW + w)*RPK + lane/CPR, chunk slot
// lane%CPR.  The lane copies the global chunk that the swizzle places in that
// slot; its column offset repeats with period NVAR in i (the swizzle period
// in rows over the rows one instruction step advances).
template <int D, int BLK>
struct DmaCfg {
  using C = Cfg<D, BLK>;
  static constexpr int PERIOD = D == 128 ? 16 : 8;            // K swizzle period in rows
  static constexpr int STEP = C::NW * C::RPK;                 // rows per instruction step
  static constexpr int NVAR = STEP % PERIOD == 0 ? 1 : PERIOD / STEP;
};

// Column byte offset (swizzled chunk * 16) of this lane's chunk for
// instruction i (i < NVAR).
template <int D, int BLK, bool IS_V>
__device__ __forceinline__ int dma_col(int i, int w, int lane) {
  using C = Cfg<D, BLK>;
  const int r = (i * C::NW + w) * C::RPK + lane / C::CPR;
  const int pc = lane % C::CPR;
  return (IS_V ? v_chunk<D>(r, pc) : k_chunk<D>(r, pc)) * 16;
}

// One K or V tile: T consecutive rows from byte `tile_off` of the head.
template <int D, int BLK>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, int tile_off, char* lds, int w, int row0,
                                         const int (&col)[DmaCfg<D, BLK>::NVAR]) {
  using C = Cfg<D, BLK>;
#pragma unroll
  for (int i = 0; i < C::NI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (i * C::NW + w) * 1024), 16,
                                             tile_off + i * C::NW * 1024 + row0 * C::ROWB +
                                                 col[i % DmaCfg<D, BLK>::NVAR],
                                             0, 0, 0);
}

// Gathered tile: instruction i copies this lane's chunk of the row at byte
// offset ro[i] (the pooled rows of a tail tile).
template <int D, int BLK>
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t rs, const int (&ro)[Cfg<D, BLK>::NI], char* lds,
                                         int w, const int (&col)[DmaCfg<D, BLK>::NVAR]) {
  using C = Cfg<D, BLK>;
#pragma unroll
  for (int i = 0; i < C::NI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (i * C::NW + w) * 1024), 16,
                                             ro[i] + col[i % DmaCfg<D, BLK>::NVAR], 0, 0, 0);
}

// S^T accumulators of one tile
template <int D, int BLK>
using SAcc = f32x16[Cfg<D, BLK>::NJS];

template <int D, int BLK>
struct State {
  f32x16 o[Cfg<D, BLK>::NOT];
  float m;   // running reference max (log2 domain, scaled)
  float l;   // this lane's partial row sum
};

// Register r of the S^T accumulator s[js] holds key key0 + 32*js + 8*(r/4)
// + 4*hh + (r%4) of the tile; kr(js, r) is that key minus key0 + 4*hh.
__device__ __forceinline__ constexpr int kr_of(int js, int r) { return 32 * js + 8 * (r >> 2) + (r & 3); }

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

// Row max of one tile's raw scores (S^T accumulators, already masked),
// over both lane halves.
template <int D, int BLK>
__device__ __forceinline__ float tile_max(const SAcc<D, BLK>& s) {
  using C = Cfg<D, BLK>;
  float mx = -INFINITY;
#pragma unroll
  for (int js = 0; js < C::NJS; ++js)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[js][r]);
  return half_max(mx);
}

// Online softmax, part 1, for one tile whose raw row max is mx: running max
// with lazy rescale of O and l.  lb is added to every logit of the tile
// (log2 n_J for tail rows).  Returns the reference max minus lb (lb while no
// key has been seen) for the exponentials.
template <int D, int BLK>
__device__ __forceinline__ float softmax_update(State<D, BLK>& st, float mx, float c, float lb) {
  using C = Cfg<D, BLK>;
  const float mxs = fmaf(mx, c, lb);
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
  return (st.m == -INFINITY ? 0.f : st.m) - lb;
}

// S^T = K Q^T for one tile held in LDS (K operands read 3 ahead).
template <int D, int BLK>
__device__ __forceinline__ void qk_tile(SAcc<D, BLK>& s, const char* Ks,
                                        const int (&kbase)[Cfg<D, BLK>::NKS],
                                        const bf16x8 (&qf)[Cfg<D, BLK>::NKS]) {
  using C = Cfg<D, BLK>;
  constexpr int NSTEP = C::NJS * C::NKS;
  constexpr int KD = 3;
#pragma unroll
  for (int js = 0; js < C::NJS; ++js) s[js] = f32x16{};
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
// NEXT_MAX: the row max of the next tile's scores (unmasked) is folded into
// the PV products' steps, one or two vector max operations beside each
// product, and returned in mx_next; the vector ALU has nothing else to do
// while those products run.
template <int D, int BLK, bool NEXT_MAX>
__device__ __forceinline__ void pipe_step(State<D, BLK>& st, const SAcc<D, BLK>& s,
                                          SAcc<D, BLK>& s_next, const char* Ks_next,
                                          const char* Vs, const int (&kbase)[Cfg<D, BLK>::NKS],
                                          const int (&vbase)[Cfg<D, BLK>::NOT],
                                          const bf16x8 (&qf)[Cfg<D, BLK>::NKS], float c, float mb,
                                          float& mx_next) {
  using C = Cfg<D, BLK>;
  constexpr int NSTEP = C::NJS * C::NKS;     // S MFMAs of one tile
  constexpr int NPAIR = 8 * C::NJS;          // element pairs (two scores) per lane and tile
  constexpr int PER = NPAIR / NSTEP;         // element pairs per step (1, or 2 for d = 64)
  static_assert(PER * NSTEP == NPAIR, "pairs spread evenly over the S steps");
  constexpr int KD = 3;                      // K operand ring depth
  constexpr int VD = 4;                      // V operand ring depth
  constexpr int NKC = 2 * C::NJS;            // 16-key PV steps of one tile
  constexpr int NPV = NKC * C::NOT;          // PV MFMAs of one tile
  uint32_t wd[NPAIR];
  float lsum = 0.f;
#pragma unroll
  for (int js = 0; js < C::NJS; ++js) s_next[js] = f32x16{};
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
    if (vi >= 0) vr[vi] = v_operand<D, BLK>(Vs, vbase, vi / NKC, vi % NKC);
    s_next[js] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s_next[js], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = step * PER + u;          // element pair
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
  // pair q = 8*ej + (r0/2) holds keys of key group ej, registers r0, r0+1;
  // PV step kc = 2*ej + h2 takes registers 8*h2 .. 8*h2 + 7 of key group ej
  bf16x8 pk[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    const int base = 8 * (kc >> 1) + 4 * (kc & 1);
    pk[kc] = __builtin_bit_cast(bf16x8, u32x4{wd[base], wd[base + 1], wd[base + 2], wd[base + 3]});
  }
  constexpr int NE = 16 * C::NJS;             // scores per lane of the next tile
  constexpr int PE = (NE + NPV - 1) / NPV;    // of them folded per PV product
  float mn = -INFINITY;
#pragma unroll
  for (int j = 0; j < NPV; ++j) {
    const bf16x8 va = vr[j % VD];
    if (j + VD < NPV) vr[j % VD] = v_operand<D, BLK>(Vs, vbase, (j + VD) / NKC, (j + VD) % NKC);
    st.o[j / NKC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pk[j % NKC], st.o[j / NKC], 0, 0, 0);
    if constexpr (NEXT_MAX) {
      // scores in accumulation order: key group 0 finishes first
#pragma unroll
      for (int u = 0; u < PE; ++u) {
        const int q = j * PE + u;
        if (q < NE) mn = fmaxf(mn, s_next[q / 16][q % 16]);
      }
      asm volatile("" ::"v"(mn));   // keeps the max inside this step
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (NEXT_MAX) mx_next = half_max(mn);
}

template <int D, int BLK>
__global__ __launch_bounds__(2 * BLK, 2) void attn_bf16_kernel(FwdArgs a) {
  using C = Cfg<D, BLK>;
  using DC = DmaCfg<D, BLK>;
  constexpr int T = C::T;
  // Double-buffered K and V tiles: tile e uses buffers K[e & 1], V[e & 1].
  // Four separate LDS objects, each named statically in every unrolled tile
  // step: the compiler can then tell that the transposed V reads of one
  // buffer do not overlap the tile loads in flight into the other, and does
  // not make the reads wait for those loads.
  __shared__ __attribute__((aligned(1024))) char K0[C::TB];
  __shared__ __attribute__((aligned(1024))) char K1[C::TB];
  __shared__ __attribute__((aligned(1024))) char V0[C::TB];
  __shared__ __attribute__((aligned(1024))) char V1[C::TB];
  // tail only: selection bitmap, then the ascending list of the eligible
  // blocks that are not listed (the pooled rows the tail tiles gather)
  __shared__ uint32_t selbits[kMaxBlocks / 32];
  __shared__ uint16_t tail_rows[kMaxBlocks];

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
  const int last_n = a.N - (a.M - 1) * BLK;
  // every listed block is eligible, so Jend - n_sel eligible blocks remain
  const int n_rest = a.approx ? Jend - n_sel : 0;
  const int n_tt = (n_rest + T - 1) / T;   // tail tiles
  // Only the ragged last block (J = M-1) and the causal diagonal (J = I)
  // need the edge mask; either is the largest index a list may hold, so in
  // an ascending list it can only be the last entry.
  int has_edge = 0;
  if (n_sel > 0) {
    const int J = list[n_sel - 1];
    has_edge = ((J + 1) * BLK > a.N || (a.causal && J >= I)) ? 1 : 0;
  }
  // tile order: [exact, unmasked) [tail but the last) [edge block) [last tail)
  const int P1 = 2 * (n_sel - has_edge);
  const int P2 = P1 + (n_tt > 0 ? n_tt - 1 : 0);
  const int P3 = P2 + 2 * has_edge;
  const int n_tiles = P3 + (n_tt > 0 ? 1 : 0);
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
  // DMA: this lane's first row and swizzled column offsets
  const int row0 = w * C::RPK + lane / C::CPR;
  int kcol[DC::NVAR], vcol[DC::NVAR];
#pragma unroll
  for (int i = 0; i < DC::NVAR; ++i) {
    kcol[i] = dma_col<D, BLK, false>(i, w, lane);
    vcol[i] = dma_col<D, BLK, true>(i, w, lane);
  }

  // Tile e: a tail tile (returns true, key = tail tile index) or an exact one
  // (key = first token).
  auto tile_src = [&](int e, int& key) -> bool {
    if (e < P1) {
      key = list[e >> 1] * BLK + (e & 1) * T;
      return false;
    }
    if (e < P2) {
      key = e - P1;
      return true;
    }
    if (e < P3) {
      key = list[n_sel - 1] * BLK + ((e - P2) & 1) * T;
      return false;
    }
    key = n_tt - 1;
    return true;
  };
  // byte offsets of the pooled rows this lane copies for tail tile tt (row 0
  // for the padding of the last tile, masked later)
  auto tail_offs = [&](int tt, int (&ro)[C::NI]) {
#pragma unroll
    for (int i = 0; i < C::NI; ++i) {
      const int r = T * tt + row0 + i * C::NW * C::RPK;
      ro[i] = (r < n_rest ? (int)tail_rows[r] : 0) * C::ROWB;
    }
  };
  auto issue_k = [&](bool tail, int key, char* dst) {
    if (!tail) {
      dma_tile<D, BLK>(krs, key * C::ROWB, dst, w, row0, kcol);
    } else {
      int ro[C::NI];
      tail_offs(key, ro);
      dma_rows<D, BLK>(tkrs, ro, dst, w, kcol);
    }
  };
  auto issue_v = [&](bool tail, int key, char* dst) {
    if (!tail) {
      dma_tile<D, BLK>(vrs, key * C::ROWB, dst, w, row0, vcol);
    } else {
      int ro[C::NI];
      tail_offs(key, ro);
      dma_rows<D, BLK>(tvrs, ro, dst, w, vcol);
    }
  };

  State<D, BLK> st;
#pragma unroll
  for (int i = 0; i < C::NOT; ++i) st.o[i] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
  const float c = a.scale_log2;

  // masks of the last tiles, in place: the edge block (end of sequence,
  // causal diagonal) or the last tail tile (padding rows, a short last
  // block's multiplicity)
  auto mask_tile = [&](f32x16 (&sv)[C::NJS], bool tail, int key) {
    if (tail) {
      const int lim = n_rest - T * key - 4 * hh;
      const int fix_kr = (last_n != BLK && tail_rows[n_rest - 1] == a.M - 1) ? lim - 1 : -1;
#pragma unroll
      for (int js = 0; js < C::NJS; ++js)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = kr_of(js, r);
          sv[js][r] = kr < lim ? (kr == fix_kr ? sv[js][r] + last_fix : sv[js][r]) : -INFINITY;
        }
    } else {
      int lim = a.N - key;
      if (a.causal) lim = min(lim, q_tok - key + 1);
      lim -= 4 * hh;
#pragma unroll
      for (int js = 0; js < C::NJS; ++js)
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[js][r] = kr_of(js, r) < lim ? sv[js][r] : -INFINITY;
    }
  };

  // Pipeline: while the softmax of tile e runs on the vector ALUs, the
  // matrix cores compute S of tile e+1; K e+2 and V e+1 load meanwhile.
  // One barrier per tile: it retires tile e's buffers and publishes the
  // loads issued during it.  (t0, k0): tile e; (t1, k1): tile e+1.
  int k0 = 0, k1 = 0;
  bool t0 = n_tiles > 0 ? tile_src(0, k0) : false;
  bool t1 = n_tiles > 1 ? tile_src(1, k1) : false;
  if (n_tiles > 0) {
    issue_k(t0, k0, K0);
    issue_v(t0, k0, V0);
  }
  if (n_tiles > 1) issue_k(t1, k1, K1);
  wait_vm();
  __syncthreads();
  f32x16 sA[C::NJS], sB[C::NJS];
  qk_tile<D, BLK>(sA, K0, kbase, qf);
  // every wave has read tile 0 from K0 before step 0 loads tile 2 into it
  __syncthreads();
  // raw row max of the current tile: in the unmasked loop each step
  // computes the next tile's beside its PV products
  float mxc = tile_max<D, BLK>(sA);

  // one tile step; Kn holds tile e+1 (read now) and receives tile e+2, Vc
  // holds tile e, Vn receives tile e+1; sc is S of tile e, sn receives S of
  // tile e+1
  // tile step; masked: whether the tile may be one of the last (masked) ones
  auto step = [&](int e, const char* Kn, char* Kc, const char* Vc, char* Vn, f32x16 (&sc)[C::NJS],
                  f32x16 (&sn)[C::NJS], auto masked) __attribute__((always_inline)) {
    int k2 = 0;
    const bool t2 = e + 2 < n_tiles ? tile_src(e + 2, k2) : false;
    if (e + 1 < n_tiles) issue_v(t1, k1, Vn);
    if (e + 2 < n_tiles) issue_k(t2, k2, Kc);
    constexpr bool MASKED = decltype(masked)::value;
    if constexpr (MASKED) {
      if (e >= P2) mask_tile(sc, t0, k0);
      mxc = tile_max<D, BLK>(sc);
    }
    const float mb = softmax_update<D, BLK>(st, mxc, c, t0 ? log2_blk : 0.f);
    // S of tile e+1 (on the last tile this reads a retired buffer and the
    // result is dropped) interleaved with the softmax of tile e
    // the product-dense part runs at raised wave priority; the other wave
    // of the SIMD fills the gaps with its masks and row maxima
    __builtin_amdgcn_s_setprio(1);
    pipe_step<D, BLK, !MASKED>(st, sc, sn, Kn, Vc, kbase, vbase, qf, c, mb, mxc);
    __builtin_amdgcn_s_setprio(0);
    wait_vm();
    __syncthreads();
    t0 = t1;
    k0 = k1;
    t1 = t2;
    k1 = k2;
  };
  // Tiles before P2 need no mask.  Their loop has no mask branch, so the S
  // accumulators of both phases stay in fixed registers (a branch that
  // rewrites them would cost a copy of S per tile at its join).
  int e = 0;
  while (e + 1 < P2) {
    step(e, K1, K0, V0, V1, sA, sB, std::false_type{});
    step(e + 1, K0, K1, V1, V0, sB, sA, std::false_type{});
    e += 2;
  }
  // the last tiles (the masked ones among them); e is even here
  while (e < n_tiles) {
    step(e, K1, K0, V0, V1, sA, sB, std::true_type{});
    if (++e >= n_tiles) break;
    step(e, K0, K1, V1, V0, sB, sA, std::true_type{});
    ++e;
  }

  // ---- epilogue: O / l in bf16.  Register r of d-tile nt holds row lq,
  // d = 32*nt + 8*(r/4) + 4*hh + (r%4); the wave's 32 rows leave through its
  // share of the free K buffers (staged row store).
  const float lt = half_sum(st.l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  // log of the denominator: sum_a exp(z_a) = lt * 2^m
  if (a.lse && q_ok && hh == 0) a.lse[(size_t)bh * a.N + q_tok] = __logf(lt) + st.m * 0.69314718055994531f;
  constexpr int WPB = C::NW / 2;                // waves per K buffer
  char* stage = (w < WPB ? K0 : K1) + (w % WPB) * 32 * C::ROWB;
#pragma unroll
  for (int nt = 0; nt < C::NOT; ++nt) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int ch = 4 * nt + q4;               // 16-byte chunk of the row
      const u32x2 x = {pack2(st.o[nt][4 * q4] * inv, st.o[nt][4 * q4 + 1] * inv),
                       pack2(st.o[nt][4 * q4 + 2] * inv, st.o[nt][4 * q4 + 3] * inv)};
      *reinterpret_cast<u32x2*>(stage + lq * C::ROWB + stage_slot<D>(lq, ch) * 16 + 8 * hh) = x;
    }
  }
  const int tok0 = I * BLK + 32 * w;            // the wave's first query token
  store_staged_rows<D, 32>(stage, a.out + ((size_t)bh * a.N + tok0) * D, a.N - tok0, lane);
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
  // 64-row query blocks up to 383 blocks per row: 16 rows per wave (four
  // waves share one K/V tile, four workgroups per CU); longer rows take the
  // two-wave pipelined kernel below, whose double-buffered tiles hide the
  // longer K/V fetches once a head's K/V outgrows the caches
  if (s.block == 64 && s.M < kPipelinedMinBlocks64)
    return launch_fwd_w16(s, p, q, k, v, tail, blk_idx, blk_cnt, out, st);
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
  if (s.block == 64) return s.D == 128 ? run<128, 64>(a, st) : run<64, 64>(a, st);
  return s.D == 128 ? run<128, 128>(a, st) : run<64, 128>(a, st);
}

}  // namespace sa
