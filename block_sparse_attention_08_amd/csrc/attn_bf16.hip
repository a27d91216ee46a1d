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
//                  routing table and "why softmax survives");
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
// K/V tiles travel HBM -> LDS with global_load_lds_dwordx4 (no registers).
// Each wave instruction fills 1 KB of LDS contiguously, so every lane picks
// the global 16-byte chunk that belongs at its LDS slot: the LDS tiles are
// row-major with 16-byte chunks XOR-swizzled (K: chunk ^ (row & 7); V:
// chunk ^ 2*(row & 3)), which keeps the MFMA operand reads free of bank
// conflicts without padding.  One K buffer and one V buffer per workgroup;
// the next K tile loads while this tile's softmax and PV run, the next V
// tile while the next S runs (two barriers per tile).  Tail tiles come from
// the float32 pooled K-bar / V-sum and are converted through registers.
// Workgroups are ordered so that each XCD receives a contiguous range of
// (kv head, query block) items, with the query heads of one KV group
// adjacent, so K/V blocks shared by neighbouring items stay in one L2.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace sa {

hipError_t launch_fwd_f32(const Shape& s, const FwdParams& p, const void* q, const void* k,
                          const void* v, const float* k_bar, const float* v_sum,
                          const int32_t* blk_idx, const int32_t* blk_cnt, void* out,
                          hipStream_t st);

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* k_bar;
  const float* v_sum;
  const int32_t* idx;
  const int32_t* cnt;
  uint16_t* out;
  int Hq, Hkv, N, M, G, total;
  float scale_log2;  // scale * log2(e)
  int causal, approx;
};

constexpr int KT = 64;  // keys per tile (a 128-token block is two tiles)

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

__device__ __forceinline__ int k_chunk(int r, int c) { return c ^ (r & 7); }
__device__ __forceinline__ int v_chunk(int r, int c) { return c ^ ((r & 3) << 1); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Wait until this wave's outstanding global loads (including the ones that
// write LDS directly) have completed.
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Byte offset, inside a KT x D tile, of the global 16-byte chunk this lane
// copies with every direct load: instruction i of wave w fills LDS chunks
// (i*NW + w)*64 + lane, i.e. rows advance by whole KB per instruction and,
// since NW*64/CPR rows is a multiple of 8, the swizzle of a lane's row is
// the same for every i.  So instruction i reads lane_off + i*NW*1024.
template <int D, int BLK, bool IS_V>
__device__ __forceinline__ int dma_lane_off(int w, int lane) {
  using C = Cfg<D, BLK>;
  const int P = w * 64 + lane;
  const int r = P / C::CPR, pc = P % C::CPR;
  const int c = IS_V ? v_chunk(r, pc) : k_chunk(r, pc);
  return r * C::ROWB + c * 16;
}

// Buffer resource over one K or V head ([N, D] bf16): loads past its last
// byte return zero, which is what the rows of a ragged last block need
// (their keys are masked and their values meet p = 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint16_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, 0x00020000);
}

// Direct HBM -> LDS load of one exact K or V tile: KT rows starting at byte
// `tile_off` of the head.
template <int D, int BLK>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, int tile_off, char* lds, int w,
                                         int lane_off) {
  using C = Cfg<D, BLK>;
#pragma unroll
  for (int i = 0; i < C::NI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (i * C::NW + w) * 1024), 16,
                                             lane_off, tile_off + i * C::NW * 1024, 0, 0);
}

// Tail tile: float32 pooled rows -> bf16 -> the same swizzled LDS layout.
// For V the rows are divided by n_J (the block's token count: `block`, or
// `last_n` for pooled row M-1), turning value sums into mean values; the
// factor n_J moves into the logit instead (see mask_tail).
template <int D, int BLK, bool IS_V>
__device__ __forceinline__ void reg_tile(const float* src, char* lds, int valid, int w, int lane,
                                         int last_row, float inv_last) {
  using C = Cfg<D, BLK>;
#pragma unroll 1
  for (int i = 0; i < C::NI; ++i) {
    const int P = (i * C::NW + w) * 64 + lane;
    const int r = P / C::CPR;
    const int pc = P % C::CPR;
    const int c = IS_V ? v_chunk(r, pc) : k_chunk(r, pc);
    u32x4 x = {0u, 0u, 0u, 0u};
    if (r < valid) {
      f32x4 lo = *reinterpret_cast<const f32x4*>(src + (size_t)r * D + 8 * c);
      f32x4 hi = *reinterpret_cast<const f32x4*>(src + (size_t)r * D + 8 * c + 4);
      if constexpr (IS_V) {
        const float f = r == last_row ? inv_last : 1.0f / (float)BLK;
        lo *= f;
        hi *= f;
      }
      x = u32x4{pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(hi[0], hi[1]), pack2(hi[2], hi[3])};
    }
    *reinterpret_cast<u32x4*>(lds + P * 16) = x;
  }
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

// Online softmax + PV for one 64-key tile (S^T accumulators s[0], s[1],
// already masked): running max with lazy rescale, exp2, bf16 pack, and
// O^T += V^T P^T with V^T read by LDS transpose loads.
template <int D, int BLK>
__device__ __forceinline__ void softmax_pv(State<D, BLK>& st, f32x16 (&s)[2], const char* Vs,
                                           const int (&vbase)[Cfg<D, BLK>::NOT], float c) {
  using C = Cfg<D, BLK>;
  float mx = -INFINITY;
#pragma unroll
  for (int js = 0; js < 2; ++js)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[js][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
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
  const float mb = st.m == -INFINITY ? 0.f : st.m;

  bf16x8 pk[4];
  float lsum = 0.f;
#pragma unroll
  for (int js = 0; js < 2; ++js) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      uint32_t wd[4];
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const int r0 = 8 * h2 + 2 * q2;
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[js][r0], c, -mb));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[js][r0 + 1], c, -mb));
        lsum += p0 + p1;
        wd[q2] = pack2(p0, p1);
      }
      pk[2 * js + h2] = __builtin_bit_cast(bf16x8, u32x4{wd[0], wd[1], wd[2], wd[3]});
    }
  }
  st.l += lsum;

#pragma unroll
  for (int nt = 0; nt < C::NOT; ++nt) {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const char* p = Vs + vbase[nt] + (16 * kc) * C::ROWB;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * C::ROWB));
      const bf16x8 va = __builtin_bit_cast(
          bf16x8, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      st.o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pk[kc], st.o[nt], 0, 0, 0);
    }
  }
}

template <int D, int BLK>
__global__ __launch_bounds__(2 * BLK, 2) void attn_bf16_kernel(FwdArgs a) {
  using C = Cfg<D, BLK>;
  __shared__ __attribute__((aligned(1024))) char Ks[KT * D * 2];
  __shared__ __attribute__((aligned(1024))) char Vs[KT * D * 2];
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

  const int n_sel = a.cnt[(size_t)bh * a.M + I];
  const int32_t* list = a.idx + ((size_t)bh * a.M + I) * a.M;
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

  // LDS byte offsets of this lane's K operand rows (per 16-wide d step) and
  // V transpose-read bases (per 32-wide d tile); tile-invariant.
  int kbase[C::NKS];
#pragma unroll
  for (int ks = 0; ks < C::NKS; ++ks) kbase[ks] = lq * C::ROWB + k_chunk(lq, 2 * ks + hh) * 16;
  int vbase[C::NOT];
  {
    const int i16 = lane & 15, grp = lane >> 4;
    const int jr = 4 * (grp >> 1) + (i16 >> 2);          // row inside a 16-key step
#pragma unroll
    for (int nt = 0; nt < C::NOT; ++nt) {
      const int n = 32 * nt + 16 * (grp & 1) + 4 * (i16 & 3);
      vbase[nt] = jr * C::ROWB + v_chunk(jr, n >> 3) * 16 + (n & 7) * 2;
    }
  }

  // first key (token index, or pooled row for tail tiles) of tile e
  auto tile_key0 = [&](int e) -> int {
    if (e < n_exact) return list[e / C::SUB] * BLK + (e % C::SUB) * KT;
    return (e - n_exact) * KT;
  };
  const int koff = dma_lane_off<D, BLK, false>(w, lane);
  const int voff = dma_lane_off<D, BLK, true>(w, lane);
  auto issue_k = [&](int e, int key0) {
    if (e < n_exact)
      dma_tile<D, BLK>(krs, key0 * C::ROWB, Ks, w, koff);
    else
      reg_tile<D, BLK, false>(a.k_bar + pp_off + (size_t)key0 * D, Ks, a.M - key0, w, lane, 0, 0.f);
  };
  auto issue_v = [&](int e, int key0) {
    if (e < n_exact)
      dma_tile<D, BLK>(vrs, key0 * C::ROWB, Vs, w, voff);
    else
      reg_tile<D, BLK, true>(a.v_sum + pp_off + (size_t)key0 * D, Vs, a.M - key0, w, lane,
                             a.M - 1 - key0, 1.0f / (float)last_n);
  };

  State<D, BLK> st;
#pragma unroll
  for (int i = 0; i < C::NOT; ++i) st.o[i] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;

  int key0 = tile_key0(0);
  issue_k(0, key0);
  issue_v(0, key0);
  wait_vm();
  __syncthreads();

  for (int e = 0; e < n_tiles; ++e) {
    const bool pseudo = e >= n_exact;
    // skip exact tiles that lie wholly past the last token (ragged last block)
    const int next_key0 = e + 1 < n_tiles ? tile_key0(e + 1) : 0;

    // ---- S^T = K Q^T
    f32x16 s[2];
#pragma unroll
    for (int js = 0; js < 2; ++js) {
      s[js] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + kbase[ks] + 32 * js * C::ROWB);
        s[js] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s[js], 0, 0, 0);
      }
    }
    wait_vm();
    __syncthreads();                 // K buffer free, V tile e landed in every wave
    if (e + 1 < n_tiles) issue_k(e + 1, next_key0);

    if (pseudo) {
      const uint32_t w0 = selbits[key0 >> 5] >> (4 * hh);
      const uint32_t w1 = selbits[(key0 >> 5) + 1] >> (4 * hh);
      mask_tail(s, Jend - key0 - 4 * hh, w0, w1, a.M - 1 - key0 - 4 * hh, bias_blk, bias_last);
    } else if (key0 + KT > a.N || (a.causal && key0 + KT > I * BLK)) {
      int lim = a.N - key0;
      if (a.causal) lim = min(lim, q_tok - key0 + 1);
      mask_exact(s, lim - 4 * hh);
    }
    softmax_pv<D, BLK>(st, s, Vs, vbase, a.scale_log2);

    wait_vm();
    __syncthreads();                 // V buffer free, K tile e+1 landed in every wave
    if (e + 1 < n_tiles) issue_v(e + 1, next_key0);
    key0 = next_key0;
  }

  // ---- epilogue: O / l, bf16, row q_tok; register r of d-tile nt holds
  // d = 32*nt + 8*(r/4) + 4*hh + (r%4).
  const float lt = st.l + __shfl_xor(st.l, 32, 64);
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
                      const void* v, const float* k_bar, const float* v_sum,
                      const int32_t* blk_idx, const int32_t* blk_cnt, void* out, hipStream_t st) {
  if (s.dtype == 0)
    return launch_fwd_f32(s, p, q, k, v, k_bar, v_sum, blk_idx, blk_cnt, out, st);
  FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.k_bar = k_bar;
  a.v_sum = v_sum;
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
  if (s.D == 128) return s.block == 128 ? run<128, 128>(a, st) : run<128, 64>(a, st);
  return s.block == 128 ? run<64, 128>(a, st) : run<64, 64>(a, st);
}

}  // namespace sa
