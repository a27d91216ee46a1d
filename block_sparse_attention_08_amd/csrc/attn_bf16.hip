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
//   S^T = K Q^T   with v_mfma_f32_32x32x16_bf16: A = K tile rows (LDS,
//                 row-major), B = the wave's Q rows (registers for the whole
//                 kernel); the accumulator puts one query row per lane
//                 (lane l and l+32 share row l%32, 16 keys each);
//   online softmax on those registers (exp2 with the scale folded in);
//   O^T += V^T P^T with P taken straight from the S registers (converted to
//                 bf16) as the B operand and V^T read from an LDS copy of the
//                 V tile stored transposed, so O^T also has one query row
//                 per lane and the rescale by e^{m_old-m} is per lane.
// K/V tiles are loaded with coalesced 16-byte loads into registers one tile
// ahead of the compute (software prefetch), then written to LDS; V is
// transposed on the way in.  The transposed V rows are padded by 16 bytes
// and their 16-byte chunks XOR-swizzled by (row/8) to keep both the
// transposing writes and the MFMA operand reads free of bank conflicts.
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

constexpr int kKPad = 8;  // bf16 elements of padding per K row
constexpr int kVPad = 8;  // bf16 elements of padding per V^T row

template <int D, int BLK>
struct Tile {
  static constexpr int NT = 2 * BLK;             // threads (BLK/32 waves)
  static constexpr int KLD = D + kKPad;          // K row stride (elements)
  static constexpr int VLD = BLK + kVPad;        // V^T row stride (elements)
  static constexpr int KU = D / 16;              // 16-byte K units per thread
  static constexpr int VU = D / 64;              // 4-row x 8-col V units per thread
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
};

// Physical element column of V^T row n for logical position pos (16-byte
// chunks XOR-swizzled by n/8).
__device__ __forceinline__ int vt_col(int n, int pos) {
  return (((pos >> 3) ^ ((n >> 3) & 7)) << 3) | (pos & 7);
}

// Logical V^T position of key j inside a tile: the 8 keys that one lane
// half feeds to one PV step are stored contiguously (see the P layout).
__device__ __forceinline__ int vt_pos(int j) {
  // j = 16*c + 8*a + 4*hb + t  ->  pos = 16*c + 8*hb + 4*a + t
  return (j & ~15) | ((j & 4) << 1) | ((j & 8) >> 1) | (j & 3);
}

template <int D, int BLK>
struct Prefetch {
  u32x4 kr[Tile<D, BLK>::KU];
  u32x4 vr[4 * Tile<D, BLK>::VU];
};

// Issue the global loads of one tile into registers.  Exact tiles come from
// bf16 K/V rows [row0, row0 + BLK) with `valid` real rows; pseudo tiles from
// the float32 pooled K-bar / V-sum rows, converted to bf16 here.
template <int D, int BLK>
__device__ __forceinline__ void load_tile(Prefetch<D, BLK>& pf, bool pseudo, const uint16_t* kx,
                                          const uint16_t* vx, const float* kp, const float* vp,
                                          int valid, int t) {
  using TL = Tile<D, BLK>;
#pragma unroll
  for (int i = 0; i < TL::KU; ++i) {
    const int u = t + i * TL::NT;
    const int r = u / TL::CPR, c = u % TL::CPR;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (r < valid) {
      if (!pseudo) {
        x = *reinterpret_cast<const u32x4*>(kx + (size_t)r * D + 8 * c);
      } else {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(kp + (size_t)r * D + 8 * c);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(kp + (size_t)r * D + 8 * c + 4);
        x = u32x4{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                  pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
      }
    }
    pf.kr[i] = x;
  }
#pragma unroll
  for (int i = 0; i < TL::VU; ++i) {
    const int u = t + i * TL::NT;
    const int rg = u / TL::CPR, c = u % TL::CPR;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int r = 4 * rg + rr;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (r < valid) {
        if (!pseudo) {
          x = *reinterpret_cast<const u32x4*>(vx + (size_t)r * D + 8 * c);
        } else {
          const f32x4 lo = *reinterpret_cast<const f32x4*>(vp + (size_t)r * D + 8 * c);
          const f32x4 hi = *reinterpret_cast<const f32x4*>(vp + (size_t)r * D + 8 * c + 4);
          x = u32x4{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                    pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
        }
      }
      pf.vr[4 * i + rr] = x;
    }
  }
}

template <int D, int BLK>
__device__ __forceinline__ void store_tile(const Prefetch<D, BLK>& pf, uint16_t* Ks, uint16_t* Vt,
                                           int t) {
  using TL = Tile<D, BLK>;
#pragma unroll
  for (int i = 0; i < TL::KU; ++i) {
    const int u = t + i * TL::NT;
    const int r = u / TL::CPR, c = u % TL::CPR;
    *reinterpret_cast<u32x4*>(Ks + r * TL::KLD + 8 * c) = pf.kr[i];
  }
#pragma unroll
  for (int i = 0; i < TL::VU; ++i) {
    const int u = t + i * TL::NT;
    const int rg = u / TL::CPR, c = u % TL::CPR;
    const int pos = vt_pos(4 * rg);
    const u32x4& r0 = pf.vr[4 * i + 0];
    const u32x4& r1 = pf.vr[4 * i + 1];
    const u32x4& r2 = pf.vr[4 * i + 2];
    const u32x4& r3 = pf.vr[4 * i + 3];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int wd = e >> 1;
      const int sh = (e & 1) * 16;
      const uint32_t a0 = (r0[wd] >> sh) & 0xFFFFu, a1 = (r1[wd] >> sh) & 0xFFFFu;
      const uint32_t a2 = (r2[wd] >> sh) & 0xFFFFu, a3 = (r3[wd] >> sh) & 0xFFFFu;
      const int n = 8 * c + e;
      *reinterpret_cast<u32x2*>(Vt + n * TL::VLD + vt_col(n, pos)) = u32x2{a0 | (a1 << 16), a2 | (a3 << 16)};
    }
  }
}

template <int D, int BLK>
__global__ __launch_bounds__(2 * BLK) void attn_bf16_kernel(FwdArgs a) {
  using TL = Tile<D, BLK>;
  constexpr int NJS = BLK / 32;   // 32-key sub-tiles per tile
  constexpr int NKS = D / 16;     // 16-wide d steps of S
  constexpr int NOT = D / 32;     // 32-wide d tiles of O
  constexpr int NKC = BLK / 16;   // 16-key steps of PV

  __shared__ __attribute__((aligned(16))) uint16_t Ks[BLK * TL::KLD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * TL::VLD];
  __shared__ uint32_t selbits[kMaxBlocks / 32];

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
  const int w = t >> 6;
  const int lq = lane & 31;   // query row inside the wave / MFMA column
  const int hh = lane >> 5;   // lane half

  const int q_tok = I * BLK + 32 * w + lq;
  const bool q_ok = q_tok < a.N;

  // Q fragment (B operand of S^T): row q_tok, d = 16*ks + 8*hh + e.
  bf16x8 qf[NKS];
  {
    const uint16_t* qrow = a.q + ((size_t)bh * a.N + (q_ok ? q_tok : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 x = q_ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * hh) : u32x4{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const int n_sel = a.cnt[(size_t)bh * a.M + I];
  const int32_t* list = a.idx + ((size_t)bh * a.M + I) * a.M;
  const int Jend = a.causal ? I + 1 : a.M;
  const int n_tail = a.approx ? (Jend + BLK - 1) / BLK : 0;
  const int n_tiles = n_sel + n_tail;

  if (a.approx) {
    for (int i = t; i < kMaxBlocks / 32; i += TL::NT) selbits[i] = 0u;
    __syncthreads();
    for (int e = t; e < n_sel; e += TL::NT) {
      const int J = list[e];
      atomicOr(&selbits[J >> 5], 1u << (J & 31));
    }
    // visible after the first barrier of the tile loop
  }

  const size_t kv_off = (size_t)(b * a.Hkv + g) * a.N * D;
  const size_t pp_off = (size_t)(b * a.Hkv + g) * a.M * D;
  const int last_n = a.N - (a.M - 1) * BLK;

  auto issue = [&](Prefetch<D, BLK>& pf, int e) {
    if (e < n_sel) {
      const int J = list[e];
      const size_t o = kv_off + (size_t)J * BLK * D;
      load_tile<D, BLK>(pf, false, a.k + o, a.v + o, nullptr, nullptr, min(BLK, a.N - J * BLK), t);
    } else {
      const int T = e - n_sel;
      const size_t o = pp_off + (size_t)T * BLK * D;
      load_tile<D, BLK>(pf, true, nullptr, nullptr, a.k_bar + o, a.v_sum + o,
                        min(BLK, a.M - T * BLK), t);
    }
  };

  f32x16 o[NOT];
#pragma unroll
  for (int i = 0; i < NOT; ++i) o[i] = f32x16{};
  float m = -INFINITY;
  float l = 0.f;

  Prefetch<D, BLK> pf;
  if (n_tiles > 0) issue(pf, 0);

  for (int e = 0; e < n_tiles; ++e) {
    __syncthreads();
    store_tile<D, BLK>(pf, Ks, Vt, t);
    __syncthreads();
    if (e + 1 < n_tiles) issue(pf, e + 1);

    const bool pseudo = e >= n_sel;
    const int J = pseudo ? (e - n_sel) : list[e];   // key block, or pooled-row tile

    // ---- S^T = K Q^T
    f32x16 s[NJS];
#pragma unroll
    for (int js = 0; js < NJS; ++js) {
      s[js] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + (32 * js + lq) * TL::KLD + 16 * ks + 8 * hh);
        s[js] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s[js], 0, 0, 0);
      }
    }

    // ---- mask, scale, running max.  Register r of sub-tile js holds key
    // (tile row) 32*js + 8*(r/4) + 4*hh + (r%4) for query row lq.
    float wgt[NJS][16];
    const bool need_mask = pseudo || (J * BLK + BLK > a.N) || (a.causal && J == I);
    float mx = -INFINITY;
#pragma unroll
    for (int js = 0; js < NJS; ++js) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jr = 32 * js + 8 * (r >> 2) + 4 * hh + (r & 3);
        float wv = 1.f;
        if (need_mask) {
          if (!pseudo) {
            const int kt = J * BLK + jr;
            wv = (kt < a.N && (!a.causal || kt <= q_tok)) ? 1.f : 0.f;
          } else {
            const int pj = J * BLK + jr;
            const bool on = pj < Jend && !((selbits[pj >> 5] >> (pj & 31)) & 1u);
            wv = on ? (pj == a.M - 1 ? (float)last_n : (float)BLK) : 0.f;
          }
        }
        wgt[js][r] = wv;
        const float z = wv > 0.f ? s[js][r] * a.scale_log2 : -INFINITY;
        s[js][r] = z;
        mx = fmaxf(mx, z);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx);
    const float ms = m_new == -INFINITY ? 0.f : m_new;
    const float corr = __builtin_amdgcn_exp2f(m - ms);

    // ---- P = exp2(z - m), row sums, bf16 pack (B operand of O^T += V^T P^T)
    bf16x8 pk[NKC];
    float lsum = 0.f;
#pragma unroll
    for (int js = 0; js < NJS; ++js) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        uint32_t wds[4];
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const int r0 = 8 * c + 2 * q2;
          const float p0 = __builtin_amdgcn_exp2f(s[js][r0] - ms);
          const float p1 = __builtin_amdgcn_exp2f(s[js][r0 + 1] - ms);
          lsum += need_mask ? (wgt[js][r0] * p0 + wgt[js][r0 + 1] * p1) : (p0 + p1);
          wds[q2] = pack_bf16x2(p0, p1);
        }
        pk[2 * js + c] = __builtin_bit_cast(bf16x8, u32x4{wds[0], wds[1], wds[2], wds[3]});
      }
    }
    l = l * corr + lsum;
    m = m_new;

    // ---- O^T = O^T * corr + V^T P^T
#pragma unroll
    for (int nt = 0; nt < NOT; ++nt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) o[nt][r] *= corr;
      const int n = 32 * nt + lq;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(Vt + n * TL::VLD + vt_col(n, 16 * kc + 8 * hh));
        o[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pk[kc], o[nt], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O / l, bf16, row q_tok; register r of d-tile nt holds
  // d = 32*nt + 8*(r/4) + 4*hh + (r%4).
  const float lt = l + __shfl_xor(l, 32, 64);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (q_ok) {
    uint16_t* orow = a.out + ((size_t)bh * a.N + q_tok) * D;
#pragma unroll
    for (int nt = 0; nt < NOT; ++nt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * nt + 8 * q4 + 4 * hh;
        const u32x2 x = {pack_bf16x2(o[nt][4 * q4] * inv, o[nt][4 * q4 + 1] * inv),
                         pack_bf16x2(o[nt][4 * q4 + 2] * inv, o[nt][4 * q4 + 3] * inv)};
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
