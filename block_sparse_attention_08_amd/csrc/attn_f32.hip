// Stage 3 for float32 inputs: exact attention over the listed key blocks
// plus the 0th-order tail, on the vector ALUs in float32.
//
// One workgroup (eight waves) per 4 query rows of a (batch, head, query
// block), sixteen lanes per query token (each owning D/16 of the head
// dimension; the dot products are summed over the sixteen lanes with four
// lane swaps).  Each wave holds all 4 rows and takes every eighth chunk of
// the keys; the eight partial softmax states are merged at the end.
// Keys are visited in chunks of 16 staged in LDS; each chunk updates the
// running max m, sum l and output o of the online softmax (FlashAttention
// tutorial, section 2: m <- max(m, max z); l <- l e^{m_old-m} + sum e^{z-m};
// o <- o e^{m_old-m} + sum e^{z-m} v; answer o / l), evaluated in base 2
// (logits scaled by log2 e, weights 2^{z-m}: the same numbers).  With the tail on, each
// eligible unlisted block J enters the same recurrence as one pseudo-key
// kbar_J with weight n_J in l and value sum SigmaV_J in o (PISA explainer,
// routing table: unselected blocks are represented by the block-mean key
// and the value sum, inside the same online softmax).
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace sa {
namespace {

constexpr int kLanes = 16;              // lanes per query row, each owning D/16 dimensions
constexpr int kRows = kWave / kLanes;   // query rows per workgroup (all of them in every wave)
constexpr int kSplit = 8;               // waves per workgroup, each folding every 8th key chunk
constexpr int kThreads = kWave * kSplit;
constexpr int kChunk = 16;              // keys staged per LDS chunk
constexpr int kSub = 16;                // keys per online-softmax update

struct FwdArgs {
  const float* q;
  const float* k;
  const float* v;
  const float* k_bar;
  const float* v_sum;
  const int32_t* idx;
  const int32_t* cnt;
  float* out;
  float* lse;
  int Hq, Hkv, N, M, block, total;
  float scale;
  int causal, approx;
};

// Sum over the 16 lanes of a DPP row (the lanes of one query row), left in
// every lane: quad swaps (lane ^ 1, lane ^ 2), then the half-row mirror
// (lane i <-> 7 - i) and the row mirror (i <-> 15 - i), each pairing lanes
// that hold disjoint partial sums.  Both lanes of a pair add the same two
// values, so all 16 lanes end with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  static_assert(kLanes == 16, "one query row per DPP row");
  x += dpp_mov<0xB1>(x);    // quad_perm [1, 0, 3, 2]
  x += dpp_mov<0x4E>(x);    // quad_perm [2, 3, 0, 1]
  x += dpp_mov<0x141>(x);   // row_half_mirror
  x += dpp_mov<0x140>(x);   // row_mirror
  return x;
}

// Per-thread share of one query row: dimensions [s*DL, (s+1)*DL) of q (pre-
// scaled) and of the output accumulator; m and l are the same in all lanes
// of a row.
template <int D>
struct State {
  static constexpr int DL = D / kLanes;
  float q[DL];
  float o[DL];
  float m, l;
};

// Fold keys [0, n) of the staged chunk into the state of this lane's row.
// visible_weight(j) gives the multiplicity of key j in l (0 masks it out);
// it is the same in all lanes of a row.  Every lane takes part (the
// lane swaps need the whole wave); rows past the sequence end hold q = 0.
template <int D, typename Vis>
__device__ __forceinline__ void fold_chunk(State<D>& st, const float (*Ks)[D], const float (*Vs)[D], int n, int sl,
                                           Vis visible_weight) {
  constexpr int DL = State<D>::DL;
  for (int j0 = 0; j0 < n; j0 += kSub) {
    float z[kSub];
    float wgt[kSub];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kSub; ++jj) {
      const int j = j0 + jj;
      wgt[jj] = j < n ? visible_weight(j) : 0.f;
      const float4* kr = reinterpret_cast<const float4*>(&Ks[j < n ? j : 0][sl * DL]);
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < DL / 4; ++c) {
        const float4 kv = kr[c];
        acc = fmaf(st.q[4 * c], kv.x, acc);
        acc = fmaf(st.q[4 * c + 1], kv.y, acc);
        acc = fmaf(st.q[4 * c + 2], kv.z, acc);
        acc = fmaf(st.q[4 * c + 3], kv.w, acc);
      }
      acc = row16_sum(acc);               // the row's partial sums
      z[jj] = wgt[jj] > 0.f ? acc : -INFINITY;
      mx = fmaxf(mx, z[jj]);
    }
    const float m_new = fmaxf(st.m, mx);
    const float ms = m_new == -INFINITY ? 0.f : m_new;
    const float corr = __builtin_amdgcn_exp2f(st.m - ms);
    float p[kSub];
    float lsum = 0.f;
#pragma unroll
    for (int jj = 0; jj < kSub; ++jj) {
      p[jj] = wgt[jj] > 0.f ? __builtin_amdgcn_exp2f(z[jj] - ms) : 0.f;
      lsum = fmaf(wgt[jj], p[jj], lsum);
    }
    st.l = st.l * corr + lsum;
#pragma unroll
    for (int c = 0; c < DL; ++c) st.o[c] *= corr;
#pragma unroll
    for (int jj = 0; jj < kSub; ++jj) {
      if (j0 + jj < n) {
        const float4* vr = reinterpret_cast<const float4*>(&Vs[j0 + jj][sl * DL]);
#pragma unroll
        for (int c = 0; c < DL / 4; ++c) {
          const float4 vv = vr[c];
          st.o[4 * c] = fmaf(p[jj], vv.x, st.o[4 * c]);
          st.o[4 * c + 1] = fmaf(p[jj], vv.y, st.o[4 * c + 1]);
          st.o[4 * c + 2] = fmaf(p[jj], vv.z, st.o[4 * c + 2]);
          st.o[4 * c + 3] = fmaf(p[jj], vv.w, st.o[4 * c + 3]);
        }
      }
    }
    st.m = m_new;
  }
}

// One chunk of rows [0, n) of a [rows, D] float32 matrix moved through one
// wave's registers: load() issues this lane's share of global loads (zeros
// past row n), store() writes them to the wave's LDS chunk.
template <int D>
struct ChunkRegs {
  static constexpr int NPF = kChunk * (D / 4) / kWave;   // float4 per lane
  static_assert(NPF * kWave == kChunk * (D / 4), "chunk staging layout");
  float4 x[NPF];
  __device__ __forceinline__ void load(const float* src, int n, int lane) {
    const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
      const int u = lane + i * kWave;
      x[i] = u < n * (D / 4) ? s4[u] : float4{0.f, 0.f, 0.f, 0.f};
    }
  }
  __device__ __forceinline__ void store(float (*dst)[D], int lane) const {
#pragma unroll
    for (int i = 0; i < NPF; ++i) reinterpret_cast<float4*>(dst[0])[lane + i * kWave] = x[i];
  }
};

// Workgroup: kRows query rows, kSplit waves.  Every wave holds all kRows
// rows (16 lanes each) and folds every kSplit-th chunk of the key sequence
// into its own running (m, l, o); the kSplit partial states are merged at
// the end (m = max_s m_s, l = sum_s l_s 2^{m_s - m}, o likewise: the online
// softmax recurrence applied to whole partial sums).  Splitting the keys
// over the waves, with no barrier inside the chunk loop, shortens each
// workgroup's chain of dependent loads and folds, and the small row count
// spreads a short sequence over many workgroups.
template <int D>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(FwdArgs a) {
  constexpr int DL = State<D>::DL;
  __shared__ __attribute__((aligned(16))) float Ks[kSplit][kChunk][D];
  __shared__ __attribute__((aligned(16))) float Vs[kSplit][kChunk][D];
  __shared__ uint32_t selbits[kMaxBlocks / 32];
  __shared__ float part[kSplit][kRows][kLanes][DL + 2];   // per wave: o, then m and l

  const int parts = a.block / kRows;            // workgroups per query block
  const int item = blockIdx.x / parts;
  const int pr = blockIdx.x - item * parts;
  const int bh = item / a.M;
  const int I = item - bh * a.M;
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int t = threadIdx.x;
  const int s = __builtin_amdgcn_readfirstlane(t / kWave);   // key split of this wave
  const int lane = t % kWave;
  const int row = lane / kLanes, sl = lane % kLanes;   // query row, dimension slice
  const int qi = I * a.block + pr * kRows + row;      // this lane's query token
  const bool active = qi < a.N;
  const size_t kvbase = (size_t)(b * a.Hkv + g) * a.N * D;

  // logits in log2 units: q scaled by scale * log2 e, weights exp2(z - m)
  const float qs = a.scale * 1.4426950408889634f;
  State<D> st;
  st.m = -INFINITY;
  st.l = 0.f;
  {
    const float4* qr = reinterpret_cast<const float4*>(a.q + ((size_t)bh * a.N + (active ? qi : 0)) * D + sl * DL);
#pragma unroll
    for (int c = 0; c < DL / 4; ++c) {
      const float4 x = active ? qr[c] : float4{0.f, 0.f, 0.f, 0.f};
      st.q[4 * c] = x.x * qs;
      st.q[4 * c + 1] = x.y * qs;
      st.q[4 * c + 2] = x.z * qs;
      st.q[4 * c + 3] = x.w * qs;
    }
#pragma unroll
    for (int c = 0; c < DL; ++c) st.o[c] = 0.f;
  }

  const int n_sel = a.cnt[(size_t)bh * a.M + I];
  const int32_t* list = a.idx + ((size_t)bh * a.M + I) * a.M;
  if (a.approx) {
    for (int w = t; w < kMaxBlocks / 32; w += kThreads) selbits[w] = 0u;
    __syncthreads();
    for (int e = t; e < n_sel; e += kThreads) {
      const int J = list[e];
      atomicOr(&selbits[J >> 5], 1u << (J & 31));
    }
    __syncthreads();
  }

  // Chunk sequence: the listed blocks (ceil(block / kChunk) chunks each),
  // then, with the tail on, the pooled rows of blocks [0, Jend) in chunks of
  // kChunk.  Wave s takes chunks s, s + kSplit, ...; its next chunk loads
  // into registers while the current one is folded from its LDS chunk.
  const int per_blk = (a.block + kChunk - 1) / kChunk;
  const int n_exact = n_sel * per_blk;
  const int Jend = a.causal ? I + 1 : a.M;
  const int n_chunks = n_exact + (a.approx ? (Jend + kChunk - 1) / kChunk : 0);
  const size_t pbase = (size_t)(b * a.Hkv + g) * a.M * D;
  auto chunk_rows = [&](int ci, int& first, int& n) {
    if (ci < n_exact) {
      const int k0 = list[ci / per_blk] * a.block;
      first = k0 + (ci % per_blk) * kChunk;
      n = min(min(a.block, a.N - k0) - (ci % per_blk) * kChunk, kChunk);
    } else {
      first = (ci - n_exact) * kChunk;
      n = min(kChunk, Jend - first);
    }
  };
  ChunkRegs<D> kr, vr;
  auto load_chunk = [&](int ci) {
    int first, n;
    chunk_rows(ci, first, n);
    if (ci < n_exact) {
      kr.load(a.k + kvbase + (size_t)first * D, n, lane);
      vr.load(a.v + kvbase + (size_t)first * D, n, lane);
    } else {
      kr.load(a.k_bar + pbase + (size_t)first * D, n, lane);
      vr.load(a.v_sum + pbase + (size_t)first * D, n, lane);
    }
  };
  if (s < n_chunks) load_chunk(s);
  for (int ci = s; ci < n_chunks; ci += kSplit) {
    // the wave's own LDS chunk: its reads of the previous chunk precede
    // these writes in the wave's instruction order
    kr.store(Ks[s], lane);
    vr.store(Vs[s], lane);
    if (ci + kSplit < n_chunks) load_chunk(ci + kSplit);
    int first, n;
    chunk_rows(ci, first, n);
    if (ci < n_exact) {
      const int causal = a.causal;
      fold_chunk<D>(st, Ks[s], Vs[s], n, sl, [&](int j) -> float { return (!causal || first + j <= qi) ? 1.f : 0.f; });
    } else {
      // 0th-order tail: eligible blocks not in the list, weight n_J
      const int M = a.M, N = a.N, blk = a.block;
      fold_chunk<D>(st, Ks[s], Vs[s], n, sl, [&](int j) -> float {
        const int J = first + j;
        if ((selbits[J >> 5] >> (J & 31)) & 1u) return 0.f;
        return J == M - 1 ? (float)(N - J * blk) : (float)blk;
      });
    }
  }

  // merge the kSplit partial states of every row
#pragma unroll
  for (int c = 0; c < DL; ++c) part[s][row][sl][c] = st.o[c];
  part[s][row][sl][DL] = st.m;
  part[s][row][sl][DL + 1] = st.l;
  __syncthreads();
  if (s == 0 && active) {
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < kSplit; ++u) m = fmaxf(m, part[u][row][sl][DL]);
    const float ms = m == -INFINITY ? 0.f : m;
    float l = 0.f;
    float o[DL];
#pragma unroll
    for (int c = 0; c < DL; ++c) o[c] = 0.f;
#pragma unroll
    for (int u = 0; u < kSplit; ++u) {
      const float w = __builtin_amdgcn_exp2f(part[u][row][sl][DL] - ms);   // 0 for an empty split
      l = fmaf(part[u][row][sl][DL + 1], w, l);
#pragma unroll
      for (int c = 0; c < DL; ++c) o[c] = fmaf(part[u][row][sl][c], w, o[c]);
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (a.lse && sl == 0) a.lse[(size_t)bh * a.N + qi] = ms * 0.6931471805599453f + logf(l);
    float4* op = reinterpret_cast<float4*>(a.out + ((size_t)bh * a.N + qi) * D + sl * DL);
#pragma unroll
    for (int c = 0; c < DL / 4; ++c)
      op[c] = float4{o[4 * c] * inv, o[4 * c + 1] * inv, o[4 * c + 2] * inv, o[4 * c + 3] * inv};
  }
}

template <int D>
hipError_t run(const FwdArgs& a, hipStream_t st) {
  const int64_t grid = (int64_t)a.total * (a.block / kRows);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_f32_kernel<D>), dim3((unsigned)grid), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const Shape& s, const FwdParams& p, const void* q, const void* k,
                          const void* v, const float* k_bar, const float* v_sum,
                          const int32_t* blk_idx, const int32_t* blk_cnt, void* out,
                          hipStream_t st) {
  FwdArgs a{};
  a.q = static_cast<const float*>(q);
  a.k = static_cast<const float*>(k);
  a.v = static_cast<const float*>(v);
  a.k_bar = k_bar;
  a.v_sum = v_sum;
  a.idx = blk_idx;
  a.cnt = blk_cnt;
  a.out = static_cast<float*>(out);
  a.lse = p.lse;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.N = s.N;
  a.M = s.M;
  a.block = s.block;
  a.total = s.B * s.Hq * s.M;
  a.scale = p.scale;
  a.causal = p.causal;
  a.approx = p.approx;
  return s.D == 128 ? run<128>(a, st) : run<64>(a, st);
}

}  // namespace sa
