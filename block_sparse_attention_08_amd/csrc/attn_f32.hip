// Stage 3 for float32 inputs: exact attention over the listed key blocks
// plus the 0th-order tail, on the vector ALUs in float32.
//
// One workgroup per (batch, head, query block), one thread per query token.
// Keys are visited in chunks of 64 staged in LDS; each chunk updates the
// running max m, sum l and output o of the online softmax (FlashAttention
// tutorial, section 2: m <- max(m, max z); l <- l e^{m_old-m} + sum e^{z-m};
// o <- o e^{m_old-m} + sum e^{z-m} v; answer o / l).  With the tail on, each
// eligible unlisted block J enters the same recurrence as one pseudo-key
// kbar_J with weight n_J in l and value sum SigmaV_J in o (PISA explainer,
// routing table: unselected blocks are represented by the block-mean key
// and the value sum, inside the same online softmax).
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace sa {
namespace {

constexpr int kThreads = 128;
constexpr int kChunk = 64;   // keys staged per LDS chunk
constexpr int kSub = 16;     // keys per online-softmax update

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

template <int D>
struct State {
  float q[D];
  float o[D];
  float m, l;
};

// Fold keys [0, n) of the staged chunk into the state.  key_pos(j) gives the
// token index used for causal masking (or -1 for pseudo-keys), weight(j) the
// multiplicity in l (0 masks the key out).
template <int D, typename Vis>
__device__ __forceinline__ void fold_chunk(State<D>& st, const float (*Ks)[D], const float (*Vs)[D],
                                           int n, Vis visible_weight) {
  for (int j0 = 0; j0 < n; j0 += kSub) {
    float z[kSub];
    float wgt[kSub];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kSub; ++jj) {
      const int j = j0 + jj;
      wgt[jj] = j < n ? visible_weight(j) : 0.f;
      float acc = 0.f;
      if (wgt[jj] > 0.f) {
#pragma unroll 16
        for (int c = 0; c < D; ++c) acc = fmaf(st.q[c], Ks[j][c], acc);
        z[jj] = acc;
      } else {
        z[jj] = -INFINITY;
      }
      mx = fmaxf(mx, z[jj]);
    }
    const float m_new = fmaxf(st.m, mx);
    const float ms = m_new == -INFINITY ? 0.f : m_new;
    const float corr = expf(st.m - ms);
    float p[kSub];
    float lsum = 0.f;
#pragma unroll
    for (int jj = 0; jj < kSub; ++jj) {
      p[jj] = wgt[jj] > 0.f ? expf(z[jj] - ms) : 0.f;
      lsum = fmaf(wgt[jj], p[jj], lsum);
    }
    st.l = st.l * corr + lsum;
#pragma unroll 8
    for (int c = 0; c < D; ++c) {
      float acc = st.o[c] * corr;
#pragma unroll
      for (int jj = 0; jj < kSub; ++jj) {
        if (j0 + jj < n) acc = fmaf(p[jj], Vs[j0 + jj][c], acc);
      }
      st.o[c] = acc;
    }
    st.m = m_new;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(FwdArgs a) {
  __shared__ float Ks[kChunk][D];
  __shared__ float Vs[kChunk][D];
  __shared__ uint32_t selbits[kMaxBlocks / 32];

  const int item = blockIdx.x;
  const int bh = item / a.M;
  const int I = item - bh * a.M;
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int t = threadIdx.x;
  const int qi = I * a.block + t;                 // this thread's query token
  const bool active = t < a.block && qi < a.N;
  const size_t kvbase = (size_t)(b * a.Hkv + g) * a.N * D;

  State<D> st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    st.q[c] = active ? a.q[((size_t)bh * a.N + qi) * D + c] * a.scale : 0.f;
    st.o[c] = 0.f;
  }

  const int n_sel = a.cnt[(size_t)bh * a.M + I];
  const int32_t* list = a.idx + ((size_t)bh * a.M + I) * a.M;
  for (int w = t; w < kMaxBlocks / 32; w += kThreads) selbits[w] = 0u;
  __syncthreads();
  for (int e = t; e < n_sel; e += kThreads) {
    const int J = list[e];
    atomicOr(&selbits[J >> 5], 1u << (J & 31));
  }

  // ---- exact blocks
  for (int e = 0; e < n_sel; ++e) {
    const int J = list[e];
    const int k0 = J * a.block;
    const int kn = min(a.block, a.N - k0);
    for (int c0 = 0; c0 < kn; c0 += kChunk) {
      const int n = min(kChunk, kn - c0);
      __syncthreads();
      for (int u = t; u < n * D; u += kThreads) {
        const int r = u / D, c = u - r * D;
        Ks[r][c] = a.k[kvbase + (size_t)(k0 + c0 + r) * D + c];
        Vs[r][c] = a.v[kvbase + (size_t)(k0 + c0 + r) * D + c];
      }
      __syncthreads();
      if (active) {
        const int first = k0 + c0;
        const int causal = a.causal;
        fold_chunk<D>(st, Ks, Vs, n, [&](int j) -> float {
          return (!causal || first + j <= qi) ? 1.f : 0.f;
        });
      }
    }
  }

  // ---- 0th-order tail: eligible blocks not in the list
  if (a.approx) {
    const int Jend = a.causal ? I + 1 : a.M;
    const size_t pbase = (size_t)(b * a.Hkv + g) * a.M * D;
    for (int c0 = 0; c0 < Jend; c0 += kChunk) {
      const int n = min(kChunk, Jend - c0);
      __syncthreads();
      for (int u = t; u < n * D; u += kThreads) {
        const int r = u / D, c = u - r * D;
        Ks[r][c] = a.k_bar[pbase + (size_t)(c0 + r) * D + c];
        Vs[r][c] = a.v_sum[pbase + (size_t)(c0 + r) * D + c];
      }
      __syncthreads();
      if (active) {
        const int M = a.M, N = a.N, blk = a.block;
        fold_chunk<D>(st, Ks, Vs, n, [&](int j) -> float {
          const int J = c0 + j;
          if ((selbits[J >> 5] >> (J & 31)) & 1u) return 0.f;
          return J == M - 1 ? (float)(N - J * blk) : (float)blk;
        });
      }
    }
  }

  if (active) {
    const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
    if (a.lse) a.lse[(size_t)bh * a.N + qi] = st.m + logf(st.l);
    float* o = a.out + ((size_t)bh * a.N + qi) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] = st.o[c] * inv;
  }
}

template <int D>
hipError_t run(const FwdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((attn_f32_kernel<D>), dim3(a.total), dim3(kThreads), 0, st, a);
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
