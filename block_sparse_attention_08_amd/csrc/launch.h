// Internal host-side launch interface between the C ABI (api.cpp) and the
// kernel translation units.  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

struct Shape {
  int B, Hq, Hkv, N, D, block, M;
  int dtype;  // 0 = f32, 1 = bf16
};

// Stage 1: block means of q and k, block sums of v (v may be null); with a
// non-null `tail` also the bf16 block means of k and of v (2 x [B,Hkv,M,D]).
hipError_t launch_pool(const Shape& s, const void* q, const void* k, const void* v,
                       float* q_bar, float* k_bar, float* v_sum, void* tail, hipStream_t st);

// Stage 2: pooled scores + selection + compaction.
struct SelectParams {
  float scale;
  int mode;        // 0 alpha, 1 density
  float alpha;
  double density;
  int causal;
  int force_diag;  // causal && approx
};
hipError_t launch_select(const Shape& s, const SelectParams& p, const float* q_bar,
                         const float* k_bar, int32_t* blk_idx, int32_t* blk_cnt, hipStream_t st);

// Stages 1 + 2 in one cooperative launch (same outputs as launch_pool then
// launch_select).
hipError_t launch_route_fused(const Shape& s, const SelectParams& p, const void* q, const void* k,
                              const void* v, float* q_bar, float* k_bar, float* v_sum, void* tail,
                              int32_t* blk_idx, int32_t* blk_cnt, hipStream_t st);

// Stage 3: attention over the listed blocks (+ 0th-order tail).
struct FwdParams {
  float scale;
  int causal;
  int approx;
  float* lse;   // optional [B, Hq, N]: natural log of each row's softmax denominator
};
hipError_t launch_fwd(const Shape& s, const FwdParams& p, const void* q, const void* k,
                      const void* v, const float* k_bar, const float* v_sum, const void* tail,
                      const int32_t* blk_idx, const int32_t* blk_cnt, void* out, hipStream_t st);

// Validation of block lists: writes [flags, bad rows, first bad row] to
// `result` (three device words; cleared by the launch itself).
hipError_t launch_check_lists(const Shape& s, int causal, int approx, const int32_t* blk_idx,
                              const int32_t* blk_cnt, uint32_t* result, hipStream_t st);

// Gradients of stage 3 (bf16 inputs).
struct BwdSizes {
  size_t lse, delta, sel_bits, col_idx, col_cnt, dk_bar, dv_bar;
};
struct BwdParams {
  float scale;
  int causal;
  int approx;
};
struct BwdPtrs {
  const void *q, *k, *v, *tail, *out, *dout;
  const int32_t *blk_idx, *blk_cnt;
  const float* lse;
  float* delta;
  uint32_t* sel_bits;
  int32_t *col_idx, *col_cnt;
  float *dk_bar, *dv_bar;
  void *dq, *dk, *dv;
};
BwdSizes bwd_sizes(const Shape& s, int approx);
hipError_t launch_bwd(const Shape& s, const BwdParams& p, const BwdPtrs& x, hipStream_t st);

// Largest number of key blocks per row the selection kernel supports.
constexpr int kMaxBlocks = 2048;

}  // namespace sa
