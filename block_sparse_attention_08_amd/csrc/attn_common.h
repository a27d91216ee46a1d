// Internal helpers shared by the bf16 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace sa {

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int KT = 64;  // keys per tile (a 128-token block is two tiles)

constexpr bf16x2 kOnes = {(__bf16)1.0f, (__bf16)1.0f};

// Masking a tile needs: none (interior exact tile), the ragged end / causal
// diagonal (edge); tail tiles of pooled rows need none but the log2(n_J)
// offset, except the last one (padding rows, a short last block).
enum { kModePlain = 0, kModeEdge = 1, kModeTail = 2, kModeTailLast = 3 };
template <int MODE>
struct ModeC { static constexpr int value = MODE; };

// two floats -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Wait until this wave's outstanding global loads (including the ones that
// write LDS directly) have completed.
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The block lists and counts stay unchanged while an attention kernel runs:
// reading them through the constant address space turns the uniform per-tile
// index reads into scalar loads, counted by lgkmcnt, so that fetching the
// next block index never waits on the K/V tile loads in flight (vmcnt).
typedef const __attribute__((address_space(4))) int32_t const_i32;
__device__ __forceinline__ const const_i32* scalar_view(const int32_t* p) {
  return (const const_i32*)p;
}

// Buffer resource over one [rows, D] bf16 head of `bytes` bytes: loads past
// the end return zero (rows of a ragged last block, pooled rows past M).
// The hardware range check of a raw buffer covers the per-lane offset plus
// the instruction's immediate, not the scalar offset, so every load here
// carries its whole offset in the per-lane operand and passes 0 as soffset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint16_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, 0x00020000);
}

// Output rows staged in LDS.  A wave's output rows are consecutive in
// memory, but its accumulator fragments hold 8-byte pieces of many rows; a
// store straight from them touches a cache line per row in every
// instruction.  Instead the wave writes its fragments into a free LDS area
// (row r at r * 2D bytes, its 16-byte chunk c in slot stage_slot(r, c), a
// swizzle that spreads a column of rows over the banks) and then stores
// whole 16-byte chunks, 64 / (D/8) consecutive rows per instruction.
template <int D>
__device__ __forceinline__ int stage_slot(int r, int c) { return c ^ (r & (D / 8 - 1)); }

// The store half: ROWS staged rows to out[0 .. nrows) (rows at or past
// nrows are not written), non-temporal (the output is not read again by the
// kernel).  The wave's own LDS writes must precede it; the fences order them
// for the other lanes of the wave.
template <int D, int ROWS>
__device__ __forceinline__ void store_staged_rows(const char* stage, uint16_t* out, int nrows, int lane) {
  constexpr int CPR = D / 8;
  constexpr int RPI = 64 / CPR;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < ROWS / RPI; ++i) {
    const int r = RPI * i + lane / CPR;
    const int c = lane % CPR;
    const u32x4 x = *reinterpret_cast<const u32x4*>(stage + r * (2 * D) + stage_slot<D>(r, c) * 16);
    if (r < nrows) __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(out + (size_t)r * D + c * 8));
  }
}

}  // namespace sa
