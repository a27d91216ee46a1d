// Achievable-rate kernels for the roofline denominators, measured on the
// machine at hand next to the datasheet peaks: a streaming read over a buffer
// much larger than the last-level cache (HBM), loops of independent bf16
// matrix-core products (MFMA) on one operand pair and on changing data, and
// a loop of 16-byte LDS reads (the operand
// path of the attention kernels).  Measurement only; nothing on the attention
// path calls them.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sa_peaks.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;                     // 16-byte loads in flight per thread and trip
constexpr size_t kChunk = (size_t)kThreads * kUnroll * 16;   // bytes per workgroup trip

// Workgroup w reads chunks w, w + grid, ...; thread t reads the vectors
// t + 256u of a chunk.  The xor of everything read decides a store that never
// happens, so no load can be dropped.
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ p, size_t chunks,
                                                        uint32_t* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t c = blockIdx.x; c < chunks; c += gridDim.x) {
    const u32x4* q = p + c * (kThreads * kUnroll) + threadIdx.x;
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x[u] = __builtin_nontemporal_load(q + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= x[u];
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[blockIdx.x & 255] = acc.x;
}

// Four independent accumulator chains per wave of v_mfma_f32_32x32x16_bf16
// (32*32*16*2 flops each).  Operands depend on the lane and a runtime value,
// the result decides a store that never happens.
constexpr int kChains = 4;
constexpr double kFlopsPerMfma = 32.0 * 32.0 * 16.0 * 2.0;

__global__ __launch_bounds__(kThreads) void mfma_kernel(int iters, float seed, uint32_t* sink) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(seed * (float)(threadIdx.x + e));
    b[e] = (__bf16)(seed * (float)(threadIdx.x - e));
  }
  f32x16 c[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[i][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kChains; ++i) c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kChains; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[i][r];
  if (s == 1234.5f) sink[blockIdx.x & 255] = __float_as_uint(s);
}

// The same products over changing data: eight operand pairs of random bits
// (bf16 values in [-2, 2)) taken in turn, B rotated against A per chain.  A
// loop on one operand pair toggles few bits in the matrix cores and draws
// less power than products over real data, and the clock the chip holds
// under load follows the power it draws; this loop gives the rate for data
// that changes with every product.  Two 256-thread workgroups per CU (the
// operand registers leave room for two waves per SIMD; four independent
// chains per wave keep the matrix core fed).
constexpr int kPairs = 8;

__global__ __launch_bounds__(kThreads) void mfma_data_kernel(int iters, uint32_t seed, uint32_t* sink) {
  bf16x8 a[kPairs], b[kPairs];
  uint32_t x = seed ^ (threadIdx.x * 2654435761u) ^ (blockIdx.x * 40503u);
#pragma unroll
  for (int u = 0; u < kPairs; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x ^= x << 13; x ^= x >> 17; x ^= x << 5;       // xorshift32
      a[u][e] = (__bf16)((float)(x & 0xFFFFu) * (1.0f / 16384.0f) - 2.0f);
      x ^= x << 13; x ^= x >> 17; x ^= x << 5;
      b[u][e] = (__bf16)((float)(x & 0xFFFFu) * (1.0f / 16384.0f) - 2.0f);
    }
  f32x16 c[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[i][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < kPairs; ++u)
#pragma unroll
      for (int i = 0; i < kChains; ++i)
        c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[(u + i) % kPairs], c[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kChains; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[i][r];
  if (s == 1234.5f) sink[blockIdx.x & 255] = __float_as_uint(s);
}

// LDS read rate: four 256-thread workgroups per CU, each filling 32 KB of
// LDS once, then per trip 16 ds_read_b128 per wave (1 KB each, contiguous
// per instruction, so free of bank conflicts) kept in flight together; an
// empty volatile statement takes every loaded vector, so no read can be
// dropped, and a compiler memory barrier per trip keeps the reads inside
// the loop.  Indexes stay below kLdsVec: base + 64*15 + 63 <= 1024 + 1023.
constexpr int kLdsVec = 2048;                  // 16-byte vectors per workgroup (32 KB)
constexpr int kLdsReads = 16;                  // reads per wave and trip

__global__ __launch_bounds__(kThreads) void lds_kernel(int iters, uint32_t* sink) {
  __shared__ u32x4 buf[kLdsVec];
  for (int i = threadIdx.x; i < kLdsVec; i += kThreads)
    buf[i] = u32x4{(uint32_t)i, (uint32_t)i + 1u, (uint32_t)i + 2u, (uint32_t)i + 3u};
  __syncthreads();
  const int lane = threadIdx.x & 63;
  for (int it = 0; it < iters; ++it) {
    const int base = (it & 1) * (kLdsVec / 2);
    u32x4 x[kLdsReads];
#pragma unroll
    for (int u = 0; u < kLdsReads; ++u) x[u] = buf[base + 64 * u + lane];
#pragma unroll
    for (int u = 0; u < kLdsReads; u += 4) asm volatile("" ::"v"(x[u]), "v"(x[u + 1]), "v"(x[u + 2]), "v"(x[u + 3]));
    asm volatile("" ::: "memory");
  }
  if (iters < 0) sink[blockIdx.x & 255] = 1u;
}

int grid_for(int per_cu) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return cus * per_cu;
}

}  // namespace

SA_PEAKS_EXPORT int sa_peak_read(const void* buf, size_t bytes, void* sink, void* stream,
                                 size_t* bytes_read) {
  if (!buf || !sink || !bytes_read) return (int)hipErrorInvalidValue;
  if (((uintptr_t)buf & 15u) != 0) return (int)hipErrorInvalidValue;
  const size_t chunks = bytes / kChunk;
  *bytes_read = chunks * kChunk;
  if (chunks == 0) return (int)hipSuccess;
  const int grid = grid_for(8);
  if (grid <= 0) return (int)hipErrorInvalidDevice;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const u32x4*)buf, chunks, (uint32_t*)sink);
  return (int)hipGetLastError();
}

SA_PEAKS_EXPORT int sa_peak_mfma_bf16(int iters, void* sink, void* stream, double* flops) {
  if (!sink || !flops || iters < 1) return (int)hipErrorInvalidValue;
  const int grid = grid_for(8);
  if (grid <= 0) return (int)hipErrorInvalidDevice;
  *flops = (double)grid * (kThreads / 64) * (double)iters * kChains * kFlopsPerMfma;
  hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, iters, 1.0e-3f,
                     (uint32_t*)sink);
  return (int)hipGetLastError();
}

SA_PEAKS_EXPORT int sa_peak_mfma_bf16_data(int iters, void* sink, void* stream, double* flops) {
  if (!sink || !flops || iters < 1) return (int)hipErrorInvalidValue;
  const int grid = grid_for(2);
  if (grid <= 0) return (int)hipErrorInvalidDevice;
  *flops = (double)grid * (kThreads / 64) * (double)iters * kPairs * kChains * kFlopsPerMfma;
  hipLaunchKernelGGL(mfma_data_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, iters, 12345u,
                     (uint32_t*)sink);
  return (int)hipGetLastError();
}

SA_PEAKS_EXPORT int sa_peak_lds_read(int iters, void* sink, void* stream, double* bytes) {
  if (!sink || !bytes || iters < 1) return (int)hipErrorInvalidValue;
  const int grid = grid_for(4);
  if (grid <= 0) return (int)hipErrorInvalidDevice;
  *bytes = (double)grid * kThreads * (double)iters * kLdsReads * 16.0;
  hipLaunchKernelGGL(lds_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, iters, (uint32_t*)sink);
  return (int)hipGetLastError();
}
