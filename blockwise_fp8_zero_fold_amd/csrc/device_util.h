// Device helpers shared by the fp8z1 kernels: slot plan access, chunk
// geometry, deterministic wave/block reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace fp8z1 {

// A block is processed as 4096 chunks of 4 consecutive elements (16 bytes of
// float32).  Chunk c covers row c / 32, columns 4 * (c % 32) .. +3.
constexpr int kChunks = kBlockElems / 4;
constexpr int kChunksPerRow = kB / 4;

// Thread count and chunk order of the per-slot sum of squares.  The fold
// (fused statistics) and the separate statistics kernel both use it, so the
// two give bit-identical per-slot sums: thread t adds chunks t, t + 256, ...
// in increasing order, the 4 elements of a chunk in increasing order, then
// the block reduction below combines the 256 partial sums in a fixed order.
constexpr int kSumThreads = 256;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Butterfly sum: every lane ends with the same value (each step adds two
// equal-order pairs, and float addition is commutative), so the result does
// not depend on scheduling.
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Max over the workgroup, broadcast to every thread.
template <int THREADS>
__device__ __forceinline__ float block_max(float v, float* lds) {
  constexpr int W = THREADS / 64;
  v = wave_max(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) lds[w] = v;
  __syncthreads();
  float r = lds[0];
#pragma unroll
  for (int i = 1; i < W; ++i) r = fmaxf(r, lds[i]);
  return r;
}

// Sum over the workgroup in a fixed order (waves' sums added in wave order);
// the result is valid in thread 0.
template <int THREADS>
__device__ __forceinline__ double block_sum(double v, double* lds) {
  constexpr int W = THREADS / 64;
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) lds[w] = v;
  __syncthreads();
  double r = 0.0;
  if (threadIdx.x == 0) {
    r = lds[0];
#pragma unroll
    for (int i = 1; i < W; ++i) r += lds[i];
  }
  return r;
}

// Square of a float32 value in float64 (exact: a 24-bit significand squared fits in 53 bits).
__device__ __forceinline__ double sq64(float x) {
  const double d = static_cast<double>(x);
  return d * d;
}

}  // namespace fp8z1
