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

// Work split of the kernels that read a slot row by row (fold, statistics):
// a slot is kStatParts parts of kPartRows rows (one 16 KB float32 part per
// workgroup, so the workgroups in flight cover a compact range), and the
// grad statistics keep one float64 partial sum per part.  The fold (fused
// statistics), the statistics pass over row-major grads and the statistics
// kernel over folded grads all use this order, so they give bit-identical
// partials: in part q, thread t adds the part's chunks t, t + 256, t + 512,
// t + 768 in increasing order, the 4 elements of a chunk in increasing order,
// then the block reduction below combines the 256 thread sums in a fixed order.
constexpr int kSumThreads = 256;
// XCDs of the part; consecutive workgroups of a launch are dealt to them in turn
constexpr int kXcds = 8;
// last-level (Infinity) cache of the part, shared by all XCDs
constexpr int64_t kLastLevelCacheBytes = 256LL << 20;
constexpr int kStatParts = FP8Z1_STAT_PARTS;
static_assert(kB % kStatParts == 0 && (kChunks / kStatParts) % kSumThreads == 0, "part split");
constexpr int kPartRows = kB / kStatParts;
constexpr int kPartChunks = kChunks / kStatParts;
constexpr int kPartPasses = kPartChunks / kSumThreads;

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

// Streaming (non-temporal) 16-byte and 4-byte accesses for data that is
// touched once per kernel: the loads and stores carry the non-temporal hint,
// so they do not displace other lines in the caches and the stores do not
// linger as dirty lines.
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 ld_stream(const float4* p) {
  const v4f_t r = __builtin_nontemporal_load(reinterpret_cast<const v4f_t*>(p));
  return make_float4(r.x, r.y, r.z, r.w);
}
__device__ __forceinline__ void st_stream(float4* p, float4 x) {
  const v4f_t r = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(r, reinterpret_cast<v4f_t*>(p));
}
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const v4u_t r = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(p));
  return make_uint4(r.x, r.y, r.z, r.w);
}
__device__ __forceinline__ void st_stream(uint4* p, uint4 x) {
  const v4u_t r = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(r, reinterpret_cast<v4u_t*>(p));
}
__device__ __forceinline__ void st_stream(uint32_t* p, uint32_t x) { __builtin_nontemporal_store(x, p); }

// Accesses to row-major params.  Their pointers come from a device array, so
// the compiler cannot tell they are global and would emit flat instructions;
// these helpers go through global-address-space pointers.  A row of a param
// whose width is not a multiple of 4 starts at an element-aligned address only:
// gfx950 under ROCm runs in unaligned-access mode, so a 16-byte load at 4-byte
// alignment is still one dwordx4 instruction; the callers only use it on bytes
// that lie inside the row segment they own.
typedef float v4f_a4_t __attribute__((ext_vector_type(4), aligned(4)));
typedef float v4f_a4_global_t __attribute__((ext_vector_type(4), aligned(4), address_space(1)));
typedef uint32_t v4u_global_t __attribute__((ext_vector_type(4), address_space(1)));
typedef uint32_t v2u_t __attribute__((ext_vector_type(2)));
typedef uint32_t v2u_a2_global_t __attribute__((ext_vector_type(2), aligned(2), address_space(1)));

// streaming 16-byte load of 4 float32 at 4-byte alignment
__device__ __forceinline__ float4 ld_global_stream_a4(const float* p) {
  const v4f_a4_t r = __builtin_nontemporal_load((const v4f_a4_global_t*)(p));
  return make_float4(r.x, r.y, r.z, r.w);
}
// the same load, cached (for data read again soon)
__device__ __forceinline__ float4 ld_global_a4(const float* p) {
  const v4f_a4_t r = *(const v4f_a4_global_t*)(p);
  return make_float4(r.x, r.y, r.z, r.w);
}
// streaming 8-byte load of 4 bfloat16 at 2-byte alignment
__device__ __forceinline__ uint2 ld_global_stream_a2x8(const uint16_t* p) {
  const v2u_t r = __builtin_nontemporal_load((const v2u_a2_global_t*)(p));
  return make_uint2(r.x, r.y);
}
// streaming 16-byte store to a 16-byte aligned address
__device__ __forceinline__ void st_global_stream(void* p, uint4 x) {
  const v4u_t r = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(r, (v4u_global_t*)(p));
}
// plain 16-byte accesses at element alignment (partial chunks and rows)
__device__ __forceinline__ float4 ld_a4(const float* p) {
  float4 r;
  __builtin_memcpy(&r, p, 16);
  return r;
}
__device__ __forceinline__ void st_a4(float* p, float4 x) { __builtin_memcpy(p, &x, 16); }
__device__ __forceinline__ void st_a1(uint8_t* p, uint4 x) { __builtin_memcpy(p, &x, 16); }

// Square of a float32 value in float64 (exact: a 24-bit significand squared fits in 53 bits).
__device__ __forceinline__ double sq64(float x) {
  const double d = static_cast<double>(x);
  return d * d;
}

}  // namespace fp8z1
