// Streaming references for the roofline.  These kernels move the bytes of a
// path kernel with the same access pattern and no arithmetic worth the name,
// so that a measured kernel can be set against the bandwidth this GPU actually
// sustains for that pattern, beside the published HBM peak.
#include <hip/hip_runtime.h>

#include "../../include/fp8z1_probe.h"
#include "device_util.h"

namespace fp8z1 {
namespace {

// plain copy, 4 KB per workgroup (256 lanes x 16 bytes), streaming accesses.
// spread = 1: workgroup b copies tile b, so the workgroups in flight cover one
// compact range; spread = S > 1: tile (b % S) * (ntiles / S) + b / S, so they
// cover S far-apart ranges, each walked in order
__global__ __launch_bounds__(256) void probe_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                         int64_t ntiles, int64_t spread) {
  const int64_t b = blockIdx.x;
  const int64_t tile = spread == 1 ? b : (b % spread) * (ntiles / spread) + b / spread;
  const int64_t i = tile * 256 + threadIdx.x;
  st_stream(dst + i, ld_stream(src + i));
}

// the update's pattern: one workgroup per 1/PARTS of a slot (64 KB / PARTS of
// each float32 array), 16 / PARTS chunks of 16 bytes per lane, the same order
// as the update kernel: per chunk read g, p, m, v and write p, m, v
// (streaming); after all chunks write 4 bytes of codes per chunk (plain
// stores, as the update does).  PARTS = 1 is the update's own tiling; smaller
// tiles show what the same mix of streams reaches when each workgroup owns
// less memory.
template <int PARTS>
__global__ __launch_bounds__(256) void probe_update_kernel(const float4* __restrict__ g, float4* __restrict__ p,
                                                           float4* __restrict__ m, float4* __restrict__ v,
                                                           uint32_t* __restrict__ q) {
  constexpr int kPasses = kChunks / 256 / PARTS;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (kChunks / PARTS);
  float keep[kPasses];
#pragma unroll
  for (int k = 0; k < kPasses; ++k) {
    const int64_t i = base + threadIdx.x + 256 * k;
    const float4 a = ld_stream(g + i), b = ld_stream(p + i), c = ld_stream(m + i), d = ld_stream(v + i);
    st_stream(p + i, make_float4(b.x + a.x, b.y + a.y, b.z + a.z, b.w + a.w));
    st_stream(m + i, make_float4(c.x + a.x, c.y + a.y, c.z + a.z, c.w + a.w));
    st_stream(v + i, make_float4(d.x + a.x, d.y + a.y, d.z + a.z, d.w + a.w));
    keep[k] = b.x + b.y + b.z + b.w;
  }
#pragma unroll
  for (int k = 0; k < kPasses; ++k) q[base + threadIdx.x + 256 * k] = __float_as_uint(keep[k]);
}

}  // namespace
}  // namespace fp8z1

using namespace fp8z1;

extern "C" int fp8z1_probe_copy(const void* src, void* dst, int64_t bytes, int64_t spread, void* stream) {
  if (!src || !dst || bytes < 0 || bytes % 4096 || reinterpret_cast<uintptr_t>(src) % 16 ||
      reinterpret_cast<uintptr_t>(dst) % 16)
    return set_error(FP8Z1_EINVAL, "probe_copy: bytes must be a multiple of 4096, buffers 16-byte aligned");
  const int64_t blocks = bytes / 4096;
  if (spread < 1 || blocks % spread)
    return set_error(FP8Z1_EINVAL, "probe_copy: spread must be >= 1 and divide bytes / 4096");
  if (blocks == 0) return FP8Z1_OK;
  if (blocks > 0x7fffffff) return set_error(FP8Z1_EINVAL, "probe_copy: too large");
  hipLaunchKernelGGL(probe_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), static_cast<uint4*>(dst),
                     blocks, spread);
  return check_hip(hipGetLastError(), "probe_copy: launch");
}

extern "C" int fp8z1_probe_update_pattern(const float* g, float* p, float* m, float* v, uint8_t* codes, int64_t nslots,
                                          int32_t parts, void* stream) {
  if (!g || !p || !m || !v || !codes || nslots < 0)
    return set_error(FP8Z1_EINVAL, "probe_update_pattern: NULL argument");
  if (parts != 1 && parts != 2 && parts != 4 && parts != 8)
    return set_error(FP8Z1_EINVAL, "probe_update_pattern: parts must be 1, 2, 4 or 8");
  const void* ptrs[5] = {g, p, m, v, codes};
  for (const void* q : ptrs)
    if (reinterpret_cast<uintptr_t>(q) % 16)
      return set_error(FP8Z1_EINVAL, "probe_update_pattern: buffers must be 16-byte aligned");
  if (nslots == 0) return FP8Z1_OK;
  if (nslots * parts > 0x7fffffff) return set_error(FP8Z1_EINVAL, "probe_update_pattern: too large");
  const dim3 grid(static_cast<unsigned>(nslots * parts));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float4* g4 = reinterpret_cast<const float4*>(g);
  float4 *p4 = reinterpret_cast<float4*>(p), *m4 = reinterpret_cast<float4*>(m), *v4 = reinterpret_cast<float4*>(v);
  uint32_t* q = reinterpret_cast<uint32_t*>(codes);
  if (parts == 1) hipLaunchKernelGGL(probe_update_kernel<1>, grid, dim3(256), 0, s, g4, p4, m4, v4, q);
  if (parts == 2) hipLaunchKernelGGL(probe_update_kernel<2>, grid, dim3(256), 0, s, g4, p4, m4, v4, q);
  if (parts == 4) hipLaunchKernelGGL(probe_update_kernel<4>, grid, dim3(256), 0, s, g4, p4, m4, v4, q);
  if (parts == 8) hipLaunchKernelGGL(probe_update_kernel<8>, grid, dim3(256), 0, s, g4, p4, m4, v4, q);
  return check_hip(hipGetLastError(), "probe_update_pattern: launch");
}
