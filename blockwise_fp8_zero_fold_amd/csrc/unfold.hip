// Unfold: the shard's 128x128-block-contiguous buffer -> row-major [E, R, C]
// params, and per-slot scales -> [E, Rb, Cb] ("面向 Blockwise FP8 量化的 ZeRO
// 优化器设计", section "参数布局变换" and the parameter/scale unfold of section
// "总结").  Only real positions are written: padding is dropped.
//
// As in the fold, whole row segments move (no element transpose).  FP8
// codes: four workgroups per slot, each a quarter of the block; a 128-byte row
// segment is 8 lanes of 16-byte stores (streaming when the row is 16-byte
// aligned, plain unaligned stores otherwise); in a partial block the chunk
// across the last real column is written byte by byte, so no byte of a
// neighbouring block's row is ever written.  float32 (used for round-trip
// checks): one workgroup per slot, the same with 4-element chunks.
#include <hip/hip_runtime.h>

#include "device_util.h"

namespace fp8z1 {
namespace {

constexpr int kUnfThreads = 256;

// FP8 codes: a workgroup moves a quarter of a block (32 rows x 128 bytes,
// 4 KB), so that the workgroups in flight cover a compact range of memory.
constexpr int kUnfRows = 32;
constexpr int kUnfParts = kB / kUnfRows;

__global__ __launch_bounds__(kUnfThreads) void unfold_e4m3_kernel(const SlotPlan* __restrict__ plan,
                                                                  const uint8_t* __restrict__ folded,
                                                                  void* const* __restrict__ dsts,
                                                                  const float* __restrict__ scales,
                                                                  float* const* __restrict__ dscales) {
  const int64_t s = blockIdx.x / kUnfParts;
  const int part = blockIdx.x % kUnfParts;
  const SlotPlan P = plan[s];
  if (P.param < 0) return;
  const int t = threadIdx.x;
  if (dscales && part == 0 && t == 0) dscales[P.param][P.soff] = scales[s];
  const int vr = P.vr, vc = P.vc;
  const int r0 = part * kUnfRows;
  const int i = t >> 3, j = 16 * (t & 7);  // 8 lanes per 128-byte row, one 16-byte chunk each
  if (r0 + i >= vr || j >= vc) return;
  const int64_t ld = P.ld;
  uint8_t* row = static_cast<uint8_t*>(dsts[P.param]) + P.off + (r0 + i) * ld;
  const uint4 x = ld_stream(reinterpret_cast<const uint4*>(folded + s * kBlockElems + (r0 + i) * kB + j));
  if (j + 16 <= vc) {
    // a chunk inside the row: one 16-byte store, at any alignment of the row
    if ((reinterpret_cast<uintptr_t>(row + j) & 15u) == 0)
      st_stream(reinterpret_cast<uint4*>(row + j), x);
    else
      st_a1(row + j, x);
  } else {
    // the chunk across the last real column: its real bytes one by one, so no
    // byte of the neighbouring block's row is written
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    for (int b = 0; b < vc - j; ++b) row[j + b] = static_cast<uint8_t>(w[b >> 2] >> (8 * (b & 3)));
  }
}

__global__ __launch_bounds__(kUnfThreads) void unfold_f32_kernel(const SlotPlan* __restrict__ plan,
                                                                 const float* __restrict__ folded,
                                                                 void* const* __restrict__ dsts,
                                                                 const float* __restrict__ scales,
                                                                 float* const* __restrict__ dscales) {
  const int64_t s = blockIdx.x;
  const SlotPlan P = plan[s];
  if (P.param < 0) return;
  const int t = threadIdx.x;
  if (dscales && t == 0) dscales[P.param][P.soff] = scales[s];
  float* dst = static_cast<float*>(dsts[P.param]) + P.off;
  const float* src = folded + s * kBlockElems;
  const int64_t ld = P.ld;
  const int vr = P.vr, vc = P.vc;
  const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll 4
  for (int q = 0; q < kChunks / kUnfThreads; ++q) {
    const int c = t + kUnfThreads * q;
    const int i = c / kChunksPerRow, j = 4 * (c % kChunksPerRow);
    if (i >= vr || j >= vc) continue;
    float* d = dst + i * ld + j;
    const float4 x = s4[c];
    if (j + 4 <= vc) {
      st_a4(d, x);
    } else {
      const float e[4] = {x.x, x.y, x.z, x.w};
      for (int b = 0; b < vc - j; ++b) d[b] = e[b];
    }
  }
}

}  // namespace
}  // namespace fp8z1

using namespace fp8z1;

extern "C" int fp8z1_unfold(const fp8z1_table* ct, const void* folded, int32_t dtype, const float* scales,
                            void* const* dst, float* const* dst_scales, void* stream) {
  fp8z1_table* t = const_cast<fp8z1_table*>(ct);
  if (!t || !folded || !dst) return set_error(FP8Z1_EINVAL, "unfold: NULL table, folded buffer or dst list");
  if (dtype != FP8Z1_E4M3 && dtype != FP8Z1_F32)
    return set_error(FP8Z1_EINVAL, "unfold: dtype must be FP8Z1_E4M3 or FP8Z1_F32");
  if (reinterpret_cast<uintptr_t>(folded) % 16) return set_error(FP8Z1_EINVAL, "unfold: folded must be 16-byte aligned");
  const bool with_scales = scales && dst_scales;
  const size_t el = dtype == FP8Z1_F32 ? 4 : 1;
  for (const fp8z1_block& e : t->entries) {
    if (e.param < 0) continue;
    const void* p = dst[e.param];
    if (!p) return set_error(FP8Z1_EINVAL, "unfold: dst pointer of param " + std::to_string(e.param) + " is NULL");
    if (reinterpret_cast<uintptr_t>(p) % el)
      return set_error(FP8Z1_EINVAL, "unfold: dst pointer of param " + std::to_string(e.param) + " is misaligned");
    if (with_scales && (!dst_scales[e.param] || reinterpret_cast<uintptr_t>(dst_scales[e.param]) % 4))
      return set_error(FP8Z1_EINVAL, "unfold: scale pointer of param " + std::to_string(e.param) + " is NULL or misaligned");
  }
  std::lock_guard<std::mutex> lock(t->mu);
  int rc = ensure_device(t, stream);
  if (rc) return rc;
  void** ddst = nullptr;
  rc = device_ptr_list(t, kRoleUnfoldDst, const_cast<const void* const*>(dst), &ddst, stream);
  if (rc) return rc;
  void** dsc = nullptr;
  if (with_scales) {
    rc = device_ptr_list(t, kRoleUnfoldScale, reinterpret_cast<const void* const*>(dst_scales), &dsc, stream);
    if (rc) return rc;
  }
  const int64_t n = t->info.shard_slots;
  if (n == 0) return FP8Z1_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == FP8Z1_E4M3)
    hipLaunchKernelGGL(unfold_e4m3_kernel, dim3(n * kUnfParts), dim3(kUnfThreads), 0, s, t->d_plan,
                       static_cast<const uint8_t*>(folded), ddst, with_scales ? scales : nullptr,
                       reinterpret_cast<float* const*>(dsc));
  else
    hipLaunchKernelGGL(unfold_f32_kernel, dim3(n), dim3(kUnfThreads), 0, s, t->d_plan,
                       static_cast<const float*>(folded), ddst, with_scales ? scales : nullptr,
                       reinterpret_cast<float* const*>(dsc));
  return check_hip(hipGetLastError(), "unfold: launch");
}
