// Unfold: the shard's 128x128-block-contiguous buffer -> row-major [E, R, C]
// params, and per-slot scales -> [E, Rb, Cb] ("面向 Blockwise FP8 量化的 ZeRO
// 优化器设计", section "参数布局变换" and the parameter/scale unfold of section
// "总结").  Only real positions are written: padding is dropped.
//
// As in the fold, whole row segments move (no element transpose).  One
// workgroup per slot.  FP8 codes: a 128-byte row segment is 8 lanes of
// 16-byte stores when the destination rows are 16-byte aligned and the
// block has all 128 columns; otherwise single-byte stores, which never touch
// a byte that belongs to a neighbouring block.  float32 (used for round-trip
// checks): the same with 16-byte / 4-byte accesses.
#include <hip/hip_runtime.h>

#include "device_util.h"

namespace fp8z1 {
namespace {

constexpr int kUnfThreads = 256;

__global__ __launch_bounds__(kUnfThreads) void unfold_e4m3_kernel(const SlotPlan* __restrict__ plan,
                                                                  const uint8_t* __restrict__ folded,
                                                                  void* const* __restrict__ dsts,
                                                                  const float* __restrict__ scales,
                                                                  float* const* __restrict__ dscales) {
  const int64_t s = blockIdx.x;
  const SlotPlan P = plan[s];
  if (P.param < 0) return;
  const int t = threadIdx.x;
  if (dscales && t == 0) dscales[P.param][P.soff] = scales[s];
  uint8_t* dst = static_cast<uint8_t*>(dsts[P.param]) + P.off;
  const uint8_t* src = folded + s * kBlockElems;
  const int64_t ld = P.ld;
  const int vr = P.vr, vc = P.vc;
  if (vc == kB && (ld % 16) == 0 && (reinterpret_cast<uintptr_t>(dst) % 16) == 0) {
    // 8 lanes per 128-byte row, 32 rows per pass
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    uint4 x[kB / 32];
#pragma unroll
    for (int q = 0; q < kB / 32; ++q) {
      const int i = (t >> 3) + 32 * q;
      if (i < vr) x[q] = s4[i * 8 + (t & 7)];
    }
#pragma unroll
    for (int q = 0; q < kB / 32; ++q) {
      const int i = (t >> 3) + 32 * q;
      if (i < vr) *reinterpret_cast<uint4*>(dst + i * ld + 16 * (t & 7)) = x[q];
    }
  } else {
    for (int idx = t; idx < kBlockElems; idx += kUnfThreads) {
      const int i = idx >> 7, j = idx & 127;
      if (i < vr && j < vc) dst[i * ld + j] = src[idx];
    }
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
  if (vc == kB && (ld % 4) == 0 && (reinterpret_cast<uintptr_t>(dst) % 16) == 0) {
    const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll 4
    for (int q = 0; q < kChunks / kUnfThreads; ++q) {
      const int c = t + kUnfThreads * q;
      const int i = c / kChunksPerRow;
      if (i < vr) *reinterpret_cast<float4*>(dst + i * ld + 4 * (c % kChunksPerRow)) = s4[c];
    }
  } else {
    for (int idx = t; idx < kBlockElems; idx += kUnfThreads) {
      const int i = idx >> 7, j = idx & 127;
      if (i < vr && j < vc) dst[i * ld + j] = src[idx];
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
  int rc = ensure_device(t);
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
    hipLaunchKernelGGL(unfold_e4m3_kernel, dim3(n), dim3(kUnfThreads), 0, s, t->d_plan,
                       static_cast<const uint8_t*>(folded), ddst, with_scales ? scales : nullptr,
                       reinterpret_cast<float* const*>(dsc));
  else
    hipLaunchKernelGGL(unfold_f32_kernel, dim3(n), dim3(kUnfThreads), 0, s, t->d_plan,
                       static_cast<const float*>(folded), ddst, with_scales ? scales : nullptr,
                       reinterpret_cast<float* const*>(dsc));
  return check_hip(hipGetLastError(), "unfold: launch");
}
