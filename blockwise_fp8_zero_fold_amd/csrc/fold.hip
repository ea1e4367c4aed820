// Fold: row-major [E, R, C] params -> the shard's 128x128-block-contiguous
// float32 buffer ("面向 Blockwise FP8 量化的 ZeRO 优化器设计", section
// "参数布局变换"; padding of section "块粒度切分").
//
// Inside a block the element order stays row-major: the fold's permute
// swaps the block-column index with the row-within-block index, so each
// 128-element row segment of the source moves whole to a contiguous 512-byte
// destination.  The kernel is therefore a segment gather, not a transpose:
// four workgroups per slot (32 rows each; XCD x takes a contiguous range of
// them), 32 lanes per row segment, 16-byte loads (at any element alignment of
// the source rows) and 16-byte stores; in a partial block only the chunk
// across the last real column is loaded element by element.  Every source
// byte is read once, every destination byte written once.  The same kernel
// without stores is the statistics pass over row-major grads.
#include <hip/hip_runtime.h>

#include "device_util.h"

namespace fp8z1 {
namespace {

constexpr int kFoldThreads = kSumThreads;  // also the statistics order

// workgroups of a fold launch: one per quarter slot, rounded up to whole XCD rounds
inline unsigned fold_grid(int64_t nslots) {
  return static_cast<unsigned>((nslots * kStatParts + kXcds - 1) / kXcds * kXcds);
}

template <typename T>
struct Src;
// load4: four consecutive elements from an element-aligned address (one vector
// load; see device_util.h), load1: one element
template <>
struct Src<float> {
  // whole chunk of a full block: one streaming 16-byte global load
  __device__ static float4 load4_full(const float* p) { return ld_global_stream_a4(p); }
  __device__ static float4 load4_full_cached(const float* p) { return ld_global_a4(p); }
  __device__ static float4 load4(const float* p) { return ld_a4(p); }
  __device__ static float load1(const float* p) { return *p; }
};
template <>
struct Src<uint16_t> {  // bfloat16 bits
  __device__ static float widen(uint32_t b) { return __uint_as_float(b << 16); }
  __device__ static float4 load4_full(const uint16_t* p) {
    const uint2 u = ld_global_stream_a2x8(p);
    return make_float4(widen(u.x & 0xffffu), widen(u.x >> 16), widen(u.y & 0xffffu), widen(u.y >> 16));
  }
  __device__ static float4 load4_full_cached(const uint16_t* p) { return load4(p); }
  __device__ static float4 load4(const uint16_t* p) {
    uint2 u;
    __builtin_memcpy(&u, p, 8);
    return make_float4(widen(u.x & 0xffffu), widen(u.x >> 16), widen(u.y & 0xffffu), widen(u.y >> 16));
  }
  __device__ static float load1(const uint16_t* p) { return widen(*p); }
};

// One workgroup per part (kPartRows rows) of a slot.  SUMSQ: also write the
// part's float64 sum of squares to part_sumsq[slot * kStatParts + part].
// WRITE = false: statistics only (the partials of a row-major grad that the
// update reads directly, without a folded copy).  KEEP: plain (cached) loads
// instead of streaming ones, so that grads which fit in the last-level cache
// are still there when the update reads them again.
template <typename T, bool SUMSQ, bool WRITE = true, bool KEEP = false>
__global__ __launch_bounds__(kFoldThreads) void fold_kernel(const SlotPlan* __restrict__ plan,
                                                            const void* const* __restrict__ srcs,
                                                            float* __restrict__ dst,
                                                            double* __restrict__ part_sumsq, int64_t nslots) {
  __shared__ double red[kFoldThreads / 64];
  // quarter slot of this workgroup: the dispatcher deals workgroups to the 8
  // XCDs in turn, so XCD x gets a contiguous range of quarter slots and
  // neighbouring blocks (which may share 128-byte lines of an unaligned
  // source row) go through one L2
  const int64_t per_xcd = static_cast<int64_t>(gridDim.x) / kXcds;  // the grid is a multiple of kXcds
  const int64_t q = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  const int64_t s = q / kStatParts;
  const int part = static_cast<int>(q % kStatParts);
  if (s >= nslots) return;  // whole workgroup
  const SlotPlan P = plan[s];
  float4* out = WRITE ? reinterpret_cast<float4*>(dst + s * kBlockElems) + part * kPartChunks : nullptr;
  const int t = threadIdx.x;
  double acc = 0.0;

  if (P.param < 0) {
    if (WRITE) {
#pragma unroll
      for (int k = 0; k < kPartPasses; ++k) out[t + kFoldThreads * k] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  } else {
    const T* src = static_cast<const T*>(srcs[P.param]) + P.off;
    const int64_t ld = P.ld;
    const int vr = P.vr, vc = P.vc;
    const int r0 = part * kPartRows;
    float4 x[kPartPasses];
    if (vr == kB && vc == kB) {
#pragma unroll
      for (int k = 0; k < kPartPasses; ++k) {
        const int c = t + kFoldThreads * k;
        const T* p = src + (r0 + c / kChunksPerRow) * ld + 4 * (c % kChunksPerRow);
        x[k] = KEEP ? Src<T>::load4_full_cached(p) : Src<T>::load4_full(p);
      }
    } else {
      // partial block: whole chunks inside the real region load as vectors, the
      // chunk across the last real column element by element, the rest is padding
#pragma unroll
      for (int k = 0; k < kPartPasses; ++k) {
        const int c = t + kFoldThreads * k;
        const int i = r0 + c / kChunksPerRow, j = 4 * (c % kChunksPerRow);
        const T* row = src + i * ld + j;
        if (i < vr && j + 4 <= vc) {
          x[k] = Src<T>::load4(row);
        } else {
          const bool rv = i < vr;
          x[k].x = (rv && j + 0 < vc) ? Src<T>::load1(row + 0) : 0.f;
          x[k].y = (rv && j + 1 < vc) ? Src<T>::load1(row + 1) : 0.f;
          x[k].z = (rv && j + 2 < vc) ? Src<T>::load1(row + 2) : 0.f;
          x[k].w = (rv && j + 3 < vc) ? Src<T>::load1(row + 3) : 0.f;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kPartPasses; ++k) {
      if (WRITE) out[t + kFoldThreads * k] = x[k];
      if (SUMSQ) {
        // padding positions hold +0 and add nothing
        acc += sq64(x[k].x);
        acc += sq64(x[k].y);
        acc += sq64(x[k].z);
        acc += sq64(x[k].w);
      }
    }
  }
  if (SUMSQ) {
    const double tot = block_sum<kFoldThreads>(acc, red);
    if (t == 0) part_sumsq[s * kStatParts + part] = tot;
  }
}

template <typename T>
hipError_t launch(const SlotPlan* plan, void** srcs, float* dst, double* sumsq, int64_t nslots,
                  hipStream_t stream) {
  if (nslots == 0) return hipSuccess;
  const dim3 grid(fold_grid(nslots));
  if (sumsq)
    hipLaunchKernelGGL((fold_kernel<T, true>), grid, dim3(kFoldThreads), 0, stream, plan, srcs, dst, sumsq, nslots);
  else
    hipLaunchKernelGGL((fold_kernel<T, false>), grid, dim3(kFoldThreads), 0, stream, plan, srcs, dst, sumsq,
                       nslots);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grad_sumsq(const SlotPlan* plan, void** grads, double* sumsq, int64_t nslots, int64_t valid_elems,
                             hipStream_t stream) {
  if (nslots == 0) return hipSuccess;
  // grads that fit in the last-level cache (256 MB on MI355X) stay there for the
  // update's second read; larger ones stream
  if (valid_elems * 4 <= kLastLevelCacheBytes)
    hipLaunchKernelGGL((fold_kernel<float, true, false, true>), dim3(fold_grid(nslots)), dim3(kFoldThreads), 0, stream,
                       plan, grads, nullptr, sumsq, nslots);
  else
    hipLaunchKernelGGL((fold_kernel<float, true, false, false>), dim3(fold_grid(nslots)), dim3(kFoldThreads), 0,
                       stream, plan, grads, nullptr, sumsq, nslots);
  return hipGetLastError();
}

}  // namespace fp8z1

using namespace fp8z1;

extern "C" int fp8z1_fold(const fp8z1_table* ct, const void* const* src, int32_t src_dtype, float* dst,
                          double* slot_sumsq, void* stream) {
  fp8z1_table* t = const_cast<fp8z1_table*>(ct);
  if (!t || !src || !(dst || slot_sumsq)) return set_error(FP8Z1_EINVAL, "fold: NULL table, src list or dst");
  if (src_dtype != FP8Z1_F32 && src_dtype != FP8Z1_BF16)
    return set_error(FP8Z1_EINVAL, "fold: src_dtype must be FP8Z1_F32 or FP8Z1_BF16");
  if (!dst && src_dtype != FP8Z1_F32)
    return set_error(FP8Z1_EINVAL, "fold: the statistics-only pass (dst NULL) takes FP8Z1_F32 grads");
  const size_t el = src_dtype == FP8Z1_F32 ? 4 : 2;
  // every param the shard holds needs a source pointer, element-aligned
  for (const fp8z1_block& e : t->entries) {
    if (e.param < 0) continue;
    const void* p = src[e.param];
    if (!p) return set_error(FP8Z1_EINVAL, "fold: src pointer of param " + std::to_string(e.param) + " is NULL");
    if (reinterpret_cast<uintptr_t>(p) % el)
      return set_error(FP8Z1_EINVAL, "fold: src pointer of param " + std::to_string(e.param) + " is misaligned");
  }
  if (reinterpret_cast<uintptr_t>(dst) % 16) return set_error(FP8Z1_EINVAL, "fold: dst must be 16-byte aligned");
  if (slot_sumsq && reinterpret_cast<uintptr_t>(slot_sumsq) % 8)
    return set_error(FP8Z1_EINVAL, "fold: slot_sumsq must be 8-byte aligned");
  if (t->info.shard_slots * kStatParts > 0x7fffffffLL) return set_error(FP8Z1_ESHAPE, "fold: too many slots");
  std::lock_guard<std::mutex> lock(t->mu);
  int rc = ensure_device(t, stream);
  if (rc) return rc;
  void** dsrc = nullptr;
  rc = device_ptr_list(t, kRoleFoldSrc, src, &dsrc, stream);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (!dst)
    e = launch_grad_sumsq(t->d_plan, dsrc, slot_sumsq, t->info.shard_slots, t->info.valid_elems, st);
  else if (src_dtype == FP8Z1_F32)
    e = launch<float>(t->d_plan, dsrc, dst, slot_sumsq, t->info.shard_slots, st);
  else
    e = launch<uint16_t>(t->d_plan, dsrc, dst, slot_sumsq, t->info.shard_slots, st);
  rc = check_hip(e, "fold: launch");
  return rc ? rc : note_use(t, stream);
}
