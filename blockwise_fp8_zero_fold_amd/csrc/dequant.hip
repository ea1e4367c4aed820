// Dequantization of row-major FP8 weights: each code times the scale of its
// 128x128 block ("面向 Blockwise FP8 量化的 ZeRO 优化器设计", section
// "Blockwise 量化": one scale per block; the scale is the dequantization
// multiplier).  Used to read back what the all-gathered FP8 weights stand
// for, e.g. to check them against the FP32 master.
#include <hip/hip_runtime.h>

#include "device_util.h"

namespace fp8z1 {
namespace {

// The hardware's conversions: OCP E4M3 code -> float32 (exact, S.1111.111 is
// NaN), float32 -> BF16 (round to nearest even, NaN kept).
__device__ __forceinline__ float e4m3_decode(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(code), 0);
}

__device__ __forceinline__ uint16_t to_bf16(float x) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x)); }

// any alignment: one workgroup per row of one expert; lanes walk the row's columns
template <bool BF16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes, const float* __restrict__ scales,
                                                      int64_t R, int64_t C, void* __restrict__ out) {
  const int64_t row = blockIdx.x;  // e * R + r
  const int64_t e = row / R, r = row % R;
  const int64_t cb = (C + kB - 1) / kB;
  const float* srow = scales + (e * ((R + kB - 1) / kB) + r / kB) * cb;
  const uint8_t* crow = codes + row * C;
  for (int64_t c = threadIdx.x; c < C; c += 256) {
    const float y = e4m3_decode(crow[c]) * srow[c / kB];
    if (BF16)
      static_cast<uint16_t*>(out)[row * C + c] = to_bf16(y);
    else
      static_cast<float*>(out)[row * C + c] = y;
  }
}

// Rows whose codes and outputs are 16-byte aligned (C a multiple of 16, aligned
// buffers): a workgroup takes kDqRows rows.  A lane turns a chunk of codes
// into one 16-byte store (FP32: 4 codes, BF16: 8), so each store instruction
// of a wave covers 1 KB of contiguous output, and loads 4 chunks before
// decoding (BF16 with 16 codes and two 16-byte stores per lane ran 7 % slower,
// FP32 with 8 chunks loaded first 3 % slower).  The codes of a chunk lie in
// one 128-column block, so they share one scale.  The codes are widened by the
// hardware's FP8 conversion and the BF16 results rounded by its BF16
// conversion; the index arithmetic is 32-bit, one division per chunk.
constexpr int kDqRows = 4;

// codes 0..3 of the word w, widened exactly, times sc (one rounding each)
__device__ __forceinline__ float4 widen4(uint32_t w, float sc) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  return make_float4(lo[0] * sc, lo[1] * sc, hi[0] * sc, hi[1] * sc);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return static_cast<uint32_t>(to_bf16(a)) | (static_cast<uint32_t>(to_bf16(b)) << 16);
}

template <bool BF16>
__global__ __launch_bounds__(256) void dequant_vec_kernel(const uint8_t* __restrict__ codes,
                                                          const float* __restrict__ scales, int32_t rows, int32_t R,
                                                          int32_t C, void* __restrict__ out) {
  constexpr int kPer = BF16 ? 8 : 4;  // codes per lane and chunk: one 16-byte store
  constexpr int kUnroll = 4;          // chunks a lane loads before it decodes
  const int32_t nchunk = C / kPer;
  const int32_t row0 = static_cast<int32_t>(blockIdx.x) * kDqRows;
  const int32_t nrows = min(kDqRows, rows - row0);
  const int32_t cb = (C + kB - 1) / kB, rb = (R + kB - 1) / kB;
  // scale row of each of the workgroup's rows
  int64_t soff[kDqRows];
#pragma unroll
  for (int j = 0; j < kDqRows; ++j) {
    const int32_t row = row0 + min(j, nrows - 1);
    const int32_t e = row / R, r = row - e * R;
    soff[j] = (static_cast<int64_t>(e) * rb + r / kB) * cb;
  }
  const int32_t total = nrows * nchunk;
  for (int32_t i0 = threadIdx.x; i0 < total; i0 += 256 * kUnroll) {
    uint4 q[kUnroll];
    int32_t jr[kUnroll], kc[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int32_t i = i0 + 256 * u;
      jr[u] = i / nchunk;
      kc[u] = i - jr[u] * nchunk;
      q[u] = make_uint4(0u, 0u, 0u, 0u);
      if (i < total) {
        const uint8_t* src = codes + static_cast<int64_t>(row0 + jr[u]) * C + kPer * kc[u];
        if (BF16) {
          const uint2 h = *reinterpret_cast<const uint2*>(src);
          q[u].x = h.x;
          q[u].y = h.y;
        } else {
          q[u].x = *reinterpret_cast<const uint32_t*>(src);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int32_t i = i0 + 256 * u;
      if (i >= total) break;
      int64_t so = soff[0];
#pragma unroll
      for (int j = 1; j < kDqRows; ++j)
        if (jr[u] == j) so = soff[j];
      const float sc = scales[so + (kPer * kc[u]) / kB];
      const int64_t o = static_cast<int64_t>(row0 + jr[u]) * C + kPer * kc[u];
      if (BF16) {
        const float4 a = widen4(q[u].x, sc), b = widen4(q[u].y, sc);
        st_stream(reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + o),
                  make_uint4(pack_bf16(a.x, a.y), pack_bf16(a.z, a.w), pack_bf16(b.x, b.y), pack_bf16(b.z, b.w)));
      } else {
        st_stream(reinterpret_cast<float4*>(static_cast<float*>(out) + o), widen4(q[u].x, sc));
      }
    }
  }
}

}  // namespace
}  // namespace fp8z1

using namespace fp8z1;

extern "C" int fp8z1_dequantize(const uint8_t* codes, const float* scales, int64_t E, int64_t R, int64_t C,
                                int32_t out_dtype, void* out, void* stream) {
  if (!codes || !scales || !out) return set_error(FP8Z1_EINVAL, "dequantize: NULL argument");
  if (E < 1 || R < 1 || C < 1) return set_error(FP8Z1_ESHAPE, "dequantize: E, R, C must be >= 1");
  if (out_dtype != FP8Z1_F32 && out_dtype != FP8Z1_BF16)
    return set_error(FP8Z1_EINVAL, "dequantize: out_dtype must be FP8Z1_F32 or FP8Z1_BF16");
  if (reinterpret_cast<uintptr_t>(scales) % 4 || reinterpret_cast<uintptr_t>(out) % (out_dtype == FP8Z1_F32 ? 4 : 2))
    return set_error(FP8Z1_EINVAL, "dequantize: misaligned scales or output");
  const int64_t rows = E * R;
  if (rows > 0x7fffffff) return set_error(FP8Z1_ESHAPE, "dequantize: more than 2^31 rows");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (C % 16 == 0 && C <= 0x7fffffff && reinterpret_cast<uintptr_t>(codes) % 16 == 0 &&
      reinterpret_cast<uintptr_t>(out) % 16 == 0) {
    const unsigned grid = static_cast<unsigned>((rows + kDqRows - 1) / kDqRows);
    const int32_t rows32 = static_cast<int32_t>(rows), R32 = static_cast<int32_t>(R), C32 = static_cast<int32_t>(C);
    if (out_dtype == FP8Z1_BF16)
      hipLaunchKernelGGL(dequant_vec_kernel<true>, dim3(grid), dim3(256), 0, s, codes, scales, rows32, R32, C32, out);
    else
      hipLaunchKernelGGL(dequant_vec_kernel<false>, dim3(grid), dim3(256), 0, s, codes, scales, rows32, R32, C32, out);
    return check_hip(hipGetLastError(), "dequantize: launch");
  }
  if (out_dtype == FP8Z1_BF16)
    hipLaunchKernelGGL(dequant_kernel<true>, dim3(static_cast<unsigned>(rows)), dim3(256), 0, s, codes, scales, R, C,
                       out);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, dim3(static_cast<unsigned>(rows)), dim3(256), 0, s, codes, scales, R, C,
                       out);
  return check_hip(hipGetLastError(), "dequantize: launch");
}
