// Dequantization of row-major FP8 weights: each code times the scale of its
// 128x128 block ("面向 Blockwise FP8 量化的 ZeRO 优化器设计", section
// "Blockwise 量化": one scale per block; the scale is the dequantization
// multiplier).  Used to read back what the all-gathered FP8 weights stand
// for, e.g. to check them against the FP32 master.
#include <hip/hip_runtime.h>

#include "device_util.h"

namespace fp8z1 {
namespace {

// OCP E4M3 code -> float32, exact: exponent field 1..15 is (1 + m/8) * 2^(e-7),
// field 0 is m * 2^-9, S.1111.111 is NaN.
__device__ __forceinline__ float e4m3_decode(uint32_t code) {
  const uint32_t sign = (code & 0x80u) << 24;
  const uint32_t e = (code >> 3) & 0xfu, m = code & 0x7u;
  float mag;
  if ((code & 0x7fu) == 0x7fu)
    mag = __uint_as_float(0x7fc00000u);
  else if (e == 0)
    mag = static_cast<float>(m) * 0.001953125f;  // m * 2^-9, exact
  else
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return __uint_as_float(__float_as_uint(mag) | sign);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);  // quiet NaN
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// one workgroup per row of one expert; lanes walk the row's columns
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
  if (out_dtype == FP8Z1_BF16)
    hipLaunchKernelGGL(dequant_kernel<true>, dim3(static_cast<unsigned>(rows)), dim3(256), 0, s, codes, scales, R, C,
                       out);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, dim3(static_cast<unsigned>(rows)), dim3(256), 0, s, codes, scales, R, C,
                       out);
  return check_hip(hipGetLastError(), "dequantize: launch");
}
