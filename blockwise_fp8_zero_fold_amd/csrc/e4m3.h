// Device FP32 -> FP8 E4M3 encoder (OCP 8-bit floating point "E4M3": exponent
// bias 7, 3 mantissa bits, largest finite 448, NaN = S.1111.111, no infinity).
//
// E4M3 is the FP8 weight format of "FP8训练技术与万亿参数模型优化实践" section
// 1.1 and of the blockwise weights of "面向 Blockwise FP8 量化的 ZeRO 优化器设计"
// section "Blockwise 量化".  Rounding: to nearest, ties to even; magnitudes of
// 448 or more (and infinities) saturate to 448; NaN keeps its sign; the sign
// of zero is kept.
//
// Integer form: for |x| >= 2^-6 (E4M3 normals) the float32 exponent/mantissa
// field is rounded to 3 mantissa bits with the usual add-half-minus-one-plus-
// lsb trick, and the exponent is re-biased from 127 to 7 (a shift of 120
// binades, 120 << 3 in the code).  Below 2^-6 the value is a multiple of 2^-9:
// |x| * 512 is exact in float32 and rint() rounds it to the integer code
// (8 = 2^-6 comes out as the smallest normal code, which is right).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8z1 {

__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a > 0x7f800000u) {
    code = 0x7fu;  // NaN
  } else if (a >= 0x43e00000u) {
    code = 0x7eu;  // >= 448 or inf: saturate
  } else if (a >= 0x3c800000u) {
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  } else {
    code = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.0f));
  }
  return sign | code;
}

}  // namespace fp8z1
