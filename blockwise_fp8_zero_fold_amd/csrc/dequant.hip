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
// buffers): a workgroup takes kDqRows rows.  FP32: a lane turns 4 codes into
// one 16-byte store, so each store instruction of a wave covers 1 KB of
// contiguous output, and loads 4 such chunks before decoding.  BF16: a lane
// turns 16 codes (one 16-byte load) into two 16-byte stores (measured faster
// for this output than 8 codes per lane).  The codes of a chunk lie in one
// 128-column block, so they share one scale.
constexpr int kDqRows = 4;

template <bool BF16>
__global__ __launch_bounds__(256) void dequant_vec_kernel(const uint8_t* __restrict__ codes,
                                                          const float* __restrict__ scales, int64_t rows, int64_t R,
                                                          int64_t C, void* __restrict__ out) {
  constexpr int kPer = BF16 ? 16 : 4;  // codes per lane and chunk (BF16: two 16-byte stores)
  constexpr int kUnroll = BF16 ? 1 : 4;  // chunks a lane loads before it decodes
  const int64_t nchunk = C / kPer;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kDqRows;
  const int64_t cb = (C + kB - 1) / kB;
  const int64_t total = min(static_cast<int64_t>(kDqRows), rows - row0) * nchunk;
  for (int64_t i0 = threadIdx.x; i0 < total; i0 += 256 * kUnroll) {
    uint4 q[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + 256 * u;
      q[u] = make_uint4(0u, 0u, 0u, 0u);
      if (i < total) {
        const uint8_t* src = codes + (row0 + i / nchunk) * C + kPer * (i % nchunk);
        if (BF16)
          q[u] = ld_stream(reinterpret_cast<const uint4*>(src));
        else
          q[u].x = *reinterpret_cast<const uint32_t*>(src);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + 256 * u;
      if (i >= total) break;
      const int64_t row = row0 + i / nchunk, k = i % nchunk;
      const int64_t e = row / R, r = row % R;
      const float sc = scales[(e * ((R + kB - 1) / kB) + r / kB) * cb + (kPer * k) / kB];
      if (BF16) {
        const uint32_t w[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
        uint32_t h[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const uint32_t lo = (w[b >> 1] >> (16 * (b & 1))) & 0xffu, hi = (w[b >> 1] >> (16 * (b & 1) + 8)) & 0xffu;
          h[b] = to_bf16(e4m3_decode(lo) * sc) | (static_cast<uint32_t>(to_bf16(e4m3_decode(hi) * sc)) << 16);
        }
        uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + row * C + kPer * k);
        st_stream(o, make_uint4(h[0], h[1], h[2], h[3]));
        st_stream(o + 1, make_uint4(h[4], h[5], h[6], h[7]));
      } else {
        const uint32_t x = q[u].x;
        st_stream(reinterpret_cast<float4*>(static_cast<float*>(out) + row * C + kPer * k),
                  make_float4(e4m3_decode(x & 0xffu) * sc, e4m3_decode((x >> 8) & 0xffu) * sc,
                              e4m3_decode((x >> 16) & 0xffu) * sc, e4m3_decode(x >> 24) * sc));
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
  if (C % 16 == 0 && reinterpret_cast<uintptr_t>(codes) % 16 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0) {
    const unsigned grid = static_cast<unsigned>((rows + kDqRows - 1) / kDqRows);
    if (out_dtype == FP8Z1_BF16)
      hipLaunchKernelGGL(dequant_vec_kernel<true>, dim3(grid), dim3(256), 0, s, codes, scales, rows, R, C, out);
    else
      hipLaunchKernelGGL(dequant_vec_kernel<false>, dim3(grid), dim3(256), 0, s, codes, scales, rows, R, C, out);
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
