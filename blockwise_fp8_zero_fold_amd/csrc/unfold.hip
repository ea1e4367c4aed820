// Unfold: the shard's 128x128-block-contiguous buffer -> row-major [E, R, C]
// params, and per-slot scales -> [E, Rb, Cb] ("面向 Blockwise FP8 量化的 ZeRO
// 优化器设计", section "参数布局变换" and the parameter/scale unfold of section
// "总结").  Only real positions are written: padding is dropped.
//
// As in the fold, whole row segments move (no element transpose).  FP8
// codes: when every block row segment starts on a 128-byte line, by blocks;
// otherwise by destination rows: the blocks of one block row that sit side
// by side in the shard fill one contiguous span of each param row, which a
// workgroup writes with aligned 16-byte stores at any alignment of the rows
// (a row segment of one block is 128 bytes, so blockwise stores into such
// rows would leave most 128-byte lines shared by two workgroups, each
// writing part of the line).
// float32 (used for round-trip checks): one workgroup per slot, 4-element
// chunks at any alignment.
#include <hip/hip_runtime.h>

#include "device_util.h"

namespace fp8z1 {
namespace {

constexpr int kUnfThreads = 256;
constexpr int kUnfBatch = 4;

// Bytes [sh, sh + 16) of the 32 bytes lo || hi (lo first), sh in [0, 16).
__device__ __forceinline__ uint4 funnel16(const uint4 lo, const uint4 hi, int sh) {
  const uint32_t d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  const int q = sh >> 2, r = 8 * (sh & 3);
  uint32_t e[5];
#pragma unroll
  for (int n = 0; n < 5; ++n) e[n] = q == 0 ? d[n] : q == 1 ? d[n + 1] : q == 2 ? d[n + 2] : d[n + 3];
  // e[n] >> r | e[n + 1] << (32 - r), with r = 0 giving e[n]
  uint32_t o[4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
    o[n] = static_cast<uint32_t>(((static_cast<uint64_t>(e[n + 1]) << 32) | e[n]) >> r);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// FP8 codes, by rows: one workgroup per work item (whole rows of a run of
// side-by-side blocks, see RowItem).  Row r of the run is `len` contiguous
// bytes of the param; the workgroup writes it as the 16-byte-aligned chunks
// that cover it.  Lane chunk k of a row starting m bytes past a 16-byte
// boundary takes run bytes [16k - m, 16k - m + 16): the folded row segments
// of the run's blocks are 128-byte runs, so those bytes are the tail of run
// chunk k - 1 and the head of run chunk k, joined with a funnel shift.  A
// lane loads only chunk k and takes chunk k - 1 from the previous lane (a
// shuffle; the first lane of a wave and the first chunk of a row load it).
// Chunks wholly inside the row are one aligned (streaming) store; the first
// and last chunk of a row are written byte by byte, only the row's own bytes,
// so no byte outside the run is ever written.  A lane takes kUnfBatch chunks
// per round and issues all their loads before any shuffle or store (an item
// of ~16 KB is one round): on the ragged shard 294 us against 325 us with one
// chunk per round, where a lane that needed chunk k - 1 itself loaded it only
// after the shuffle.
__global__ __launch_bounds__(kUnfThreads) void unfold_rows_e4m3_kernel(const RowItem* __restrict__ items,
                                                                       const uint8_t* __restrict__ folded,
                                                                       void* const* __restrict__ dsts,
                                                                       const float* __restrict__ scales,
                                                                       float* const* __restrict__ dscales) {
  const RowItem it = items[blockIdx.x];
  const int t = threadIdx.x;
  if (dscales && it.row0 == 0)
    for (int b = t; b < it.nblk; b += kUnfThreads) dscales[it.param][it.soff + b] = scales[it.slot + b];
  uint8_t* base = static_cast<uint8_t*>(dsts[it.param]) + it.off;
  const uint8_t* src = folded + static_cast<int64_t>(it.slot) * kBlockElems + static_cast<int64_t>(it.row0) * kB;
  const int len = it.len;
  const int nq = 8 * it.nblk;        // 16-byte chunks of the run's folded row segments
  const int kc = (len + 30) / 16;    // chunks a row of len bytes can touch at any alignment
  const int total = it.rows * kc;
  // kUnfBatch chunks per lane per round, every load of the round (the chunk, and
  // chunk k - 1 where no lane has it) issued before any shuffle or store
  constexpr int U = kUnfBatch;
  for (int c0 = t; c0 < total; c0 += U * kUnfThreads) {
    uint4 hi[U], lo[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kUnfThreads;
      const int r = c / kc, k = c - r * kc;
      const uint8_t* srow = src + r * kB;
      const int m = static_cast<int>(reinterpret_cast<uintptr_t>(base + static_cast<int64_t>(r) * it.ld) & 15u);
      const bool act = c < total && 16 * k - m < len;
      // run chunk q of row r: block q / 8 of the run, bytes 16 (q % 8) of its row segment
      hi[u] = act && k < nq ? ld_stream(reinterpret_cast<const uint4*>(srow + static_cast<int64_t>(k >> 3) * kBlockElems +
                                                                    16 * (k & 7)))
                            : make_uint4(0u, 0u, 0u, 0u);
      const bool own_lo = m && act && k > 0 && (threadIdx.x & 63) == 0;  // no previous lane to take it from
      lo[u] = own_lo ? ld_stream(reinterpret_cast<const uint4*>(srow + static_cast<int64_t>((k - 1) >> 3) * kBlockElems +
                                                             16 * ((k - 1) & 7)))
                     : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kUnfThreads;
      uint4 prev;  // chunk k - 1 of the row is the previous lane's chunk (all lanes take part)
      prev.x = __shfl_up(hi[u].x, 1);
      prev.y = __shfl_up(hi[u].y, 1);
      prev.z = __shfl_up(hi[u].z, 1);
      prev.w = __shfl_up(hi[u].w, 1);
      const int r = c / kc, k = c - r * kc;
      uint8_t* row = base + static_cast<int64_t>(r) * it.ld;
      const int m = static_cast<int>(reinterpret_cast<uintptr_t>(row) & 15u);
      const int x0 = 16 * k - m;  // run byte of the chunk's first byte (> -16)
      if (c >= total || x0 >= len) continue;
      const bool from_lane = (threadIdx.x & 63) != 0 && k > 0;
      const uint4 x = m ? funnel16(from_lane ? prev : lo[u], hi[u], 16 - m) : hi[u];
      uint8_t* d = row + x0;  // 16-byte aligned
      if (x0 >= 0 && x0 + 16 <= len) {
        st_global_stream(d, x);
      } else {
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        const int b0 = x0 < 0 ? -x0 : 0, b1 = len - x0 < 16 ? len - x0 : 16;
        for (int b = b0; b < b1; ++b) d[b] = static_cast<uint8_t>(w[b >> 2] >> (8 * (b & 3)));
      }
    }
  }
}

// FP8 codes, by blocks (used when every row segment of the call starts on a
// 128-byte line, so no line is shared by two workgroups): a workgroup of one
// wave moves a sixteenth of a block (8 rows x 128 bytes, 1 KB), so that the
// workgroups in flight cover a compact range of memory; 8 lanes per row, 16
// bytes each.  (4 KB per workgroup of 256 lanes took 2-3 % longer, 8 and
// 16 KB with two or four rows per lane 12-17 %.)
constexpr int kUnfRows = 8;
constexpr int kUnfParts = kB / kUnfRows;
constexpr int kUnfBlkThreads = 8 * kUnfRows;

__global__ __launch_bounds__(kUnfBlkThreads) void unfold_blocks_e4m3_kernel(const SlotPlan* __restrict__ plan,
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
      st_global_stream(row + j, x);
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
  if (t->info.shard_slots * kUnfParts > 0x7fffffffLL) return set_error(FP8Z1_ESHAPE, "unfold: too many slots");
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
  const bool f32 = dtype == FP8Z1_F32;
  rc = device_ptr_list(t, f32 ? kRoleUnfoldDstF32 : kRoleUnfoldDst, const_cast<const void* const*>(dst), &ddst, stream);
  if (rc) return rc;
  void** dsc = nullptr;
  if (with_scales) {
    rc = device_ptr_list(t, f32 ? kRoleUnfoldScaleF32 : kRoleUnfoldScale,
                         reinterpret_cast<const void* const*>(dst_scales), &dsc, stream);
    if (rc) return rc;
  }
  const int64_t n = t->info.shard_slots;
  if (n == 0) return FP8Z1_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == FP8Z1_E4M3) {
    // by blocks when every held param's rows and block row segments start on
    // a 128-byte line (C a multiple of 128, destination 128-byte aligned),
    // else by rows
    bool lines = true;
    for (size_t p = 0; p < t->shapes.size() && lines; ++p)
      if (t->held[p]) lines = t->shapes[p].C % 128 == 0 && reinterpret_cast<uintptr_t>(dst[p]) % 128 == 0;
    if (lines)
      hipLaunchKernelGGL(unfold_blocks_e4m3_kernel, dim3(static_cast<unsigned>(n * kUnfParts)), dim3(kUnfBlkThreads), 0, s,
                         t->d_plan,
                         static_cast<const uint8_t*>(folded), ddst, with_scales ? scales : nullptr,
                         reinterpret_cast<float* const*>(dsc));
    else if (t->n_rows > 0)
      hipLaunchKernelGGL(unfold_rows_e4m3_kernel, dim3(static_cast<unsigned>(t->n_rows)), dim3(kUnfThreads), 0, s,
                         t->d_rows, static_cast<const uint8_t*>(folded), ddst, with_scales ? scales : nullptr,
                         reinterpret_cast<float* const*>(dsc));
  } else
    hipLaunchKernelGGL(unfold_f32_kernel, dim3(static_cast<unsigned>(n)), dim3(kUnfThreads), 0, s, t->d_plan,
                       static_cast<const float*>(folded), ddst, with_scales ? scales : nullptr,
                       reinterpret_cast<float* const*>(dsc));
  rc = check_hip(hipGetLastError(), "unfold: launch");
  return rc ? rc : note_use(t, stream);
}
