// The optimizer step on one rank's folded shard, and its state.
//
// "面向 Blockwise FP8 量化的 ZeRO 优化器设计", section "总结": after the reduced
// grads are folded and sliced, the rank updates its FP32 master and then
// quantizes it into FP8 weights and one scale per 128x128 block.
// "DeepSpeed ZeRO 优化": step order global norm -> loss-scale update ->
// unscale/clip -> optimizer step (section 3.2), clip coefficient
// max_norm / (norm + 1e-6) (section 7), dynamic loss scaling (section 6),
// overflow = inf/NaN in the grads, which skips the step (section 9, Q6).
//
// Kernels, all on the caller's stream, no host synchronization:
//   K1 sumsq_kernel   one workgroup per quarter slot: float64 sum of squares
//                     of its real grads -> workspace[4 * slot + part] (level 1)
//   K2 finalize_kernel one workgroup of 1024 lanes: fixed-order float64 sum
//                     of the part sums + the other ranks' sum -> overflow flag, clip and
//                     unscale factor k, bias-correction scalars, loss scale;
//                     written to the device state                (level 2)
//   K3 update          one workgroup per slot: AdamW on g, p, m, v (16-byte
//                     streaming loads and stores), the updated block kept in
//                     registers, block amax (wave shuffles + LDS), scale,
//                     E4M3 codes.  Returns at once when K2 flagged a skip.
//                     update_full_kernel (1024 lanes) takes the full-block
//                     slots: it issues every load of its block before any
//                     arithmetic and every store after it; update_kernel
//                     (512 lanes) takes partial blocks and padding slots, and
//                     every slot of a small shard.
// K1 is left out when no statistics are needed, or when the fold already
// wrote the per-quarter sums (fused statistics).
#include <hip/hip_runtime.h>

#include <cmath>

#include "device_util.h"
#include "e4m3.h"

namespace fp8z1 {
namespace {

// ---------------------------------------------------------------- K1

// one workgroup per part of a slot, the order of the fold's fused statistics
__global__ __launch_bounds__(kSumThreads) void sumsq_kernel(const SlotPlan* __restrict__ plan,
                                                            const float* __restrict__ grad,
                                                            double* __restrict__ out) {
  __shared__ double red[kSumThreads / 64];
  const int64_t s = blockIdx.x / kStatParts;
  const int part = blockIdx.x % kStatParts;
  const SlotPlan P = plan[s];
  const int t = threadIdx.x;
  double acc = 0.0;
  if (P.param >= 0) {
    const float4* g = reinterpret_cast<const float4*>(grad + s * kBlockElems) + part * kPartChunks;
    const int vr = P.vr, vc = P.vc;
    const int r0 = part * kPartRows;
    if (vr == kB && vc == kB) {
#pragma unroll
      for (int k = 0; k < kPartPasses; ++k) {
        const float4 x = g[t + kSumThreads * k];
        acc += sq64(x.x);
        acc += sq64(x.y);
        acc += sq64(x.z);
        acc += sq64(x.w);
      }
    } else {
#pragma unroll
      for (int k = 0; k < kPartPasses; ++k) {
        const int c = t + kSumThreads * k;
        const int i = r0 + c / kChunksPerRow, j = 4 * (c % kChunksPerRow);
        if (i < vr && j < vc) {
          const float4 x = g[c];
          // masked positions add +0, exactly what the fold's zero padding adds
          acc += j + 0 < vc ? sq64(x.x) : 0.0;
          acc += j + 1 < vc ? sq64(x.y) : 0.0;
          acc += j + 2 < vc ? sq64(x.z) : 0.0;
          acc += j + 3 < vc ? sq64(x.w) : 0.0;
        } else {
          acc += 0.0;
          acc += 0.0;
          acc += 0.0;
          acc += 0.0;
        }
      }
    }
  }
  const double tot = block_sum<kSumThreads>(acc, red);
  if (t == 0) out[s * kStatParts + part] = tot;
}

// ---------------------------------------------------------------- K2

struct FinalizeArgs {
  double extra_sumsq;
  const double* global_sumsq;  // device; when set, the global sum itself (partials unused)
  int64_t nslots;
  float lr, beta1, beta2, weight_decay, max_grad_norm;
  float growth_factor, backoff_factor;
  int32_t growth_interval;
  int32_t loss_scaling;
  int32_t have_stats;
  int32_t extra_found_inf;
};

constexpr int kFinThreads = 1024;
constexpr int kFinAcc = 8;  // independent accumulators per lane (loads in flight)

// Level 2 of the sum of squares: the shard's partials (one per quarter slot)
// summed in a fixed order.  Partial i goes to lane i % 1024, accumulator
// (i / 1024) % 8 of that lane, each accumulator adding its partials in
// increasing order; a lane adds its 8 accumulators in order, then the block
// reduction combines the lanes.  (One dependent chain of loads per lane made
// this a latency-bound 0.25 ms for the 229,376 partials of the full step.)
__device__ __forceinline__ double sum_partials(const double* __restrict__ partial, int64_t count, double* red) {
  double acc[kFinAcc];
#pragma unroll
  for (int u = 0; u < kFinAcc; ++u) acc[u] = 0.0;
  int64_t i = threadIdx.x;
  for (; i + (kFinAcc - 1) * kFinThreads < count; i += kFinAcc * kFinThreads) {
    double x[kFinAcc];
#pragma unroll
    for (int u = 0; u < kFinAcc; ++u) x[u] = partial[i + u * kFinThreads];
#pragma unroll
    for (int u = 0; u < kFinAcc; ++u) acc[u] += x[u];
  }
  // the last partial round: fewer than kFinAcc partials left for this lane
#pragma unroll
  for (int u = 0; u < kFinAcc - 1; ++u)
    if (i + u * kFinThreads < count) acc[u] += partial[i + u * kFinThreads];
  double tot = acc[0];
#pragma unroll
  for (int u = 1; u < kFinAcc; ++u) tot += acc[u];
  return block_sum<kFinThreads>(tot, red);
}

__global__ __launch_bounds__(kFinThreads) void shard_sumsq_kernel(const double* __restrict__ partial, int64_t count,
                                                                  double* __restrict__ out) {
  __shared__ double red[kFinThreads / 64];
  const double tot = sum_partials(partial, count, red);
  if (threadIdx.x == 0) *out = tot;
}

__global__ __launch_bounds__(kFinThreads) void finalize_kernel(const double* __restrict__ partial,
                                                               fp8z1_state* __restrict__ st, FinalizeArgs a) {
  __shared__ double red[kFinThreads / 64];
  const bool own = a.have_stats && !a.global_sumsq;  // uniform over the workgroup
  const double local = own ? sum_partials(partial, a.nslots * kStatParts, red) : 0.0;
  if (threadIdx.x != 0) return;

  fp8z1_state S = *st;
  const double scale = a.loss_scaling ? static_cast<double>(S.loss_scale) : 1.0;
  double glob = 0.0;
  bool found = false;
  if (a.have_stats) {
    glob = a.global_sumsq ? *a.global_sumsq : local + a.extra_sumsq;
    found = !isfinite(glob) || a.extra_found_inf != 0;
  }
  S.global_sumsq = glob;
  S.found_inf = found ? 1 : 0;
  if (found) {
    S.skipped_total += 1;
    if (a.loss_scaling) {
      S.loss_scale = static_cast<float>(scale * static_cast<double>(a.backoff_factor));
      S.good_steps = 0;
    }
    *st = S;
    return;
  }
  double coef = 1.0;
  if (a.max_grad_norm > 0.0f) {
    const double norm = sqrt(glob) / scale;
    const double c = static_cast<double>(a.max_grad_norm) / (norm + 1e-6);
    if (c < 1.0) coef = c;
  }
  S.k = static_cast<float>(coef / scale);
  S.step += 1;
  S.beta1_pow = S.beta1_pow * static_cast<double>(a.beta1);
  S.beta2_pow = S.beta2_pow * static_cast<double>(a.beta2);
  S.step_size = static_cast<float>(static_cast<double>(a.lr) / (1.0 - S.beta1_pow));
  S.bc2_sqrt = static_cast<float>(sqrt(1.0 - S.beta2_pow));
  S.decay = static_cast<float>(1.0 - static_cast<double>(a.lr) * static_cast<double>(a.weight_decay));
  if (a.loss_scaling) {
    S.good_steps += 1;
    if (S.good_steps >= a.growth_interval) {
      S.loss_scale = static_cast<float>(scale * static_cast<double>(a.growth_factor));
      S.good_steps = 0;
    }
  }
  *st = S;
}

__global__ void state_init_kernel(fp8z1_state* st, float loss_scale) {
  fp8z1_state S;
  S.step = 0;
  S.beta1_pow = 1.0;
  S.beta2_pow = 1.0;
  S.global_sumsq = 0.0;
  S.loss_scale = loss_scale;
  S.k = 1.0f;
  S.step_size = 0.0f;
  S.bc2_sqrt = 1.0f;
  S.decay = 1.0f;
  S.good_steps = 0;
  S.found_inf = 0;
  S.skipped_total = 0;
  *st = S;
}

// ---------------------------------------------------------------- K3

struct UpdateArgs {
  float beta1, beta2, one_minus_beta1, one_minus_beta2, eps;
  int32_t pow2_scale;
  int64_t nslots;
  int32_t cache_codes;  // 1: plain stores for the codes, 0: streaming stores
};

// Block scale from the block's amax.  Default: amax / 448 (the largest E4M3
// value), 1 for an all-zero block.  Power-of-two rule (the E8M0 shared scale of
// the OCP microscaling formats): 2^(floor(log2 amax) - 8), 8 being the
// exponent of the largest E4M3 binade, clamped to the E8M0 range from 2^-127.
__device__ __forceinline__ float block_scale(float amax, bool pow2) {
  if (!(amax > 0.0f)) return 1.0f;
  if (!pow2) return amax / 448.0f;
  const uint32_t u = __float_as_uint(amax);
  if (u >= 0x7f800000u) return amax;  // +inf
  const uint32_t ef = u >> 23;
  // floor(log2 amax): the exponent field for normals; from the leading bit of the
  // mantissa for subnormals (value = m * 2^-149)
  const int k = ef ? static_cast<int>(ef) - 127 : (31 - __clz(static_cast<int>(u & 0x7fffffu))) - 149;
  const int x = max(k - 8, -127);
  return x >= -126 ? __uint_as_float(static_cast<uint32_t>(x + 127) << 23) : __uint_as_float(1u << (x + 149));
}

struct Moments {
  float p, m, v;
};

// One element of the AdamW update, one float32 rounding per operation.
__device__ __forceinline__ Moments adamw1(float g_raw, float p, float m, float v, float k, float decay,
                                          float step_size, float bc2, const UpdateArgs& a) {
  const float g = g_raw * k;
  const float m1 = a.beta1 * m + a.one_minus_beta1 * g;
  const float v1 = a.beta2 * v + a.one_minus_beta2 * (g * g);
  // __builtin_sqrtf lowers to the correctly rounded sequence (hardware sqrt,
  // then a one-ulp correction from the fma residuals); __fsqrt_rn lowers to the
  // bare hardware sqrt here, which is off by one ulp on some inputs.
  const float den = __builtin_sqrtf(v1) / bc2 + a.eps;
  const float p1 = p * decay - step_size * (m1 / den);
  return {p1, m1, v1};
}

__device__ __forceinline__ uint32_t pack_codes(float4 x, float s) {
  return e4m3_encode(x.x / s) | (e4m3_encode(x.y / s) << 8) | (e4m3_encode(x.z / s) << 16) |
         (e4m3_encode(x.w / s) << 24);
}

// Where the update reads the grads from: the folded shard (the fold ran
// before), or the row-major params directly (the fold happens on read and no
// folded copy of the grads is written).
template <bool ROWMAJOR>
struct GradSrc {
  const float4* folded;  // this slot's folded grads (!ROWMAJOR)
  const float* rows;     // element (0, 0) of this slot's block (ROWMAJOR)
  int64_t ld;            // row stride (ROWMAJOR)

  // the 4 elements of chunk c (all real)
  __device__ __forceinline__ float4 chunk(int c) const {
    if (!ROWMAJOR) return ld_stream(folded + c);
    return ld_global_stream_a4(rows + (c / kChunksPerRow) * ld + 4 * (c % kChunksPerRow));
  }
  // element e of chunk c, which is column j of row i
  __device__ __forceinline__ float elem(int c, int i, int j, int e) const {
    if (ROWMAJOR) return rows[i * ld + j];
    return reinterpret_cast<const float*>(folded + c)[e];
  }
};

// Pointers of one slot's g, p, m, v and codes.
template <bool ROWMAJOR>
struct SlotPtrs {
  GradSrc<ROWMAJOR> g;
  float4 *p, *m, *v;
  uint32_t* codes;
};

template <bool ROWMAJOR>
__device__ __forceinline__ SlotPtrs<ROWMAJOR> slot_ptrs(const SlotPlan& P, int64_t s, const float* grad,
                                                       void* const* grad_rows, float* master, float* mom1,
                                                       float* mom2, uint8_t* fp8) {
  SlotPtrs<ROWMAJOR> r;
  const int64_t base = s * (kBlockElems / 4);
  if (ROWMAJOR) {
    r.g.folded = nullptr;
    r.g.rows = P.param >= 0 ? static_cast<const float*>(grad_rows[P.param]) + P.off : nullptr;
    r.g.ld = P.ld;
  } else {
    r.g.folded = reinterpret_cast<const float4*>(grad) + base;
    r.g.rows = nullptr;
    r.g.ld = 0;
  }
  r.p = reinterpret_cast<float4*>(master) + base;
  r.m = reinterpret_cast<float4*>(mom1) + base;
  r.v = reinterpret_cast<float4*>(mom2) + base;
  r.codes = reinterpret_cast<uint32_t*>(fp8 + s * kBlockElems);
  return r;
}

// Slot of workgroup b: entry b of the launch's slot list, or slot b.  The
// plain order keeps the workgroups in flight on one compact window of slots
// (giving each XCD a contiguous range of slots instead ran the ragged shard's
// update 6 % slower, the MoE shard's 10 %).
__device__ __forceinline__ int64_t launch_slot(const int32_t* slots) {
  const int64_t b = blockIdx.x;
  return slots ? slots[b] : b;
}

// Full blocks.  1024 lanes, each with 4 chunks (16 elements) of the block: all
// 16 loads of a lane (g, then p, m, v) are issued before any arithmetic, and
// the stores of p, m and v follow the arithmetic as one group; the scheduling
// barriers keep the compiler from interleaving them.  The workgroup so asks for
// its whole block (4 x 64 KB) at once, and one workgroup per CU (97 VGPRs) is
// in flight: on the MoE shard this ran 10 % faster than 512 lanes with loads
// and stores interleaved per chunk (two workgroups per CU), and faster than
// the same with 512 lanes (its 32 loads per lane leave one workgroup of 8
// waves per CU) or with the next slot's loads overlapping the current slot's
// stores in a persistent grid.
constexpr int kFullThreads = 1024;
constexpr int kFullPasses = kChunks / kFullThreads;

template <bool ROWMAJOR>
__global__ __launch_bounds__(kFullThreads) void update_full_kernel(
    const SlotPlan* __restrict__ plan, const fp8z1_state* __restrict__ st, const float* __restrict__ grad,
    void* const* __restrict__ grad_rows, float* __restrict__ master, float* __restrict__ mom1,
    float* __restrict__ mom2, uint8_t* __restrict__ fp8, float* __restrict__ scales, UpdateArgs a,
    const int32_t* __restrict__ slots) {
  __shared__ float red[kFullThreads / 64];
  if (st->found_inf) return;  // skipped step: nothing changes
  const float k = st->k, decay = st->decay, step_size = st->step_size, bc2 = st->bc2_sqrt;
  const int64_t s = launch_slot(slots);
  const SlotPlan P = plan[s];
  const SlotPtrs<ROWMAJOR> X = slot_ptrs<ROWMAJOR>(P, s, grad, grad_rows, master, mom1, mom2, fp8);
  const int t = threadIdx.x;
  float4 g[kFullPasses], p[kFullPasses], m[kFullPasses], v[kFullPasses];
#pragma unroll
  for (int q = 0; q < kFullPasses; ++q) g[q] = X.g.chunk(t + kFullThreads * q);
#pragma unroll
  for (int q = 0; q < kFullPasses; ++q) p[q] = ld_stream(X.p + t + kFullThreads * q);
#pragma unroll
  for (int q = 0; q < kFullPasses; ++q) m[q] = ld_stream(X.m + t + kFullThreads * q);
#pragma unroll
  for (int q = 0; q < kFullPasses; ++q) v[q] = ld_stream(X.v + t + kFullThreads * q);
  __builtin_amdgcn_sched_barrier(0);
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < kFullPasses; ++q) {
    const Moments e0 = adamw1(g[q].x, p[q].x, m[q].x, v[q].x, k, decay, step_size, bc2, a);
    const Moments e1 = adamw1(g[q].y, p[q].y, m[q].y, v[q].y, k, decay, step_size, bc2, a);
    const Moments e2 = adamw1(g[q].z, p[q].z, m[q].z, v[q].z, k, decay, step_size, bc2, a);
    const Moments e3 = adamw1(g[q].w, p[q].w, m[q].w, v[q].w, k, decay, step_size, bc2, a);
    p[q] = make_float4(e0.p, e1.p, e2.p, e3.p);
    m[q] = make_float4(e0.m, e1.m, e2.m, e3.m);
    v[q] = make_float4(e0.v, e1.v, e2.v, e3.v);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(e0.p), fabsf(e1.p)), fmaxf(fabsf(e2.p), fabsf(e3.p))));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < kFullPasses; ++q) st_stream(X.p + t + kFullThreads * q, p[q]);
#pragma unroll
  for (int q = 0; q < kFullPasses; ++q) st_stream(X.m + t + kFullThreads * q, m[q]);
#pragma unroll
  for (int q = 0; q < kFullPasses; ++q) st_stream(X.v + t + kFullThreads * q, v[q]);
  __builtin_amdgcn_sched_barrier(0);
  amax = block_max<kFullThreads>(amax, red);
  const float scale = block_scale(amax, a.pow2_scale != 0);
  // codes of a shard up to about twice the last-level cache: plain (cached)
  // stores, so that the unfold which follows finds many of them still in the
  // cache; larger ones stream
  if (a.cache_codes) {
#pragma unroll
    for (int q = 0; q < kFullPasses; ++q) X.codes[t + kFullThreads * q] = pack_codes(p[q], scale);
  } else {
#pragma unroll
    for (int q = 0; q < kFullPasses; ++q) st_stream(X.codes + t + kFullThreads * q, pack_codes(p[q], scale));
  }
  if (t == 0) scales[s] = scale;
}

// Any slot: full blocks, partial blocks and padding slots.  512 lanes, 8
// chunks per lane, loads and stores per chunk (68 VGPRs, several workgroups
// per CU: on a small shard, or on the few partial blocks of a large one, the
// full-block kernel's one workgroup per CU leaves too few rounds).
constexpr int kUpdThreads = 512;
constexpr int kUpdPasses = kChunks / kUpdThreads;

template <bool ROWMAJOR>
__global__ __launch_bounds__(kUpdThreads) void update_kernel(const SlotPlan* __restrict__ plan,
                                                             const fp8z1_state* __restrict__ st,
                                                             const float* __restrict__ grad,
                                                             void* const* __restrict__ grad_rows,
                                                             float* __restrict__ master, float* __restrict__ mom1,
                                                             float* __restrict__ mom2, uint8_t* __restrict__ fp8,
                                                             float* __restrict__ scales, UpdateArgs a,
                                                             const int32_t* __restrict__ slots) {
  __shared__ float red[kUpdThreads / 64];
  if (st->found_inf) return;  // skipped step: nothing changes
  const float k = st->k, decay = st->decay, step_size = st->step_size, bc2 = st->bc2_sqrt;
  const int64_t s = launch_slot(slots);
  const SlotPlan P = plan[s];
  const int t = threadIdx.x;
  const SlotPtrs<ROWMAJOR> X = slot_ptrs<ROWMAJOR>(P, s, grad, grad_rows, master, mom1, mom2, fp8);
  uint32_t* codes = X.codes;
  if (P.param < 0) {
#pragma unroll
    for (int q = 0; q < kUpdPasses; ++q) codes[t + kUpdThreads * q] = 0u;
    if (t == 0) scales[s] = 1.0f;
    return;
  }
  const GradSrc<ROWMAJOR>& G = X.g;
  float4* p4 = X.p;
  float4* m4 = X.m;
  float4* v4 = X.v;

  float4 pn[kUpdPasses];
  float amax = 0.0f;
  const int vr = P.vr, vc = P.vc;
  const bool full = vr == kB && vc == kB;
  if (full) {
#pragma unroll
    for (int q = 0; q < kUpdPasses; ++q) {
      const int c = t + kUpdThreads * q;
      const float4 g = G.chunk(c), p = ld_stream(p4 + c), m = ld_stream(m4 + c), v = ld_stream(v4 + c);
      const Moments e0 = adamw1(g.x, p.x, m.x, v.x, k, decay, step_size, bc2, a);
      const Moments e1 = adamw1(g.y, p.y, m.y, v.y, k, decay, step_size, bc2, a);
      const Moments e2 = adamw1(g.z, p.z, m.z, v.z, k, decay, step_size, bc2, a);
      const Moments e3 = adamw1(g.w, p.w, m.w, v.w, k, decay, step_size, bc2, a);
      pn[q] = make_float4(e0.p, e1.p, e2.p, e3.p);
      st_stream(p4 + c, pn[q]);
      st_stream(m4 + c, make_float4(e0.m, e1.m, e2.m, e3.m));
      st_stream(v4 + c, make_float4(e0.v, e1.v, e2.v, e3.v));
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(e0.p), fabsf(e1.p)), fmaxf(fabsf(e2.p), fabsf(e3.p))));
    }
  } else {
    // partial block: chunks wholly inside the real region go as in a full
    // block; in the chunk across the last real column, padding positions are
    // neither used nor changed (their loaded values are written back as they
    // were); padding counts 0 in amax
#pragma unroll
    for (int q = 0; q < kUpdPasses; ++q) {
      const int c = t + kUpdThreads * q;
      const int i = c / kChunksPerRow, j = 4 * (c % kChunksPerRow);
      pn[q] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < vr && j + 4 <= vc) {
        const float4 g = G.chunk(c), p = ld_stream(p4 + c), m = ld_stream(m4 + c), v = ld_stream(v4 + c);
        const Moments e0 = adamw1(g.x, p.x, m.x, v.x, k, decay, step_size, bc2, a);
        const Moments e1 = adamw1(g.y, p.y, m.y, v.y, k, decay, step_size, bc2, a);
        const Moments e2 = adamw1(g.z, p.z, m.z, v.z, k, decay, step_size, bc2, a);
        const Moments e3 = adamw1(g.w, p.w, m.w, v.w, k, decay, step_size, bc2, a);
        pn[q] = make_float4(e0.p, e1.p, e2.p, e3.p);
        st_stream(p4 + c, pn[q]);
        st_stream(m4 + c, make_float4(e0.m, e1.m, e2.m, e3.m));
        st_stream(v4 + c, make_float4(e0.v, e1.v, e2.v, e3.v));
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(e0.p), fabsf(e1.p)), fmaxf(fabsf(e2.p), fabsf(e3.p))));
      } else if (i < vr && j < vc) {
        // the chunk across the last real column: its real elements one by one
        float* pf = reinterpret_cast<float*>(p4 + c);
        float* mf = reinterpret_cast<float*>(m4 + c);
        float* vf = reinterpret_cast<float*>(v4 + c);
        float qn[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (j + e < vc) {
            const Moments r = adamw1(G.elem(c, i, j + e, e), pf[e], mf[e], vf[e], k, decay, step_size, bc2, a);
            pf[e] = r.p;
            mf[e] = r.m;
            vf[e] = r.v;
            qn[e] = r.p;
            amax = fmaxf(amax, fabsf(r.p));
          }
        }
        pn[q] = make_float4(qn[0], qn[1], qn[2], qn[3]);
      }
    }
  }

  amax = block_max<kUpdThreads>(amax, red);
  const float scale = block_scale(amax, a.pow2_scale != 0);
  if (full) {
    if (a.cache_codes) {
#pragma unroll
      for (int q = 0; q < kUpdPasses; ++q) codes[t + kUpdThreads * q] = pack_codes(pn[q], scale);
    } else {
#pragma unroll
      for (int q = 0; q < kUpdPasses; ++q) st_stream(codes + t + kUpdThreads * q, pack_codes(pn[q], scale));
    }
  } else {
#pragma unroll
    for (int q = 0; q < kUpdPasses; ++q) {
      const int c = t + kUpdThreads * q;
      const int i = c / kChunksPerRow, j = 4 * (c % kChunksPerRow);
      uint32_t w = 0u;
      if (i < vr && j < vc) {
        w = pack_codes(pn[q], scale);
        // padding positions get code 0
        const int nvalid = vc - j;
        if (nvalid < 4) w &= (1u << (8 * nvalid)) - 1u;
      }
      codes[c] = w;
    }
  }
  if (t == 0) scales[s] = scale;
}

__global__ void encode_kernel(const float* __restrict__ in, uint8_t* __restrict__ out, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) out[i] = static_cast<uint8_t>(e4m3_encode(in[i]));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) % 16) == 0; }

}  // namespace
}  // namespace fp8z1

using namespace fp8z1;

extern "C" int fp8z1_state_init(const fp8z1_hparams* hp, fp8z1_state* d_state, void* stream) {
  if (!hp || !d_state) return set_error(FP8Z1_EINVAL, "state_init: NULL argument");
  if (reinterpret_cast<uintptr_t>(d_state) % 8) return set_error(FP8Z1_EINVAL, "state_init: state must be 8-byte aligned");
  const float s0 = hp->loss_scaling ? hp->init_scale : 1.0f;
  if (hp->loss_scaling && !(s0 > 0.0f && std::isfinite(s0)))
    return set_error(FP8Z1_EINVAL, "state_init: init_scale must be finite and > 0");
  hipLaunchKernelGGL(state_init_kernel, dim3(1), dim3(1), 0, static_cast<hipStream_t>(stream), d_state, s0);
  return check_hip(hipGetLastError(), "state_init: launch");
}

extern "C" int fp8z1_step_workspace_bytes(const fp8z1_table* t, size_t* bytes) {
  if (!t || !bytes) return set_error(FP8Z1_EINVAL, "step_workspace_bytes: NULL argument");
  *bytes = static_cast<size_t>(t->info.shard_slots) * kStatParts * sizeof(double);
  return FP8Z1_OK;
}

extern "C" int fp8z1_shard_sumsq(const fp8z1_table* t, const double* d_partials, double* d_sum, void* stream) {
  if (!t || !d_sum || (!d_partials && t->info.shard_slots > 0))
    return set_error(FP8Z1_EINVAL, "shard_sumsq: NULL argument");
  if (reinterpret_cast<uintptr_t>(d_partials) % 8 || reinterpret_cast<uintptr_t>(d_sum) % 8)
    return set_error(FP8Z1_EINVAL, "shard_sumsq: partials and sum must be 8-byte aligned");
  const int64_t count = t->info.shard_slots * kStatParts;
  hipLaunchKernelGGL(shard_sumsq_kernel, dim3(1), dim3(kFinThreads), 0, static_cast<hipStream_t>(stream), d_partials,
                     count, d_sum);
  return check_hip(hipGetLastError(), "shard_sumsq: launch");
}

namespace {

int step_impl(fp8z1_table* t, const fp8z1_hparams* hp, fp8z1_state* d_state, const float* grad,
              const void* const* grad_rows, float* master, float* m, float* v, uint8_t* fp8, float* scales,
              void* d_workspace, size_t workspace_bytes, int32_t presummed, void* stream) {
  const char* who = grad_rows ? "step_rowmajor" : "step";
  if (!t || !hp || !d_state || !(grad || grad_rows) || !master || !m || !v || !fp8 || !scales)
    return set_error(FP8Z1_EINVAL, std::string(who) + ": NULL argument");
  if ((grad && !aligned16(grad)) || !aligned16(master) || !aligned16(m) || !aligned16(v) || !aligned16(fp8))
    return set_error(FP8Z1_EINVAL, std::string(who) + ": grad, master, m, v and fp8 must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(scales) % 4 || reinterpret_cast<uintptr_t>(d_state) % 8)
    return set_error(FP8Z1_EINVAL, std::string(who) + ": misaligned scales or state");
  if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f && hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
    return set_error(FP8Z1_EINVAL, std::string(who) + ": betas must be in [0, 1)");
  if (!(hp->eps > 0.0f) || !std::isfinite(hp->lr) || !std::isfinite(hp->weight_decay))
    return set_error(FP8Z1_EINVAL, std::string(who) + ": eps must be > 0, lr and weight_decay finite");
  if (std::isnan(hp->max_grad_norm)) return set_error(FP8Z1_EINVAL, std::string(who) + ": max_grad_norm is NaN");
  if (hp->loss_scaling && hp->growth_interval < 1)
    return set_error(FP8Z1_EINVAL, std::string(who) + ": growth_interval must be >= 1");
  if (hp->loss_scaling && !(hp->growth_factor > 0.0f && std::isfinite(hp->growth_factor) &&
                            hp->backoff_factor > 0.0f && std::isfinite(hp->backoff_factor)))
    return set_error(FP8Z1_EINVAL, std::string(who) + ": growth_factor and backoff_factor must be finite and > 0");
  if (hp->scale_rule != FP8Z1_SCALE_AMAX && hp->scale_rule != FP8Z1_SCALE_POW2)
    return set_error(FP8Z1_EINVAL, std::string(who) + ": scale_rule must be FP8Z1_SCALE_AMAX or FP8Z1_SCALE_POW2");
  if (grad_rows) {
    for (const fp8z1_block& e : t->entries) {
      if (e.param < 0) continue;
      const void* p = grad_rows[e.param];
      if (!p || reinterpret_cast<uintptr_t>(p) % 4)
        return set_error(FP8Z1_EINVAL, std::string(who) + ": grad pointer of param " + std::to_string(e.param) +
                                           " is NULL or misaligned");
    }
  }
  const bool stats = hp->max_grad_norm > 0.0f || hp->loss_scaling != 0;
  const bool given = stats && hp->d_global_sumsq != nullptr;  // global sum from the caller, on the device
  const int64_t n = t->info.shard_slots;
  if (n * kStatParts > 0x7fffffffLL) return set_error(FP8Z1_ESHAPE, std::string(who) + ": too many slots");
  if (given && reinterpret_cast<uintptr_t>(hp->d_global_sumsq) % 8)
    return set_error(FP8Z1_EINVAL, std::string(who) + ": misaligned d_global_sumsq");
  if (stats && !given) {
    if (!d_workspace) return set_error(FP8Z1_EINVAL, std::string(who) + ": statistics need the workspace");
    if (workspace_bytes < static_cast<size_t>(n) * kStatParts * sizeof(double))
      return set_error(FP8Z1_EINVAL, std::string(who) + ": workspace smaller than fp8z1_step_workspace_bytes()");
    if (reinterpret_cast<uintptr_t>(d_workspace) % 8)
      return set_error(FP8Z1_EINVAL, std::string(who) + ": misaligned workspace");
  }
  std::lock_guard<std::mutex> lock(t->mu);
  int rc = ensure_device(t, stream);
  if (rc) return rc;
  void** drows = nullptr;
  if (grad_rows) {
    rc = device_ptr_list(t, kRoleStepGrad, grad_rows, &drows, stream);
    if (rc) return rc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  double* partial = static_cast<double*>(d_workspace);
  if (stats && !given && !presummed && n > 0) {
    if (grad_rows)
      rc = check_hip(launch_grad_sumsq(t->d_plan, drows, partial, n, t->info.valid_elems, s),
                     "step: statistics launch");
    else {
      hipLaunchKernelGGL(sumsq_kernel, dim3(static_cast<unsigned>(n * kStatParts)), dim3(kSumThreads), 0, s,
                         t->d_plan, grad, partial);
      rc = check_hip(hipGetLastError(), "step: statistics launch");
    }
    if (rc) return rc;
  }
  FinalizeArgs fa;
  fa.extra_sumsq = hp->extra_sumsq;
  fa.global_sumsq = given ? hp->d_global_sumsq : nullptr;
  fa.nslots = n;
  fa.lr = hp->lr;
  fa.beta1 = hp->beta1;
  fa.beta2 = hp->beta2;
  fa.weight_decay = hp->weight_decay;
  fa.max_grad_norm = hp->max_grad_norm;
  fa.growth_factor = hp->growth_factor;
  fa.backoff_factor = hp->backoff_factor;
  fa.growth_interval = hp->growth_interval;
  fa.loss_scaling = hp->loss_scaling ? 1 : 0;
  fa.have_stats = stats ? 1 : 0;
  fa.extra_found_inf = hp->extra_found_inf ? 1 : 0;
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(kFinThreads), 0, s, partial, d_state, fa);
  rc = check_hip(hipGetLastError(), "step: finalize launch");
  if (rc) return rc;
  if (n == 0) return note_use(t, stream);
  UpdateArgs ua;
  ua.beta1 = hp->beta1;
  ua.beta2 = hp->beta2;
  ua.one_minus_beta1 = static_cast<float>(1.0 - static_cast<double>(hp->beta1));
  ua.one_minus_beta2 = static_cast<float>(1.0 - static_cast<double>(hp->beta2));
  ua.eps = hp->eps;
  ua.pow2_scale = hp->scale_rule == FP8Z1_SCALE_POW2 ? 1 : 0;
  ua.cache_codes = n * kBlockElems <= 2 * kLastLevelCacheBytes;
  // full blocks first (all slots in order when every slot is one), then the
  // partial blocks and padding slots.  The full-block kernel holds one
  // workgroup per CU; below kManyFullSlots slots that leaves few rounds, and
  // small launches take the general kernel, which holds several (on the dense
  // shard's 3,440 slots the two ran within 0.5 % of each other).
  constexpr int64_t kManyFullSlots = 8192;
  auto launch = [&](bool full, const int32_t* list, int64_t count) {
    if (count == 0) return;
    full = full && count >= kManyFullSlots;
    ua.nslots = count;
    const unsigned grid = static_cast<unsigned>(count);
    if (grad_rows && full)
      hipLaunchKernelGGL(update_full_kernel<true>, dim3(grid), dim3(kFullThreads), 0, s, t->d_plan, d_state, nullptr,
                         drows, master, m, v, fp8, scales, ua, list);
    else if (grad_rows)
      hipLaunchKernelGGL(update_kernel<true>, dim3(grid), dim3(kUpdThreads), 0, s, t->d_plan, d_state, nullptr, drows,
                         master, m, v, fp8, scales, ua, list);
    else if (full)
      hipLaunchKernelGGL(update_full_kernel<false>, dim3(grid), dim3(kFullThreads), 0, s, t->d_plan, d_state, grad,
                         nullptr, master, m, v, fp8, scales, ua, list);
    else
      hipLaunchKernelGGL(update_kernel<false>, dim3(grid), dim3(kUpdThreads), 0, s, t->d_plan, d_state, grad, nullptr,
                         master, m, v, fp8, scales, ua, list);
  };
  if (t->n_other_slots == 0) {
    launch(true, nullptr, n);
  } else {
    launch(true, t->d_full_slots, t->n_full_slots);
    rc = check_hip(hipGetLastError(), "step: update launch");
    if (rc) return rc;
    launch(false, t->d_other_slots, t->n_other_slots);
  }
  rc = check_hip(hipGetLastError(), "step: update launch");
  return rc ? rc : note_use(t, stream);
}

}  // namespace

extern "C" int fp8z1_step(const fp8z1_table* ct, const fp8z1_hparams* hp, fp8z1_state* d_state, const float* grad,
                          float* master, float* m, float* v, uint8_t* fp8, float* scales, void* d_workspace,
                          size_t workspace_bytes, int32_t presummed, void* stream) {
  if (!grad) return set_error(FP8Z1_EINVAL, "step: NULL argument");
  return step_impl(const_cast<fp8z1_table*>(ct), hp, d_state, grad, nullptr, master, m, v, fp8, scales, d_workspace,
                   workspace_bytes, presummed, stream);
}

extern "C" int fp8z1_step_rowmajor(const fp8z1_table* ct, const fp8z1_hparams* hp, fp8z1_state* d_state,
                                   const void* const* grads, float* master, float* m, float* v, uint8_t* fp8,
                                   float* scales, void* d_workspace, size_t workspace_bytes, void* stream) {
  if (!grads) return set_error(FP8Z1_EINVAL, "step_rowmajor: NULL argument");
  return step_impl(const_cast<fp8z1_table*>(ct), hp, d_state, nullptr, grads, master, m, v, fp8, scales,
                   d_workspace, workspace_bytes, 0, stream);
}

// ---------------------------------------------------------------- no allocation
//
// The statistics partials of fp8z1_step_rowmajor_noalloc: a file-scope device
// array, one copy per GPU.  In host code `scratch` names a host-side stand-in,
// not device memory; its device address on each GPU comes from
// hipGetSymbolAddress, taken once per device (with that device current) at the
// first call there, and only that address is passed to kernels.
namespace {
constexpr int64_t kNoallocSlots = FP8Z1_NOALLOC_MAX_SLOTS;
static __device__ __align__(256) double scratch[kNoallocSlots * kStatParts];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
double* g_scratch_ptr[kMaxDevices] = {};

int scratch_on_device(double** out) {
  int dev = -1;
  int rc = check_hip(hipGetDevice(&dev), "step_rowmajor_noalloc: hipGetDevice");
  if (rc) return rc;
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(FP8Z1_EDEVICE, "step_rowmajor_noalloc: device index " + std::to_string(dev) + " beyond " +
                                         std::to_string(kMaxDevices));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    rc = check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "step_rowmajor_noalloc: hipGetSymbolAddress");
    if (rc) return rc;
    g_scratch_ptr[dev] = static_cast<double*>(p);
  }
  *out = g_scratch_ptr[dev];
  return FP8Z1_OK;
}
}  // namespace

extern "C" int fp8z1_step_rowmajor_noalloc(const fp8z1_table* ct, const fp8z1_hparams* hp, fp8z1_state* d_state,
                                           const void* const* grads, float* master, float* m, float* v, uint8_t* fp8,
                                           float* scales, void* stream) {
  fp8z1_table* t = const_cast<fp8z1_table*>(ct);
  if (!t || !hp || !grads) return set_error(FP8Z1_EINVAL, "step_rowmajor_noalloc: NULL argument");
  if (t->info.shard_slots > kNoallocSlots)
    return set_error(FP8Z1_ESHAPE, "step_rowmajor_noalloc: the table has " + std::to_string(t->info.shard_slots) +
                                       " slots, more than FP8Z1_NOALLOC_MAX_SLOTS (" + std::to_string(kNoallocSlots) +
                                       "); use fp8z1_step_rowmajor with a workspace");
  {
    std::lock_guard<std::mutex> lock(t->mu);
    if (t->device < 0)
      return set_error(FP8Z1_EINVAL,
                       "step_rowmajor_noalloc: the table is not set up on a device yet (setting it up allocates); "
                       "make one other GPU call with it first, e.g. the init fp8z1_fold");
  }
  double* ws = nullptr;
  const int rc = scratch_on_device(&ws);
  if (rc) return rc;
  return step_impl(t, hp, d_state, nullptr, grads, master, m, v, fp8, scales, ws,
                   static_cast<size_t>(kNoallocSlots) * kStatParts * sizeof(double), 0, stream);
}

extern "C" int fp8z1_encode_e4m3(const float* in, uint8_t* out, int64_t n, void* stream) {
  if (n < 0 || (n > 0 && (!in || !out))) return set_error(FP8Z1_EINVAL, "encode_e4m3: bad arguments");
  if (n == 0) return FP8Z1_OK;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  if (blocks > 0x7fffffff) return set_error(FP8Z1_EINVAL, "encode_e4m3: n too large for one launch");
  hipLaunchKernelGGL(encode_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads), 0,
                     static_cast<hipStream_t>(stream), in, out, n);
  return check_hip(hipGetLastError(), "encode_e4m3: launch");
}
