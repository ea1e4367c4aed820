// Shard lookup table (host only): block-wise and param-wise splits.
//
// "面向 Blockwise FP8 量化的 ZeRO 优化器设计", section "块粒度切分": params are
// cut in 128x128 units, each quantized dimension padded up to a multiple of
// 128, and a lookup table keeps the real sizes and the padding so that the
// optimizer can walk the params inside a 1-D buffer.  Section "参数粒度切分":
// params sorted by size go greedily to DP buckets, each bucket padded up to
// the largest one.  The readings where the text is silent are the ones stated
// in fp8z1.h (block order, tail padding, greedy tie-breaks).
#include <algorithm>
#include <cstring>
#include <new>
#include <stdexcept>
#include <numeric>

#include "internal.h"

namespace {
thread_local std::string g_last_error;
}

namespace fp8z1 {

int set_error(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

}  // namespace fp8z1

using namespace fp8z1;

extern "C" const char* fp8z1_status_string(int status) {
  switch (status) {
    case FP8Z1_OK: return "ok";
    case FP8Z1_EINVAL: return "invalid argument";
    case FP8Z1_ENOMEM: return "out of memory";
    case FP8Z1_EHIP: return "HIP runtime error";
    case FP8Z1_ESHAPE: return "unsupported or mismatched shape";
    case FP8Z1_EDEVICE: return "table bound to another device";
    default: return "unknown status";
  }
}

extern "C" const char* fp8z1_last_error(void) { return g_last_error.c_str(); }

namespace {

struct Grid {
  int64_t E, Rb, Cb, nb;
};

Grid grid_of(const fp8z1_shape& s) {
  Grid g;
  g.E = s.E;
  g.Rb = (s.R + kB - 1) / kB;
  g.Cb = (s.C + kB - 1) / kB;
  g.nb = g.E * g.Rb * g.Cb;
  return g;
}

// Block number `b` (0 <= b < nb) of param `pid`, in (expert, block_row, block_col) order.
fp8z1_block block_of(int32_t pid, const fp8z1_shape& s, const Grid& g, int64_t b) {
  fp8z1_block e{};
  e.param = pid;
  e.expert = static_cast<int32_t>(b / (g.Rb * g.Cb));
  int64_t rem = b % (g.Rb * g.Cb);
  int64_t br = rem / g.Cb, bc = rem % g.Cb;
  e.brow = static_cast<uint16_t>(br);
  e.bcol = static_cast<uint16_t>(bc);
  e.vrows = static_cast<uint8_t>(std::min<int64_t>(kB, s.R - kB * br));
  e.vcols = static_cast<uint8_t>(std::min<int64_t>(kB, s.C - kB * bc));
  e.reserved = 0;
  return e;
}

fp8z1_block pad_entry() {
  fp8z1_block e{};
  e.param = -1;
  return e;
}

// Greedy param-wise assignment: largest first (ties by id), each param to the
// least loaded bucket (ties to the lowest bucket index).
std::vector<int32_t> greedy_buckets(const std::vector<int64_t>& sizes, int32_t dp) {
  std::vector<int32_t> order(sizes.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    if (sizes[a] != sizes[b]) return sizes[a] > sizes[b];
    return a < b;
  });
  std::vector<int64_t> load(dp, 0);
  std::vector<int32_t> owner(sizes.size(), 0);
  for (int32_t p : order) {
    int32_t best = 0;
    for (int32_t b = 1; b < dp; ++b)
      if (load[b] < load[best]) best = b;
    owner[p] = best;
    load[best] += sizes[p];
  }
  return owner;
}

}  // namespace

extern "C" int fp8z1_build_table(const fp8z1_shape* shapes, int32_t n_params, int32_t dp, int32_t rank,
                                 int32_t split, fp8z1_table** out) {
  if (!out) return set_error(FP8Z1_EINVAL, "build_table: out is NULL");
  *out = nullptr;
  if (!shapes || n_params < 1) return set_error(FP8Z1_EINVAL, "build_table: need n_params >= 1 shapes");
  if (dp < 1) return set_error(FP8Z1_EINVAL, "build_table: dp must be >= 1");
  if (!(rank == FP8Z1_ALL_RANKS || (rank >= 0 && rank < dp)))
    return set_error(FP8Z1_EINVAL, "build_table: rank must be in [0, dp) or FP8Z1_ALL_RANKS");
  if (split != FP8Z1_SPLIT_BLOCK && split != FP8Z1_SPLIT_PARAM)
    return set_error(FP8Z1_EINVAL, "build_table: split must be FP8Z1_SPLIT_BLOCK or FP8Z1_SPLIT_PARAM");

  std::vector<Grid> grids(n_params);
  int64_t nb_total = 0;
  for (int32_t p = 0; p < n_params; ++p) {
    const fp8z1_shape& s = shapes[p];
    if (s.E < 1 || s.R < 1 || s.C < 1)
      return set_error(FP8Z1_ESHAPE, "build_table: param " + std::to_string(p) + " has a dimension < 1");
    if (s.R >= (int64_t(1) << 23) || s.C >= (int64_t(1) << 23) || s.E >= (int64_t(1) << 31))
      return set_error(FP8Z1_ESHAPE, "build_table: param " + std::to_string(p) + " exceeds R, C < 2^23, E < 2^31");
    grids[p] = grid_of(s);
    if (grids[p].nb >= (int64_t(1) << 31))
      return set_error(FP8Z1_ESHAPE, "build_table: param " + std::to_string(p) + " has 2^31 or more blocks");
    nb_total += grids[p].nb;
  }

  fp8z1_table* t = new (std::nothrow) fp8z1_table();
  if (!t) return set_error(FP8Z1_ENOMEM, "build_table: host allocation failed");
  t->shapes.assign(shapes, shapes + n_params);

  int64_t spr = 0;
  try {
    if (split == FP8Z1_SPLIT_BLOCK) {
      spr = (nb_total + dp - 1) / dp;
      const int64_t first = rank == FP8Z1_ALL_RANKS ? 0 : int64_t(rank) * spr;
      const int64_t n = rank == FP8Z1_ALL_RANKS ? int64_t(dp) * spr : spr;
      t->entries.reserve(n);
      int64_t base = 0;  // global slot of the current param's first block
      for (int32_t p = 0; p < n_params && int64_t(t->entries.size()) < n; ++p) {
        const int64_t lo = std::max<int64_t>(first, base), hi = std::min<int64_t>(first + n, base + grids[p].nb);
        for (int64_t g = lo; g < hi; ++g) t->entries.push_back(block_of(p, shapes[p], grids[p], g - base));
        base += grids[p].nb;
      }
      while (int64_t(t->entries.size()) < n) t->entries.push_back(pad_entry());
      t->info.shard_first_slot = first;
    } else {
      std::vector<int64_t> sizes(n_params);
      for (int32_t p = 0; p < n_params; ++p) sizes[p] = grids[p].nb;
      std::vector<int32_t> owner = greedy_buckets(sizes, dp);
      std::vector<int64_t> load(dp, 0);
      for (int32_t p = 0; p < n_params; ++p) load[owner[p]] += sizes[p];
      spr = *std::max_element(load.begin(), load.end());
      const int32_t r0 = rank == FP8Z1_ALL_RANKS ? 0 : rank;
      const int32_t r1 = rank == FP8Z1_ALL_RANKS ? dp : rank + 1;
      t->entries.reserve((r1 - r0) * spr);
      for (int32_t b = r0; b < r1; ++b) {
        for (int32_t p = 0; p < n_params; ++p)
          if (owner[p] == b)
            for (int64_t k = 0; k < grids[p].nb; ++k) t->entries.push_back(block_of(p, shapes[p], grids[p], k));
        for (int64_t k = load[b]; k < spr; ++k) t->entries.push_back(pad_entry());
      }
      t->info.shard_first_slot = int64_t(r0) * spr;
    }
  } catch (const std::bad_alloc&) {
    delete t;
    return set_error(FP8Z1_ENOMEM, "build_table: host allocation failed");
  } catch (const std::length_error&) {  // more entries than a vector can hold
    delete t;
    return set_error(FP8Z1_ENOMEM, "build_table: table too large for host memory");
  }

  int64_t valid = 0;
  t->held.assign(static_cast<size_t>(n_params), 0);
  for (const fp8z1_block& e : t->entries) {
    valid += int64_t(e.vrows) * int64_t(e.vcols);
    if (e.param >= 0) t->held[e.param] = 1;
  }
  t->info.split = split;
  t->info.dp = dp;
  t->info.rank = rank;
  t->info.n_params = n_params;
  t->info.total_blocks = nb_total;
  t->info.slots_per_rank = spr;
  t->info.shard_slots = int64_t(t->entries.size());
  t->info.valid_elems = valid;
  t->info.pad_elems = t->info.shard_slots * kBlockElems - valid;
  *out = t;
  return FP8Z1_OK;
}

extern "C" int fp8z1_table_info_get(const fp8z1_table* t, fp8z1_table_info* out) {
  if (!t || !out) return set_error(FP8Z1_EINVAL, "table_info_get: NULL argument");
  *out = t->info;
  return FP8Z1_OK;
}

extern "C" int fp8z1_table_entries(const fp8z1_table* t, const fp8z1_block** entries) {
  if (!t || !entries) return set_error(FP8Z1_EINVAL, "table_entries: NULL argument");
  *entries = t->entries.empty() ? nullptr : t->entries.data();
  return FP8Z1_OK;
}
