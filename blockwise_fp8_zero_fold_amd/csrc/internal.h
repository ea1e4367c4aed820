// Internal definitions shared by the fp8z1 library sources (not part of the ABI).
#pragma once

#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/fp8z1.h"

namespace fp8z1 {

constexpr int kB = FP8Z1_BLOCK;          // block edge
constexpr int kBlockElems = kB * kB;     // 16384 elements per block

// Per-slot launch record kept on the device, derived from the 16-byte ABI
// entry and the param shapes so that a kernel needs one 32-byte load per
// slot.  `off` is the element offset of the block's (0, 0) element in its
// param's row-major [E, R, C] buffer, `ld` the row stride C, `soff` the
// offset of the block's scale in the param's [E, Rb, Cb] scale array.
struct SlotPlan {
  int64_t off;
  int64_t ld;
  int32_t param;  // -1: padding slot
  int32_t soff;
  uint16_t vr, vc;
  uint32_t pad;
};
static_assert(sizeof(SlotPlan) == 32, "SlotPlan is 32 bytes");

// Unfold work item: `rows` consecutive rows of a run of blocks that sit side
// by side in one block row of a param (consecutive slots, consecutive block
// columns).  Row i of such a run is one contiguous span of `len` real
// elements of the param's row-major buffer, so a workgroup can write it with
// aligned stores whatever the alignment of the row.  `off` is the element
// offset of the item's first row at the run's first block column, `slot` the
// run's first slot, `row0` the item's first row within the block row, `soff`
// the scale offset of the run's first block.
struct RowItem {
  int64_t off;
  int64_t ld;
  int32_t param;
  int32_t slot;
  int32_t len;
  int32_t nblk;
  int32_t row0;
  int32_t rows;
  int32_t soff;
  int32_t pad;
};
static_assert(sizeof(RowItem) == 48, "RowItem is 48 bytes");

// Size of an unfold work item: all side-by-side blocks of the run (a split
// run would leave the 128-byte lines at the cut shared by two workgroups),
// and as many of their rows as fit about kRowItemBytes bytes of FP8 output.
constexpr int kRowItemBytes = 16384;

// One pointer list per kind of call, so that a call of one kind cannot retarget a
// captured graph of another kind (the FP8 and the FP32 unfold have their own).
enum PtrRole {
  kRoleFoldSrc = 0,
  kRoleUnfoldDst = 1,
  kRoleUnfoldScale = 2,
  kRoleStepGrad = 3,
  kRoleUnfoldDstF32 = 4,
  kRoleUnfoldScaleF32 = 5,
  kNumRoles = 6
};

// Device-side pointer list for one role: a pinned host mirror, the device
// array and an event marking the end of the last upload from the mirror.
struct PtrCache {
  const void** host = nullptr;  // pinned
  void** dev = nullptr;
  void* done = nullptr;  // hipEvent_t
  bool valid = false;
};

}  // namespace fp8z1

struct fp8z1_table {
  fp8z1_table_info info{};
  std::vector<fp8z1_shape> shapes;
  std::vector<fp8z1_block> entries;
  // device state, created at the first GPU use
  std::mutex mu;
  int device = -1;
  fp8z1::SlotPlan* d_plan = nullptr;
  fp8z1::RowItem* d_rows = nullptr;  // unfold work items
  int64_t n_rows = 0;
  // slot lists of the update: full blocks, and the rest (partial blocks and
  // padding slots); both empty when every slot is a full block
  int32_t* d_full_slots = nullptr;
  int32_t* d_other_slots = nullptr;
  int64_t n_full_slots = 0, n_other_slots = 0;
  std::vector<char> held;  // per param: the table holds a block of it
  fp8z1::PtrCache ptrs[fp8z1::kNumRoles];
  // recorded on the caller's stream after the launches of every uncaptured
  // call that uses the table's device arrays; release waits for it (calls on
  // one table are on one stream or ordered by the caller, so the last one
  // finishing means all have)
  void* last_use = nullptr;  // hipEvent_t
};

namespace fp8z1 {

int set_error(int status, const std::string& msg);
// Bind the table to the current device and upload its plan (first call only;
// refused while `stream` is being captured).
int ensure_device(fp8z1_table* t, void* stream);
// Upload (if changed) a host list of n_params device pointers; returns the device
// array.  A change is refused while `stream` is being captured.
int device_ptr_list(fp8z1_table* t, PtrRole role, const void* const* host_list, void*** out, void* stream);
int check_hip(int hip_status, const char* what);
// Record the table's last-use event on `stream` (nothing inside a capture).
int note_use(fp8z1_table* t, void* stream);

}  // namespace fp8z1

#ifdef __HIPCC__
#include <hip/hip_runtime.h>
namespace fp8z1 {
// Per-slot float64 sums of squares of row-major FP32 grads (no folded copy),
// in the same order as the fold's fused statistics.
hipError_t launch_grad_sumsq(const SlotPlan* plan, void** grads, double* sumsq, int64_t nslots, int64_t valid_elems,
                             hipStream_t stream);
}  // namespace fp8z1
#endif
