// Device side of a table handle: the per-slot launch plan, the per-param
// pointer lists, release; and state copies to and from the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "internal.h"

namespace fp8z1 {

int check_hip(int hip_status, const char* what) {
  const hipError_t e = static_cast<hipError_t>(hip_status);
  if (e == hipSuccess) return FP8Z1_OK;
  return set_error(FP8Z1_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

// The set-up below allocates, copies synchronously and waits on events, none
// of which may happen while `stream` is being captured into a graph; the
// callers ask this only on those slow paths, so a captured call costs nothing.
static int refuse_in_capture(void* stream, const char* what) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  int rc = check_hip(hipStreamIsCapturing(static_cast<hipStream_t>(stream), &st), "hipStreamIsCapturing");
  if (rc) return rc;
  if (st != hipStreamCaptureStatusNone)
    return set_error(FP8Z1_EINVAL, std::string(what) +
                                       " inside a stream capture: make the same call once outside the capture first");
  return FP8Z1_OK;
}

int ensure_device(fp8z1_table* t, void* stream) {
  int dev = -1;
  int rc = check_hip(hipGetDevice(&dev), "hipGetDevice");
  if (rc) return rc;
  if (t->device >= 0) {
    if (dev != t->device)
      return set_error(FP8Z1_EDEVICE, "table is bound to device " + std::to_string(t->device) + ", current is " +
                                           std::to_string(dev));
    return FP8Z1_OK;
  }
  rc = refuse_in_capture(stream, "first device use of a table");
  if (rc) return rc;
  const size_t n = t->entries.size();
  std::vector<SlotPlan> plan(n);
  for (size_t s = 0; s < n; ++s) {
    const fp8z1_block& e = t->entries[s];
    SlotPlan& p = plan[s];
    std::memset(&p, 0, sizeof(p));
    p.param = e.param;
    if (e.param < 0) continue;
    const fp8z1_shape& sh = t->shapes[e.param];
    const int64_t rb = (sh.R + kB - 1) / kB, cb = (sh.C + kB - 1) / kB;
    p.off = (int64_t(e.expert) * sh.R + int64_t(kB) * e.brow) * sh.C + int64_t(kB) * e.bcol;
    p.ld = sh.C;
    p.soff = static_cast<int32_t>((int64_t(e.expert) * rb + e.brow) * cb + e.bcol);
    p.vr = e.vrows;
    p.vc = e.vcols;
  }
  // unfold work items: runs of side-by-side blocks of one block row, cut into
  // groups of whole rows of about kRowItemBytes bytes of FP8 output
  std::vector<RowItem> rows;
  for (size_t s = 0; s < n;) {
    const fp8z1_block& e = t->entries[s];
    if (e.param < 0) {
      ++s;
      continue;
    }
    size_t s1 = s + 1;
    while (s1 < n && t->entries[s1].param == e.param && t->entries[s1].expert == e.expert &&
           t->entries[s1].brow == e.brow && t->entries[s1].bcol == t->entries[s1 - 1].bcol + 1)
      ++s1;
    const fp8z1_shape& sh = t->shapes[e.param];
    const int32_t nblk = static_cast<int32_t>(s1 - s);
    const int32_t len = kB * (nblk - 1) + t->entries[s1 - 1].vcols;
    const int32_t vr = e.vrows;
    const int32_t per = std::max(1, std::min(vr, kRowItemBytes / len));
    for (int32_t r0 = 0; r0 < vr; r0 += per) {
      RowItem it;
      std::memset(&it, 0, sizeof(it));
      it.off = (int64_t(e.expert) * sh.R + int64_t(kB) * e.brow + r0) * sh.C + int64_t(kB) * e.bcol;
      it.ld = sh.C;
      it.param = e.param;
      it.slot = static_cast<int32_t>(s);
      it.len = len;
      it.nblk = nblk;
      it.row0 = r0;
      it.rows = std::min(per, vr - r0);
      it.soff = plan[s].soff;
      rows.push_back(it);
    }
    s = s1;
  }
  if (rows.size() > 0x7fffffffULL) return set_error(FP8Z1_ESHAPE, "table: too many unfold work items");
  // update slot lists: full blocks apart from the rest, so that the update's
  // full-block kernel carries no partial-block code
  std::vector<int32_t> full_slots, other_slots;
  for (size_t s = 0; s < n; ++s) {
    const fp8z1_block& e = t->entries[s];
    (e.param >= 0 && e.vrows == kB && e.vcols == kB ? full_slots : other_slots).push_back(static_cast<int32_t>(s));
  }
  if (other_slots.empty()) full_slots.clear();  // all full: the update runs over the slots in order
  // (a failed earlier attempt may have left some of these allocated: keep them)
  for (int r = 0; r < kNumRoles; ++r) {
    PtrCache& c = t->ptrs[r];
    const size_t bytes = sizeof(void*) * t->shapes.size();
    if (!c.host)
      rc = check_hip(hipHostMalloc(reinterpret_cast<void**>(&c.host), bytes, hipHostMallocDefault), "hipHostMalloc");
    if (!rc && !c.dev) rc = check_hip(hipMalloc(reinterpret_cast<void**>(&c.dev), bytes), "hipMalloc");
    if (!rc && !c.done)
      rc = check_hip(hipEventCreateWithFlags(reinterpret_cast<hipEvent_t*>(&c.done), hipEventDisableTiming),
                     "hipEventCreate");
    if (rc) return rc;
    c.valid = false;
  }
  if (!t->last_use) {
    rc = check_hip(hipEventCreateWithFlags(reinterpret_cast<hipEvent_t*>(&t->last_use), hipEventDisableTiming),
                   "hipEventCreate");
    if (rc) return rc;
  }
  if (n) {
    if (!t->d_plan)
      rc = check_hip(hipMalloc(reinterpret_cast<void**>(&t->d_plan), n * sizeof(SlotPlan)), "hipMalloc(plan)");
    if (rc) return rc;
    rc = check_hip(hipMemcpy(t->d_plan, plan.data(), n * sizeof(SlotPlan), hipMemcpyHostToDevice), "hipMemcpy(plan)");
    if (rc) return rc;
  }
  if (!rows.empty()) {
    if (!t->d_rows)
      rc = check_hip(hipMalloc(reinterpret_cast<void**>(&t->d_rows), rows.size() * sizeof(RowItem)),
                     "hipMalloc(unfold items)");
    if (rc) return rc;
    rc = check_hip(hipMemcpy(t->d_rows, rows.data(), rows.size() * sizeof(RowItem), hipMemcpyHostToDevice),
                   "hipMemcpy(unfold items)");
    if (rc) return rc;
  }
  t->n_rows = static_cast<int64_t>(rows.size());
  for (int which = 0; which < 2; ++which) {
    std::vector<int32_t>& list = which ? other_slots : full_slots;
    int32_t*& dst = which ? t->d_other_slots : t->d_full_slots;
    if (list.empty()) continue;
    if (!dst) rc = check_hip(hipMalloc(reinterpret_cast<void**>(&dst), list.size() * sizeof(int32_t)), "hipMalloc(slots)");
    if (rc) return rc;
    rc = check_hip(hipMemcpy(dst, list.data(), list.size() * sizeof(int32_t), hipMemcpyHostToDevice), "hipMemcpy(slots)");
    if (rc) return rc;
  }
  t->n_full_slots = static_cast<int64_t>(full_slots.size());
  t->n_other_slots = static_cast<int64_t>(other_slots.size());
  t->device = dev;
  return FP8Z1_OK;
}

int note_use(fp8z1_table* t, void* stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  int rc = check_hip(hipStreamIsCapturing(static_cast<hipStream_t>(stream), &st), "hipStreamIsCapturing");
  if (rc || st != hipStreamCaptureStatusNone || !t->last_use) return rc;
  return check_hip(hipEventRecord(static_cast<hipEvent_t>(t->last_use), static_cast<hipStream_t>(stream)),
                   "hipEventRecord(table use)");
}

int device_ptr_list(fp8z1_table* t, PtrRole role, const void* const* host_list, void*** out, void* stream) {
  PtrCache& c = t->ptrs[role];
  const size_t bytes = sizeof(void*) * t->shapes.size();
  if (!c.valid || std::memcmp(c.host, host_list, bytes) != 0) {
    int rc = refuse_in_capture(stream, "new param pointers");
    if (rc) return rc;
    hipEvent_t ev = static_cast<hipEvent_t>(c.done);
    if (c.valid) {
      // the previous upload may still be reading the pinned mirror
      rc = check_hip(hipEventSynchronize(ev), "hipEventSynchronize");
      if (rc) return rc;
    }
    std::memcpy(c.host, host_list, bytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    rc = check_hip(hipMemcpyAsync(c.dev, c.host, bytes, hipMemcpyHostToDevice, s), "hipMemcpyAsync(pointer list)");
    if (!rc) rc = check_hip(hipEventRecord(ev, s), "hipEventRecord");
    if (rc) {
      c.valid = false;
      return rc;
    }
    c.valid = true;
  }
  *out = c.dev;
  return FP8Z1_OK;
}

}  // namespace fp8z1

using namespace fp8z1;

extern "C" void fp8z1_table_free(fp8z1_table* t) {
  if (!t) return;
  bool any = t->d_plan != nullptr || t->d_rows != nullptr || t->d_full_slots != nullptr ||
             t->d_other_slots != nullptr || t->last_use != nullptr;
  for (int r = 0; r < kNumRoles; ++r) any = any || t->ptrs[r].host || t->ptrs[r].dev || t->ptrs[r].done;
  if (any) {  // device resources exist only after a GPU call used the table
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (t->device >= 0 && cur != t->device) (void)hipSetDevice(t->device);
    // pending uploads and the kernels of the table's last call must have
    // finished (only this table's own work is waited for)
    for (int r = 0; r < kNumRoles; ++r)
      if (t->ptrs[r].done) (void)hipEventSynchronize(static_cast<hipEvent_t>(t->ptrs[r].done));
    if (t->last_use) {
      (void)hipEventSynchronize(static_cast<hipEvent_t>(t->last_use));
      (void)hipEventDestroy(static_cast<hipEvent_t>(t->last_use));
    }
    for (int r = 0; r < kNumRoles; ++r) {
      PtrCache& c = t->ptrs[r];
      if (c.host) (void)hipHostFree(c.host);
      if (c.dev) (void)hipFree(c.dev);
      if (c.done) (void)hipEventDestroy(static_cast<hipEvent_t>(c.done));
    }
    if (t->d_plan) (void)hipFree(t->d_plan);
    if (t->d_rows) (void)hipFree(t->d_rows);
    if (t->d_full_slots) (void)hipFree(t->d_full_slots);
    if (t->d_other_slots) (void)hipFree(t->d_other_slots);
    if (t->device >= 0 && cur >= 0 && cur != t->device) (void)hipSetDevice(cur);
  }
  delete t;
}

extern "C" int fp8z1_state_read(const fp8z1_state* d_state, fp8z1_state* out, void* stream) {
  if (!d_state || !out) return set_error(FP8Z1_EINVAL, "state_read: NULL argument");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = check_hip(hipMemcpyAsync(out, d_state, sizeof(fp8z1_state), hipMemcpyDeviceToHost, s), "state_read: copy");
  if (rc) return rc;
  return check_hip(hipStreamSynchronize(s), "state_read: sync");
}

extern "C" int fp8z1_state_write(fp8z1_state* d_state, const fp8z1_state* in, void* stream) {
  if (!d_state || !in) return set_error(FP8Z1_EINVAL, "state_write: NULL argument");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = check_hip(hipMemcpyAsync(d_state, in, sizeof(fp8z1_state), hipMemcpyHostToDevice, s), "state_write: copy");
  if (rc) return rc;
  return check_hip(hipStreamSynchronize(s), "state_write: sync");
}
