// C ABI of libmla_mxfp4.so: argument validation, device checks, the plan
// registry and kernel launches. Errors are returned as status codes with a
// thread-local message, the C counterpart of the input checks on page
// "kernelbot-amd-mixed-mla-608791" (check_mla_inputs / check_hip_error).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>

#include "mla_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(MLA_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

struct DeviceInfo {
  bool queried = false;
  bool is_gfx950 = false;
  int num_cus = 0;
  size_t lds_per_block = 0;
};

std::mutex g_mu;
std::unordered_map<int, DeviceInfo> g_devices;

// What a decode call needs to launch without reading the device-side plan.
struct PlanEntry {
  int device;
  int32_t num_slots;
  int32_t num_reduce;
  int32_t wide_reduce;   // reduce kernel shape (see DecodeArgs)
  int32_t off_lse;
  int32_t off_out;
  size_t workspace_bytes;
};
std::unordered_map<uintptr_t, PlanEntry> g_plans;

int current_device(int* dev, DeviceInfo* info) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceInfo& d = g_devices[*dev];
  if (!d.queried) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, *dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    d.is_gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.num_cus = prop.multiProcessorCount;
    d.lds_per_block = prop.sharedMemPerBlock;
    d.queried = true;
  }
  *info = d;
  if (!d.is_gfx950) return fail(MLA_ERR_DEVICE, "the current HIP device is not gfx950 (MI355X)");
  if (d.lds_per_block < mla::decode_lds_bytes() || d.lds_per_block < mla::decode_dense_lds_bytes() ||
      d.lds_per_block < mla::decode_24_lds_bytes())
    return fail(MLA_ERR_DEVICE, "device LDS per workgroup is smaller than the decode kernel needs");
  return MLA_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID: return "MLA_ERR_INVALID";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    case MLA_ERR_DEVICE: return "MLA_ERR_DEVICE";
    case MLA_ERR_NOT_PLANNED: return "MLA_ERR_NOT_PLANNED";
    default: return "MLA_ERR_UNKNOWN";
  }
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

int mla_device_num_cus(int32_t* num_cus) {
  if (num_cus == nullptr) return fail(MLA_ERR_INVALID, "num_cus is null");
  int dev;
  DeviceInfo info;
  const int st = current_device(&dev, &info);
  if (st != MLA_OK) return st;
  *num_cus = info.num_cus;
  return MLA_OK;
}

int mla_workspace_bytes(int32_t batch, int64_t total_kv, int32_t num_cus, size_t* bytes) {
  if (bytes == nullptr) return fail(MLA_ERR_INVALID, "bytes is null");
  if (batch < 0) return fail(MLA_ERR_INVALID, "batch must be >= 0");
  if (total_kv < 0 || total_kv > INT32_MAX) return fail(MLA_ERR_INVALID, "total_kv must be in [0, 2^31)");
  if (num_cus <= 0) {
    const int st = mla_device_num_cus(&num_cus);
    if (st != MLA_OK) return st;
  }
  // the plans a bound covers address their partials with int32 offsets
  // (mla_plan_device refuses the same layout)
  if (mla::device_layout(batch, total_kv, num_cus).off_out > INT32_MAX)
    return fail(MLA_ERR_INVALID, "these sizes exceed the int32 offsets of a plan");
  *bytes = mla::workspace_bound(batch, total_kv, num_cus);
  return MLA_OK;
}

int mla_plan_host(const int32_t* kv_indptr_host, int32_t batch, int32_t num_cus, int32_t* words,
                  size_t capacity_words, size_t* num_words, size_t* workspace_bytes) {
  if (num_words == nullptr || workspace_bytes == nullptr)
    return fail(MLA_ERR_INVALID, "num_words / workspace_bytes is null");
  mla::PlanResult p;
  std::string err;
  const int st = mla::build_plan(kv_indptr_host, batch, num_cus, &p, &err);
  if (st != MLA_OK) return fail(st, err);
  *num_words = p.words.size();
  *workspace_bytes = p.workspace_bytes;
  if (capacity_words < p.words.size() || (words == nullptr && !p.words.empty()))
    return fail(MLA_ERR_WORKSPACE, "word buffer too small for the plan");
  if (!p.words.empty()) std::memcpy(words, p.words.data(), p.words.size() * sizeof(int32_t));
  return MLA_OK;
}

int mla_plan_cus(const int32_t* kv_indptr_host, int32_t batch, int32_t num_cus, void* workspace,
                 size_t workspace_bytes, void* stream) {
  int dev;
  DeviceInfo info;
  int st = current_device(&dev, &info);
  if (st != MLA_OK) return st;
  if (num_cus <= 0) num_cus = info.num_cus;
  if (workspace == nullptr || !aligned(workspace, mla::kAlignBytes))
    return fail(MLA_ERR_INVALID, "workspace must be a non-null 256-byte aligned device pointer");
  mla::PlanResult p;
  std::string err;
  st = mla::build_plan(kv_indptr_host, batch, num_cus, &p, &err);
  if (st != MLA_OK) return fail(st, err);
  if (p.workspace_bytes > workspace_bytes) {
    char buf[160];
    std::snprintf(buf, sizeof(buf), "workspace too small: plan needs %zu bytes, got %zu",
                  p.workspace_bytes, workspace_bytes);
    return fail(MLA_ERR_WORKSPACE, buf);
  }
  hipError_t e = hipMemcpyAsync(workspace, p.words.data(), p.words.size() * sizeof(int32_t),
                                hipMemcpyHostToDevice, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(plan)");
  e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize(plan)");
  {
    std::lock_guard<std::mutex> lk(g_mu);
    // more than 16 partials per merged sequence on average: the wide merge
    const int32_t wide = p.num_partials > 16 * p.num_reduce ? 1 : 0;
    g_plans[(uintptr_t)workspace] = PlanEntry{dev, p.num_slots, p.num_reduce, wide, p.off_lse, p.off_out,
                                              p.workspace_bytes};
  }
  return MLA_OK;
}

int mla_plan_device(const int32_t* kv_indptr_dev, int32_t batch, int64_t max_total_kv, int32_t num_cus,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int dev;
  DeviceInfo info;
  int st = current_device(&dev, &info);
  if (st != MLA_OK) return st;
  if (num_cus <= 0) num_cus = info.num_cus;
  if (batch < 0) return fail(MLA_ERR_INVALID, "batch must be >= 0");
  if (max_total_kv < 0 || max_total_kv > INT32_MAX)
    return fail(MLA_ERR_INVALID, "max_total_kv must be in [0, 2^31)");
  if (kv_indptr_dev == nullptr || !aligned(kv_indptr_dev, 4))
    return fail(MLA_ERR_INVALID, "kv_indptr must be a non-null 4-byte aligned device pointer");
  if (workspace == nullptr || !aligned(workspace, mla::kAlignBytes))
    return fail(MLA_ERR_INVALID, "workspace must be a non-null 256-byte aligned device pointer");
  const mla::DeviceLayout l = mla::device_layout(batch, max_total_kv, num_cus);
  if (l.off_out > INT32_MAX) return fail(MLA_ERR_INVALID, "plan offsets exceed int32");
  if ((size_t)l.total_bytes > workspace_bytes) {
    char buf[160];
    std::snprintf(buf, sizeof(buf), "workspace too small: the bounds need %lld bytes, got %zu",
                  (long long)l.total_bytes, workspace_bytes);
    return fail(MLA_ERR_WORKSPACE, buf);
  }
  hipError_t e = (hipError_t)mla::launch_plan_device(kv_indptr_dev, batch, num_cus, max_total_kv, l,
                                                      workspace, stream);
  if (e != hipSuccess) return hip_fail(e, "mla_plan_kernel launch");
  {
    // the decode launches for the bounds; its kernels read the actual
    // counts from the plan words
    std::lock_guard<std::mutex> lk(g_mu);
    // counts are only known on the device: a batch smaller than 1/16 of the
    // slots may split its sequences into more than 16 partials each
    const int32_t wide = (int64_t)batch * 16 < l.slots ? 1 : 0;
    g_plans[(uintptr_t)workspace] = PlanEntry{dev, (int32_t)l.slots, batch, wide, (int32_t)l.off_lse,
                                              (int32_t)l.off_out, (size_t)l.total_bytes};
  }
  return MLA_OK;
}

int mla_plan(const int32_t* kv_indptr_host, int32_t batch, void* workspace, size_t workspace_bytes,
             void* stream) {
  return mla_plan_cus(kv_indptr_host, batch, 0, workspace, workspace_bytes, stream);
}

int mla_plan_release(void* workspace) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_plans.erase((uintptr_t)workspace) == 0)
    return fail(MLA_ERR_NOT_PLANNED, "workspace has no plan to release");
  return MLA_OK;
}

}  // extern "C"

namespace {

enum class KvFormat { kMxfp4, kFp8, kBf16, kMxfp4_24 };

// Shared validation and launch of the three cache formats: the plan, the
// partial layout and the reduce kernel are the same for all of them.
int decode_common(KvFormat fmt, const void* q, const void* kv, const void* kv_scale,
                  const int32_t* kv_indices, const int32_t* kv_indptr, void* out, float sm_scale,
                  void* workspace, void* stream, bool gather = false,
                  const int32_t* page_indptr = nullptr, int32_t page_size = 1,
                  const int32_t* kv_start = nullptr) {
  // The registry is consulted before any HIP call: a workspace that was
  // never planned, or was released, is refused without touching the device.
  PlanEntry pe;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_plans.find((uintptr_t)workspace);
    if (it == g_plans.end())
      return fail(MLA_ERR_NOT_PLANNED, "workspace was not prepared by mla_plan (or was released)");
    pe = it->second;
  }
  int dev;
  DeviceInfo info;
  int st = current_device(&dev, &info);
  if (st != MLA_OK) return st;
  if (pe.device != dev) return fail(MLA_ERR_INVALID, "workspace was planned on another device");
  if (!std::isfinite(sm_scale)) return fail(MLA_ERR_INVALID, "sm_scale must be finite");
  const bool any_work = pe.num_slots > 0 || pe.num_reduce > 0;
  if (any_work) {
    if (out == nullptr || !aligned(out, 16)) return fail(MLA_ERR_INVALID, "out must be non-null and 16-byte aligned");
    if (kv_indptr == nullptr || !aligned(kv_indptr, 4)) return fail(MLA_ERR_INVALID, "kv_indptr must be non-null and 4-byte aligned");
  }
  if (pe.num_slots > 0) {
    if (q == nullptr || !aligned(q, 16)) return fail(MLA_ERR_INVALID, "q must be non-null and 16-byte aligned");
    const char* kv_name = (fmt == KvFormat::kMxfp4 || fmt == KvFormat::kMxfp4_24) ? "kv_packed"
                          : fmt == KvFormat::kFp8                                 ? "kv_fp8"
                                                                                  : "kv_bf16";
    if (kv == nullptr || !aligned(kv, 16))
      return fail(MLA_ERR_INVALID, std::string(kv_name) + " must be non-null and 16-byte aligned");
    if (fmt == KvFormat::kMxfp4 && kv_scale == nullptr) return fail(MLA_ERR_INVALID, "kv_scale must be non-null");
    if (fmt == KvFormat::kMxfp4_24 && (kv_scale == nullptr || !aligned(kv_scale, 8)))
      return fail(MLA_ERR_INVALID, "kv_scale must be a non-null 8-byte aligned device pointer (24-scale rows)");
    if (gather) {
      if (kv_indices == nullptr || !aligned(kv_indices, 4))
        return fail(MLA_ERR_INVALID, "kv_indices must be a non-null 4-byte aligned device pointer");
      if (fmt == KvFormat::kMxfp4 && !aligned(kv_scale, 2))
        return fail(MLA_ERR_INVALID, "kv_scale must be 2-byte aligned for a gathered cache");
      if (page_size < 1) return fail(MLA_ERR_INVALID, "page_size must be >= 1");
    }
    if (fmt == KvFormat::kFp8 && (kv_scale == nullptr || !aligned(kv_scale, 4)))
      return fail(MLA_ERR_INVALID, "kv_scale must be a non-null 4-byte aligned device pointer");
  }
  mla::DecodeArgs a;
  a.q = q;
  a.kv_packed = (const uint8_t*)kv;
  a.kv_scale = (const uint8_t*)kv_scale;
  a.kv_indptr = kv_indptr;
  a.kv_indices = gather ? kv_indices : nullptr;
  a.page_indptr = gather ? page_indptr : nullptr;
  a.page_size = gather ? page_size : 1;
  a.kv_start = gather ? nullptr : kv_start;
  a.out = out;
  a.plan = (const int32_t*)workspace;
  a.part_lse = (float*)((uint8_t*)workspace + pe.off_lse);
  a.part_out = (float*)((uint8_t*)workspace + pe.off_out);
  a.score_scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  a.num_slots = pe.num_slots;
  a.num_reduce = pe.num_reduce;
  a.wide_reduce = pe.wide_reduce;
  const int gmax = info.num_cus * MLA_PLAN_WG_PER_CU;
  a.grid = pe.num_slots < gmax ? pe.num_slots : gmax;
  hipError_t e;
  if (fmt == KvFormat::kMxfp4) {
    e = (hipError_t)mla::launch_decode(a, stream);
    if (e != hipSuccess) return hip_fail(e, "mla_decode_kernel launch");
  } else if (fmt == KvFormat::kMxfp4_24) {
    e = (hipError_t)mla::launch_decode_24(a, stream);
    if (e != hipSuccess) return hip_fail(e, "mla_decode_mxfp4_24_kernel launch");
  } else {
    e = (hipError_t)mla::launch_decode_dense(a, fmt == KvFormat::kFp8, (const float*)kv_scale, stream);
    if (e != hipSuccess) return hip_fail(e, "mla_decode_dense_kernel launch");
  }
  e = (hipError_t)mla::launch_reduce(a, stream);
  if (e != hipSuccess) return hip_fail(e, "mla_reduce_kernel launch");
  return MLA_OK;
}

// A shared-rows call needs its start rows.
bool starts_ok(const int32_t* kv_start) {
  if (kv_start == nullptr || !aligned(kv_start, 4)) {
    fail(MLA_ERR_INVALID, "kv_start must be a non-null 4-byte aligned device pointer");
    return false;
  }
  return true;
}

// A page-table call needs its page offsets (checked before the plan, so an
// empty batch reports the missing array too).
bool page_table_ok(const int32_t* page_indptr) {
  if (page_indptr == nullptr || !aligned(page_indptr, 4)) {
    fail(MLA_ERR_INVALID, "page_indptr must be a non-null 4-byte aligned device pointer");
    return false;
  }
  return true;
}

}  // namespace

extern "C" {

int mla_decode_mxfp4(const void* q, const void* kv_packed, const void* kv_scale,
                     const int32_t* kv_indptr, void* out, float sm_scale, void* workspace,
                     void* stream) {
  return decode_common(KvFormat::kMxfp4, q, kv_packed, kv_scale, nullptr, kv_indptr, out, sm_scale, workspace,
                       stream);
}

int mla_decode_mxfp4_24(const void* q, const void* kv_packed, const void* kv_scale, const int32_t* kv_indptr,
                        void* out, float sm_scale, void* workspace, void* stream) {
  return decode_common(KvFormat::kMxfp4_24, q, kv_packed, kv_scale, nullptr, kv_indptr, out, sm_scale, workspace,
                       stream);
}

int mla_decode_mxfp4_noalloc(const void* q, const void* kv_packed, const void* kv_scale,
                             const int32_t* kv_indptr, int32_t batch, void* out, float sm_scale,
                             void* stream) {
  if (batch < 0) return fail(MLA_ERR_INVALID, "batch must be >= 0");
  if (!std::isfinite(sm_scale)) return fail(MLA_ERR_INVALID, "sm_scale must be finite");
  if (kv_indptr == nullptr || !aligned(kv_indptr, 4))
    return fail(MLA_ERR_INVALID, "kv_indptr must be a non-null 4-byte aligned device pointer");
  if (batch > 0) {
    if (q == nullptr || !aligned(q, 16)) return fail(MLA_ERR_INVALID, "q must be non-null and 16-byte aligned");
    if (kv_packed == nullptr || !aligned(kv_packed, 16))
      return fail(MLA_ERR_INVALID, "kv_packed must be non-null and 16-byte aligned");
    if (kv_scale == nullptr) return fail(MLA_ERR_INVALID, "kv_scale must be non-null");
    if (out == nullptr || !aligned(out, 16)) return fail(MLA_ERR_INVALID, "out must be non-null and 16-byte aligned");
  }
  int dev;
  DeviceInfo info;
  int st = current_device(&dev, &info);
  if (st != MLA_OK) return st;
  // the plan is laid out for any offsets of `batch` sequences (up to 2^31 - 1
  // tokens), as mla_plan_device lays it out for its bounds
  const mla::DeviceLayout l = mla::device_layout(batch, INT32_MAX, info.num_cus);
  if ((size_t)l.total_bytes > mla::kNoAllocScratchBytes || l.off_out > INT32_MAX) {
    char buf[200];
    std::snprintf(buf, sizeof(buf),
                  "batch %d needs %lld bytes of plan and partials; the static scratch holds %zu bytes",
                  (int)batch, (long long)l.total_bytes, mla::kNoAllocScratchBytes);
    return fail(MLA_ERR_WORKSPACE, buf);
  }
  void* ws = nullptr;
  hipError_t e = (hipError_t)mla::noalloc_scratch(dev, &ws);
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  if (batch == 0) return MLA_OK;
  e = (hipError_t)mla::launch_plan_device(kv_indptr, batch, info.num_cus, INT32_MAX, l, ws, stream);
  if (e != hipSuccess) return hip_fail(e, "mla_plan_kernel launch");
  mla::DecodeArgs a;
  a.q = q;
  a.kv_packed = (const uint8_t*)kv_packed;
  a.kv_scale = (const uint8_t*)kv_scale;
  a.kv_indptr = kv_indptr;
  a.kv_indices = nullptr;
  a.page_indptr = nullptr;
  a.page_size = 1;
  a.kv_start = nullptr;
  a.out = out;
  a.plan = (const int32_t*)ws;
  a.part_lse = (float*)((uint8_t*)ws + l.off_lse);
  a.part_out = (float*)((uint8_t*)ws + l.off_out);
  a.score_scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  a.num_slots = (int32_t)l.slots;
  a.num_reduce = batch;
  // the counts are only known on the device (as for mla_plan_device)
  a.wide_reduce = (int64_t)batch * 16 < l.slots ? 1 : 0;
  const int gmax = info.num_cus * MLA_PLAN_WG_PER_CU;
  a.grid = a.num_slots < gmax ? a.num_slots : gmax;
  e = (hipError_t)mla::launch_decode(a, stream);
  if (e != hipSuccess) return hip_fail(e, "mla_decode_kernel launch");
  e = (hipError_t)mla::launch_reduce(a, stream);
  if (e != hipSuccess) return hip_fail(e, "mla_reduce_kernel launch");
  return MLA_OK;
}

int mla_decode_mxfp4_paged(const void* q, const void* kv_packed, const void* kv_scale,
                           const int32_t* kv_indices, const int32_t* kv_indptr, void* out, float sm_scale,
                           void* workspace, void* stream) {
  return decode_common(KvFormat::kMxfp4, q, kv_packed, kv_scale, kv_indices, kv_indptr, out, sm_scale,
                       workspace, stream, true);
}

int mla_decode_fp8(const void* q, const void* kv_fp8, const float* kv_scale, const int32_t* kv_indptr,
                   void* out, float sm_scale, void* workspace, void* stream) {
  return decode_common(KvFormat::kFp8, q, kv_fp8, kv_scale, nullptr, kv_indptr, out, sm_scale, workspace, stream);
}

int mla_decode_bf16(const void* q, const void* kv_bf16, const int32_t* kv_indptr, void* out,
                    float sm_scale, void* workspace, void* stream) {
  return decode_common(KvFormat::kBf16, q, kv_bf16, nullptr, nullptr, kv_indptr, out, sm_scale, workspace, stream);
}

int mla_decode_fp8_paged(const void* q, const void* kv_fp8, const float* kv_scale, const int32_t* kv_indices,
                         const int32_t* kv_indptr, void* out, float sm_scale, void* workspace, void* stream) {
  return decode_common(KvFormat::kFp8, q, kv_fp8, kv_scale, kv_indices, kv_indptr, out, sm_scale, workspace,
                       stream, true);
}

int mla_decode_bf16_paged(const void* q, const void* kv_bf16, const int32_t* kv_indices,
                          const int32_t* kv_indptr, void* out, float sm_scale, void* workspace, void* stream) {
  return decode_common(KvFormat::kBf16, q, kv_bf16, nullptr, kv_indices, kv_indptr, out, sm_scale, workspace,
                       stream, true);
}

int mla_decode_mxfp4_page_table(const void* q, const void* kv_packed, const void* kv_scale,
                                const int32_t* page_indices, const int32_t* page_indptr, int32_t page_size,
                                const int32_t* kv_indptr, void* out, float sm_scale, void* workspace,
                                void* stream) {
  if (!page_table_ok(page_indptr)) return MLA_ERR_INVALID;
  return decode_common(KvFormat::kMxfp4, q, kv_packed, kv_scale, page_indices, kv_indptr, out, sm_scale,
                       workspace, stream, true, page_indptr, page_size);
}

int mla_decode_fp8_page_table(const void* q, const void* kv_fp8, const float* kv_scale,
                              const int32_t* page_indices, const int32_t* page_indptr, int32_t page_size,
                              const int32_t* kv_indptr, void* out, float sm_scale, void* workspace,
                              void* stream) {
  if (!page_table_ok(page_indptr)) return MLA_ERR_INVALID;
  return decode_common(KvFormat::kFp8, q, kv_fp8, kv_scale, page_indices, kv_indptr, out, sm_scale, workspace,
                       stream, true, page_indptr, page_size);
}

int mla_decode_mxfp4_starts(const void* q, const void* kv_packed, const void* kv_scale, const int32_t* kv_start,
                            const int32_t* kv_indptr, void* out, float sm_scale, void* workspace, void* stream) {
  if (!starts_ok(kv_start)) return MLA_ERR_INVALID;
  return decode_common(KvFormat::kMxfp4, q, kv_packed, kv_scale, nullptr, kv_indptr, out, sm_scale, workspace,
                       stream, false, nullptr, 1, kv_start);
}

int mla_decode_fp8_starts(const void* q, const void* kv_fp8, const float* kv_scale, const int32_t* kv_start,
                          const int32_t* kv_indptr, void* out, float sm_scale, void* workspace, void* stream) {
  if (!starts_ok(kv_start)) return MLA_ERR_INVALID;
  return decode_common(KvFormat::kFp8, q, kv_fp8, kv_scale, nullptr, kv_indptr, out, sm_scale, workspace, stream,
                       false, nullptr, 1, kv_start);
}

int mla_decode_bf16_starts(const void* q, const void* kv_bf16, const int32_t* kv_start, const int32_t* kv_indptr,
                           void* out, float sm_scale, void* workspace, void* stream) {
  if (!starts_ok(kv_start)) return MLA_ERR_INVALID;
  return decode_common(KvFormat::kBf16, q, kv_bf16, nullptr, nullptr, kv_indptr, out, sm_scale, workspace, stream,
                       false, nullptr, 1, kv_start);
}

int mla_decode_bf16_page_table(const void* q, const void* kv_bf16, const int32_t* page_indices,
                               const int32_t* page_indptr, int32_t page_size, const int32_t* kv_indptr,
                               void* out, float sm_scale, void* workspace, void* stream) {
  if (!page_table_ok(page_indptr)) return MLA_ERR_INVALID;
  return decode_common(KvFormat::kBf16, q, kv_bf16, nullptr, page_indices, kv_indptr, out, sm_scale, workspace,
                       stream, true, page_indptr, page_size);
}

}  // extern "C"
