// libfathom C ABI: argument validation, workspace carving, kernel launches.
// The declarations, with argument meaning, layout, ownership and error
// behaviour, are in include/fathom.h.  Every check below runs on the host
// before any HIP call, so an invalid call launches nothing.

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <vector>

#include "fathom.h"
#include "fathom_internal.h"

using namespace fathom;

// Scratch memory of fathom_allocate_scan_topk_noalloc: a static device array
// that each GPU the library runs on holds until the process ends.  Host code
// never uses the array's name as an address (on the host it names a stand-in,
// not device memory): its device address is taken once per device with
// hipGetSymbolAddress and kept per device.
static __device__ __align__(256) unsigned char scratch[FATHOM_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return FATHOM_OK;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(FATHOM_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int check_store(const fathom_store_desc* s) {
  if (!s) return fail(FATHOM_ERR_INVALID_ARG, "store descriptor is NULL");
  if (s->num_kv_heads < 1) return fail(FATHOM_ERR_INVALID_ARG, "num_kv_heads must be >= 1");
  if (s->d != kD) return fail(FATHOM_ERR_UNSUPPORTED, "d = %d: only d = %d is supported", s->d, kD);
  if (s->n < 1) return fail(FATHOM_ERR_INVALID_ARG, "n must be >= 1");
  if (s->n > kMaxKeys)
    return fail(FATHOM_ERR_UNSUPPORTED, "n = %lld exceeds the supported %lld keys per head",
                static_cast<long long>(s->n), static_cast<long long>(kMaxKeys));
  const int64_t words = (s->n + 31) / 32;
  if (s->ldw < words || s->ldw % 4 != 0)
    return fail(FATHOM_ERR_INVALID_ARG, "ldw = %lld must be >= ceil(n/32) = %lld and a multiple of 4",
                static_cast<long long>(s->ldw), static_cast<long long>(words));
  // The scan addresses a head's plane block with 32-bit byte offsets (row
  // offsets and the buffer resource's record count), so one head's block
  // must stay below 4 GiB.
  const int64_t head_bytes = int64_t(kD) * kPlanes * s->ldw * 4;
  if (head_bytes > kMaxHeadBytes)
    return fail(FATHOM_ERR_UNSUPPORTED, "one head's plane block is %lld bytes, above the %lld addressable (ldw = %lld)",
                static_cast<long long>(head_bytes), static_cast<long long>(kMaxHeadBytes),
                static_cast<long long>(s->ldw));
  if (s->lengths && !aligned(s->lengths, 4)) return fail(FATHOM_ERR_INVALID_ARG, "lengths must be 4-byte aligned");
  if (static_cast<int64_t>(s->num_kv_heads) * head_bytes > kMaxStoreBytes)
    return fail(FATHOM_ERR_UNSUPPORTED, "plane store of %lld bytes is above the supported %lld bytes",
                static_cast<long long>(static_cast<int64_t>(s->num_kv_heads) * head_bytes),
                static_cast<long long>(kMaxStoreBytes));
  return FATHOM_OK;
}

// Workspace layouts (every section 256-byte aligned).
struct PackLayout {
  size_t kmin, kmax, s1, s2, total;
};
PackLayout pack_layout(int H) {
  const size_t cnt = static_cast<size_t>(H) * kD;
  PackLayout L{};
  size_t off = 0;
  L.kmin = off; off = round_up(off + cnt * 4, 256);
  L.kmax = off; off = round_up(off + cnt * 4, 256);
  L.s1 = off;   off = round_up(off + cnt * 8, 256);
  L.s2 = off;   off = round_up(off + cnt * 8, 256);
  L.total = off;
  return L;
}

struct ScanLayout {
  size_t theta, count, sample, cand, tables, rescue, rescue_cnt, rescue_hist, rescue_done, total;
  int rescue_wgs;
};
ScanLayout scan_layout(int num_q, int64_t n, int k) {
  const size_t Q = static_cast<size_t>(num_q);
  ScanLayout L{};
  L.rescue_wgs = rescue_wgs_for(n);
  const size_t R = static_cast<size_t>(L.rescue_wgs);
  size_t off = 0;
  L.theta = off;  off = round_up(off + Q * 4, 256);
  L.count = off;  off = round_up(off + Q * 4, 256);
  L.sample = off; off = round_up(off + Q * kSampleMaxKeys * 4, 256);
  L.cand = off;   off = round_up(off + Q * kCandCap * 8, 256);
  L.tables = off; off = round_up(off + Q * kChunkTableBytes, 256);
  L.rescue = off; off = round_up(off + size_t(kRescueSlots) * R * size_t(k) * 8, 256);
  L.rescue_cnt = off;  off = round_up(off + size_t(kRescueSlots) * R * 8, 256);
  L.rescue_hist = off; off = round_up(off + size_t(kRescueSlots) * kRescueHistBins * 4, 256);
  L.rescue_done = off; off = round_up(off + size_t(kRescueSlots) * 4, 256);
  L.total = off;
  return L;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch` per device

// events of the staged host-resident call: (ready, freed) per staging slot,
// and the allocation's
std::mutex g_staged_mu;
hipEvent_t g_staged_events[5] = {};

// kernel timing record
std::mutex g_timing_mu;
bool g_timing_on = false;
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_events;   // created on enable
size_t g_events_used = 0;
constexpr size_t kMaxTimed = 4096;

}  // namespace

namespace {

int scan_impl(const char* where, const uint32_t* planes, const float* lo, const float* step,
              const fathom_store_desc* store, const float* q, const uint8_t* alloc, int32_t num_q,
              int32_t group, int32_t k, int32_t* out_idx, float* out_score, float* all_scores,
              void* workspace, size_t workspace_bytes, void* hip_stream, const float* var, int32_t budget_bits,
              uint8_t* alloc_out) {
  int st = check_store(store);
  if (st != FATHOM_OK) return st;
  if (!planes || !lo || !step || !q || !out_idx || !out_score)
    return fail(FATHOM_ERR_INVALID_ARG, "planes, lo, step, q, out_idx and out_score must be non-NULL");
  if (var) {
    if (!alloc_out) return fail(FATHOM_ERR_INVALID_ARG, "alloc must be non-NULL");
    if (budget_bits < 0 || budget_bits > kPlanes * kD)
      return fail(FATHOM_ERR_INVALID_ARG, "budget_bits = %d outside [0, %d]", budget_bits, kPlanes * kD);
    if (!aligned(q, 8) || !aligned(var, 8) || !aligned(alloc_out, 2))
      return fail(FATHOM_ERR_INVALID_ARG, "q and var must be 8-byte aligned, alloc 2-byte aligned");
  } else if (!alloc) {
    return fail(FATHOM_ERR_INVALID_ARG, "alloc must be non-NULL");
  }
  if (num_q < 1 || group < 1) return fail(FATHOM_ERR_INVALID_ARG, "num_q and group must be >= 1");
  if (static_cast<int64_t>(store->num_kv_heads) * group != num_q)
    return fail(FATHOM_ERR_INVALID_ARG, "num_q = %d must equal num_kv_heads (%d) * group (%d)", num_q,
                store->num_kv_heads, group);
  if (k < 1 || k > store->n) return fail(FATHOM_ERR_INVALID_ARG, "k = %d outside [1, n]", k);
  if (k > FATHOM_MAX_K) return fail(FATHOM_ERR_UNSUPPORTED, "k = %d exceeds FATHOM_MAX_K (%d)", k, FATHOM_MAX_K);
  if (!aligned(planes, 16)) return fail(FATHOM_ERR_INVALID_ARG, "planes must be 16-byte aligned");
  if (!aligned(lo, 4) || !aligned(step, 4) || !aligned(q, 4) || !aligned(out_idx, 4) ||
      !aligned(out_score, 4) || (all_scores && !aligned(all_scores, 4)))
    return fail(FATHOM_ERR_INVALID_ARG, "float and int32 arrays must be 4-byte aligned");
  const ScanLayout L = scan_layout(num_q, store->n, k);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < L.total)
    return fail(FATHOM_ERR_WORKSPACE, "scan needs a 256-byte aligned workspace of %zu bytes (got %zu)",
                L.total, workspace_bytes);
  char* w = static_cast<char*>(workspace);
  ScanWorkspace ws{reinterpret_cast<float*>(w + L.theta), reinterpret_cast<uint32_t*>(w + L.count),
                   reinterpret_cast<float*>(w + L.sample), reinterpret_cast<uint2*>(w + L.cand),
                   static_cast<void*>(w + L.tables), reinterpret_cast<uint2*>(w + L.rescue),
                   reinterpret_cast<uint2*>(w + L.rescue_cnt), reinterpret_cast<uint32_t*>(w + L.rescue_hist),
                   reinterpret_cast<uint32_t*>(w + L.rescue_done),
                   L.rescue_wgs};

  ScanTiming timing;
  bool timed = false;
  {
    std::lock_guard<std::mutex> lock(g_timing_mu);
    if (g_timing_on && g_events_used < g_events.size()) {
      timing.start = g_events[g_events_used].first;
      timing.stop = g_events[g_events_used].second;
      ++g_events_used;
      timed = true;
    }
  }
  hipError_t e = launch_scan_topk(planes, lo, step, store->num_kv_heads, store->n, store->lengths, store->ldw, q,
                                  alloc,
                                  num_q, group, k, out_idx, out_score, all_scores, ws,
                                  timed ? &timing : nullptr, static_cast<hipStream_t>(hip_stream), var,
                                  budget_bits, alloc_out);
  if (e != hipSuccess) return hip_fail(e, where);
  return ok();
}

size_t attend_bytes(int num_q, int k) {
  const size_t b = size_t(num_q) * size_t(attend_splits(k)) * size_t(kD + 2) * sizeof(float);
  return (b + 255) / 256 * 256;
}

}  // namespace

extern "C" {

int64_t fathom_plane_ldw(int64_t n) {
  if (n < 1) return -1;
  const int64_t words = (n + 31) / 32;
  return (words + 3) / 4 * 4;
}

size_t fathom_workspace_bytes(int32_t op, const fathom_store_desc* store, int32_t num_q, int32_t k) {
  if (check_store(store) != FATHOM_OK) return 0;
  if (op == FATHOM_OP_PACK) return pack_layout(store->num_kv_heads).total;
  if (op == FATHOM_OP_SCAN) {
    if (num_q < 1 || k < 1 || k > kMaxK) return 0;
    return scan_layout(num_q, store->n, k).total;
  }
  if (op == FATHOM_OP_ATTEND) {
    if (num_q < 1 || k < 1 || k > kMaxK) return 0;
    return attend_bytes(num_q, k);
  }
  return 0;
}

int fathom_pack_planes(const float* keys, int64_t stride_head, int64_t stride_token,
                       const fathom_store_desc* store, uint32_t* planes, float* lo, float* step,
                       float* var, void* workspace, size_t workspace_bytes, void* hip_stream) {
  int st = check_store(store);
  if (st != FATHOM_OK) return st;
  if (!keys || !planes || !lo || !step) return fail(FATHOM_ERR_INVALID_ARG, "keys, planes, lo and step must be non-NULL");
  if (!aligned(keys, 16)) return fail(FATHOM_ERR_INVALID_ARG, "keys must be 16-byte aligned");
  if (stride_token < kD || stride_token % 4 != 0)
    return fail(FATHOM_ERR_INVALID_ARG, "stride_token must be >= d and a multiple of 4");
  if (store->num_kv_heads > 1 && (stride_head < store->n * stride_token || stride_head % 4 != 0))
    return fail(FATHOM_ERR_INVALID_ARG, "stride_head must be >= n * stride_token and a multiple of 4");
  if (!aligned(planes, 16)) return fail(FATHOM_ERR_INVALID_ARG, "planes must be 16-byte aligned");
  if (!aligned(lo, 4) || !aligned(step, 4) || (var && !aligned(var, 4)))
    return fail(FATHOM_ERR_INVALID_ARG, "lo, step and var must be 4-byte aligned");
  const PackLayout L = pack_layout(store->num_kv_heads);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < L.total)
    return fail(FATHOM_ERR_WORKSPACE, "pack needs a 256-byte aligned workspace of %zu bytes (got %zu)",
                L.total, workspace_bytes);
  char* w = static_cast<char*>(workspace);
  PackWorkspace ws{reinterpret_cast<uint32_t*>(w + L.kmin), reinterpret_cast<uint32_t*>(w + L.kmax),
                   reinterpret_cast<unsigned long long*>(w + L.s1),
                   reinterpret_cast<unsigned long long*>(w + L.s2)};
  hipError_t e = launch_pack(keys, store->num_kv_heads > 1 ? stride_head : 0, stride_token,
                             store->num_kv_heads, store->n, store->lengths, store->ldw, planes, lo, step, var, ws,
                             static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "fathom_pack_planes launch");
  return ok();
}

int fathom_append_keys(const float* keys, int64_t stride_head, int64_t stride_token, int32_t m,
                       const fathom_store_desc* store, uint32_t* planes, const float* lo, const float* step,
                       void* hip_stream) {
  int st = check_store(store);
  if (st != FATHOM_OK) return st;
  if (!keys || !planes || !lo || !step) return fail(FATHOM_ERR_INVALID_ARG, "keys, planes, lo and step must be non-NULL");
  if (m < 1) return fail(FATHOM_ERR_INVALID_ARG, "m must be >= 1");
  if (store->n + m > store->ldw * 32)
    return fail(FATHOM_ERR_INVALID_ARG, "n + m = %lld exceeds the rows' capacity %lld",
                static_cast<long long>(store->n + m), static_cast<long long>(store->ldw * 32));
  if (store->n + m > kMaxKeys)
    return fail(FATHOM_ERR_UNSUPPORTED, "n + m = %lld above %lld", static_cast<long long>(store->n + m),
                static_cast<long long>(kMaxKeys));
  if (stride_token < kD) return fail(FATHOM_ERR_INVALID_ARG, "stride_token must be >= d");
  if (store->num_kv_heads > 1 && stride_head < int64_t(m) * stride_token)
    return fail(FATHOM_ERR_INVALID_ARG, "stride_head must be >= m * stride_token");
  if (!aligned(keys, 4) || !aligned(planes, 16) || !aligned(lo, 4) || !aligned(step, 4))
    return fail(FATHOM_ERR_INVALID_ARG, "keys, lo and step must be 4-byte aligned, planes 16-byte aligned");
  hipError_t e = launch_append(keys, stride_head, stride_token, m, store->num_kv_heads, store->n, store->lengths,
                               store->ldw, planes, lo, step, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "fathom_append_keys launch");
  return ok();
}

int fathom_allocate(const float* q, int32_t num_q, int32_t group, const float* var,
                    const fathom_store_desc* store, int32_t budget_bits, uint8_t* alloc,
                    void* hip_stream) {
  int st = check_store(store);
  if (st != FATHOM_OK) return st;
  if (!q || !var || !alloc) return fail(FATHOM_ERR_INVALID_ARG, "q, var and alloc must be non-NULL");
  if (num_q < 1 || group < 1) return fail(FATHOM_ERR_INVALID_ARG, "num_q and group must be >= 1");
  if (static_cast<int64_t>(store->num_kv_heads) * group != num_q)
    return fail(FATHOM_ERR_INVALID_ARG, "num_q = %d must equal num_kv_heads (%d) * group (%d)", num_q,
                store->num_kv_heads, group);
  if (budget_bits < 0 || budget_bits > kPlanes * kD)
    return fail(FATHOM_ERR_INVALID_ARG, "budget_bits = %d outside [0, %d]", budget_bits, kPlanes * kD);
  if (!aligned(q, 8) || !aligned(var, 8) || !aligned(alloc, 2))
    return fail(FATHOM_ERR_INVALID_ARG, "q and var must be 8-byte aligned, alloc 2-byte aligned");
  hipError_t e = launch_allocate(q, num_q, group, var, budget_bits, alloc, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "fathom_allocate launch");
  return ok();
}

int fathom_control_allocate(const float* q, int32_t num_q, int32_t mode, int32_t budget_bits, uint8_t* alloc,
                            void* hip_stream) {
  if (!q || !alloc) return fail(FATHOM_ERR_INVALID_ARG, "q and alloc must be non-NULL");
  if (num_q < 1) return fail(FATHOM_ERR_INVALID_ARG, "num_q must be >= 1");
  if (mode != FATHOM_CONTROL_UNIFORM && mode != FATHOM_CONTROL_TOP_CHANNELS)
    return fail(FATHOM_ERR_INVALID_ARG, "unknown control mode %d", mode);
  if (budget_bits < 0 || budget_bits > kPlanes * kD)
    return fail(FATHOM_ERR_INVALID_ARG, "budget_bits = %d outside [0, %d]", budget_bits, kPlanes * kD);
  if (!aligned(q, 8) || !aligned(alloc, 2))
    return fail(FATHOM_ERR_INVALID_ARG, "q must be 8-byte aligned, alloc 2-byte aligned");
  hipError_t e = launch_control_allocate(q, num_q, mode, budget_bits, alloc, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "fathom_control_allocate launch");
  return ok();
}

int fathom_scan_topk(const uint32_t* planes, const float* lo, const float* step,
                     const fathom_store_desc* store, const float* q, const uint8_t* alloc,
                     int32_t num_q, int32_t group, int32_t k, int32_t* out_idx, float* out_score,
                     float* all_scores, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return scan_impl("fathom_scan_topk launch", planes, lo, step, store, q, alloc, num_q, group, k, out_idx,
                   out_score, all_scores, workspace, workspace_bytes, hip_stream, nullptr, 0, nullptr);
}

int fathom_allocate_scan_topk(const uint32_t* planes, const float* lo, const float* step, const float* var,
                              const fathom_store_desc* store, const float* q, int32_t num_q, int32_t group,
                              int32_t budget_bits, int32_t k, uint8_t* alloc, int32_t* out_idx,
                              float* out_score, void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!var) return fail(FATHOM_ERR_INVALID_ARG, "var must be non-NULL");
  return scan_impl("fathom_allocate_scan_topk launch", planes, lo, step, store, q, nullptr, num_q, group, k,
                   out_idx, out_score, nullptr, workspace, workspace_bytes, hip_stream, var, budget_bits, alloc);
}

int fathom_allocate_scan_topk_noalloc(const uint32_t* planes, const float* lo, const float* step, const float* var,
                                      const fathom_store_desc* store, const float* q, int32_t num_q, int32_t group,
                                      int32_t budget_bits, int32_t k, uint8_t* alloc, int32_t* out_idx,
                                      float* out_score, void* hip_stream) {
  if (!var) return fail(FATHOM_ERR_INVALID_ARG, "var must be non-NULL");
  if (num_q < 1 || num_q > FATHOM_NOALLOC_MAX_Q)
    return fail(FATHOM_ERR_UNSUPPORTED, "num_q = %d outside [1, %d] for the allocation-free call", num_q,
                FATHOM_NOALLOC_MAX_Q);
  if (!store || k < 1 || k > kMaxK) return fail(FATHOM_ERR_INVALID_ARG, "store must be non-NULL and 1 <= k <= %d", kMaxK);
  const size_t need = scan_layout(num_q, store->n, k).total;
  if (need > FATHOM_NOALLOC_SCRATCH_BYTES)
    return fail(FATHOM_ERR_UNSUPPORTED, "the call needs %zu scratch bytes, above the static %d", need,
                FATHOM_NOALLOC_SCRATCH_BYTES);
  int device = -1;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (device < 0 || device >= kMaxDevices) return fail(FATHOM_ERR_UNSUPPORTED, "device %d above %d", device, kMaxDevices);
  void* ptr = nullptr;
  {
    // set-up, once per device with that device current: the array's device
    // address (each GPU holds its own copy at its own address)
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      if (!p || !aligned(p, 256)) return fail(FATHOM_ERR_HIP, "static scratch has no 256-byte aligned address");
      g_scratch_ptr[device] = p;
    }
    ptr = g_scratch_ptr[device];
  }
  return scan_impl("fathom_allocate_scan_topk_noalloc launch", planes, lo, step, store, q, nullptr, num_q, group,
                   k, out_idx, out_score, nullptr, ptr, FATHOM_NOALLOC_SCRATCH_BYTES, hip_stream, var, budget_bits,
                   alloc);
}

int fathom_allocate_scan_topk_staged(const uint32_t* planes_host, const float* lo, const float* step,
                                     const float* var, const fathom_store_desc* store, const float* q, int32_t num_q,
                                     int32_t group, int32_t budget_bits, int32_t k, uint8_t* alloc, int32_t* out_idx,
                                     float* out_score, uint32_t* staging, size_t staging_bytes, void* workspace,
                                     size_t workspace_bytes, int32_t mode, void* hip_stream, void* copy_stream) {
  int st = check_store(store);
  if (st != FATHOM_OK) return st;
  if (!planes_host || !lo || !step || !var || !q || !alloc || !out_idx || !out_score || !staging)
    return fail(FATHOM_ERR_INVALID_ARG, "pointers must be non-NULL");
  if (mode != FATHOM_STAGE_COPY_ENGINE && mode != FATHOM_STAGE_GATHER)
    return fail(FATHOM_ERR_INVALID_ARG, "unknown staging mode %d", mode);
  if (num_q < 1 || group < 1) return fail(FATHOM_ERR_INVALID_ARG, "num_q and group must be >= 1");
  if (static_cast<int64_t>(store->num_kv_heads) * group != num_q)
    return fail(FATHOM_ERR_INVALID_ARG, "num_q = %d must equal num_kv_heads (%d) * group (%d)", num_q,
                store->num_kv_heads, group);
  if (budget_bits < 0 || budget_bits > kPlanes * kD)
    return fail(FATHOM_ERR_INVALID_ARG, "budget_bits = %d outside [0, %d]", budget_bits, kPlanes * kD);
  if (k < 1 || k > store->n) return fail(FATHOM_ERR_INVALID_ARG, "k = %d outside [1, n]", k);
  if (k > FATHOM_MAX_K) return fail(FATHOM_ERR_UNSUPPORTED, "k = %d exceeds FATHOM_MAX_K (%d)", k, FATHOM_MAX_K);
  if (!aligned(q, 8) || !aligned(var, 8) || !aligned(alloc, 2) || !aligned(planes_host, 16) ||
      !aligned(staging, 256) || !aligned(lo, 4) || !aligned(step, 4) || !aligned(out_idx, 4) ||
      !aligned(out_score, 4))
    return fail(FATHOM_ERR_INVALID_ARG, "misaligned pointer (q, var 8; alloc 2; planes 16; staging 256 bytes)");
  const int64_t head_words = int64_t(kD) * kPlanes * store->ldw;
  if (staging_bytes < size_t(2 * head_words * 4))
    return fail(FATHOM_ERR_WORKSPACE, "staging needs two head blocks: %lld bytes (got %zu)",
                static_cast<long long>(2 * head_words * 4), staging_bytes);
  const ScanLayout L = scan_layout(group, store->n, k);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < L.total)
    return fail(FATHOM_ERR_WORKSPACE, "staged scan needs a 256-byte aligned workspace of %zu bytes (got %zu)",
                L.total, workspace_bytes);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipStream_t cstream = static_cast<hipStream_t>(copy_stream);
  const uint32_t* planes_dev = nullptr;   // device view of the pinned store (gather mode)
  if (mode == FATHOM_STAGE_GATHER) {
    void* dp = nullptr;
    hipError_t e = hipHostGetDevicePointer(&dp, const_cast<uint32_t*>(planes_host), 0);
    if (e != hipSuccess) return hip_fail(e, "hipHostGetDevicePointer (planes_host must be pinned host memory)");
    planes_dev = static_cast<const uint32_t*>(dp);
  }
  // events (ready, freed) per staging slot and one for the allocation,
  // created once
  {
    std::lock_guard<std::mutex> lock(g_staged_mu);
    for (int i = 0; i < 5; ++i) {
      if (g_staged_events[i]) continue;
      hipError_t e = hipEventCreateWithFlags(&g_staged_events[i], hipEventDisableTiming);
      if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
    }
  }
  hipEvent_t* ready = &g_staged_events[0];
  hipEvent_t* freed = &g_staged_events[2];
  hipEvent_t ev_alloc = g_staged_events[4];
  // 1. the allocation
  hipError_t e = launch_allocate(q, num_q, group, var, budget_bits, alloc, stream);
  if (e != hipSuccess) return hip_fail(e, "fathom_allocate_scan_topk_staged allocate launch");
  std::vector<uint8_t> alloc_h;
  if (mode == FATHOM_STAGE_COPY_ENGINE) {
    // the copy commands need the union on the host: this thread waits
    alloc_h.resize(size_t(num_q) * kD);
    e = hipMemcpyAsync(alloc_h.data(), alloc, alloc_h.size(), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "allocation readback");
  } else {
    e = hipEventRecord(ev_alloc, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(cstream, ev_alloc, 0);
    if (e != hipSuccess) return hip_fail(e, "allocation event");
  }
  char* w = static_cast<char*>(workspace);
  ScanWorkspace ws{reinterpret_cast<float*>(w + L.theta), reinterpret_cast<uint32_t*>(w + L.count),
                   reinterpret_cast<float*>(w + L.sample), reinterpret_cast<uint2*>(w + L.cand),
                   static_cast<void*>(w + L.tables), reinterpret_cast<uint2*>(w + L.rescue),
                   reinterpret_cast<uint2*>(w + L.rescue_cnt), reinterpret_cast<uint32_t*>(w + L.rescue_hist),
                   reinterpret_cast<uint32_t*>(w + L.rescue_done), L.rescue_wgs};
  // copy-engine mode: a copy costs a fixed ~11 us besides its bytes (about
  // 640 KB at the link's rate), so two runs are joined when the rows between
  // them cost less than that
  const int64_t join_rows = std::max<int64_t>(0, (int64_t(640) << 10) / (store->ldw * 4));
  for (int h = 0; h < store->num_kv_heads; ++h) {
    const int slot = h & 1;
    uint32_t* dst_head = staging + slot * head_words;
    // 2. wait until the scan that last read the slot (two heads back, or the
    // previous call's) has finished
    e = hipStreamWaitEvent(cstream, freed[slot], 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent (slot free)");
    if (mode == FATHOM_STAGE_GATHER) {
      e = launch_stage_union(planes_dev + int64_t(h) * head_words, dst_head, alloc + int64_t(h) * group * kD, group,
                             store->ldw, cstream);
      if (e != hipSuccess) return hip_fail(e, "stage_union launch");
    } else {
      // the head's union runs: rows j < u_c of channel c are contiguous, and
      // so are consecutive channels while u_c = 4
      const uint32_t* src_head = planes_host + int64_t(h) * head_words;
      int64_t run_lo = -1, run_hi = -1;   // rows [run_lo, run_hi)
      auto flush = [&]() -> hipError_t {
        if (run_hi <= run_lo) return hipSuccess;
        return hipMemcpyAsync(dst_head + run_lo * store->ldw, src_head + run_lo * store->ldw,
                              size_t((run_hi - run_lo) * store->ldw * 4), hipMemcpyHostToDevice, cstream);
      };
      for (int c = 0; c < kD && e == hipSuccess; ++c) {
        int u = 0;
        for (int g = 0; g < group; ++g)
          u = std::max<int>(u, std::min<int>(alloc_h[size_t(h * group + g) * kD + c], kPlanes));
        if (u == 0) continue;
        const int64_t lo_row = int64_t(c) * kPlanes;
        if (run_hi >= 0 && lo_row - run_hi <= join_rows) {
          run_hi = lo_row + u;   // joins the run (with the rows between)
        } else {
          e = flush();
          run_lo = lo_row;
          run_hi = lo_row + u;
        }
      }
      if (e == hipSuccess) e = flush();
      if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (union run)");
    }
    e = hipEventRecord(ready[slot], cstream);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, ready[slot], 0);
    if (e != hipSuccess) return hip_fail(e, "staging events");
    // 3. the head's scan from the staged slot
    e = launch_scan_topk(dst_head, lo + int64_t(h) * kD, step + int64_t(h) * kD, 1, store->n,
                         store->lengths ? store->lengths + h : nullptr, store->ldw, q + int64_t(h) * group * kD,
                         alloc + int64_t(h) * group * kD, group, group, k, out_idx + int64_t(h) * group * k,
                         out_score + int64_t(h) * group * k, nullptr, ws, nullptr, stream);
    if (e != hipSuccess) return hip_fail(e, "fathom_allocate_scan_topk_staged scan launch");
    e = hipEventRecord(freed[slot], stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord (slot free)");
  }
  return ok();
}

int fathom_sparse_attention(const uint16_t* k_rows, const uint16_t* v_rows, int64_t stride_head,
                            int64_t stride_token, const fathom_store_desc* store, const float* q,
                            const int32_t* idx, int32_t num_q, int32_t group, int32_t k, float scale,
                            float* out, void* workspace, size_t workspace_bytes, void* hip_stream) {
  int st = check_store(store);
  if (st != FATHOM_OK) return st;
  if (!k_rows || !v_rows || !q || !idx || !out)
    return fail(FATHOM_ERR_INVALID_ARG, "k_rows, v_rows, q, idx and out must be non-NULL");
  if (num_q < 1 || group < 1) return fail(FATHOM_ERR_INVALID_ARG, "num_q and group must be >= 1");
  if (static_cast<int64_t>(store->num_kv_heads) * group != num_q)
    return fail(FATHOM_ERR_INVALID_ARG, "num_q = %d must equal num_kv_heads (%d) * group (%d)", num_q,
                store->num_kv_heads, group);
  if (k < 1 || k > store->n) return fail(FATHOM_ERR_INVALID_ARG, "k = %d outside [1, n]", k);
  if (k > kMaxK) return fail(FATHOM_ERR_UNSUPPORTED, "k = %d above %d", k, kMaxK);
  if (!std::isfinite(scale)) return fail(FATHOM_ERR_INVALID_ARG, "scale must be finite");
  if (!aligned(k_rows, 16) || !aligned(v_rows, 16))
    return fail(FATHOM_ERR_INVALID_ARG, "k_rows and v_rows must be 16-byte aligned");
  if (stride_token < kD || stride_token % 8 != 0)
    return fail(FATHOM_ERR_INVALID_ARG, "stride_token must be >= d and a multiple of 8");
  if (store->num_kv_heads > 1 && (stride_head < store->n * stride_token || stride_head % 8 != 0))
    return fail(FATHOM_ERR_INVALID_ARG, "stride_head must be >= n * stride_token and a multiple of 8");
  if (!aligned(q, 4) || !aligned(idx, 4) || !aligned(out, 4))
    return fail(FATHOM_ERR_INVALID_ARG, "q, idx and out must be 4-byte aligned");
  const size_t need = attend_bytes(num_q, k);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need)
    return fail(FATHOM_ERR_WORKSPACE, "attention needs a 256-byte aligned workspace of %zu bytes (got %zu)", need,
                workspace_bytes);
  hipError_t e = launch_attend(k_rows, v_rows, stride_head, stride_token, store->n, store->lengths, q, idx, num_q,
                               group, k, scale,
                               static_cast<float*>(workspace), out, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "fathom_sparse_attention launch");
  return ok();
}

int fathom_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* hip_stream) {
  if (!src || !sink) return fail(FATHOM_ERR_INVALID_ARG, "src and sink must be non-NULL");
  if (bytes < 16 || bytes % 16 != 0) return fail(FATHOM_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  if (!aligned(src, 16) || !aligned(sink, 4)) return fail(FATHOM_ERR_INVALID_ARG, "src must be 16-byte aligned");
  hipError_t e = launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "fathom_stream_read launch");
  return ok();
}

int32_t fathom_stream_read_sink_words(void) { return stream_read_blocks(); }

int fathom_host_device_pointer(void* pinned_host, void** device_ptr) {
  if (!pinned_host || !device_ptr) return fail(FATHOM_ERR_INVALID_ARG, "pointers must be non-NULL");
  hipError_t e = hipHostGetDevicePointer(device_ptr, pinned_host, 0);
  if (e != hipSuccess) return hip_fail(e, "hipHostGetDevicePointer");
  return ok();
}

const char* fathom_status_string(int32_t status) {
  switch (status) {
    case FATHOM_OK: return "ok";
    case FATHOM_ERR_INVALID_ARG: return "invalid argument";
    case FATHOM_ERR_UNSUPPORTED: return "unsupported";
    case FATHOM_ERR_WORKSPACE: return "workspace missing or too small";
    case FATHOM_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* fathom_last_error(void) { return g_last_error; }

int fathom_timing_enable(int32_t enable) {
  std::lock_guard<std::mutex> lock(g_timing_mu);
  if (enable && g_events.empty()) {
    g_events.reserve(kMaxTimed);
    for (size_t i = 0; i < kMaxTimed; ++i) {
      hipEvent_t a = nullptr, b = nullptr;
      hipError_t e = hipEventCreate(&a);
      if (e == hipSuccess) e = hipEventCreate(&b);
      if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
      g_events.emplace_back(a, b);
    }
  }
  g_timing_on = enable != 0;
  return ok();
}

int fathom_timing_read(double* total_ms, int32_t* launches) {
  if (!total_ms || !launches) return fail(FATHOM_ERR_INVALID_ARG, "outputs must be non-NULL");
  std::lock_guard<std::mutex> lock(g_timing_mu);
  double sum = 0.0;
  for (size_t i = 0; i < g_events_used; ++i) {
    hipError_t e = hipEventSynchronize(g_events[i].second);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, g_events[i].first, g_events[i].second);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    sum += ms;
  }
  *total_ms = sum;
  *launches = static_cast<int32_t>(g_events_used);
  g_events_used = 0;
  return ok();
}

}  // extern "C"
