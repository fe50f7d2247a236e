// gdn_replay_rollback_verify_flush_noalloc: the one-call step for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops
// that must not allocate, harnesses that forbid it). The only scratch the step
// needs beyond its inputs and outputs is its array of arrival counters
// (gdn_replay_cache::sync); this entry point takes them from a library-owned
// device array instead of the caller's buffer.
//
// The array is a file-scope device variable: every GPU the library runs on
// holds one copy of it until the process ends. Host code never passes the
// variable's name to a kernel (on the host it is a stand-in, not a device
// address): the first call on a device, with that device current, looks up the
// device copy's address with hipGetSymbolAddress and keeps it per device, and
// every launch takes that address.
//
// The counters are zero when the code object is loaded, and every completed
// call leaves each counter it touched at zero (the last workgroup to count in
// resets it), so each call starts from zeros without a clearing launch. Calls
// on one GPU share the array: calls that overlap in time on one GPU (other
// streams, other threads) race on the counters and must not be issued.
#include <hip/hip_runtime.h>

#include <climits>
#include <mutex>

#include "internal.h"

namespace {

// int32 counters: 256 KiB per device
constexpr int64_t kScratchEntries = GDN_REPLAY_NOALLOC_SYNC_ENTRIES;

static __device__ __align__(256) int32_t scratch[kScratchEntries];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
int32_t *g_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

// Address of the current device's copy of `scratch`, looked up on its first
// use on that device; null on failure.
int32_t *scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = static_cast<int32_t *>(p);
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

int gdn_replay_rollback_verify_flush_noalloc(const gdn_replay_cache *c, int32_t num_reqs,
                                             const int32_t *slot_idx, const int32_t *num_accepted,
                                             const int32_t *prev_draft_lens, int32_t prev_draft,
                                             const int32_t *draft_lens, int32_t draft_len,
                                             int32_t min_len, const void *q, const void *k,
                                             const void *v, const float *alpha, const float *beta,
                                             float *out, hipStream_t stream) {
  if (!c) return GDN_EINVAL;
  // The caller's counter fields are ignored. Check every argument first with a
  // stand-in for the counters (never dereferenced: nothing is launched).
  gdn_replay_cache cc = *c;
  cc.sync = reinterpret_cast<int32_t *>(uintptr_t(256));
  cc.sync_len = INT32_MAX;
  int st = gdnr::rollback_verify_flush_call(&cc, num_reqs, slot_idx, num_accepted,
                                            prev_draft_lens, prev_draft, draft_lens, draft_len,
                                            min_len, q, k, v, alpha, beta, out, stream, true);
  if (st != GDN_OK || num_reqs == 0) return st;
  // the cache's counters must fit the library's array
  const int64_t need = gdnr::sync_entries(cc.num_slots, cc.num_k_heads);
  if (need > kScratchEntries) return GDN_EUNSUPPORTED;
  int32_t *ptr = scratch_of_current_device();
  if (!ptr) return GDN_EHIP;
  cc.sync = ptr;
  cc.sync_len = static_cast<int32_t>(kScratchEntries);
  return gdnr::rollback_verify_flush_call(&cc, num_reqs, slot_idx, num_accepted, prev_draft_lens,
                                          prev_draft, draft_lens, draft_len, min_len, q, k, v,
                                          alpha, beta, out, stream, false);
}

}  // extern "C"
