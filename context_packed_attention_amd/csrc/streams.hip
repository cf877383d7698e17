// Side streams for running independent launches of one call concurrently
// (the backward of short shares runs its dK/dV launch beside its dQ launch):
// per calling thread and device, MAX_SIDE streams of default priority with a
// fork event and one join event each, created on first use and never
// released (a thread-exit hook could run after the HIP runtime has shut down
// at process exit; each thread that calls the library on a device holds
// MAX_SIDE streams and MAX_SIDE + 1 events there until the process ends). A
// fork is an event recorded on the caller's stream that the side streams wait
// on; a join records an event on every side stream that the caller's stream
// waits on (graph capture records the same pattern as a fork and a join).
#include <hip/hip_runtime.h>

#include <atomic>

#include "internal.h"

namespace cpattn {

namespace {
struct SideSetStore {
  SideSet set[64];
};
}  // namespace

cp_attn_status side_set(int device, SideSet** out) {
  static thread_local SideSetStore store;
  if (device < 0 || device >= 64) return fail(CP_ATTN_ERR_INVALID_ARG, "device index out of range");
  SideSet& ss = store.set[device];
  if (!ss.ready) {
    cp_attn_status rc = hip_check(hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming), "hipEventCreate(fork)");
    for (int i = 0; rc == CP_ATTN_OK && i < MAX_SIDE; ++i) {
      rc = hip_check(hipStreamCreateWithFlags(&ss.s[i], hipStreamNonBlocking), "hipStreamCreate(side)");
      if (rc == CP_ATTN_OK) rc = hip_check(hipEventCreateWithFlags(&ss.join[i], hipEventDisableTiming), "hipEventCreate(join)");
    }
    if (rc != CP_ATTN_OK) {
      if (ss.fork) (void)hipEventDestroy(ss.fork);
      for (int i = 0; i < MAX_SIDE; ++i) {
        if (ss.join[i]) (void)hipEventDestroy(ss.join[i]);
        if (ss.s[i]) (void)hipStreamDestroy(ss.s[i]);
      }
      ss = SideSet{};
      return rc;
    }
    ss.ready = true;
  }
  *out = &ss;
  return CP_ATTN_OK;
}

cp_attn_status fork_to(SideSet* ss, hipStream_t st, int n) {
  cp_attn_status rc = hip_check(hipEventRecord(ss->fork, st), "hipEventRecord(fork)");
  for (int i = 0; rc == CP_ATTN_OK && i < n; ++i) rc = hip_check(hipStreamWaitEvent(ss->s[i], ss->fork, 0), "hipStreamWaitEvent(fork)");
  return rc;
}

cp_attn_status join_from(SideSet* ss, hipStream_t st, int n) {
  cp_attn_status rc = CP_ATTN_OK;
  for (int i = 0; rc == CP_ATTN_OK && i < n; ++i) {
    rc = hip_check(hipEventRecord(ss->join[i], ss->s[i]), "hipEventRecord(join)");
    if (rc == CP_ATTN_OK) rc = hip_check(hipStreamWaitEvent(st, ss->join[i], 0), "hipStreamWaitEvent(join)");
  }
  return rc;
}

int cu_count(int device) {
  static std::atomic<int> cached[64] = {};
  if (device < 0 || device >= 64) return 256;
  int n = cached[device].load(std::memory_order_relaxed);
  if (!n) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || n <= 0) n = 256;
    cached[device].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool short_launches(long long max_blocks, int device) { return max_blocks < 4LL * 2 * cu_count(device); }

}  // namespace cpattn
