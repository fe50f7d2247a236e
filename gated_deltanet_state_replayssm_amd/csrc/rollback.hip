// Pointer-only rollback: commit the accepted prefix of the last appended draft.
//
// "The inference stack behind OCRia" (LlamaIndex), section "Making speculative
// verification cheaper": on rejection only the buffer pointer moves, keeping
// the accepted prefix, so no state is restored. The draft was appended behind
// the committed window by verify, so committing a tokens is len += a.
#include "device_common.h"
#include "internal.h"

namespace gdnr {

namespace {

__global__ __launch_bounds__(256) void rollback_kernel(RollbackArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.num_reqs) return;
  const CacheView &c = a.c;
  const int s = a.slot_idx[i];
  if (s < 0 || s >= c.num_slots) {
    raise_err(c.err, GDN_DERR_SLOT);
    return;
  }
  const int head = c.head[s], n = c.len[s];
  if (head < 0 || head >= c.cap || n < 0 || n > c.cap) {
    raise_err(c.err, GDN_DERR_POINTER);
    return;
  }
  const int D = request_draft(a.draft_lens, i, a.draft);
  if (D < 0) {
    raise_err(c.err, GDN_DERR_DRAFT);
    return;
  }
  const int acc = a.num_accepted[i];
  if (acc < 0 || acc > D) {
    raise_err(c.err, GDN_DERR_ACCEPT);
    return;
  }
  if (n + acc > c.cap) {
    raise_err(c.err, GDN_DERR_CAPACITY);
    return;
  }
  c.len[s] = n + acc;
}

}  // namespace

hipError_t launch_rollback(const RollbackArgs &a, hipStream_t stream) {
  const int block = 256;
  dim3 grid((a.num_reqs + block - 1) / block);
  hipLaunchKernelGGL(rollback_kernel, grid, dim3(block), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdnr
