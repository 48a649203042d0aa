// Post-accept KV cache compaction for gfx950: validation of keep / n_keep, then the race-free
// gather of compact_rows.h.

#include "compact_rows.h"
#include "kernels.h"

#include "../../include/ddtree.h"

namespace ddtree {
namespace {

__global__ void __launch_bounds__(kCompactThreads) compact_kv_kernel(CompactArgs a) {
  __shared__ int keep_s[kMaxQ];
  __shared__ int bad_s;
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = a.n_keep[s];
  if (tid == 0) bad_s = 0;
  __syncthreads();
  if (n < 0 || n > a.keep_stride || n > kMaxQ) {  // uniform over the workgroup
    if (tid == 0 && a.status != nullptr) atomicOr(a.status, DDTREE_STATUS_BAD_KEEP);
    return;
  }
  const int P = a.prefix_lens != nullptr ? a.prefix_lens[s] : a.prefix_len;
  if (P < 0 || P > a.kv_rows) {  // uniform over the workgroup
    if (tid == 0 && a.status != nullptr) atomicOr(a.status, DDTREE_STATUS_BAD_PREFIX);
    return;
  }
  if (tid < n) {
    const int32_t* kp = a.keep + (size_t)s * a.keep_stride;
    const int k = kp[tid];
    bool ok = k >= 0 && (long long)P + k < (long long)a.kv_rows;
    if (tid > 0) ok = ok && kp[tid - 1] < k;
    keep_s[tid] = k;
    if (!ok) bad_s = 1;
  }
  __syncthreads();
  if (bad_s) {
    if (tid == 0 && a.status != nullptr) atomicOr(a.status, DDTREE_STATUS_BAD_KEEP);
    return;
  }

  compact_rows(a.ckv, a.kpe, (size_t)s * a.kv_rows + P, keep_s, n);
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<CompactArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(compact_kv_kernel), dim3((unsigned)a.n_streams),
                         dim3(kCompactThreads), args, 0, stream);
}

}  // namespace ddtree
