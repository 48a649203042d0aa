// Post-accept KV cache compaction for gfx950: validation of keep / n_keep, then the race-free
// gather of compact_rows.h.

#include "compact_rows.h"
#include "kernels.h"

#include "../../include/ddtree.h"

namespace ddtree {
namespace {

__global__ void __launch_bounds__(kCompactThreads) compact_kv_kernel(CompactArgs a) {
  __shared__ int keep_s[kMaxQ];
  __shared__ int bad_s, first_s;
  const int s = blockIdx.x;
  const int P = a.prefix_lens != nullptr ? a.prefix_lens[s] : a.prefix_len;
  const int n = a.n_keep[s];
  const int why = load_keep(a.keep + (size_t)s * a.keep_stride, n, a.keep_stride, P, a.kv_rows, keep_s, &bad_s,
                            &first_s);
  if (why != 0) {
    if (threadIdx.x == 0 && a.status != nullptr) atomicOr(a.status, why);
    return;
  }
  compact_rows(a.ckv, a.kpe, (size_t)s * a.kv_rows + P, keep_s, first_s, n);
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<CompactArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(compact_kv_kernel), dim3((unsigned)a.n_streams),
                         dim3(kCompactThreads), args, 0, stream);
}

}  // namespace ddtree
