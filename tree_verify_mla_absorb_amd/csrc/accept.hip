// Greedy acceptance of verified draft trees, alone or fused with KV compaction, for gfx950.
//
// The walk (accept_walk.h) follows "The Microsecond Verdict: Validating a DDTree Kernel Fix Under
// Time Pressure", sections "The Crash That Demanded a Fix" and "What Was Learned".  The fused
// kernel then moves the accepted rows to the front of the tree block with the race-free gather
// of compact_rows.h, in the same launch.

#include "accept_walk.h"
#include "compact_rows.h"
#include "kernels.h"

#include "../../include/ddtree.h"

namespace ddtree {
namespace {

__device__ __forceinline__ void write_outputs(const AcceptArgs& a, int s, int lane, const Walk& w) {
  write_walk(w, lane, a.keep + (size_t)s * a.keep_stride, a.n_keep + s,
             a.next_token == nullptr ? nullptr : a.next_token + s, a.status);
}

// One wave per stream.
__global__ void __launch_bounds__(64) tree_accept_kernel(AcceptArgs a) {
  const int s = blockIdx.x;
  const int lane = threadIdx.x;
  const Walk w = accept_walk(a.parents, a.draft, a.target, a.q_len, s, lane);
  write_outputs(a, s, lane, w);
}

// One workgroup per stream: wave 0 walks, then all waves gather the accepted rows.  With
// per-stream prefix lengths, the stream's entry is then advanced by the accepted count: the
// accepted rows are committed, and the next tree goes after them.
__global__ void __launch_bounds__(kCompactThreads) accept_compact_kernel(AcceptArgs a) {
  __shared__ int keep_s[kMaxQ];
  __shared__ int n_s, first_s;
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int P = a.prefix_lens != nullptr ? a.prefix_lens[s] : a.prefix_len;
  if (tid < 64) {
    const Walk w = accept_walk(a.parents, a.draft, a.target, a.q_len, s, tid);
    write_outputs(a, s, tid, w);
    if (tid < w.n) keep_s[tid] = w.my_node;
    const int first = rows_in_place(w.my_node, tid, w.n);
    if (tid == 0) {
      n_s = w.n;
      first_s = first;
    }
  }
  __syncthreads();
  const int n = n_s;
  if (n == 0) return;  // malformed tree: the cache is left untouched
  if (P < 0 || (long long)P + a.q_len > (long long)a.kv_rows) {  // uniform over the workgroup
    if (tid == 0 && a.status != nullptr) atomicOr(a.status, DDTREE_STATUS_BAD_PREFIX);
    return;
  }
  compact_rows(a.ckv, a.kpe, (size_t)s * a.kv_rows + P, keep_s, first_s, n);
  if (a.prefix_lens != nullptr && tid == 0) a.prefix_lens[s] = P + n;
}

}  // namespace

hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<AcceptArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(tree_accept_kernel), dim3((unsigned)a.n_streams), dim3(64),
                         args, 0, stream);
}

hipError_t launch_accept_compact(const AcceptArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<AcceptArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(accept_compact_kernel), dim3((unsigned)a.n_streams),
                         dim3(kCompactThreads), args, 0, stream);
}

}  // namespace ddtree
