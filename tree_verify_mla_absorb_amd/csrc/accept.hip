// Greedy acceptance of verified draft trees, alone or fused with KV compaction, for gfx950.
//
// "The Microsecond Verdict: Validating a DDTree Kernel Fix Under Time Pressure", sections "The
// Crash That Demanded a Fix" and "What Was Learned": tree_accept walks the accepted path from the
// root -- the longest run on which drafter and target agree -- and records it, with the walk
// capped at q_len nodes.  Rule: from the current node c the walk moves to the lowest-index child
// j (parents[j] == c) whose draft token equals the target's token at c, and stops when no child
// matches; its outputs are the path, its length, and the target's token at the last node.
//
// A tree holds at most 64 nodes, so one wave holds the whole tree, node j in lane j.  Each level
// of the walk is one wave-wide ballot over (parents[j] == c && draft[j] == target[c]); the lowest
// set bit is the accepted child.  Child indices exceed their parent's (validated first), so the
// walk visits strictly increasing nodes and ends within q_len - 1 levels for any input.
//
// The fused kernel then moves the accepted rows to the front of the tree block with the
// race-free gather of compact_rows.h, in the same launch.

#include "compact_rows.h"
#include "kernels.h"

#include "../../include/ddtree.h"

namespace ddtree {
namespace {

struct Walk {
  int n;        // accepted nodes (0: malformed tree)
  int next;     // target token at the last accepted node (-1: malformed tree)
  int my_node;  // path[lane] for lane < n
};

// One wave; every lane calls it.  Reads row s of parents / draft / target.
__device__ __forceinline__ Walk accept_walk(const AcceptArgs& a, int s, int lane) {
  const int Q = a.q_len;
  const bool in = lane < Q;
  const size_t row = (size_t)s * Q + lane;
  const int p = in ? a.parents[row] : -2;
  const int d = in ? a.draft[row] : 0;
  const int tg = in ? a.target[row] : 0;
  const bool ok = !in || (lane == 0 ? p == -1 : (p >= 0 && p < lane));
  Walk w{0, -1, 0};
  if (__builtin_amdgcn_ballot_w64(!ok) != 0) return w;  // uniform
  int cur = 0, n = 1;
  for (int level = 1; level < Q; ++level) {
    const int tc = __shfl(tg, cur);
    const unsigned long long m = __builtin_amdgcn_ballot_w64(in && p == cur && d == tc);
    if (m == 0) break;
    cur = (int)__builtin_ctzll(m);
    if (lane == n) w.my_node = cur;
    ++n;
  }
  w.n = n;
  w.next = __shfl(tg, cur);
  return w;
}

__device__ __forceinline__ void write_outputs(const AcceptArgs& a, int s, int lane, const Walk& w) {
  if (lane < w.n) a.keep[(size_t)s * a.keep_stride + lane] = w.my_node;
  if (lane == 0) {
    a.n_keep[s] = w.n;
    if (a.next_token != nullptr) a.next_token[s] = w.next;
    if (w.n == 0 && a.status != nullptr) atomicOr(a.status, DDTREE_STATUS_BAD_PARENTS);
  }
}

// One wave per stream.
__global__ void __launch_bounds__(64) tree_accept_kernel(AcceptArgs a) {
  const int s = blockIdx.x;
  const int lane = threadIdx.x;
  const Walk w = accept_walk(a, s, lane);
  write_outputs(a, s, lane, w);
}

// One workgroup per stream: wave 0 walks, then all waves gather the accepted rows.  With
// per-stream prefix lengths, the stream's entry is then advanced by the accepted count: the
// accepted rows are committed, and the next tree goes after them.
__global__ void __launch_bounds__(kCompactThreads) accept_compact_kernel(AcceptArgs a) {
  __shared__ int keep_s[kMaxQ];
  __shared__ int n_s;
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int P = a.prefix_lens != nullptr ? a.prefix_lens[s] : a.prefix_len;
  if (tid < 64) {
    const Walk w = accept_walk(a, s, tid);
    write_outputs(a, s, tid, w);
    if (tid < w.n) keep_s[tid] = w.my_node;
    if (tid == 0) n_s = w.n;
  }
  __syncthreads();
  const int n = n_s;
  if (n == 0) return;  // malformed tree: the cache is left untouched
  if (P < 0 || (long long)P + a.q_len > (long long)a.kv_rows) {  // uniform over the workgroup
    if (tid == 0 && a.status != nullptr) atomicOr(a.status, DDTREE_STATUS_BAD_PREFIX);
    return;
  }
  compact_rows(a.ckv, a.kpe, (size_t)s * a.kv_rows + P, keep_s, n);
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
