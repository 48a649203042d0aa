// Post-accept compaction of all layers' caches in one launch, for gfx950.
//
// "Race Conditions, Buffer Aliasing, and the Architecture of a Native DDTree Inference Engine":
// section "The Cache Compaction Problem" defines the gather of the accepted tree rows, and the
// closing section ("The Broader Significance") lists the fused compaction gather among the
// optimisations deferred for later.  Every layer keeps its own latent cache, and the same
// accepted path moves the same rows in each of them, so one step compacts as many caches as the
// model has layers.
//
// One workgroup per (stream, group of layers): it takes the stream's accepted path -- from the
// caller's keep / n_keep, or by walking the tree itself (accept_walk.h; each workgroup repeats
// the walk over 3 x q_len ints instead of synchronising the grid) -- and runs the race-free
// gather of compact_rows.h over its layers, as many per round trip as the registers hold (a
// path that moves m rows fits floor(18 / ceil(72 m / 256)) layers).  The workgroups of the
// first group write the acceptance outputs and the status bits.  Per-stream prefix lengths are
// advanced by a second, one-thread-per-stream launch: inside the first, other workgroups may
// still be reading a stream's entry.

#include "accept_walk.h"
#include "compact_rows.h"
#include "kernels.h"

#include "../../include/ddtree.h"

namespace ddtree {
namespace {

__device__ __forceinline__ int prefix_of(const LayersArgs& a, int s) {
  return a.prefix_lens != nullptr ? a.prefix_lens[s] : a.prefix_len;
}

// The caches of layers layer0, layer0 + 1, ... from the pointer tables.
struct TableCaches {
  const LayersArgs& a;
  int layer0;
  __device__ uint16_t* ckv(int g) const { return a.ckv[layer0 + g]; }
  __device__ uint16_t* kpe(int g) const { return a.kpe[layer0 + g]; }
};

// Rows [first, n) of stream s move in every layer of this workgroup's group.
__device__ __forceinline__ void gather_group(const LayersArgs& a, int s, int P, const int* keep_s, int first, int n) {
  const int m = n - first;
  if (m <= 0) return;
  const int slots = (m * kChunksRow + kCompactThreads - 1) / kCompactThreads;
  const int per_round = kCompactPerThread / slots;  // >= 1: m <= 64 needs at most 18 slots
  const int l_begin = blockIdx.y * a.layers_per_wg;
  const int l_end = min(a.n_layers, l_begin + a.layers_per_wg);
  for (int l = l_begin; l < l_end; l += per_round)  // rounds touch disjoint layers: no barrier between them
    gather_rows(TableCaches{a, l}, min(per_round, l_end - l), (size_t)s * a.kv_rows + P, keep_s, first, m);
}

__global__ void __launch_bounds__(kCompactThreads) compact_layers_kernel(LayersArgs a) {
  __shared__ int keep_s[kMaxQ];
  __shared__ int bad_s, first_s;
  const int s = blockIdx.x;
  const int P = prefix_of(a, s);
  const int n = a.n_keep[s];
  const int why =
      load_keep(a.keep + (size_t)s * a.keep_stride, n, a.keep_stride, P, a.kv_rows, keep_s, &bad_s, &first_s);
  if (why != 0) {
    if (blockIdx.y == 0 && threadIdx.x == 0 && a.status != nullptr) atomicOr(a.status, why);
    return;
  }
  gather_group(a, s, P, keep_s, first_s, n);
}

// A stream's rows move when its tree is well formed (n > 0) and its tree block lies inside the
// cache; the prefix advance below applies the same test.
__device__ __forceinline__ bool block_in_cache(int P, int q_len, int kv_rows) {
  return P >= 0 && (long long)P + q_len <= (long long)kv_rows;
}

__global__ void __launch_bounds__(kCompactThreads) accept_compact_layers_kernel(LayersArgs a) {
  __shared__ int keep_s[kMaxQ];
  __shared__ int n_s, first_s;
  const int s = blockIdx.x;
  const int tid = threadIdx.x;
  const int P = prefix_of(a, s);
  if (tid < 64) {
    const Walk w = accept_walk(a.parents, a.draft, a.target, a.q_len, s, tid);
    if (blockIdx.y == 0)
      write_walk(w, tid, a.keep + (size_t)s * a.keep_stride, a.n_keep + s,
                 a.next_token == nullptr ? nullptr : a.next_token + s, a.status);
    if (tid < w.n) keep_s[tid] = w.my_node;
    const int first = rows_in_place(w.my_node, tid, w.n);
    if (tid == 0) {
      n_s = w.n;
      first_s = first;
    }
  }
  __syncthreads();
  const int n = n_s;
  if (n == 0) return;  // malformed tree: the caches are left untouched
  if (!block_in_cache(P, a.q_len, a.kv_rows)) {  // uniform over the workgroup
    if (blockIdx.y == 0 && tid == 0 && a.status != nullptr) atomicOr(a.status, DDTREE_STATUS_BAD_PREFIX);
    return;
  }
  gather_group(a, s, P, keep_s, first_s, n);
}

__global__ void __launch_bounds__(256) advance_prefixes_kernel(int32_t* prefix_lens, const int32_t* n_keep,
                                                               int q_len, int kv_rows, int n_streams) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= n_streams) return;
  const int P = prefix_lens[s];
  const int n = n_keep[s];
  if (n > 0 && block_in_cache(P, q_len, kv_rows)) prefix_lens[s] = P + n;
}

int groups(const LayersArgs& a) { return (a.n_layers + a.layers_per_wg - 1) / a.layers_per_wg; }

}  // namespace

hipError_t launch_compact_layers(const LayersArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<LayersArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(compact_layers_kernel),
                         dim3((unsigned)a.n_streams, (unsigned)groups(a)), dim3(kCompactThreads), args, 0, stream);
}

hipError_t launch_accept_compact_layers(const LayersArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<LayersArgs*>(&a)};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(accept_compact_layers_kernel),
                                 dim3((unsigned)a.n_streams, (unsigned)groups(a)), dim3(kCompactThreads), args, 0,
                                 stream);
  if (e != hipSuccess || a.prefix_lens == nullptr) return e;
  int32_t* pl = a.prefix_lens;
  const int32_t* nk = a.n_keep;
  int q_len = a.q_len, kv_rows = a.kv_rows, n_streams = a.n_streams;
  void* args2[] = {&pl, &nk, &q_len, &kv_rows, &n_streams};
  return hipLaunchKernel(reinterpret_cast<const void*>(advance_prefixes_kernel),
                         dim3((unsigned)((a.n_streams + 255) / 256)), dim3(256), args2, 0, stream);
}

}  // namespace ddtree
