// Post-accept KV cache compaction for gfx950.
//
// "Race Conditions, Buffer Aliasing, and the Architecture of a Native DDTree Inference Engine",
// section "The Cache Compaction Problem": the accepted path's rows move from prefix + keep[i] to
// prefix + i.  Since the path is strictly increasing, keep[i] >= i, yet a parallel in-place
// gather still races: the thread copying row prefix + keep[j] can read a row that another
// thread i' = keep[j] is already overwriting.  The pages gather into scratch and copy back.
//
// Here one workgroup owns a stream and holds every kept row in registers (at most 64 rows x
// 1152 B, 18 x 16 B per thread) before any row is written: all reads complete, a workgroup
// barrier, then all writes.  No reader can observe a write, whatever the schedule, and no
// second pass over HBM is needed.  Rows with keep[i] == i (always the root) are skipped.

#include "kernels.h"

#include "../../include/ddtree.h"

namespace ddtree {
namespace {

constexpr int kChunksLat = kDLat * 2 / 16;    // 64 chunks of 16 B per latent row
constexpr int kChunksRope = kDRope * 2 / 16;  // 8 chunks per rotary row
constexpr int kChunksRow = kChunksLat + kChunksRope;
constexpr int kThreads = 256;
constexpr int kPerThread = (kMaxQ * kChunksRow + kThreads - 1) / kThreads;  // 18

__global__ void __launch_bounds__(kThreads) compact_kv_kernel(CompactArgs a) {
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
  if (tid < n) {
    const int32_t* kp = a.keep + (size_t)s * a.keep_stride;
    const int k = kp[tid];
    bool ok = k >= 0 && (long long)a.prefix_len + k < (long long)a.kv_rows;
    if (tid > 0) ok = ok && kp[tid - 1] < k;
    keep_s[tid] = k;
    if (!ok) bad_s = 1;
  }
  __syncthreads();
  if (bad_s) {
    if (tid == 0 && a.status != nullptr) atomicOr(a.status, DDTREE_STATUS_BAD_KEEP);
    return;
  }

  const size_t row0 = (size_t)s * a.kv_rows + a.prefix_len;
  uint4* ckv = reinterpret_cast<uint4*>(a.ckv);
  uint4* kpe = reinterpret_cast<uint4*>(a.kpe);
  const int total = n * kChunksRow;

  uint4 v[kPerThread];
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int c = tid + j * kThreads;
    if (c < total) {
      const int i = c / kChunksRow;
      const int part = c - i * kChunksRow;
      const int src = keep_s[i];
      if (src != i) {
        v[j] = part < kChunksLat ? ckv[(row0 + src) * kChunksLat + part]
                                 : kpe[(row0 + src) * kChunksRope + (part - kChunksLat)];
      }
    }
  }
  // Every kept row of this stream is now in registers; only then does anything get written.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int c = tid + j * kThreads;
    if (c < total) {
      const int i = c / kChunksRow;
      const int part = c - i * kChunksRow;
      if (keep_s[i] != i) {
        if (part < kChunksLat)
          ckv[(row0 + i) * kChunksLat + part] = v[j];
        else
          kpe[(row0 + i) * kChunksRope + (part - kChunksLat)] = v[j];
      }
    }
  }
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<CompactArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(compact_kv_kernel), dim3((unsigned)a.n_streams),
                         dim3(kThreads), args, 0, stream);
}

}  // namespace ddtree
