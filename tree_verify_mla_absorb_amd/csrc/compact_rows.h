// The race-free in-place row gather shared by the compaction kernels.
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
#pragma once

#include "kernels.h"

#include "../../include/ddtree.h"

namespace ddtree {

constexpr int kCompactThreads = 256;
constexpr int kChunksLat = kDLat * 2 / 16;    // 64 chunks of 16 B per latent row
constexpr int kChunksRope = kDRope * 2 / 16;  // 8 chunks per rotary row
constexpr int kChunksRow = kChunksLat + kChunksRope;
constexpr int kCompactPerThread = (kMaxQ * kChunksRow + kCompactThreads - 1) / kCompactThreads;  // 18

// 16-byte chunk as a native vector: an array of these stays in VGPRs (HIP's uint4 is a struct
// with a union, which keeps the array below in scratch memory and serialises its loads).
typedef unsigned int Chunk16 __attribute__((ext_vector_type(4)));

// Moves rows row0 + keep_s[i] to row0 + i for i < n (n <= kMaxQ, keep_s strictly increasing, in
// LDS and visible to every thread).  Called by all kCompactThreads threads of the workgroup.
__device__ __forceinline__ void compact_rows(uint16_t* ckv16, uint16_t* kpe16, size_t row0, const int* keep_s, int n) {
  const int tid = threadIdx.x;
  Chunk16* ckv = reinterpret_cast<Chunk16*>(ckv16);
  Chunk16* kpe = reinterpret_cast<Chunk16*>(kpe16);
  const int total = n * kChunksRow;
  Chunk16 v[kCompactPerThread];
#pragma unroll
  for (int j = 0; j < kCompactPerThread; ++j) {
    const int c = tid + j * kCompactThreads;
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
  for (int j = 0; j < kCompactPerThread; ++j) {
    const int c = tid + j * kCompactThreads;
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

// Reads a caller-given keep row (n entries) into keep_s and checks it against the stream's prefix
// P: n in [0, min(keep_stride, kMaxQ)], P in [0, kv_rows], entries strictly increasing, first
// >= 0, last row P + keep[n-1] < kv_rows.  Returns 0 when the gather may run, else the status
// bit that says why not.  Called by every thread of the workgroup with the same n and P; the
// result is uniform.  bad_s is a workgroup-shared int.
__device__ __forceinline__ int load_keep(const int32_t* keep_row, int n, int keep_stride, int P, int kv_rows,
                                         int* keep_s, int* bad_s) {
  const int tid = threadIdx.x;
  if (n < 0 || n > keep_stride || n > kMaxQ) return DDTREE_STATUS_BAD_KEEP;
  if (P < 0 || P > kv_rows) return DDTREE_STATUS_BAD_PREFIX;
  if (tid == 0) *bad_s = 0;
  __syncthreads();
  if (tid < n) {
    const int k = keep_row[tid];
    bool ok = k >= 0 && (long long)P + k < (long long)kv_rows;
    if (tid > 0) ok = ok && keep_row[tid - 1] < k;
    keep_s[tid] = k;
    if (!ok) *bad_s = 1;
  }
  __syncthreads();
  return *bad_s ? DDTREE_STATUS_BAD_KEEP : 0;
}

}  // namespace ddtree
