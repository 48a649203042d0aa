// The race-free in-place row gather shared by the compaction kernels.
//
// "Race Conditions, Buffer Aliasing, and the Architecture of a Native DDTree Inference Engine",
// section "The Cache Compaction Problem": the accepted path's rows move from prefix + keep[i] to
// prefix + i.  Since the path is strictly increasing, keep[i] >= i, yet a parallel in-place
// gather still races: the thread copying row prefix + keep[j] can read a row that another
// thread i' = keep[j] is already overwriting.  The pages gather into scratch and copy back.
//
// Here one workgroup owns a stream (in one or more caches) and holds every moved row in registers
// (at most 64 rows x 1152 B, 18 x 16 B per thread) before any row is written: all reads complete,
// a workgroup barrier, then all writes.  No reader can observe a write, whatever the schedule,
// and no second pass over HBM is needed.  Rows with keep[i] == i (always the root, and only ever
// a leading run) are skipped, so a short accepted path also moves few bytes; the registers that
// a long path would need then hold the rows of several caches (model layers) at once.
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

// Moves rows of G caches at once: in cache g (caches.ckv(g) / caches.kpe(g)), row
// row0 + keep_s[first + r] goes to row0 + first + r for r < m.  keep_s is in LDS, visible to every
// thread, strictly increasing, and keep_s[i] == i for i < first (those rows stay).  Each cache's
// m * 72 chunks of 16 B take `slots` = ceil(m * 72 / 256) register slots per thread, and
// G * slots <= kCompactPerThread; the cache of a slot is the same for the whole workgroup, so its
// pointers are uniform.  Called by all kCompactThreads threads of the workgroup.
template <class Caches>
__device__ __forceinline__ void gather_rows(const Caches& caches, int G, size_t row0, const int* keep_s, int first,
                                            int m) {
  // Opaque copies, so that a caller's loop over rounds of caches does not hoist the per-slot
  // index work out of the loop and hold it in registers across all rounds.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int per_cache = m * kChunksRow;
  int slots = (per_cache + kCompactThreads - 1) / kCompactThreads;
  asm volatile("" : "+s"(slots));
  Chunk16 v[kCompactPerThread];
  {
    int g = 0, j = 0;  // uniform: the cache and the slot within it of register slot jj
#pragma unroll
    for (int jj = 0; jj < kCompactPerThread; ++jj) {
      const int c = tid + j * kCompactThreads;
      if (g < G && c < per_cache) {
        const int r = c / kChunksRow;
        const int part = c - r * kChunksRow;
        const size_t src = row0 + keep_s[first + r];
        v[jj] = part < kChunksLat ? reinterpret_cast<const Chunk16*>(caches.ckv(g))[src * kChunksLat + part]
                                  : reinterpret_cast<const Chunk16*>(caches.kpe(g))[src * kChunksRope + (part - kChunksLat)];
      }
      if (++j == slots) {
        j = 0;
        ++g;
      }
    }
  }
  // Every moved row of these caches is now in registers; only then does anything get written.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  // The store addresses are recomputed rather than kept from the loads: holding 18 slots'
  // indices across the barrier would cost more registers (and occupancy) than recomputing them.
  int tid2 = tid;
  asm volatile("" : "+v"(tid2));
  int g = 0, j = 0;
#pragma unroll
  for (int jj = 0; jj < kCompactPerThread; ++jj) {
    const int c = tid2 + j * kCompactThreads;
    if (g < G && c < per_cache) {
      const int r = c / kChunksRow;
      const int part = c - r * kChunksRow;
      const size_t dst = row0 + first + r;
      if (part < kChunksLat)
        reinterpret_cast<Chunk16*>(caches.ckv(g))[dst * kChunksLat + part] = v[jj];
      else
        reinterpret_cast<Chunk16*>(caches.kpe(g))[dst * kChunksRope + (part - kChunksLat)] = v[jj];
    }
    if (++j == slots) {
      j = 0;
      ++g;
    }
  }
}

// Caches: a single one.
struct OneCache {
  uint16_t* c;
  uint16_t* k;
  __device__ uint16_t* ckv(int) const { return c; }
  __device__ uint16_t* kpe(int) const { return k; }
};

// The leading rows of keep_s[0..n) that stay in place (keep_s[i] == i); from the first moved row
// on, every row moves (a strictly increasing keep with keep[i] > i keeps keep[i'] > i' after it).
// Called by wave 0 only, lanes < 64.
__device__ __forceinline__ int rows_in_place(int my_keep, int lane, int n) {
  const unsigned long long moved = __builtin_amdgcn_ballot_w64(lane < n && my_keep != lane);
  return moved == 0 ? n : (int)__builtin_ctzll(moved);
}

// Moves rows row0 + keep_s[i] to row0 + i for i < n in one cache (n <= kMaxQ; keep_s strictly
// increasing and visible to every thread; rows [0, first) stay).
__device__ __forceinline__ void compact_rows(uint16_t* ckv16, uint16_t* kpe16, size_t row0, const int* keep_s, int first,
                                             int n) {
  gather_rows(OneCache{ckv16, kpe16}, 1, row0, keep_s, first, n - first);
}

// Reads a caller-given keep row (n entries) into keep_s and checks it against the stream's prefix
// P: n in [0, min(keep_stride, kMaxQ)], P in [0, kv_rows], entries strictly increasing, first
// >= 0, last row P + keep[n-1] < kv_rows.  Returns 0 when the gather may run, else the status
// bit that says why not; *first_s receives the count of leading rows that stay in place (valid
// when 0 is returned).  Called by every thread of the workgroup with the same n and P; the
// result is uniform.  bad_s and first_s are workgroup-shared ints.
__device__ __forceinline__ int load_keep(const int32_t* keep_row, int n, int keep_stride, int P, int kv_rows,
                                         int* keep_s, int* bad_s, int* first_s) {
  const int tid = threadIdx.x;
  if (n < 0 || n > keep_stride || n > kMaxQ) return DDTREE_STATUS_BAD_KEEP;
  if (P < 0 || P > kv_rows) return DDTREE_STATUS_BAD_PREFIX;
  if (tid == 0) *bad_s = 0;
  __syncthreads();
  if (tid < 64) {
    const int k = tid < n ? keep_row[tid] : 0;
    if (tid < n) {
      bool ok = k >= 0 && (long long)P + k < (long long)kv_rows;
      if (tid > 0) ok = ok && keep_row[tid - 1] < k;
      keep_s[tid] = k;
      if (!ok) *bad_s = 1;
    }
    const int first = rows_in_place(k, tid, n);
    if (tid == 0) *first_s = first;
  }
  __syncthreads();
  return *bad_s ? DDTREE_STATUS_BAD_KEEP : 0;
}

}  // namespace ddtree
