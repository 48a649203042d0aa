// Writing the draft tree's key/value rows into the latent cache at their offset, for gfx950.
//
// "Race Conditions, Buffer Aliasing, and the Architecture of a Native DDTree Inference Engine":
// section "Scratch Buffer Architecture: Managing Transformer Activations" has the key/value
// projection's un-normalised output go through RMSNorm straight into the cache at its offset;
// section "Assumptions, Input Knowledge, and Output Knowledge" names the model family (MLA with
// RMSNorm and NeoX rotary embeddings); section "The Cache Compaction Problem" puts tree node i at
// cache row P + i.  Per node, from its 576 projection outputs (fp32):
//   latent row  ckv[P + i] = bf16( x[0:512] / sqrt(mean(x[0:512]^2) + eps) * w )
//   rotary row  kpe[P + i] = bf16( NeoX rotation of x[512:576] at position P + depth(i) )
// with the caller's rotation tables cos / sin [rows][32]: pair (j, j + 32) turns by the angle of
// row pos, column j.  Rounding to bf16 is to nearest, ties to even.
//
// One wave per (stream, node).  The wave first ranks the whole tree (node j in lane j): six
// pointer-jumping steps give every node's depth (a tree has at most 64 nodes, depth < 64), after
// the one-ballot check that every parent is an earlier node.  Lane l then owns latent values
// [8l, 8l + 8) (two 16-byte loads and one 16-byte store) and rotary value l.  The sum of squares
// is a wave butterfly in fp32.  A stream whose tree is malformed, whose block leaves the cache,
// or whose deepest position has no table row is left untouched and flagged.

#include "kernels.h"

#include "../../include/ddtree.h"

namespace ddtree {
namespace {

constexpr int kAppendWaves = 4;  // nodes per workgroup

typedef float F32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int U32x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bits, round to nearest, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ unsigned bf16_rne(float f) {
  const unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, __shfl_xor(v, m));
  return v;
}

__global__ void __launch_bounds__(64 * kAppendWaves) append_tree_kv_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x;
  const int i = blockIdx.y * kAppendWaves + (threadIdx.x >> 6);
  const int Q = a.q_len;
  if (i >= Q) return;  // uniform over the wave

  // Depths of the whole tree, node j in lane j.
  const bool in = lane < Q;
  const int p = in ? a.parents[(size_t)s * Q + lane] : -1;
  const bool ok = !in || (lane == 0 ? p == -1 : (p >= 0 && p < lane));
  const bool tree_ok = __builtin_amdgcn_ballot_w64(!ok) == 0;
  int up = (lane == 0 || !in || !tree_ok) ? lane : p;  // the root and idle lanes point at themselves
  int depth = (lane == 0 || !in || !tree_ok) ? 0 : 1;
#pragma unroll
  for (int k = 0; k < 6; ++k) {  // after k steps: distance to the 2^k-th ancestor, capped at the root
    const int d_up = __shfl(depth, up);
    const int up_up = __shfl(up, up);
    depth += d_up;
    up = up_up;
  }
  const int P = a.prefix_lens != nullptr ? a.prefix_lens[s] : a.prefix_len;
  const int deepest = wave_max(depth);
  int why = 0;
  if (!tree_ok)
    why = DDTREE_STATUS_BAD_PARENTS;
  else if (P < 0 || (long long)P + Q > (long long)a.kv_rows)
    why = DDTREE_STATUS_BAD_PREFIX;
  else if ((long long)P + deepest >= (long long)a.rope_rows)
    why = DDTREE_STATUS_BAD_POSITION;
  if (why != 0) {  // uniform over the stream: every wave of it takes the same decision
    if (i == 0 && lane == 0 && a.status != nullptr) atomicOr(a.status, why);
    return;
  }
  const int pos = P + __builtin_amdgcn_readlane(depth, i);  // i is the wave's node: a lane read

  const float* x = a.kv + ((size_t)s * Q + i) * (kDLat + kDRope);
  const F32x4 x0 = *reinterpret_cast<const F32x4*>(x + 8 * lane);
  const F32x4 x1 = *reinterpret_cast<const F32x4*>(x + 8 * lane + 4);
  const F32x4 w0 = *reinterpret_cast<const F32x4*>(a.weight + 8 * lane);
  const F32x4 w1 = *reinterpret_cast<const F32x4*>(a.weight + 8 * lane + 4);
  const float own = x[kDLat + lane];
  const float other = x[kDLat + (lane ^ 32)];
  const int j = lane & 31;
  const float c = a.rope_cos[(size_t)pos * 32 + j];
  const float sn = a.rope_sin[(size_t)pos * 32 + j];

  float ss = x0.x * x0.x + x0.y * x0.y + x0.z * x0.z + x0.w * x0.w;
  ss += x1.x * x1.x + x1.y * x1.y + x1.z * x1.z + x1.w * x1.w;
  ss = wave_sum(ss);
  const float r = rsqrtf(ss * (1.0f / kDLat) + a.eps);
  U32x4 packed;
  packed.x = bf16_rne(x0.x * r * w0.x) | (bf16_rne(x0.y * r * w0.y) << 16);
  packed.y = bf16_rne(x0.z * r * w0.z) | (bf16_rne(x0.w * r * w0.w) << 16);
  packed.z = bf16_rne(x1.x * r * w1.x) | (bf16_rne(x1.y * r * w1.y) << 16);
  packed.w = bf16_rne(x1.z * r * w1.z) | (bf16_rne(x1.w * r * w1.w) << 16);
  const size_t row = (size_t)s * a.kv_rows + P + i;
  *reinterpret_cast<U32x4*>(a.ckv + row * kDLat + 8 * lane) = packed;

  // NeoX: out[j] = x[j] c - x[j+32] s for the first half, out[j+32] = x[j+32] c + x[j] s.
  const float rot = lane < 32 ? own * c - other * sn : own * c + other * sn;
  a.kpe[row * kDRope + lane] = (uint16_t)bf16_rne(rot);
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<AppendArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(append_tree_kv_kernel),
                         dim3((unsigned)a.n_streams, (unsigned)((a.q_len + kAppendWaves - 1) / kAppendWaves)),
                         dim3(64 * kAppendWaves), args, 0, stream);
}

}  // namespace ddtree
