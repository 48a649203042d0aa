// Best-first draft-tree construction for gfx950.
//
// "Building the Foundation: Architecting a Native CUDA DDTree Inference Engine", sections
// "Tie-Breaking and Numerical Precision", "The Single-Threaded Heap Design" and "Assumptions
// Underlying the Design": the builder expands a best-first heap of candidates keyed by float32
// cumulative log-weight, ties in insertion order; a popped candidate becomes the next node and
// offers its next sibling (log-weight logw - lp[d-1][r] + lp[d-1][r+1], in that order) and its
// first child (logw + lp[d][0]); it emits parents, tokens, depths, log-weights, the child /
// sibling links and the visibility (ancestor) relation.
//
// The pages keep the heap on one thread.  Here one wave holds the whole candidate pool instead:
// at most 1 + 2 (budget - 1) <= 125 candidates ever exist, two slots per lane, slot = insertion
// number.  A pop is a 64-lane max-reduction (DPP row shifts and broadcasts, no LDS round trip)
// of order-preserving keys of the log-weights, and two ballots pick the earliest-inserted
// candidate among equal weights -- exactly the heap's order.  Node i's outputs live in lane i
// and are filled as the node is appended: its ancestor mask is its parent's (read across lanes)
// plus its own bit, and the retrieve links chain each parent's children in append order.
// The drafter's log-probabilities and tokens of the request are staged in LDS once.

#include "kernels.h"

#include "../../include/ddtree.h"

namespace ddtree {
namespace {

constexpr int kBuildMaxD = 64;
constexpr int kBuildMaxK = 64;

// float -> uint32 with the same order (finite values; larger float, larger key, never 0).
__device__ __forceinline__ unsigned ordered_key(float w) {
  const unsigned u = __float_as_uint(w);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ unsigned dpp_max(unsigned v) {
  return max(v, (unsigned)__builtin_amdgcn_update_dpp((int)v, (int)v, kCtrl, kRowMask, 0xF, false));
}

// Maximum of v over the 64 lanes, returned to every lane.
__device__ __forceinline__ unsigned wave_max_u32(unsigned v) {
  v = dpp_max<0x111>(v);  // row_shr:1
  v = dpp_max<0x112>(v);  // row_shr:2
  v = dpp_max<0x114>(v);  // row_shr:4
  v = dpp_max<0x118>(v);  // row_shr:8   -> lane 15 of each row: the row's maximum
  v = dpp_max<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v = dpp_max<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3 -> lane 63: the wave's maximum
  return __builtin_amdgcn_readlane(v, 63);
}

__global__ void __launch_bounds__(64) tree_build_kernel(BuildArgs a) {
  __shared__ float lp_s[kBuildMaxD * kBuildMaxK];
  __shared__ int tok_s[kBuildMaxD * kBuildMaxK];
  const int s = blockIdx.x;
  const int lane = threadIdx.x;
  const int D = a.depth, K = a.topk, B = a.budget;
  const size_t base = (size_t)s * D * K;
  for (int i = lane; i < D * K; i += 64) {
    lp_s[i] = a.lp[base + i];
    tok_s[i] = a.tok[base + i];
  }
  __syncthreads();

  // candidate slots (slot c: lane c % 64, sub-slot c / 64)
  bool live[2] = {false, false};
  float cw[2] = {0.f, 0.f};
  int cd[2] = {0, 0}, cr[2] = {0, 0}, cp[2] = {0, 0};
  // node `lane`
  int my_parent = -1, my_depth = 0, my_rank = 0, my_tok = -1, my_fc = -1, my_ns = -1, my_last = -1;
  float my_w = 0.f;
  unsigned long long my_anc = lane == 0 ? 1ull : 0ull;
  if (lane == 0) {
    my_tok = a.root_tok != nullptr ? a.root_tok[s] : -1;
    live[0] = true;
    cw[0] = lp_s[0];
    cd[0] = 1;
  }
  int n = 1, n_ins = 1;
  for (int step = 0; step < B; ++step) {
    const unsigned k0 = live[0] ? ordered_key(cw[0]) : 0u;
    const unsigned k1 = live[1] ? ordered_key(cw[1]) : 0u;
    const unsigned m = wave_max_u32(max(k0, k1));
    if (m == 0) break;  // no candidate left (top-1 chain shorter than the budget)
    const unsigned long long b0 = __builtin_amdgcn_ballot_w64(k0 == m);
    const unsigned long long b1 = __builtin_amdgcn_ballot_w64(k1 == m);
    const int ins = b0 != 0 ? (int)__builtin_ctzll(b0) : 64 + (int)__builtin_ctzll(b1);
    const int owner = ins & 63, sub = ins >> 6;
    const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(sub ? cw[1] : cw[0]), owner));
    const int d = __builtin_amdgcn_readlane(sub ? cd[1] : cd[0], owner);
    const int r = __builtin_amdgcn_readlane(sub ? cr[1] : cr[0], owner);
    const int p = __builtin_amdgcn_readlane(sub ? cp[1] : cp[0], owner);
    if (lane == owner) live[sub] = false;
    const int idx = n++;
    // append node idx
    // the parent's mask, read across lanes as two 32-bit halves (zero-extended: bit 31 of the
    // low half is a node, not a sign)
    const unsigned long long pa =
        (unsigned long long)(unsigned)__builtin_amdgcn_readlane((int)(unsigned)(my_anc & 0xffffffffu), p) |
        ((unsigned long long)(unsigned)__builtin_amdgcn_readlane((int)(unsigned)(my_anc >> 32), p) << 32);
    const int prev = __builtin_amdgcn_readlane(my_last, p);
    if (lane == idx) {
      my_parent = p;
      my_depth = d;
      my_rank = r;
      my_tok = tok_s[(d - 1) * K + r];
      my_w = w;
      my_anc = pa | (1ull << idx);
    }
    if (prev >= 0) {
      if (lane == prev) my_ns = idx;
    } else if (lane == p) {
      my_fc = idx;
    }
    if (lane == p) my_last = idx;
    if (step + 1 == B) break;  // no further pops: nothing to offer
    // offer the next sibling, then the first child
    if (r + 1 < K) {
      const float ws = (w - lp_s[(d - 1) * K + r]) + lp_s[(d - 1) * K + r + 1];
      if (lane == (n_ins & 63)) {
        const int c = n_ins >> 6;
        live[c] = true;
        cw[c] = ws;
        cd[c] = d;
        cr[c] = r + 1;
        cp[c] = p;
      }
      ++n_ins;
    }
    if (d < D) {
      const float wc = w + lp_s[d * K];
      if (lane == (n_ins & 63)) {
        const int c = n_ins >> 6;
        live[c] = true;
        cw[c] = wc;
        cd[c] = d + 1;
        cr[c] = 0;
        cp[c] = idx;
      }
      ++n_ins;
    }
  }
  const size_t row = (size_t)s * (B + 1) + lane;
  if (lane < n) {
    a.parents[row] = my_parent;
    a.tokens[row] = my_tok;
    if (a.depths != nullptr) a.depths[row] = my_depth;
    if (a.logw != nullptr) a.logw[row] = my_w;
    if (a.first_child != nullptr) a.first_child[row] = my_fc;
    if (a.next_sibling != nullptr) a.next_sibling[row] = my_ns;
    if (a.anc != nullptr) a.anc[row] = my_anc;
  }
  if (lane == 0) a.n_nodes[s] = n;
}

}  // namespace

hipError_t launch_build(const BuildArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<BuildArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(tree_build_kernel), dim3((unsigned)a.n_streams), dim3(64),
                         args, 0, stream);
}

}  // namespace ddtree
