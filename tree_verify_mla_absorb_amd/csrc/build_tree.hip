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
// plus its own bit.  The retrieve links come from the parents in one pass at the end.
// The drafter's log-probabilities and tokens of the request are staged in LDS once.

#include "kernels.h"

#include "../../include/ddtree.h"

namespace ddtree {
namespace {

constexpr int kBuildMaxD = 64;
constexpr int kBuildMaxK = 64;

// float -> uint32 with the same order (finite values; larger float, larger key, never 0).
// -0.0 takes +0.0's key: the two compare equal, so their order is the insertion order.
__device__ __forceinline__ unsigned ordered_key(float w) {
  unsigned u = __float_as_uint(w);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Maximum of v over the 64 lanes, returned to every lane: row shifts by 1, 2, 4, 8 leave each
// row's maximum in its lane 15, then row broadcasts of lane 15 into rows 1, 3 and of lane 31
// into rows 2, 3 leave the wave's maximum in lane 63.  Each step is one max with a DPP source; a
// lane without a source (or outside the row mask) is not written and keeps its value.  A DPP
// read of a VGPR written by the previous VALU instruction needs two wait states (s_nop 1), and
// so does the lane read that follows.
__device__ __forceinline__ unsigned wave_max_u32(unsigned v) {
  asm volatile(
      "s_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      "s_nop 1"
      : "+v"(v));
  return __builtin_amdgcn_readlane(v, 63);
}

// kOneSlot: budget <= 32, so at most 1 + 2 (budget - 1) <= 63 candidates ever exist and every
// one fits in sub-slot 0; the second sub-slot's keys, ballot and inserts are compiled out.
template <bool kOneSlot>
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

  // Candidate slots (slot c: lane c % 64, sub-slot c / 64), one register per field and
  // sub-slot: a candidate's weight, depth, rank and parent.  Updates are per-lane selects, not
  // branches, so a pop costs a few dozen wave instructions.
  float w0 = 0.f, w1 = 0.f;
  int d0 = 0, d1 = 0, r0 = 0, r1 = 0, p0 = 0, p1 = 0;
  bool l0 = lane == 0, l1 = false;  // live; slot 0 = the root's first child
  if (lane == 0) {
    w0 = lp_s[0];
    d0 = 1;
  }
  // node `lane`
  int my_parent = -1, my_depth = 0, my_rank = 0, my_tok = lane == 0 && a.root_tok != nullptr ? a.root_tok[s] : -1;
  float my_w = 0.f;
  unsigned long long my_anc = lane == 0 ? 1ull : 0ull;
  int n = 1, n_ins = 1;
  for (int step = 0; step < B; ++step) {
    const unsigned k0 = l0 ? ordered_key(w0) : 0u;
    const unsigned k1 = (!kOneSlot && l1) ? ordered_key(w1) : 0u;
    const unsigned m = wave_max_u32(max(k0, k1));
    if (m == 0) break;  // no candidate left (top-1 chain shorter than the budget)
    const unsigned long long b0 = __builtin_amdgcn_ballot_w64(k0 == m);
    const unsigned long long b1 = kOneSlot ? 0ull : __builtin_amdgcn_ballot_w64(k1 == m);
    int d, r, p;
    float w;
    if (kOneSlot || b0 != 0) {  // uniform: the earliest-inserted maximum sits in sub-slot 0 of lane `owner`
      const int owner = (int)__builtin_ctzll(b0);
      w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(w0), owner));
      d = __builtin_amdgcn_readlane(d0, owner);
      r = __builtin_amdgcn_readlane(r0, owner);
      p = __builtin_amdgcn_readlane(p0, owner);
      l0 = l0 && lane != owner;
    } else {
      const int owner = (int)__builtin_ctzll(b1);
      w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(w1), owner));
      d = __builtin_amdgcn_readlane(d1, owner);
      r = __builtin_amdgcn_readlane(r1, owner);
      p = __builtin_amdgcn_readlane(p1, owner);
      l1 = l1 && lane != owner;
    }
    const int idx = n++;
    // append node idx: the parent's mask, read across lanes as two 32-bit halves
    // (zero-extended: bit 31 of the low half is a node, not a sign)
    const unsigned long long pa =
        (unsigned long long)(unsigned)__builtin_amdgcn_readlane((int)(unsigned)(my_anc & 0xffffffffu), p) |
        ((unsigned long long)(unsigned)__builtin_amdgcn_readlane((int)(unsigned)(my_anc >> 32), p) << 32);
    // the node's token and the three log-probabilities its offers need, read together (indices
    // clamped into the table) so that one LDS wait covers them all
    const int t = tok_s[(d - 1) * K + r];
    const float lp_r = lp_s[(d - 1) * K + r];
    const float lp_n = lp_s[(d - 1) * K + min(r + 1, K - 1)];
    const float lp_c = lp_s[min(d, D - 1) * K];
    const bool me = lane == idx;
    my_parent = me ? p : my_parent;
    my_depth = me ? d : my_depth;
    my_rank = me ? r : my_rank;
    my_tok = me ? t : my_tok;
    my_w = me ? w : my_w;
    my_anc = me ? (pa | (1ull << idx)) : my_anc;
    // offer the next sibling (the pages' float32 expression, in this order), then the first child.
    // The last pop's offers are made too (nothing reads the pool after the loop; in the one-slot
    // form the last child may take slot 64, which lands on slot 0 and is never read): without a
    // branch here the reads above are not sunk below it.
    const bool has_sib = r + 1 < K, has_child = d < D;
    const float ws = has_sib ? (w - lp_r) + lp_n : 0.f;
    const float wc = has_child ? w + lp_c : 0.f;
    const int slot_s = n_ins, slot_c = n_ins + (has_sib ? 1 : 0);
    n_ins = slot_c + (has_child ? 1 : 0);
    // per lane: does this lane own the sibling's / the child's slot, in sub-slot 0 or 1?
    const bool own_s = has_sib && lane == (slot_s & 63), own_c = has_child && lane == (slot_c & 63);
    const bool s_in0 = own_s && (kOneSlot || slot_s < 64), s_in1 = !kOneSlot && own_s && slot_s >= 64;
    const bool c_in0 = own_c && (kOneSlot || slot_c < 64), c_in1 = !kOneSlot && own_c && slot_c >= 64;
    w0 = s_in0 ? ws : (c_in0 ? wc : w0);
    d0 = s_in0 ? d : (c_in0 ? d + 1 : d0);
    r0 = s_in0 ? r + 1 : (c_in0 ? 0 : r0);
    p0 = s_in0 ? p : (c_in0 ? idx : p0);
    l0 = l0 || s_in0 || c_in0;
    w1 = s_in1 ? ws : (c_in1 ? wc : w1);
    d1 = s_in1 ? d : (c_in1 ? d + 1 : d1);
    r1 = s_in1 ? r + 1 : (c_in1 ? 0 : r1);
    p1 = s_in1 ? p : (c_in1 ? idx : p1);
    l1 = l1 || s_in1 || c_in1;
  }
  // Retrieve links from a (parent, rank) table: the children of a node are appended in rank
  // order 0, 1, 2, ... (rank r + 1 is offered only once rank r is popped), so its first child is
  // entry (node, 0) and a node's next sibling is entry (parent, rank + 1); -1 where none.
  __shared__ __attribute__((aligned(16))) int link_s[kBuildMaxD * kBuildMaxK];  // [parent < 64][rank < 64]
  typedef int I32x4 __attribute__((ext_vector_type(4)));
  for (int e = 4 * lane; e < n * 64; e += 4 * 64) *reinterpret_cast<I32x4*>(link_s + e) = I32x4{-1, -1, -1, -1};
  __syncthreads();
  if (lane > 0 && lane < n) link_s[my_parent * 64 + my_rank] = lane;
  __syncthreads();
  const int my_fc = lane < n ? link_s[lane * 64] : -1;
  const int my_ns = (lane > 0 && lane < n && my_rank + 1 < K) ? link_s[my_parent * 64 + my_rank + 1] : -1;
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
  const void* kernel = a.budget <= 32 ? reinterpret_cast<const void*>(tree_build_kernel<true>)
                                      : reinterpret_cast<const void*>(tree_build_kernel<false>);
  return hipLaunchKernel(kernel, dim3((unsigned)a.n_streams), dim3(64), args, 0, stream);
}

}  // namespace ddtree
