// The greedy acceptance walk over one verified draft tree, shared by the acceptance kernels.
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
#pragma once

#include "kernels.h"

#include "../../include/ddtree.h"

namespace ddtree {

struct Walk {
  int n;        // accepted nodes (0: malformed tree)
  int next;     // target token at the last accepted node (-1: malformed tree)
  int my_node;  // path[lane] for lane < n
};

// One wave; every lane calls it.  Reads row s of parents / draft / target ([.][q_len] int32).
__device__ __forceinline__ Walk accept_walk(const int32_t* parents, const int32_t* draft, const int32_t* target,
                                            int q_len, int s, int lane) {
  const bool in = lane < q_len;
  const size_t row = (size_t)s * q_len + lane;
  const int p = in ? parents[row] : -2;
  const int d = in ? draft[row] : 0;
  const int tg = in ? target[row] : 0;
  const bool ok = !in || (lane == 0 ? p == -1 : (p >= 0 && p < lane));
  Walk w{0, -1, 0};
  if (__builtin_amdgcn_ballot_w64(!ok) != 0) return w;  // uniform
  // cur is wave-uniform (the lowest bit of a ballot), so the target token at cur is a lane read,
  // not an LDS permute round trip per level
  int cur = 0, n = 1;
  for (int level = 1; level < q_len; ++level) {
    const int tc = __builtin_amdgcn_readlane(tg, cur);
    const unsigned long long m = __builtin_amdgcn_ballot_w64(in && p == cur && d == tc);
    if (m == 0) break;
    cur = (int)__builtin_ctzll(m);
    if (lane == n) w.my_node = cur;
    ++n;
  }
  w.n = n;
  w.next = __builtin_amdgcn_readlane(tg, cur);
  return w;
}

// Writes one stream's walk: keep_row[0..n), *n_keep, *next_token (when given) and, for a
// malformed tree, the BAD_PARENTS status bit.  Every lane of the walking wave calls it.
__device__ __forceinline__ void write_walk(const Walk& w, int lane, int32_t* keep_row, int32_t* n_keep,
                                           int32_t* next_token, int32_t* status) {
  if (lane < w.n) keep_row[lane] = w.my_node;
  if (lane == 0) {
    *n_keep = w.n;
    if (next_token != nullptr) *next_token = w.next;
    if (w.n == 0 && status != nullptr) atomicOr(status, DDTREE_STATUS_BAD_PARENTS);
  }
}

}  // namespace ddtree
