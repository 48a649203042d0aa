// Internal launch interface between the C ABI shim and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ddtree.h"

namespace ddtree {

constexpr int kHeads = 64;
constexpr int kDLat = 512;
constexpr int kDRope = 64;
constexpr int kMaxQ = 64;

// verify_attn tiling: one workgroup = 4 waves = 2 tree nodes x 64 heads; keys are staged into
// LDS 32 rows at a time.
constexpr int kQueriesPerWG = 2;
constexpr int kTileKeys = 32;
constexpr int kWGThreads = 256;

// The launch holds two groups of workgroups.  Group 0: node pairs (2p, 2p + 1), p < q_len / 2.
// Group 1 (odd q_len only): the last node alone.  Dispatch order: lead1 workgroups of group 1,
// all of group 0, the rest of group 1.  Each group has its own key-range split count;
// a group with more than one split writes (out, lse) partials that a merge pass combines.
//   group 0 partial rows: ((s * n_pairs + p) * 2 + node_in_pair) * 64 + head
//   group 1 partial rows: s * 64 + head
struct VerifyArgs {
  const uint16_t* q_lat;
  const uint16_t* q_pe;
  const uint16_t* ckv;
  const uint16_t* kpe;
  const int32_t* parents;
  float* out;
  float* lse;
  float* part_out[2];  // [splits][rows of the group][512] when that group is split
  float* part_lse[2];  // [splits][rows of the group]
  int32_t* status;
  const int32_t* prefix_lens;  // per-stream prefix lengths, or null: prefix_len for every stream
  int prefix_len;      // the prefix length, or with prefix_lens its upper bound
  int q_len;
  int n_streams;
  int kv_rows;
  int n_pairs;         // q_len / 2
  int n_tiles;         // ceil((prefix_len + q_len) / kTileKeys), the longest stream
  int splits[2];
  int tiles_per_split[2];
  int wg_count0;       // workgroups of group 0
  int lead1;           // group-1 workgroups dispatched before group 0 (the rest follow it)
  float scale_log2e;   // softmax scale * log2(e)
};

hipError_t launch_verify(const VerifyArgs& a, int wg_total, hipStream_t stream);

// One merge launch covers the partial rows of both groups: group 0's rows first, then group
// 1's (row numbering above).  A group that is not split has no rows here.
struct CombineArgs {
  const float* part_out[2];
  const float* part_lse[2];
  float* out;
  float* lse;
  long long rows[2];   // partial rows of each group, 0 when the group is not split
  int n_splits[2];
  int n_pairs;
  int q_len;
};

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

struct CompactArgs {
  uint16_t* ckv;
  uint16_t* kpe;
  const int32_t* keep;
  const int32_t* n_keep;
  int32_t* status;
  const int32_t* prefix_lens;  // per-stream prefix lengths, or null: prefix_len
  int kv_rows;
  int n_streams;
  int prefix_len;
  int keep_stride;
};

hipError_t launch_compact(const CompactArgs& a, hipStream_t stream);

struct AcceptArgs {
  const int32_t* parents;  // [n_streams][q_len]
  const int32_t* draft;    // [n_streams][q_len]
  const int32_t* target;   // [n_streams][q_len]
  int32_t* keep;           // [n_streams][keep_stride]
  int32_t* n_keep;         // [n_streams]
  int32_t* next_token;     // [n_streams] or null
  int32_t* status;         // or null
  uint16_t* ckv;           // fused compaction only
  uint16_t* kpe;
  int32_t* prefix_lens;    // fused, per stream: read, then advanced by n_keep; or null
  int kv_rows;
  int prefix_len;
  int q_len;
  int n_streams;
  int keep_stride;
};

hipError_t launch_accept(const AcceptArgs& a, hipStream_t stream);

struct BuildArgs {
  const float* lp;            // [n_streams][depth][topk], decreasing within a position
  const int32_t* tok;         // [n_streams][depth][topk]
  const int32_t* root_tok;    // [n_streams] or null
  int32_t* parents;           // [n_streams][budget + 1]
  int32_t* tokens;            // [n_streams][budget + 1]
  int32_t* n_nodes;           // [n_streams]
  int32_t* depths;            // [n_streams][budget + 1] or null
  float* logw;                // [n_streams][budget + 1] or null
  int32_t* first_child;       // [n_streams][budget + 1] or null
  int32_t* next_sibling;      // [n_streams][budget + 1] or null
  unsigned long long* anc;    // [n_streams][budget + 1] or null
  int depth;                  // 1..64
  int topk;                   // 1..64
  int budget;                 // 1..63
  int n_streams;
};

hipError_t launch_build(const BuildArgs& a, hipStream_t stream);
hipError_t launch_accept_compact(const AcceptArgs& a, hipStream_t stream);

// Compaction of every layer's cache in one launch.  All layers share n_streams and kv_rows;
// workgroup (s, group) = (blockIdx.x, blockIdx.y) handles layers [group * layers_per_wg, ...).
// The pointer tables travel in the kernel arguments (2 KB at kMaxLayers = 128).
constexpr int kMaxLayers = DDTREE_MAX_LAYERS;

struct LayersArgs {
  uint16_t* ckv[kMaxLayers];
  uint16_t* kpe[kMaxLayers];
  const int32_t* parents;  // acceptance: [n_streams][q_len] (with draft / target)
  const int32_t* draft;
  const int32_t* target;
  int32_t* keep;           // [n_streams][keep_stride]: written by acceptance, else read
  int32_t* n_keep;         // [n_streams]: written by acceptance, else read
  int32_t* next_token;     // acceptance only, or null
  int32_t* status;         // or null
  int32_t* prefix_lens;    // per stream, or null: prefix_len for every stream
  int kv_rows;
  int prefix_len;
  int q_len;               // acceptance only
  int n_streams;
  int keep_stride;
  int n_layers;
  int layers_per_wg;
};

// The tree's cache rows from the key/value projection's output (RMSNorm + NeoX rotation).
struct AppendArgs {
  const float* kv;             // [n_streams][q_len][576]
  const float* weight;         // [512]
  const float* rope_cos;       // [rope_rows][32]
  const float* rope_sin;       // [rope_rows][32]
  const int32_t* parents;      // [n_streams][q_len]
  const int32_t* prefix_lens;  // per stream, or null: prefix_len
  uint16_t* ckv;
  uint16_t* kpe;
  int32_t* status;             // or null
  float eps;
  int prefix_len;
  int q_len;
  int n_streams;
  int kv_rows;
  int rope_rows;
};

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);

// keep / n_keep given: validated per stream, then gathered in every layer.
hipError_t launch_compact_layers(const LayersArgs& a, hipStream_t stream);
// Acceptance, then the gather in every layer; with prefix_lens, a second launch advances them.
hipError_t launch_accept_compact_layers(const LayersArgs& a, hipStream_t stream);

}  // namespace ddtree
