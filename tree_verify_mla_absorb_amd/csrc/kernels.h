// Internal launch interface between the C ABI shim and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ddtree {

constexpr int kHeads = 64;
constexpr int kDLat = 512;
constexpr int kDRope = 64;
constexpr int kMaxQ = 64;

// verify_attn tiling: one workgroup = 4 waves = 2 tree queries x 64 heads; keys are staged
// into LDS 64 rows at a time.
constexpr int kQueriesPerWG = 2;
constexpr int kTileKeys = 64;
constexpr int kWGThreads = 256;

struct VerifyArgs {
  const uint16_t* q_lat;
  const uint16_t* q_pe;
  const uint16_t* ckv;
  const uint16_t* kpe;
  const int32_t* parents;
  float* out;          // final output (no split) -- or nullptr when partials are written
  float* lse;
  float* part_out;     // [splits][S][Q][64][512] (split > 1)
  float* part_lse;     // [splits][S][Q][64]
  int32_t* status;
  int prefix_len;
  int q_len;
  int n_streams;
  int kv_rows;
  int n_qgroups;       // ceil(q_len / 2)
  int n_splits;
  int tiles_per_split;
  int n_tiles;         // ceil((prefix_len + q_len) / 64)
  float scale_log2e;   // softmax scale * log2(e)
};

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);

struct CombineArgs {
  const float* part_out;
  const float* part_lse;
  float* out;
  float* lse;
  int rows;            // S * Q * 64
  int n_splits;
};

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

struct CompactArgs {
  uint16_t* ckv;
  uint16_t* kpe;
  const int32_t* keep;
  const int32_t* n_keep;
  int32_t* status;
  int kv_rows;
  int n_streams;
  int prefix_len;
  int keep_stride;
};

hipError_t launch_compact(const CompactArgs& a, hipStream_t stream);

}  // namespace ddtree
