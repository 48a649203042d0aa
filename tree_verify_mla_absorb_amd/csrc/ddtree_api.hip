// C ABI of the library: argument validation, launch planning, kernel launches.
// Validation reads no device memory and never synchronises; see include/ddtree.h for the
// contract of every entry point.

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../include/ddtree.h"
#include "kernels.h"

namespace {

using ddtree::kDLat;
using ddtree::kDRope;
using ddtree::kHeads;
using ddtree::kMaxQ;
using ddtree::kQueriesPerWG;
using ddtree::kTileKeys;

constexpr int kMaxSplits = 32;
constexpr long long kMaxGrid = 0x7fffffffLL;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

int cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

struct Plan {
  int n_qgroups = 0;
  int n_tiles = 0;
  int n_splits = 1;
  int tiles_per_split = 0;
};

bool shape_ok(int prefix_len, int q_len, int n_streams) {
  return prefix_len >= 0 && q_len >= 1 && q_len <= kMaxQ && n_streams >= 1 &&
         (long long)prefix_len + q_len <= 0x7fffffffLL - kTileKeys;
}

// Key-range split count.  Each (stream, query pair) unit walks n_tiles key tiles; splitting
// lets small launches fill the GPU at the price of a merge pass over fp32 partials.  The
// automatic choice minimises a simple time model: rounds of workgroups over the CUs times
// tiles per workgroup, plus the partial traffic of the merge expressed in tile-times.
Plan make_plan(int prefix_len, int q_len, int n_streams, int num_splits) {
  Plan p;
  p.n_qgroups = (q_len + kQueriesPerWG - 1) / kQueriesPerWG;
  p.n_tiles = (prefix_len + q_len + kTileKeys - 1) / kTileKeys;
  const long long units = (long long)n_streams * p.n_qgroups;
  int want;
  if (num_splits > 0) {
    want = num_splits;
  } else {
    const int cus = cu_count();
    // One tile of one unit is ~17.8 MFLOP, ~2.2 us on one CU.  Each (unit, split) partial
    // costs 0.5 MB of HBM traffic (128 rows x 2 KiB written, then read by the merge), ~64 ns
    // of the whole GPU's bandwidth: ~0.03 tile-times.  Plus a fixed cost for the second launch.
    double best = 1e300;
    want = 1;
    for (int sp = 1; sp <= kMaxSplits && sp <= p.n_tiles; ++sp) {
      const int tps = (p.n_tiles + sp - 1) / sp;
      const int eff = (p.n_tiles + tps - 1) / tps;
      const double rounds = ceil((double)units * eff / cus);
      const double merge = eff > 1 ? 0.03 * (double)units * eff + 0.5 : 0.0;
      const double cost = rounds * tps + merge;
      if (cost < best - 1e-9) {
        best = cost;
        want = sp;
      }
    }
  }
  if (want > kMaxSplits) want = kMaxSplits;
  if (want > p.n_tiles) want = p.n_tiles;
  if (want < 1) want = 1;
  p.tiles_per_split = (p.n_tiles + want - 1) / want;
  p.n_splits = (p.n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;  // every split non-empty
  return p;
}

size_t part_out_bytes(const Plan& p, int q_len, int n_streams) {
  return (size_t)p.n_splits * n_streams * q_len * kHeads * kDLat * sizeof(float);
}
size_t workspace_bytes_for(const Plan& p, int q_len, int n_streams) {
  if (p.n_splits <= 1) return 0;
  const size_t lse_bytes = (size_t)p.n_splits * n_streams * q_len * kHeads * sizeof(float);
  return part_out_bytes(p, q_len, n_streams) + lse_bytes;
}

}  // namespace

extern "C" {

int ddtree_version(void) { return DDTREE_VERSION; }

const char* ddtree_status_string(int code) {
  switch (code) {
    case DDTREE_OK: return "ok";
    case DDTREE_ERR_NULL: return "a required pointer is NULL";
    case DDTREE_ERR_SHAPE: return "a size argument is out of range";
    case DDTREE_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case DDTREE_ERR_ALIAS: return "an output range overlaps an input range";
    case DDTREE_ERR_WORKSPACE: return "workspace missing or too small";
    case DDTREE_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int ddtree_verify_attn_num_splits(int prefix_len, int q_len, int n_streams, int num_splits) {
  if (!shape_ok(prefix_len, q_len, n_streams) || num_splits < 0) return DDTREE_ERR_SHAPE;
  return make_plan(prefix_len, q_len, n_streams, num_splits).n_splits;
}

size_t ddtree_verify_attn_workspace_size(int prefix_len, int q_len, int n_streams, int num_splits) {
  if (!shape_ok(prefix_len, q_len, n_streams) || num_splits < 0) return 0;
  const Plan p = make_plan(prefix_len, q_len, n_streams, num_splits);
  return workspace_bytes_for(p, q_len, n_streams);
}

int ddtree_verify_attn_ex(const void* q_lat, const void* q_pe, const void* ckv, const void* kpe,
                          int prefix_len, const int32_t* parents, int q_len, int n_streams,
                          float* out_lat, float* lse, int kv_rows, float scale, int num_splits,
                          void* workspace, size_t workspace_bytes, int32_t* dev_status,
                          hipStream_t stream) {
  if (!q_lat || !q_pe || !ckv || !kpe || !parents || !out_lat || !lse) return DDTREE_ERR_NULL;
  if (!shape_ok(prefix_len, q_len, n_streams) || num_splits < 0) return DDTREE_ERR_SHAPE;
  if (kv_rows < prefix_len + q_len) return DDTREE_ERR_SHAPE;
  if (!aligned16(q_lat) || !aligned16(q_pe) || !aligned16(ckv) || !aligned16(kpe) || !aligned16(out_lat) ||
      !aligned4(lse) || !aligned4(parents) || (dev_status && !aligned4(dev_status)))
    return DDTREE_ERR_ALIGN;
  if (!(scale > 0.f) || !isfinite(scale)) scale = 1.0f / sqrtf(192.0f);

  const size_t rows_q = (size_t)n_streams * q_len * kHeads;
  const Range r_out = range_of(out_lat, rows_q * kDLat * sizeof(float));
  const Range r_lse = range_of(lse, rows_q * sizeof(float));
  const Range inputs[] = {
      range_of(q_lat, rows_q * kDLat * 2), range_of(q_pe, rows_q * kDRope * 2),
      range_of(ckv, (size_t)n_streams * kv_rows * kDLat * 2),
      range_of(kpe, (size_t)n_streams * kv_rows * kDRope * 2),
      range_of(parents, (size_t)n_streams * q_len * sizeof(int32_t))};
  for (const Range& in : inputs)
    if (overlap(in, r_out) || overlap(in, r_lse)) return DDTREE_ERR_ALIAS;
  if (overlap(r_out, r_lse)) return DDTREE_ERR_ALIAS;

  const Plan plan = make_plan(prefix_len, q_len, n_streams, num_splits);
  const long long blocks = (long long)n_streams * plan.n_qgroups * plan.n_splits;
  if (blocks > kMaxGrid) return DDTREE_ERR_SHAPE;

  ddtree::VerifyArgs a{};
  a.q_lat = static_cast<const uint16_t*>(q_lat);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.ckv = static_cast<const uint16_t*>(ckv);
  a.kpe = static_cast<const uint16_t*>(kpe);
  a.parents = parents;
  a.status = dev_status;
  a.prefix_len = prefix_len;
  a.q_len = q_len;
  a.n_streams = n_streams;
  a.kv_rows = kv_rows;
  a.n_qgroups = plan.n_qgroups;
  a.n_splits = plan.n_splits;
  a.tiles_per_split = plan.tiles_per_split;
  a.n_tiles = plan.n_tiles;
  a.scale_log2e = scale * 1.4426950408889634f;

  if (plan.n_splits > 1) {
    const size_t need = workspace_bytes_for(plan, q_len, n_streams);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return DDTREE_ERR_WORKSPACE;
    const Range r_ws = range_of(workspace, need);
    for (const Range& in : inputs)
      if (overlap(in, r_ws)) return DDTREE_ERR_ALIAS;
    if (overlap(r_ws, r_out) || overlap(r_ws, r_lse)) return DDTREE_ERR_ALIAS;
    a.part_out = static_cast<float*>(workspace);
    a.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + part_out_bytes(plan, q_len, n_streams));
    a.out = nullptr;
    a.lse = nullptr;
  } else {
    a.out = out_lat;
    a.lse = lse;
  }
  if (ddtree::launch_verify(a, stream) != hipSuccess) return DDTREE_ERR_HIP;
  if (plan.n_splits > 1) {
    ddtree::CombineArgs c{};
    c.part_out = a.part_out;
    c.part_lse = a.part_lse;
    c.out = out_lat;
    c.lse = lse;
    c.rows = (int)rows_q;
    c.n_splits = plan.n_splits;
    if ((long long)rows_q * 128 / 256 + 1 > kMaxGrid) return DDTREE_ERR_SHAPE;
    if (ddtree::launch_combine(c, stream) != hipSuccess) return DDTREE_ERR_HIP;
  }
  return DDTREE_OK;
}

int ddtree_verify_attn(const void* q_lat, const void* q_pe, const void* ckv, const void* kpe,
                       int prefix_len, const int32_t* parents, int q_len, int n_streams,
                       float* out_lat, float* lse, hipStream_t stream) {
  return ddtree_verify_attn_ex(q_lat, q_pe, ckv, kpe, prefix_len, parents, q_len, n_streams, out_lat, lse,
                               prefix_len + q_len, 0.f, 1, nullptr, 0, nullptr, stream);
}

int ddtree_compact_kv(const ddtree_kv_cache* cache, int prefix_len, const int32_t* keep,
                      const int32_t* n_keep, int keep_stride, int32_t* dev_status, hipStream_t stream) {
  if (!cache || !cache->ckv || !cache->kpe || !keep || !n_keep) return DDTREE_ERR_NULL;
  if (cache->n_streams < 1 || cache->kv_rows < 1 || prefix_len < 0 || prefix_len > cache->kv_rows ||
      keep_stride < 1)
    return DDTREE_ERR_SHAPE;
  if (!aligned16(cache->ckv) || !aligned16(cache->kpe) || !aligned4(keep) || !aligned4(n_keep) ||
      (dev_status && !aligned4(dev_status)))
    return DDTREE_ERR_ALIGN;
  if (overlap(range_of(cache->ckv, (size_t)cache->n_streams * cache->kv_rows * kDLat * 2),
              range_of(cache->kpe, (size_t)cache->n_streams * cache->kv_rows * kDRope * 2)))
    return DDTREE_ERR_ALIAS;
  ddtree::CompactArgs a{};
  a.ckv = static_cast<uint16_t*>(cache->ckv);
  a.kpe = static_cast<uint16_t*>(cache->kpe);
  a.keep = keep;
  a.n_keep = n_keep;
  a.status = dev_status;
  a.kv_rows = cache->kv_rows;
  a.n_streams = cache->n_streams;
  a.prefix_len = prefix_len;
  a.keep_stride = keep_stride;
  if (ddtree::launch_compact(a, stream) != hipSuccess) return DDTREE_ERR_HIP;
  return DDTREE_OK;
}

}  // extern "C"
