// C ABI of the library: argument validation, launch planning, kernel launches.
// Validation reads no device memory and never synchronises; see include/ddtree.h for the
// contract of every entry point.

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/ddtree.h"
#include "kernels.h"

namespace {

using ddtree::kDLat;
using ddtree::kDRope;
using ddtree::kHeads;
using ddtree::kMaxQ;
using ddtree::kQueriesPerWG;
using ddtree::kTileKeys;

constexpr int kMaxSplits = 64;
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
  int n_pairs = 0;     // node pairs per stream (group 0)
  int has_odd = 0;     // 1 when q_len is odd (group 1: the last node alone)
  int n_tiles = 0;
  int splits[2] = {1, 1};
  int tiles_per_split[2] = {0, 0};
  long long wgs[2] = {0, 0};
  long long part_rows[2] = {0, 0};
};

bool shape_ok(int prefix_len, int q_len, int n_streams) {
  // kv rows are addressed with 32-bit byte offsets inside one stream's cache
  return prefix_len >= 0 && q_len >= 1 && q_len <= kMaxQ && n_streams >= 1 &&
         (long long)prefix_len + q_len <= (1LL << 21);
}

// Normalise a requested split count: every split gets the same number of tiles and none is
// empty.
void set_splits(Plan& p, int g, int want) {
  if (want > kMaxSplits) want = kMaxSplits;
  if (want > p.n_tiles) want = p.n_tiles;
  if (want < 1) want = 1;
  p.tiles_per_split[g] = (p.n_tiles + want - 1) / want;
  p.splits[g] = (p.n_tiles + p.tiles_per_split[g] - 1) / p.tiles_per_split[g];
}

// Estimated time of a plan, in units of one workgroup-tile (32 keys x 128 query-heads, about
// 9 MFLOP, ~1-1.5 us on one CU).  When every workgroup fits on the CUs at once, the longest one
// decides.  Otherwise, when group 0 fills whole rounds, group 1 adds rounds of its own; else the
// estimate is the larger of group 0's own rounds and the list-scheduling bound (total work /
// CUs + one group-1 workgroup).  A split group pays for its partials: 2 KiB per row written and
// read back by the merge, plus the split workgroup's own Q load (~0.09 tile-times per 128 rows
// of one split, fitted to forced-split sweeps of a long single stream); a launch with any split
// group pays about 3 tile-times once for the merge launch that covers both groups (measured: a
// merge costs ~3 us).
double plan_cost(const Plan& p, long long units0, long long units1, int cus) {
  const double c0 = p.tiles_per_split[0], c1 = p.tiles_per_split[1];
  const long long n0 = units0 * p.splits[0], n1 = units1 * p.splits[1];
  const double end0 = n0 ? (double)((n0 + cus - 1) / cus) * c0 : 0.0;
  double t = end0;
  if (n0 + n1 <= cus) {
    t = fmax(n0 ? c0 : 0.0, n1 ? c1 : 0.0);
  } else if (n1) {
    if (n0 % cus == 0)
      t = end0 + (double)((n1 + cus - 1) / cus) * c1;
    else
      t = fmax(end0, ((double)n0 * c0 + (double)n1 * c1) / cus + c1);
  }
  const bool split0 = n0 && p.splits[0] > 1, split1 = n1 && p.splits[1] > 1;
  if (split0) t += 0.09 * (double)n0;
  if (split1) t += 0.045 * (double)n1;
  if (split0 || split1) t += 3.0;  // one merge launch covers both groups
  return t;
}

// Workgroup counts and partial rows of a plan whose split counts are set.
void finish_plan(Plan& p, long long units0, long long units1) {
  p.wgs[0] = units0 * p.splits[0];
  p.wgs[1] = units1 * p.splits[1];
  p.part_rows[0] = units0 * 2 * kHeads;
  p.part_rows[1] = units1 * kHeads;
}

size_t workspace_bytes_for(const Plan& p);

// The split plan for these sizes.  An automatic plan (num_splits == 0) only considers plans
// whose partials fit in ws_cap bytes (the unsplit plan needs none, so one always fits).
Plan make_plan(int prefix_len, int q_len, int n_streams, int num_splits, size_t ws_cap = (size_t)-1) {
  Plan p;
  p.n_pairs = q_len / 2;
  p.has_odd = q_len & 1;
  p.n_tiles = (prefix_len + q_len + kTileKeys - 1) / kTileKeys;
  const long long units0 = (long long)n_streams * p.n_pairs;
  const long long units1 = (long long)n_streams * p.has_odd;
  if (num_splits > 0) {
    set_splits(p, 0, num_splits);
    set_splits(p, 1, num_splits);
  } else {
    const int cus = cu_count();
    // Group 1's candidate split counts, normalised once: 1..8 and the larger powers of two
    // (plus, per group-0 count below, that count: the odd node's workgroups then run as long as
    // the pairs').
    int c_splits[12], c_tps[12], n_cand = 0;
    auto add_candidate = [&](int want) {
      Plan q = p;
      set_splits(q, 1, want);
      for (int k = 0; k < n_cand; ++k)
        if (c_splits[k] == q.splits[1] && c_tps[k] == q.tiles_per_split[1]) return;
      c_splits[n_cand] = q.splits[1];
      c_tps[n_cand] = q.tiles_per_split[1];
      ++n_cand;
    };
    if (units1 == 0) {
      add_candidate(1);
    } else {
      for (int s1 = 1; s1 <= 8; ++s1) add_candidate(s1);
      for (int s1 = 16; s1 <= kMaxSplits; s1 *= 2) add_candidate(s1);
    }
    double best = 1e300;
    Plan trial = p;
    auto consider = [&](int splits1, int tps1) {
      trial.splits[1] = splits1;
      trial.tiles_per_split[1] = tps1;
      if (ws_cap != (size_t)-1) {
        finish_plan(trial, units0, units1);
        if (workspace_bytes_for(trial) > ws_cap) return;
      }
      const double c = plan_cost(trial, units0, units1, cus);
      if (c < best - 1e-9) {
        best = c;
        p.splits[0] = trial.splits[0];
        p.tiles_per_split[0] = trial.tiles_per_split[0];
        p.splits[1] = trial.splits[1];
        p.tiles_per_split[1] = trial.tiles_per_split[1];
      }
    };
    for (int s0 = 1; s0 <= 32 && s0 <= p.n_tiles; ++s0) {
      if (units0 == 0 && s0 > 1) break;
      set_splits(trial, 0, s0);
      if (trial.splits[0] != s0) continue;
      for (int k = 0; k < n_cand; ++k) consider(c_splits[k], c_tps[k]);
      if (units1 != 0 && s0 > 8 && (s0 & (s0 - 1)) != 0) {
        Plan q = p;
        set_splits(q, 1, s0);
        consider(q.splits[1], q.tiles_per_split[1]);
      }
    }
  }
  if (p.tiles_per_split[0] == 0) set_splits(p, 0, 1);
  if (p.tiles_per_split[1] == 0) set_splits(p, 1, 1);
  finish_plan(p, units0, units1);
  return p;
}

// Workspace: [group 0 out partials][group 1 out partials][group 0 lse][group 1 lse], each part
// present only when its group is split, every part 256-byte aligned.
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t part_out_bytes(const Plan& p, int g) {
  return p.splits[g] > 1 && p.wgs[g] ? align256((size_t)p.splits[g] * p.part_rows[g] * kDLat * sizeof(float)) : 0;
}
size_t part_lse_bytes(const Plan& p, int g) {
  return p.splits[g] > 1 && p.wgs[g] ? align256((size_t)p.splits[g] * p.part_rows[g] * sizeof(float)) : 0;
}
size_t workspace_bytes_for(const Plan& p) {
  return part_out_bytes(p, 0) + part_out_bytes(p, 1) + part_lse_bytes(p, 0) + part_lse_bytes(p, 1);
}

// Split count reported to callers: the larger of the two groups'.
int reported_splits(const Plan& p) {
  int n = 1;
  for (int g = 0; g < 2; ++g)
    if (p.wgs[g] && p.splits[g] > n) n = p.splits[g];
  return n;
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
  return reported_splits(make_plan(prefix_len, q_len, n_streams, num_splits));
}

size_t ddtree_verify_attn_workspace_size(int prefix_len, int q_len, int n_streams, int num_splits) {
  if (!shape_ok(prefix_len, q_len, n_streams) || num_splits < 0) return 0;
  return workspace_bytes_for(make_plan(prefix_len, q_len, n_streams, num_splits));
}

namespace {

// Split partials of ddtree_verify_attn_noalloc, for callers that cannot allocate: one array per
// GPU, held until the process ends.  Host code never passes the array's name to a kernel (on the
// host it only stands in for the symbol); it passes the device address that hipGetSymbolAddress
// reports for the GPU the launch runs on (the stream's), looked up once per device with that
// device current.
constexpr size_t kScratchBytes = DDTREE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices] = {};

// The scratch address on the GPU of `stream` (the current GPU for the null stream), or an error
// code.  The first call for a device makes that device current for the lookup and restores the
// caller's device afterwards.
int scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return DDTREE_ERR_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return DDTREE_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return DDTREE_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_dev[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return DDTREE_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return DDTREE_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return DDTREE_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return DDTREE_ERR_HIP;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return DDTREE_OK;
}

// ddtree_verify_attn_ex and ddtree_verify_attn_ragged: prefix_lens == nullptr means every stream
// has prefix_len rows of prefix; otherwise prefix_len bounds the per-stream device values.
// use_scratch (ddtree_verify_attn_noalloc): the partials go to this GPU's scratch array instead
// of a caller workspace, and the plan is restricted to partials that fit there.
int verify_impl(const void* q_lat, const void* q_pe, const void* ckv, const void* kpe, int prefix_len,
                const int32_t* prefix_lens, const int32_t* parents, int q_len, int n_streams, float* out_lat,
                float* lse, int kv_rows, float scale, int num_splits, void* workspace, size_t workspace_bytes,
                int32_t* dev_status, hipStream_t stream, bool use_scratch = false) {
  if (!q_lat || !q_pe || !ckv || !kpe || !parents || !out_lat || !lse) return DDTREE_ERR_NULL;
  if (!shape_ok(prefix_len, q_len, n_streams) || num_splits < 0) return DDTREE_ERR_SHAPE;
  if (kv_rows < prefix_len + q_len) return DDTREE_ERR_SHAPE;
  if (!aligned16(q_lat) || !aligned16(q_pe) || !aligned16(ckv) || !aligned16(kpe) || !aligned16(out_lat) ||
      !aligned4(lse) || !aligned4(parents) || (dev_status && !aligned4(dev_status)) ||
      (prefix_lens && !aligned4(prefix_lens)))
    return DDTREE_ERR_ALIGN;
  if (kv_rows > (1 << 21)) return DDTREE_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) scale = 1.0f / sqrtf(192.0f);

  const size_t rows_q = (size_t)n_streams * q_len * kHeads;
  const Range r_out = range_of(out_lat, rows_q * kDLat * sizeof(float));
  const Range r_lse = range_of(lse, rows_q * sizeof(float));
  const Range inputs[] = {
      range_of(q_lat, rows_q * kDLat * 2), range_of(q_pe, rows_q * kDRope * 2),
      range_of(ckv, (size_t)n_streams * kv_rows * kDLat * 2),
      range_of(kpe, (size_t)n_streams * kv_rows * kDRope * 2),
      range_of(parents, (size_t)n_streams * q_len * sizeof(int32_t)),
      range_of(prefix_lens, prefix_lens ? (size_t)n_streams * sizeof(int32_t) : 0)};
  for (const Range& in : inputs)
    if (overlap(in, r_out) || overlap(in, r_lse)) return DDTREE_ERR_ALIAS;
  if (overlap(r_out, r_lse)) return DDTREE_ERR_ALIAS;

  const Plan plan = make_plan(prefix_len, q_len, n_streams, num_splits, use_scratch ? kScratchBytes : (size_t)-1);
  const long long blocks = plan.wgs[0] + plan.wgs[1];
  if (blocks > kMaxGrid) return DDTREE_ERR_SHAPE;

  ddtree::VerifyArgs a{};
  a.q_lat = static_cast<const uint16_t*>(q_lat);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.ckv = static_cast<const uint16_t*>(ckv);
  a.kpe = static_cast<const uint16_t*>(kpe);
  a.parents = parents;
  a.out = out_lat;
  a.lse = lse;
  a.status = dev_status;
  a.prefix_lens = prefix_lens;
  a.prefix_len = prefix_len;
  a.q_len = q_len;
  a.n_streams = n_streams;
  a.kv_rows = kv_rows;
  a.n_pairs = plan.n_pairs;
  a.n_tiles = plan.n_tiles;
  for (int g = 0; g < 2; ++g) {
    a.splits[g] = plan.splits[g];
    a.tiles_per_split[g] = plan.tiles_per_split[g];
  }
  a.wg_count0 = (int)plan.wgs[0];
  // Half of group 1 (whole groups of 8, one per XCD) goes first: see the kernel's dispatch
  // order.  Only worth it with enough group-1 workgroups to shift a sizeable set of CUs.
  a.lead1 = (plan.wgs[0] > 0 && plan.wgs[1] >= 16) ? (int)((plan.wgs[1] / 2) & ~7LL) : 0;
  a.scale_log2e = scale * 1.4426950408889634f;

  const size_t need = workspace_bytes_for(plan);
  if (use_scratch) {
    if (need > kScratchBytes) return DDTREE_ERR_WORKSPACE;  // a forced split count too large
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      const int rc = scratch_address(stream, &workspace);
      if (rc != DDTREE_OK) return rc;
      workspace_bytes = kScratchBytes;
    }
  }
  if (need > 0) {
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return DDTREE_ERR_WORKSPACE;
    const Range r_ws = range_of(workspace, need);
    for (const Range& in : inputs)
      if (overlap(in, r_ws)) return DDTREE_ERR_ALIAS;
    if (overlap(r_ws, r_out) || overlap(r_ws, r_lse)) return DDTREE_ERR_ALIAS;
    char* w = static_cast<char*>(workspace);
    for (int g = 0; g < 2; ++g) {
      a.part_out[g] = part_out_bytes(plan, g) ? reinterpret_cast<float*>(w) : nullptr;
      w += part_out_bytes(plan, g);
    }
    for (int g = 0; g < 2; ++g) {
      a.part_lse[g] = part_lse_bytes(plan, g) ? reinterpret_cast<float*>(w) : nullptr;
      w += part_lse_bytes(plan, g);
    }
  }
  if (ddtree::launch_verify(a, (int)blocks, stream) != hipSuccess) return DDTREE_ERR_HIP;
  if (a.part_out[0] || a.part_out[1]) {  // one merge launch for every split group
    ddtree::CombineArgs c{};
    for (int g = 0; g < 2; ++g) {
      c.part_out[g] = a.part_out[g];
      c.part_lse[g] = a.part_lse[g];
      c.rows[g] = a.part_out[g] ? plan.part_rows[g] : 0;
      c.n_splits[g] = plan.splits[g];
    }
    c.out = out_lat;
    c.lse = lse;
    c.n_pairs = plan.n_pairs;
    c.q_len = q_len;
    if (ddtree::launch_combine(c, stream) != hipSuccess) return DDTREE_ERR_HIP;
  }
  return DDTREE_OK;
}

}  // namespace

int ddtree_verify_attn_ex(const void* q_lat, const void* q_pe, const void* ckv, const void* kpe,
                          int prefix_len, const int32_t* parents, int q_len, int n_streams,
                          float* out_lat, float* lse, int kv_rows, float scale, int num_splits,
                          void* workspace, size_t workspace_bytes, int32_t* dev_status,
                          hipStream_t stream) {
  return verify_impl(q_lat, q_pe, ckv, kpe, prefix_len, nullptr, parents, q_len, n_streams, out_lat, lse, kv_rows,
                     scale, num_splits, workspace, workspace_bytes, dev_status, stream);
}

int ddtree_verify_attn_ragged(const void* q_lat, const void* q_pe, const void* ckv, const void* kpe,
                              const int32_t* prefix_lens, int max_prefix_len, const int32_t* parents, int q_len,
                              int n_streams, float* out_lat, float* lse, int kv_rows, float scale,
                              int num_splits, void* workspace, size_t workspace_bytes, int32_t* dev_status,
                              hipStream_t stream) {
  if (!prefix_lens) return DDTREE_ERR_NULL;
  return verify_impl(q_lat, q_pe, ckv, kpe, max_prefix_len, prefix_lens, parents, q_len, n_streams, out_lat, lse,
                     kv_rows, scale, num_splits, workspace, workspace_bytes, dev_status, stream);
}

int ddtree_verify_attn_noalloc(const void* q_lat, const void* q_pe, const void* ckv, const void* kpe,
                               int prefix_len, const int32_t* parents, int q_len, int n_streams, float* out_lat,
                               float* lse, int kv_rows, float scale, int num_splits, int32_t* dev_status,
                               hipStream_t stream) {
  return verify_impl(q_lat, q_pe, ckv, kpe, prefix_len, nullptr, parents, q_len, n_streams, out_lat, lse, kv_rows,
                     scale, num_splits, nullptr, 0, dev_status, stream, true);
}

int ddtree_verify_attn(const void* q_lat, const void* q_pe, const void* ckv, const void* kpe,
                       int prefix_len, const int32_t* parents, int q_len, int n_streams,
                       float* out_lat, float* lse, hipStream_t stream) {
  return ddtree_verify_attn_ex(q_lat, q_pe, ckv, kpe, prefix_len, parents, q_len, n_streams, out_lat, lse,
                               prefix_len + q_len, 0.f, 1, nullptr, 0, nullptr, stream);
}

namespace {

int compact_impl(const ddtree_kv_cache* cache, int prefix_len, const int32_t* prefix_lens, const int32_t* keep,
                 const int32_t* n_keep, int keep_stride, int32_t* dev_status, hipStream_t stream) {
  if (!cache || !cache->ckv || !cache->kpe || !keep || !n_keep) return DDTREE_ERR_NULL;
  if (cache->n_streams < 1 || cache->kv_rows < 1 || prefix_len < 0 || prefix_len > cache->kv_rows ||
      keep_stride < 1)
    return DDTREE_ERR_SHAPE;
  if (!aligned16(cache->ckv) || !aligned16(cache->kpe) || !aligned4(keep) || !aligned4(n_keep) ||
      (dev_status && !aligned4(dev_status)) || (prefix_lens && !aligned4(prefix_lens)))
    return DDTREE_ERR_ALIGN;
  const Range ckv = range_of(cache->ckv, (size_t)cache->n_streams * cache->kv_rows * kDLat * 2);
  const Range kpe = range_of(cache->kpe, (size_t)cache->n_streams * cache->kv_rows * kDRope * 2);
  if (overlap(ckv, kpe)) return DDTREE_ERR_ALIAS;
  const Range small[3] = {range_of(keep, (size_t)cache->n_streams * keep_stride * 4),
                          range_of(n_keep, (size_t)cache->n_streams * 4),
                          range_of(prefix_lens, prefix_lens ? (size_t)cache->n_streams * 4 : 0)};
  for (const Range& r : small)
    if (overlap(r, ckv) || overlap(r, kpe)) return DDTREE_ERR_ALIAS;
  ddtree::CompactArgs a{};
  a.ckv = static_cast<uint16_t*>(cache->ckv);
  a.kpe = static_cast<uint16_t*>(cache->kpe);
  a.keep = keep;
  a.n_keep = n_keep;
  a.status = dev_status;
  a.prefix_lens = prefix_lens;
  a.kv_rows = cache->kv_rows;
  a.n_streams = cache->n_streams;
  a.prefix_len = prefix_len;
  a.keep_stride = keep_stride;
  if (ddtree::launch_compact(a, stream) != hipSuccess) return DDTREE_ERR_HIP;
  return DDTREE_OK;
}

}  // namespace

int ddtree_compact_kv(const ddtree_kv_cache* cache, int prefix_len, const int32_t* keep,
                      const int32_t* n_keep, int keep_stride, int32_t* dev_status, hipStream_t stream) {
  return compact_impl(cache, prefix_len, nullptr, keep, n_keep, keep_stride, dev_status, stream);
}

int ddtree_compact_kv_ragged(const ddtree_kv_cache* cache, const int32_t* prefix_lens, const int32_t* keep,
                             const int32_t* n_keep, int keep_stride, int32_t* dev_status, hipStream_t stream) {
  if (!prefix_lens) return DDTREE_ERR_NULL;
  return compact_impl(cache, 0, prefix_lens, keep, n_keep, keep_stride, dev_status, stream);
}

}  // extern "C"

namespace {

// Shared argument checks of the acceptance calls.  Returns DDTREE_OK or an error code.
int check_accept(const int32_t* parents, const int32_t* draft_tokens, const int32_t* target_tokens, int q_len,
                 int n_streams, int32_t* keep, int keep_stride, int32_t* n_keep, int32_t* next_token,
                 int32_t* dev_status) {
  if (!parents || !draft_tokens || !target_tokens || !keep || !n_keep) return DDTREE_ERR_NULL;
  if (q_len < 1 || q_len > kMaxQ || n_streams < 1 || keep_stride < q_len) return DDTREE_ERR_SHAPE;
  if (!aligned4(parents) || !aligned4(draft_tokens) || !aligned4(target_tokens) || !aligned4(keep) ||
      !aligned4(n_keep) || (next_token && !aligned4(next_token)) || (dev_status && !aligned4(dev_status)))
    return DDTREE_ERR_ALIGN;
  const size_t in_bytes = (size_t)n_streams * q_len * 4;
  const Range ins[3] = {range_of(parents, in_bytes), range_of(draft_tokens, in_bytes), range_of(target_tokens, in_bytes)};
  Range outs[3] = {range_of(keep, (size_t)n_streams * keep_stride * 4), range_of(n_keep, (size_t)n_streams * 4),
                   range_of(next_token, next_token ? (size_t)n_streams * 4 : 0)};
  const int n_out = next_token ? 3 : 2;
  for (int o = 0; o < n_out; ++o) {
    for (const Range& r : ins)
      if (overlap(outs[o], r)) return DDTREE_ERR_ALIAS;
    for (int o2 = o + 1; o2 < n_out; ++o2)
      if (overlap(outs[o], outs[o2])) return DDTREE_ERR_ALIAS;
  }
  return DDTREE_OK;
}

ddtree::AcceptArgs accept_args(const int32_t* parents, const int32_t* draft_tokens, const int32_t* target_tokens,
                               int q_len, int n_streams, int32_t* keep, int keep_stride, int32_t* n_keep,
                               int32_t* next_token, int32_t* dev_status) {
  ddtree::AcceptArgs a{};
  a.parents = parents;
  a.draft = draft_tokens;
  a.target = target_tokens;
  a.keep = keep;
  a.n_keep = n_keep;
  a.next_token = next_token;
  a.status = dev_status;
  a.q_len = q_len;
  a.n_streams = n_streams;
  a.keep_stride = keep_stride;
  return a;
}

}  // namespace

int ddtree_tree_accept(const int32_t* parents, const int32_t* draft_tokens, const int32_t* target_tokens,
                       int q_len, int n_streams, int32_t* keep, int keep_stride, int32_t* n_keep,
                       int32_t* next_token, int32_t* dev_status, hipStream_t stream) {
  const int rc = check_accept(parents, draft_tokens, target_tokens, q_len, n_streams, keep, keep_stride, n_keep,
                              next_token, dev_status);
  if (rc != DDTREE_OK) return rc;
  const ddtree::AcceptArgs a = accept_args(parents, draft_tokens, target_tokens, q_len, n_streams, keep,
                                           keep_stride, n_keep, next_token, dev_status);
  if (ddtree::launch_accept(a, stream) != hipSuccess) return DDTREE_ERR_HIP;
  return DDTREE_OK;
}

namespace {

int accept_compact_impl(const ddtree_kv_cache* cache, int prefix_len, int32_t* prefix_lens, const int32_t* parents,
                        const int32_t* draft_tokens, const int32_t* target_tokens, int q_len, int32_t* keep,
                        int keep_stride, int32_t* n_keep, int32_t* next_token, int32_t* dev_status,
                        hipStream_t stream) {
  if (!cache || !cache->ckv || !cache->kpe) return DDTREE_ERR_NULL;
  int rc = check_accept(parents, draft_tokens, target_tokens, q_len, cache->n_streams, keep, keep_stride,
                        n_keep, next_token, dev_status);
  if (rc != DDTREE_OK) return rc;
  if (cache->n_streams < 1 || cache->kv_rows < 1 || prefix_len < 0 ||
      (long long)prefix_len + q_len > (long long)cache->kv_rows)
    return DDTREE_ERR_SHAPE;
  if (!aligned16(cache->ckv) || !aligned16(cache->kpe) || (prefix_lens && !aligned4(prefix_lens)))
    return DDTREE_ERR_ALIGN;
  const Range ckv = range_of(cache->ckv, (size_t)cache->n_streams * cache->kv_rows * kDLat * 2);
  const Range kpe = range_of(cache->kpe, (size_t)cache->n_streams * cache->kv_rows * kDRope * 2);
  if (overlap(ckv, kpe)) return DDTREE_ERR_ALIAS;
  const size_t in_bytes = (size_t)cache->n_streams * q_len * 4;
  const Range r_pl = range_of(prefix_lens, prefix_lens ? (size_t)cache->n_streams * 4 : 0);
  const Range others[7] = {range_of(parents, in_bytes), range_of(draft_tokens, in_bytes),
                           range_of(target_tokens, in_bytes),
                           range_of(keep, (size_t)cache->n_streams * keep_stride * 4),
                           range_of(n_keep, (size_t)cache->n_streams * 4),
                           range_of(next_token, next_token ? (size_t)cache->n_streams * 4 : 0), r_pl};
  for (const Range& r : others)
    if (overlap(r, ckv) || overlap(r, kpe)) return DDTREE_ERR_ALIAS;
  for (int o = 0; o < 6; ++o)
    if (overlap(others[o], r_pl)) return DDTREE_ERR_ALIAS;
  ddtree::AcceptArgs a = accept_args(parents, draft_tokens, target_tokens, q_len, cache->n_streams, keep,
                                     keep_stride, n_keep, next_token, dev_status);
  a.ckv = static_cast<uint16_t*>(cache->ckv);
  a.kpe = static_cast<uint16_t*>(cache->kpe);
  a.kv_rows = cache->kv_rows;
  a.prefix_len = prefix_len;
  a.prefix_lens = prefix_lens;
  if (ddtree::launch_accept_compact(a, stream) != hipSuccess) return DDTREE_ERR_HIP;
  return DDTREE_OK;
}

}  // namespace

int ddtree_accept_compact(const ddtree_kv_cache* cache, int prefix_len, const int32_t* parents,
                          const int32_t* draft_tokens, const int32_t* target_tokens, int q_len,
                          int32_t* keep, int keep_stride, int32_t* n_keep, int32_t* next_token,
                          int32_t* dev_status, hipStream_t stream) {
  return accept_compact_impl(cache, prefix_len, nullptr, parents, draft_tokens, target_tokens, q_len, keep,
                             keep_stride, n_keep, next_token, dev_status, stream);
}

int ddtree_accept_compact_ragged(const ddtree_kv_cache* cache, int32_t* prefix_lens, const int32_t* parents,
                                 const int32_t* draft_tokens, const int32_t* target_tokens, int q_len,
                                 int32_t* keep, int keep_stride, int32_t* n_keep, int32_t* next_token,
                                 int32_t* dev_status, hipStream_t stream) {
  if (!prefix_lens) return DDTREE_ERR_NULL;
  return accept_compact_impl(cache, 0, prefix_lens, parents, draft_tokens, target_tokens, q_len, keep, keep_stride,
                             n_keep, next_token, dev_status, stream);
}

namespace {

// Shared checks of the multi-layer calls: the layer table, its common geometry, alignment, and
// that no two caches (and no cache and small array) overlap.  Fills the pointer tables of `a`.
int check_layers(const ddtree_kv_cache* caches, int n_layers, const Range* small, int n_small,
                 ddtree::LayersArgs* a) {
  if (!caches) return DDTREE_ERR_NULL;
  if (n_layers < 1 || n_layers > ddtree::kMaxLayers) return DDTREE_ERR_SHAPE;
  const int kv_rows = caches[0].kv_rows, n_streams = caches[0].n_streams;
  if (kv_rows < 1 || n_streams < 1) return DDTREE_ERR_SHAPE;
  Range r[2 * ddtree::kMaxLayers];
  for (int l = 0; l < n_layers; ++l) {
    const ddtree_kv_cache& c = caches[l];
    if (!c.ckv || !c.kpe) return DDTREE_ERR_NULL;
    if (c.kv_rows != kv_rows || c.n_streams != n_streams) return DDTREE_ERR_SHAPE;
    if (!aligned16(c.ckv) || !aligned16(c.kpe)) return DDTREE_ERR_ALIGN;
    r[2 * l] = range_of(c.ckv, (size_t)n_streams * kv_rows * kDLat * 2);
    r[2 * l + 1] = range_of(c.kpe, (size_t)n_streams * kv_rows * kDRope * 2);
    a->ckv[l] = static_cast<uint16_t*>(c.ckv);
    a->kpe[l] = static_cast<uint16_t*>(c.kpe);
  }
  // No two caches overlap: sorted by start, each range must end before the next one starts.
  std::sort(r, r + 2 * n_layers, [](const Range& x, const Range& y) { return x.lo < y.lo; });
  for (int i = 0; i + 1 < 2 * n_layers; ++i)
    if (overlap(r[i], r[i + 1])) return DDTREE_ERR_ALIAS;
  for (int i = 0; i < 2 * n_layers; ++i)
    for (int k = 0; k < n_small; ++k)
      if (overlap(r[i], small[k])) return DDTREE_ERR_ALIAS;
  a->kv_rows = kv_rows;
  a->n_streams = n_streams;
  a->n_layers = n_layers;
  // Layers per workgroup: about four resident workgroups per compute unit in all, so that the
  // whole grid is in flight at once and each workgroup pays the load -> barrier -> store latency
  // about once.
  const long long target = 4LL * cu_count();
  const long long per = ((long long)n_layers * n_streams + target - 1) / target;
  a->layers_per_wg = (int)(per < 1 ? 1 : (per > n_layers ? n_layers : per));
  return DDTREE_OK;
}

}  // namespace

int ddtree_compact_kv_layers(const ddtree_kv_cache* caches, int n_layers, int prefix_len, const int32_t* prefix_lens,
                             const int32_t* keep, const int32_t* n_keep, int keep_stride, int32_t* dev_status,
                             hipStream_t stream) {
  if (!caches || !keep || !n_keep) return DDTREE_ERR_NULL;
  if (keep_stride < 1 || (!prefix_lens && prefix_len < 0)) return DDTREE_ERR_SHAPE;
  if (!aligned4(keep) || !aligned4(n_keep) || (dev_status && !aligned4(dev_status)) ||
      (prefix_lens && !aligned4(prefix_lens)))
    return DDTREE_ERR_ALIGN;
  const int n_streams = caches[0].n_streams;
  if (n_streams < 1) return DDTREE_ERR_SHAPE;
  const Range small[4] = {range_of(keep, (size_t)n_streams * keep_stride * 4), range_of(n_keep, (size_t)n_streams * 4),
                          range_of(prefix_lens, prefix_lens ? (size_t)n_streams * 4 : 0),
                          range_of(dev_status, dev_status ? 4 : 0)};
  ddtree::LayersArgs a{};
  const int rc = check_layers(caches, n_layers, small, 4, &a);
  if (rc != DDTREE_OK) return rc;
  if (!prefix_lens && prefix_len > a.kv_rows) return DDTREE_ERR_SHAPE;
  a.keep = const_cast<int32_t*>(keep);  // read only in this call
  a.n_keep = const_cast<int32_t*>(n_keep);
  a.status = dev_status;
  a.prefix_lens = const_cast<int32_t*>(prefix_lens);
  a.prefix_len = prefix_lens ? 0 : prefix_len;
  a.keep_stride = keep_stride;
  if (ddtree::launch_compact_layers(a, stream) != hipSuccess) return DDTREE_ERR_HIP;
  return DDTREE_OK;
}

int ddtree_accept_compact_layers(const ddtree_kv_cache* caches, int n_layers, int prefix_len, int32_t* prefix_lens,
                                 const int32_t* parents, const int32_t* draft_tokens, const int32_t* target_tokens,
                                 int q_len, int32_t* keep, int keep_stride, int32_t* n_keep, int32_t* next_token,
                                 int32_t* dev_status, hipStream_t stream) {
  if (!caches) return DDTREE_ERR_NULL;
  const int n_streams = caches[0].n_streams;
  if (n_streams < 1) return DDTREE_ERR_SHAPE;
  int rc = check_accept(parents, draft_tokens, target_tokens, q_len, n_streams, keep, keep_stride, n_keep,
                        next_token, dev_status);
  if (rc != DDTREE_OK) return rc;
  if (prefix_lens && !aligned4(prefix_lens)) return DDTREE_ERR_ALIGN;
  const size_t in_bytes = (size_t)n_streams * q_len * 4;
  const Range small[8] = {range_of(parents, in_bytes), range_of(draft_tokens, in_bytes),
                          range_of(target_tokens, in_bytes), range_of(keep, (size_t)n_streams * keep_stride * 4),
                          range_of(n_keep, (size_t)n_streams * 4),
                          range_of(next_token, next_token ? (size_t)n_streams * 4 : 0),
                          range_of(dev_status, dev_status ? 4 : 0),
                          range_of(prefix_lens, prefix_lens ? (size_t)n_streams * 4 : 0)};
  for (int o = 0; o < 7; ++o)
    if (overlap(small[o], small[7])) return DDTREE_ERR_ALIAS;
  ddtree::LayersArgs a{};
  rc = check_layers(caches, n_layers, small, 8, &a);
  if (rc != DDTREE_OK) return rc;
  const int p0 = prefix_lens ? 0 : prefix_len;
  if (p0 < 0 || (long long)p0 + q_len > (long long)a.kv_rows) return DDTREE_ERR_SHAPE;
  a.parents = parents;
  a.draft = draft_tokens;
  a.target = target_tokens;
  a.keep = keep;
  a.n_keep = n_keep;
  a.next_token = next_token;
  a.status = dev_status;
  a.prefix_lens = prefix_lens;
  a.prefix_len = p0;
  a.q_len = q_len;
  a.keep_stride = keep_stride;
  if (ddtree::launch_accept_compact_layers(a, stream) != hipSuccess) return DDTREE_ERR_HIP;
  return DDTREE_OK;
}

int ddtree_append_tree_kv(const ddtree_kv_cache* cache, int prefix_len, const int32_t* prefix_lens,
                          const int32_t* parents, int q_len, const float* kv, const float* norm_weight, float eps,
                          const float* rope_cos, const float* rope_sin, int rope_rows, int32_t* dev_status,
                          hipStream_t stream) {
  if (!cache || !cache->ckv || !cache->kpe || !parents || !kv || !norm_weight || !rope_cos || !rope_sin)
    return DDTREE_ERR_NULL;
  const int S = cache->n_streams;
  if (S < 1 || cache->kv_rows < 1 || q_len < 1 || q_len > kMaxQ || q_len > cache->kv_rows || rope_rows < 1 ||
      !(eps >= 0.f) || !isfinite(eps))
    return DDTREE_ERR_SHAPE;
  if (!prefix_lens && (prefix_len < 0 || (long long)prefix_len + q_len > (long long)cache->kv_rows))
    return DDTREE_ERR_SHAPE;
  if (!aligned16(cache->ckv) || !aligned16(cache->kpe) || !aligned16(kv) || !aligned16(norm_weight) ||
      !aligned4(rope_cos) || !aligned4(rope_sin) || !aligned4(parents) || (prefix_lens && !aligned4(prefix_lens)) ||
      (dev_status && !aligned4(dev_status)))
    return DDTREE_ERR_ALIGN;
  const Range ckv = range_of(cache->ckv, (size_t)S * cache->kv_rows * kDLat * 2);
  const Range kpe = range_of(cache->kpe, (size_t)S * cache->kv_rows * kDRope * 2);
  if (overlap(ckv, kpe)) return DDTREE_ERR_ALIAS;
  const Range ins[7] = {range_of(kv, (size_t)S * q_len * (kDLat + kDRope) * 4), range_of(norm_weight, kDLat * 4),
                        range_of(rope_cos, (size_t)rope_rows * 32 * 4), range_of(rope_sin, (size_t)rope_rows * 32 * 4),
                        range_of(parents, (size_t)S * q_len * 4),
                        range_of(prefix_lens, prefix_lens ? (size_t)S * 4 : 0),
                        range_of(dev_status, dev_status ? 4 : 0)};
  for (const Range& r : ins)
    if (overlap(r, ckv) || overlap(r, kpe)) return DDTREE_ERR_ALIAS;
  if (overlap(ins[6], ins[0]) || overlap(ins[6], ins[4]) || overlap(ins[6], ins[5])) return DDTREE_ERR_ALIAS;
  ddtree::AppendArgs a{};
  a.kv = kv;
  a.weight = norm_weight;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.parents = parents;
  a.prefix_lens = prefix_lens;
  a.ckv = static_cast<uint16_t*>(cache->ckv);
  a.kpe = static_cast<uint16_t*>(cache->kpe);
  a.status = dev_status;
  a.eps = eps;
  a.prefix_len = prefix_lens ? 0 : prefix_len;
  a.q_len = q_len;
  a.n_streams = S;
  a.kv_rows = cache->kv_rows;
  a.rope_rows = rope_rows;
  if (ddtree::launch_append(a, stream) != hipSuccess) return DDTREE_ERR_HIP;
  return DDTREE_OK;
}

int ddtree_tree_build(const float* logprobs, const int32_t* topk_tokens, const int32_t* root_tokens, int depth,
                      int topk, int budget, int n_streams, int32_t* parents, int32_t* node_tokens,
                      int32_t* n_nodes, int32_t* depths, float* logw, int32_t* first_child,
                      int32_t* next_sibling, uint64_t* anc, hipStream_t stream) {
  if (!logprobs || !topk_tokens || !parents || !node_tokens || !n_nodes) return DDTREE_ERR_NULL;
  if (depth < 1 || depth > 64 || topk < 1 || topk > 64 || budget < 1 || budget > kMaxQ - 1 || n_streams < 1)
    return DDTREE_ERR_SHAPE;
  if (!aligned4(logprobs) || !aligned4(topk_tokens) || (root_tokens && !aligned4(root_tokens)) ||
      !aligned4(parents) || !aligned4(node_tokens) || !aligned4(n_nodes) || (depths && !aligned4(depths)) ||
      (logw && !aligned4(logw)) || (first_child && !aligned4(first_child)) ||
      (next_sibling && !aligned4(next_sibling)) || (anc && (reinterpret_cast<uintptr_t>(anc) & 7u)))
    return DDTREE_ERR_ALIGN;
  const size_t q = (size_t)budget + 1, S = (size_t)n_streams;
  const size_t in_bytes = S * depth * topk * 4;
  const Range ins[3] = {range_of(logprobs, in_bytes), range_of(topk_tokens, in_bytes),
                        range_of(root_tokens, root_tokens ? S * 4 : 0)};
  const Range outs[8] = {range_of(parents, S * q * 4), range_of(node_tokens, S * q * 4), range_of(n_nodes, S * 4),
                         range_of(depths, depths ? S * q * 4 : 0), range_of(logw, logw ? S * q * 4 : 0),
                         range_of(first_child, first_child ? S * q * 4 : 0),
                         range_of(next_sibling, next_sibling ? S * q * 4 : 0), range_of(anc, anc ? S * q * 8 : 0)};
  for (int o = 0; o < 8; ++o) {
    for (const Range& r : ins)
      if (overlap(outs[o], r)) return DDTREE_ERR_ALIAS;
    for (int o2 = o + 1; o2 < 8; ++o2)
      if (overlap(outs[o], outs[o2])) return DDTREE_ERR_ALIAS;
  }
  ddtree::BuildArgs a{};
  a.lp = logprobs;
  a.tok = topk_tokens;
  a.root_tok = root_tokens;
  a.parents = parents;
  a.tokens = node_tokens;
  a.n_nodes = n_nodes;
  a.depths = depths;
  a.logw = logw;
  a.first_child = first_child;
  a.next_sibling = next_sibling;
  a.anc = reinterpret_cast<unsigned long long*>(anc);
  a.depth = depth;
  a.topk = topk;
  a.budget = budget;
  a.n_streams = n_streams;
  if (ddtree::launch_build(a, stream) != hipSuccess) return DDTREE_ERR_HIP;
  return DDTREE_OK;
}
