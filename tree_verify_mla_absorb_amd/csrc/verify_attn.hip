// Tree-verify MLA-absorb attention for gfx950 (MI355X).
//
// The operation ("Race Conditions, Buffer Aliasing, and the Architecture of a Native DDTree
// Inference Engine", section "The Mission: A Native DDTree Engine"): every draft-tree node of a
// stream, for all 64 heads, attends over one latent KV cache shared by the heads -- the
// committed prefix followed by the appended tree block (section "The Cache Compaction Problem":
// node i lives in row prefix + i and a parent index is always smaller than its child's).  A node
// sees the whole prefix plus its own ancestor-or-self tree rows.
//
// The pages' first kernel re-read the shared latent cache once per head ("The Microsecond
// Verdict", section "The Timeout That Tells a Story": 64x the bandwidth).  Here each key tile is
// staged into LDS once per workgroup and consumed by all 128 query-head rows of that workgroup
// as bf16 MFMA contractions:
//
//   S^T[key, qh] = K[key, 0:576] . Q^T[0:576, qh]          (A = K from LDS, B = Q)
//   O^T[dim, qh] += V^T[dim, key] . P^T[key, qh]            (A = V^T via LDS transpose reads,
//                                                            B = P^T, published through LDS)
//
// Computing S^T (keys as MFMA rows) puts one query-head column in each lane, so the softmax
// statistics are per-lane values plus one cross-half exchange, and the accumulator layout of
// S^T is already the B-operand layout the PV product needs (the key order inside each 16-key
// contraction is permuted identically on the V side).
//
// Workgroup = 4 waves over 2 tree nodes x 64 heads = 4 head blocks of 32 query-heads.  For the
// scores, wave w owns head block w: node (first + w / 2), heads 32 (w & 1) .. +31, so the tree
// mask is wave-uniform -- one 64-bit ancestor-or-self mask, built from one load of parents[]
// by a fixed number of pointer-jumping steps, so no input can make it run long (the bounded-
// walk lesson of "The Microsecond Verdict", section "The Crash That Demanded a Fix").  For the
// value product the waves split the 512 latent dims instead
// (wave w: dims 128 w .. +127 of all four head blocks) and share the probabilities through
// LDS, so each V^T fragment read feeds four MFMAs.
//
// Pipeline, per 32-key tile t (one workgroup barrier per tile):
//   wait for tile t's rows, barrier, start staging tile t + 1 (three LDS stages in a ring),
//   scores of tile t, then the value product of tile t - 1 (whose probabilities were published
//   before the barrier) next to the softmax of tile t, then publish tile t's probabilities.

#include "kernels.h"

#include <math.h>

#include "../../include/ddtree.h"

namespace ddtree {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float F32x4 __attribute__((ext_vector_type(4)));

// LDS layout.
//   stage s (ring of three), one 32-key tile each:
//     latent: 32 rows x 1040 B (1024 B of c_kv + 16 B pad).  Key k lives in row rho(k), rho
//         swapping the two 2-bit halves of k's low nibble.  With the pad, the 16 rows read by
//         one ds_read_b128 phase land on 16 distinct bank quads and the 4 rows x 64 B read by
//         32 lanes of a ds_read_b64_tr_b16 land on 4 distinct 16-bank groups; every address is
//         a per-lane base plus an immediate.
//     rotary: chunk-major, [16-byte chunk 8][key 32][16 B]: the 16 keys read by one
//         ds_read_b128 phase are 256 contiguous bytes.
//   P buffers (two): bf16 probabilities of a tile, [head block 4][16-key slice 2][lane 64][16 B],
//       written by the wave that computed the scores and read by all four waves.
//   rotary queries: [wave 4][k-step 4][lane 64][16 B], staged once.
constexpr int kRowBytesGlobal = kDLat * 2;                // 1024 B per c_kv row in HBM
constexpr int kRowStride = kRowBytesGlobal + 16;          // 1040 B per latent row in LDS
constexpr int kRopeRowBytes = kDRope * 2;                 // 128 B per k_pe row in HBM
constexpr int kLatBytes = kTileKeys * kRowStride;         // 33280 B
constexpr int kRopeBytes = kTileKeys * kRopeRowBytes;     // 4096 B
constexpr int kStageBytes = kLatBytes + kRopeBytes;       // 37376 B
constexpr int kStages = 3;
constexpr int kPBytes = 4 * 2 * 64 * 16;                  // 8 KiB per buffer
constexpr int kPOff = kStages * kStageBytes;
constexpr int kQpeOff = kPOff + 2 * kPBytes;
constexpr int kSmemBytes = kQpeOff + 4 * 4 * 64 * 16;     // 144896 B
// Output transpose area of a wave at the end: 32 rows x (128 fp32 + 16 B pad), inside the stages.
constexpr int kTRow = 128 * 4 + 16;
static_assert(4 * 32 * kTRow <= kPOff, "the output transpose areas must not reach the P buffers");
// Scores are exponentiated against a per-head reference max taken from the first 32 keys.
// If the true max ends above ref + kRefHi or below ref - kRefLo (log2 units) the workgroup
// repeats its key range once with the exact max as reference.  Inside the window every
// probability stays within [2^-kRefLo, 2^kRefHi] of the reference, far from fp32/bf16 limits,
// and no accumulator is ever rescaled.
constexpr float kRefHi = 64.0f;
constexpr float kRefLo = 32.0f;
constexpr float kLn2 = 0.69314718055994530942f;
// Buffer resource word 3 for gfx9-family raw (untyped, stride 0) buffers.
constexpr int kBufferDword3 = 0x00020000;
// s_waitcnt immediate for vmcnt(0) alone (gfx9 encoding: expcnt and lgkmcnt fields at their
// maximum).  Issued through the builtin, the compiler's own wait tracking sees it and drops
// any later wait it would otherwise place inside the key loop for its own loads.
constexpr int kWaitVmcnt0 = 0x0F70;
// Score operands read ahead of the MFMA that consumes them, in k-steps.
constexpr int kKAhead = 4;
// Staging instructions per wave and tile: 8 latent rows and one rotary instruction.
constexpr int kStageInstrs = kTileKeys / 4 + 1;
// Staging instructions of the next tile issued inside the score chain (one every kDmaEvery
// k-steps); the rest go into the first value steps.
constexpr int kDmaEvery = 5;
constexpr int kDmaInScores = 7;
// In a one-node workgroup the two waves of a head block split its score chain: waves 0, 1 take
// the 4 rotary and the first 14 latent k-steps, waves 2, 3 the last 18 latent ones, and the
// halves meet through LDS.  A half chain carries a staging instruction every kDmaEveryHalf
// k-steps, kDmaInHalf of them.
constexpr int kSplitStep = 18;
constexpr int kDmaEveryHalf = 3;
constexpr int kDmaInHalf = 6;
// Value step that reads the probabilities of the second 16-key slice.
constexpr int kP1Step = 3;

static_assert(kTileKeys == 32, "the layout above is written for 32-key tiles");

__device__ __forceinline__ int rho(int k) { return (k & ~15) | ((k & 3) << 2) | ((k >> 2) & 3); }

// Raw buffer resource over `bytes` bytes at `base` (stride 0, untyped).
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, unsigned bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  return i32x4{(int)(unsigned)a, (int)((a >> 32) & 0xffffu), (int)bytes, kBufferDword3};
}

// One wave instruction of direct global->LDS staging: lane i's 16 bytes at
// rsrc + soff + voff land at LDS byte lds_addr + 16 i.  Issued from asm so that the compiler
// neither orders later LDS reads of other stages behind it nor folds it into its own wait
// counting; the consumer waits on vmcnt explicitly and crosses a workgroup barrier before
// reading the stage this wrote.  The loop issues no other vector-memory instruction.
__device__ __forceinline__ void dma16(unsigned lds_addr, i32x4 rsrc, int voff, int soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

// One k-step of the score chain, S^T += K Q^T, with the accumulator in VGPRs.  Issued from
// asm because the compiler gives every MFMA of this kernel an AGPR accumulator, and an AGPR
// score tile would evict a block of O^T (which fills all 256 AGPRs) on every key tile.  The
// chain accumulates in place (the source C operand is the destination itself, which the
// matrix core forwards back to back); the first step starts from 0.  The last step ends with
// 18 wait states so that the VALU reads of the scores that follow see the final result
// (an 8-pass XDL result needs 12 before a VALU read on gfx950).
__device__ __forceinline__ void score_step(f32x16& st, const bf16x8& k, const bf16x8& q, bool first, bool last) {
  if (first)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(st) : "v"(k), "v"(q));
  else if (last)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 1"
                 : "+v"(st) : "v"(k), "v"(q));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(st) : "v"(k), "v"(q));
}

// Combine the two lane halves that hold the same head (lanes l and l ^ 32).
__device__ __forceinline__ float half_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float half_sum(float x) { return x + __shfl_xor(x, 32); }

// Ragged launches: the stream that logical stream ls stands for.  Each XCD runs a contiguous
// run of logical streams; with per-stream prefixes of different lengths, runs of consecutive
// streams carry unequal work and the busiest XCD sets the launch time.  So the streams are
// ranked by prefix length (longest first, ties by index; an invalid entry counts as 0) and the
// ranks are dealt to the 8 runs in snake order -- runs 0..7 take ranks 0..7, runs 7..0 ranks
// 8..15, and so on, with a last partial round for n_streams % 8 -- which evens out the runs'
// totals; within a run the streams come longest first.  One stream per lane: at most 64 streams.
// Every wave of the launch computes the same mapping.
__device__ __forceinline__ int balanced_stream(const int32_t* prefix_lens, int n_streams, int max_prefix, int ls,
                                               int lane) {
  const int S = n_streams;
  int len = -1;
  if (lane < S) {
    const int pv = prefix_lens[lane];
    len = (pv < 0 || pv > max_prefix) ? 0 : pv;
  }
  int rank = 0;
  for (int j = 0; j < S; ++j) {
    const int lj = __builtin_amdgcn_readlane(len, j);
    rank += (lj > len || (lj == len && j < lane)) ? 1 : 0;
  }
  // run b holds S / 8 streams from the full rounds, plus one from the partial round when that
  // round (forward after an even number of full rounds, backward after an odd one) reaches it
  const int full = S >> 3, part = S & 7;
  int b = 0, start = 0;
  for (; b < 7; ++b) {
    const int extra = part == 0 ? 0 : ((full & 1) == 0 ? (b < part) : (b >= 8 - part));
    if (ls < start + full + extra) break;
    start += full + extra;
  }
  const int i = ls - start;
  const int rk = 8 * i + ((i & 1) ? 7 - b : b);
  const unsigned long long m = __builtin_amdgcn_ballot_w64(lane < S && rank == rk);
  return m != 0 ? (int)__builtin_ctzll(m) : ls;
}

template <bool B>
struct Flag {
  static constexpr bool value = B;
};
// k-steps [A, B) of the score chain
template <int A, int B>
struct Steps {
  static constexpr int u0 = A, u1 = B;
};

__global__ void __attribute__((amdgpu_flat_work_group_size(kWGThreads, kWGThreads),
                               amdgpu_waves_per_eu(1, 1)))
verify_attn_kernel(VerifyArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmemBytes];
  __shared__ int redo_s;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c32 = lane & 31;
  const int g = lane >> 5;

  // Group and position of this workgroup.  Dispatch order: the first lead1 workgroups of group
  // 1, all of group 0, then the rest of group 1.  Workgroups of equal length run in lockstep,
  // and their Q loads at the start and output stores at the end then hit HBM all at once; the
  // short group-1 workgroups in front shift half of the compute units by one of them, so the
  // two halves reach those bursts at different times.  Workgroup b is dispatched to XCD b % 8;
  // within a group the index is renumbered so that each XCD runs a contiguous run of (stream,
  // node pair, split) units: the workgroups of one stream then share that XCD's L2 while they
  // stream the same key tiles, and the light workgroups of group 1 spread over all XCDs.  In a
  // ragged launch the logical stream is mapped to a real one by length (balanced_stream).
  const int b_id = (int)blockIdx.x;
  const int grp = (b_id >= a.lead1 && b_id < a.lead1 + a.wg_count0) ? 0 : 1;
  const int j = grp == 0 ? b_id - a.lead1 : (b_id < a.lead1 ? b_id : b_id - a.wg_count0);
  const int cnt = grp == 0 ? a.wg_count0 : (int)gridDim.x - a.wg_count0;
  const int xcd = j & 7;
  const int per = cnt >> 3, rem = cnt & 7;
  const int logical = xcd * per + min(xcd, rem) + (j >> 3);
  const int n_split = a.splits[grp];
  const int sp = logical % n_split;
  const int unit = logical / n_split;
  const int ls = grp == 0 ? unit / max(a.n_pairs, 1) : unit;  // logical stream
  const int s = (a.prefix_lens != nullptr && a.n_streams <= 64)
                    ? balanced_stream(a.prefix_lens, a.n_streams, a.prefix_len, ls, lane)
                    : ls;
  const int pair = grp == 0 ? unit - ls * a.n_pairs : 0;
  const int q0 = grp == 0 ? 2 * pair : a.q_len - 1;  // first node of the workgroup
  const int n_nodes = grp == 0 ? 2 : 1;

  // Prefix length of this stream: uniform, or read per stream (bounded by prefix_len; a value
  // outside [0, prefix_len] is flagged, its stream computed with an empty prefix and poisoned).
  int P = a.prefix_len;
  bool bad_prefix = false;
  if (a.prefix_lens != nullptr) {
    const int pv = __builtin_amdgcn_readfirstlane(a.prefix_lens[s]);
    bad_prefix = pv < 0 || pv > a.prefix_len;
    P = bad_prefix ? 0 : pv;
  }
  const int Q = a.q_len;
  const int L = P + Q;
  const int qi = q0 + (wave >> 1);
  const bool active = (wave >> 1) < n_nodes;  // group 1: head blocks 2, 3 compute a copy
  const int qc = active ? qi : q0;
  const int head = (wave & 1) * 32 + c32;
  // row of (node q0 + k, head h) in this group's partial buffers
  auto part_row = [&](int k, int h) { return grp == 0 ? ((s * a.n_pairs + pair) * 2 + k) * kHeads + h : s * kHeads + h; };

  // Ancestor-or-self masks of the whole tree, node j in lane j, from one load of parents[]:
  // six pointer-jumping steps (mask |= mask[up]; up = up[up]) cover any chain of at most 64
  // nodes.  A node whose parent entry is not an earlier node (or a root with a parent) links
  // to itself, so its chain stops there, as a walk that stops at the bad entry would.
  uint64_t anc;
  bool bad;
  {
    const bool in = lane < Q;
    const int pn = in ? a.parents[(size_t)s * Q + lane] : -1;
    const bool ok = !in || (lane == 0 ? pn == -1 : (pn >= 0 && pn < lane));
    bad = __builtin_amdgcn_ballot_w64(!ok) != 0;
    int up = (in && ok && lane != 0) ? pn : lane;
    unsigned lo = in ? (lane < 32 ? 1u << lane : 0u) : 0u;
    unsigned hi = in ? (lane >= 32 ? 1u << (lane - 32) : 0u) : 0u;
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      lo |= __shfl(lo, up);
      hi |= __shfl(hi, up);
      up = __shfl(up, up);
    }
    anc = (uint64_t)(unsigned)__builtin_amdgcn_readlane((int)lo, qc) |
          ((uint64_t)(unsigned)__builtin_amdgcn_readlane((int)hi, qc) << 32);
  }
  if (bad && a.status != nullptr && threadIdx.x == 0) atomicOr(a.status, DDTREE_STATUS_BAD_PARENTS);
  if (bad_prefix && a.status != nullptr && threadIdx.x == 0) atomicOr(a.status, DDTREE_STATUS_BAD_PREFIX);

  // Staging of this stream's cache rows.  A latent row is one wave instruction (64 lanes x
  // 16 B); the rotary instruction of wave w moves 16-byte chunks 2w, 2w + 1 of all 32 rows
  // (lanes 0-31: chunk 2w, lanes 32-63: chunk 2w + 1, lane & 31 = key).  Rows past the end of
  // the cache are clamped to the last row: their scores are masked out.
  const i32x4 ckv_rs = buffer_rsrc(a.ckv + (size_t)s * a.kv_rows * kDLat, (unsigned)a.kv_rows * kDLat * 2);
  const i32x4 kpe_rs = buffer_rsrc(a.kpe + (size_t)s * a.kv_rows * kDRope, (unsigned)a.kv_rows * kDRope * 2);
  const i32x4 ckv_none = buffer_rsrc(a.ckv, 0u), kpe_none = buffer_rsrc(a.kpe, 0u);
  const unsigned smem_base = (unsigned)(size_t)((__attribute__((address_space(3))) unsigned char*)smem);
  const int lane16 = lane << 4;
  const int rope_lane = (lane & 31) * kRopeRowBytes + (lane >> 5) * 16;  // key row + chunk parity
  // Wave instruction j of staging tile t into stage stg: j < 8 moves latent row 8 wave + j,
  // j = 8 the wave's rotary chunks.  With empty resources (0 bytes) every lane is out of
  // range: the instruction reads no memory, which lets the key loop issue it unconditionally.
  auto stage_part = [&](int t, int stg, int j, const i32x4& crs, const i32x4& krs) __attribute__((always_inline)) {
    const unsigned base = smem_base + stg * kStageBytes;
    const int key0 = t * kTileKeys;
    if (j < kTileKeys / 4) {
      const int row = wave * (kTileKeys / 4) + j;
      const int key = min(key0 + rho(row), L - 1);  // rho is its own inverse
      dma16(__builtin_amdgcn_readfirstlane(base + row * kRowStride), crs, lane16,
            __builtin_amdgcn_readfirstlane(key * kRowBytesGlobal));
    } else {
      // rotary: keys past the end are clamped per lane
      const int over = key0 + (lane & 31) - (L - 1);
      const int voff = rope_lane - (over > 0 ? over * kRopeRowBytes : 0);
      dma16(__builtin_amdgcn_readfirstlane(base + kLatBytes + wave * 1024), krs, voff,
            __builtin_amdgcn_readfirstlane(key0 * kRopeRowBytes + wave * 32));
    }
  };
  auto stage_tile = [&](int t, int stg) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kStageInstrs; ++j) stage_part(t, stg, j, ckv_rs, kpe_rs);
  };

  // Per-lane LDS byte offsets (k-step, slice and block parts are immediates).
  //  K reads: key c32 -> row rho(c32); 16-byte chunk 2 ks + g.
  const int k_off = rho(c32) * kRowStride + (g << 4);
  //  rotary K reads: key c32, chunk 2 ks + g
  const int r_off = kLatBytes + g * 512 + c32 * 16;
  //  rotary Q reads
  const unsigned char* const qpe_lds = smem + kQpeOff + wave * 4096 + lane16;
  //  V^T transpose reads.  A ds_read_b64_tr_b16 serves 16 lanes from 4 rows x 4 chunks of 4
  //  bf16: lane (4 r + q) of a 16-lane group points at key r, dims 4q..4q+3 of the group's 16
  //  dims, and output lane j receives dim j of those 4 keys.  For a 16-key slice the two reads
  //  cc = 0, 1 take keys 8cc + 4g + r of the slice (the order in which the S^T accumulator
  //  hands keys to the B operand), which rho maps to rows 4r + 2cc + g of the slice.
  const int r4 = (lane >> 2) & 3;
  const int q4 = lane & 3;
  const int tr_off = (4 * r4 + g) * kRowStride + ((((lane >> 4) & 1) << 1 | (q4 >> 1)) << 4) + ((q4 & 1) << 3) +
                     wave * 256;  // this wave's 128 latent dims

  f32x16 o[4][4];        // [head block][32-dim block]: dims 128 wave + 32 db + 8 (i / 4) + 4 g + i % 4
  float m_ref = 0.f;     // reference max (log2 units) of this lane's head, equal in both halves
  // This lane's share of the denominator, summed over the bf16-rounded probabilities that the
  // value product multiplies: out = sum p~ v / sum p~ is then a convex combination of the value
  // rows, and a row dominated by one key reproduces that key's row whatever its probability
  // rounded to.  (An fp32 sum of the unrounded probabilities leaves that rounding, up to 2^-8
  // relative, in the output.)  lse takes the same sum, within 2^-8 relative of the exact one,
  // i.e. within 0.004 in natural-log units.
  float l_run = 0.f;
  float mx_run = -INFINITY;
  const float cs = a.scale_log2e;
  // This split's tiles of this stream (a split past a short stream's end is empty: it writes
  // lse = -inf and a zero output, which the merge weighs by 0).
  const int t_begin = sp * a.tiles_per_split[grp];
  const int t_end = min((L + kTileKeys - 1) / kTileKeys, t_begin + a.tiles_per_split[grp]);
  const int t_mask = max(t_begin, min(t_end, P / kTileKeys));  // first tile holding tree keys

  // Q^T fragments of this wave's head block: lane holds head `head`, dims 16 ks + 8 g .. +7.
  // The 32 latent k-steps stay in VGPRs for the whole key range; the 4 rotary k-steps are
  // staged once into LDS (the register file is full: O^T alone takes all 256 AGPRs).  They are
  // loaded in the first pass, right behind the first tile's staging, so that one wait covers
  // both.
  bf16x8 qf[32];


  // ---- S^T of a tile held in stage stg: 4 rotary + 32 latent k-steps (k-steps [U0, U1) of
  //      them for a half chain)
  auto score_mma = [&](int stg, auto&& hook, auto&& dma, auto steps_tag) __attribute__((always_inline)) -> f32x16 {
    constexpr int U0 = decltype(steps_tag)::u0, U1 = decltype(steps_tag)::u1;
    constexpr int kEvery = U1 - U0 == 36 ? kDmaEvery : kDmaEveryHalf;
    constexpr int kIn = U1 - U0 == 36 ? kDmaInScores : kDmaInHalf;
    const unsigned char* st_base = smem + stg * kStageBytes;
    // k-step u: the 4 rotary k-steps first (both operands in LDS), then the 32 latent ones
    // (Q in registers).
    auto kfrag = [&](int u) __attribute__((always_inline)) -> bf16x8 {
      return u < 4 ? *reinterpret_cast<const bf16x8*>(st_base + r_off + u * 1024)
                   : *reinterpret_cast<const bf16x8*>(st_base + k_off + (u - 4) * 32);
    };
    auto qpe_frag = [&](int u) __attribute__((always_inline)) -> bf16x8 {
      return *reinterpret_cast<const bf16x8*>(qpe_lds + u * 1024);
    };
    // Operands are read kKAhead k-steps ahead of their MFMA; a scheduling barrier after each
    // k-step keeps that order (left alone, the scheduler moves each read next to its use and
    // every MFMA waits out a full LDS latency).  dma(j) issues staging instruction j of the
    // next tile every kDmaEvery k-steps: a wave that issues them back to back stalls for most
    // of their transfer, one spread between MFMAs costs little.  hook() issues the first reads
    // of the value product.
    bf16x8 kb[kKAhead], qb[4];
#pragma unroll
    for (int u = U0; u < U0 + kKAhead; ++u) {
      kb[(u - U0) % kKAhead] = kfrag(u);
      if (u < 4) qb[u] = qpe_frag(u);
    }
#pragma unroll
    for (int u = U0 + kKAhead; u < 4; ++u) qb[u] = qpe_frag(u);
    f32x16 st;
    bf16x8 kprev, qprev;
#pragma unroll
    for (int u = U0; u < U1; ++u) {
      const int v = u - U0;
      const bf16x8 kcur = kb[v % kKAhead];
      const bf16x8 qcur = u < 4 ? qb[u] : qf[u - 4];
      if (u + kKAhead < U1) kb[v % kKAhead] = kfrag(u + kKAhead);
      if (v % kEvery == 1 && v / kEvery < kIn) dma(v / kEvery);
      if (u == U1 - 2) hook();
      score_step(st, kcur, qcur, u == U0, u == U1 - 1);
      // The compiler cannot see inside the asm MFMA, so it would treat the operand registers as
      // free once the asm is issued.  They stay in use until the next MFMA of the chain has
      // issued -- and that one waits for this one's result, so by then every operand read is
      // done -- and no later write (VALU or LDS) can reach them while the matrix core reads them.
      if (u > U0) asm volatile("" ::"v"(kprev), "v"(qprev));
      kprev = kcur;
      qprev = qcur;
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("" ::"v"(kprev), "v"(qprev));
    return st;
  };

  // ---- running sum plus rounded probabilities e, e + 1 (e even) of a tile
  auto sum_pair = [](const bf16x8 (&pb)[2], int e, float sum) __attribute__((always_inline)) -> float {
    const bf16x2 pr = {pb[e >> 3][e & 7], pb[e >> 3][(e & 7) + 1]};
    return __builtin_amdgcn_fdot2_f32_bf16(pr, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, sum, false);
  };
  // ---- probabilities of accumulator entries 2 k, 2 k + 1 of tile t (entry i holds key
  //      8 (i / 4) + 4 g + i % 4 of the tile): visibility, running raw max, exp2 against the
  //      reference, bf16 packing, and the running sum of the rounded probabilities.
  auto prob_pair = [&](const f32x16& st, int t, int k, auto masked_tag, bf16x8 (&pb)[2], float& psum,
                       float& mx) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked_tag)::value;
#pragma unroll
    for (int e = 2 * k; e < 2 * k + 2; ++e) {
      float x = st[e];
      if constexpr (kMasked) {
        const int rel = t * kTileKeys + 4 * g - P + 8 * (e >> 2) + (e & 3);
        const unsigned sh = (unsigned)min(max(rel, 0), 63);
        const bool vis = (rel < 0) | ((rel < Q) & (unsigned)((anc >> sh) & 1ull));
        x = vis ? x : -INFINITY;
      }
      mx = fmaxf(mx, x);
      const float pv = __builtin_amdgcn_exp2f(fmaf(x, cs, -m_ref));
      pb[e >> 3][e & 7] = (__bf16)pv;
    }
    // The previous rounded pair joins the sum (one dot2 with (1, 1)).  One pair late, so that
    // it never waits for this pair's exponentials and packing; the last pair of the tile is
    // added by the caller.
    if (k > 0) psum = sum_pair(pb, 2 * k - 2, psum);
  };
  auto publish = [&](int pbuf, int u, const bf16x8& v) __attribute__((always_inline)) {
    *reinterpret_cast<bf16x8*>(smem + kPOff + pbuf * kPBytes + wave * 2048 + lane16 + u * 1024) = v;
  };

  // ---- values of a tile held in stage stg with probabilities in pbuf: O^T += V^T P^T,
  //      2 slices of 16 keys x 4 dim blocks = 8 steps of 4 MFMAs (one per head block).
  //      value_prologue reads the first operands (P of slice 0, V^T of step 0); step k reads V^T
  //      of step k + 1 (and, at k = kP1Step, P of slice 1), and side(k) -- VALU work of the next
  //      tile -- shares step k with the MFMAs.  A scheduling barrier closes each step.
  auto vfrag = [&](int stg, int k) __attribute__((always_inline)) -> bf16x8 {
    const unsigned char* vp = smem + stg * kStageBytes + tr_off + (k >> 2) * 16 * kRowStride + (k & 3) * 64;
    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vp);
    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 2 * kRowStride));
    return __builtin_bit_cast(bf16x8, s16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
  };
  auto pfrag = [&](int pbuf, int hb, int slice) __attribute__((always_inline)) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(smem + kPOff + pbuf * kPBytes + hb * 2048 + slice * 1024 + lane16);
  };
  // kHalf: a workgroup of one node (group 1), whose head blocks 2 and 3 only repeat 0 and 1 --
  // their value product is skipped (their outputs are never written).
  auto value_prologue = [&](int stg, int pbuf, bf16x8 (&p0)[4], bf16x8& vf, auto half_tag)
                            __attribute__((always_inline)) {
    constexpr int kNhb = decltype(half_tag)::value ? 2 : 4;
#pragma unroll
    for (int hb = 0; hb < kNhb; ++hb) p0[hb] = pfrag(pbuf, hb, 0);
    vf = vfrag(stg, 0);
  };
  auto values = [&](int stg, int pbuf, bf16x8 (&p0)[4], bf16x8& vf, auto&& side, auto half_tag)
                    __attribute__((always_inline)) {
    constexpr int kNhb = decltype(half_tag)::value ? 2 : 4;
    bf16x8 p1[4];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const bf16x8 vcur = vf;
      if (k + 1 < 8) vf = vfrag(stg, k + 1);
      if (k == kP1Step) {
#pragma unroll
        for (int hb = 0; hb < kNhb; ++hb) p1[hb] = pfrag(pbuf, hb, 1);
      }
#pragma unroll
      for (int hb = 0; hb < kNhb; ++hb)
        o[hb][k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vcur, k < 4 ? p0[hb] : p1[hb], o[hb][k & 3], 0, 0, 0);
      side(k);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto no_side = [](int) __attribute__((always_inline)) {};
  auto no_hook = []() __attribute__((always_inline)) {};

  // ---- one pipeline step: tile t's rows are in stage (t - t_begin) % 3 (staged one step
  //      earlier); the previous tile's probabilities are in P buffer (t - t_begin + 1) & 1.
  //      A steady step runs the value product of tile t - 1 with the softmax of tile t spread
  //      between its MFMAs.  The first step of a pass has no previous tile; on the first pass it
  //      also sets the reference max from this tile before any exponential.
  auto step = [&](int t, auto masked_tag, auto first_tag, auto set_ref_tag, auto half_tag)
                  __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first_tag)::value;
    constexpr bool kSetRef = decltype(set_ref_tag)::value;
    constexpr bool kMasked = decltype(masked_tag)::value;
    constexpr bool kHalf = decltype(half_tag)::value;
    // staging instructions of the next tile issued inside the score chain
    constexpr int kIn = kHalf ? kDmaInHalf : kDmaInScores;
    const int i = t - t_begin;
    const int stg = i % kStages;
    const int pbuf = i & 1;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();  // tile t staged and published tile t - 1 visible; tile t - 2 released
    const bool stage_next = t + 1 < t_end;
    const i32x4 crs = stage_next ? ckv_rs : ckv_none, krs = stage_next ? kpe_rs : kpe_none;
    auto dma = [&](int j) __attribute__((always_inline)) { stage_part(t + 1, (i + 1) % kStages, j, crs, krs); };
    bf16x8 p0[4], vf;
    const int prev_stg = (i + 2) % kStages, prev_pbuf = (i + 1) & 1;
    f32x16 st;
    auto chain = [&](auto&& hook) __attribute__((always_inline)) {
      if constexpr (!kHalf) {
        st = score_mma(stg, hook, dma, Steps<0, 36>{});
      } else {
        // a one-node workgroup: waves w and w + 2 split head block w's chain, and wave w + 2
        // hands its partial scores to wave w through LDS (its own rotary-query area, unused
        // here), behind a barrier that waits for LDS writes only -- the next tile's staging
        // stays in flight
        if (wave < 2)
          st = score_mma(stg, hook, dma, Steps<0, kSplitStep>{});
        else
          st = score_mma(stg, hook, dma, Steps<kSplitStep, 36>{});
        F32x4* xb = reinterpret_cast<F32x4*>(smem + kQpeOff + (2 + (wave & 1)) * 4096) + lane;
        if (wave >= 2) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) xb[i4 * 64] = F32x4{st[4 * i4], st[4 * i4 + 1], st[4 * i4 + 2], st[4 * i4 + 3]};
        }
        // lgkmcnt(0) only: this wave's LDS writes are done; vmcnt is left alone, so the next
        // tile's staging stays in flight across the barrier
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if (wave < 2) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const F32x4 x = xb[i4 * 64];
            st[4 * i4] += x[0];
            st[4 * i4 + 1] += x[1];
            st[4 * i4 + 2] += x[2];
            st[4 * i4 + 3] += x[3];
          }
        }
      }
    };
    if constexpr (kFirst) {
#pragma unroll
      for (int j = kIn; j < kStageInstrs; ++j) dma(j);  // no value steps to carry them
      chain(no_hook);
    } else {
      chain([&]() __attribute__((always_inline)) { value_prologue(prev_stg, prev_pbuf, p0, vf, half_tag); });
    }
    // in a one-node workgroup only waves 0, 1 hold whole scores: the softmax is theirs
    const bool soft = !kHalf || wave < 2;
    bf16x8 pb[2];
    float psum = 0.f, mx = -INFINITY;
    if constexpr (kFirst) {
      if constexpr (kSetRef) {
        float m = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float x = st[e];
          if constexpr (kMasked) {
            const int rel = t * kTileKeys + 4 * g - P + 8 * (e >> 2) + (e & 3);
            const unsigned sh = (unsigned)min(max(rel, 0), 63);
            const bool vis = (rel < 0) | ((rel < Q) & (unsigned)((anc >> sh) & 1ull));
            x = vis ? x : -INFINITY;
          }
          m = fmaxf(m, x);
        }
        const float m0 = half_max(m * cs);
        m_ref = m0 == -INFINITY ? 0.f : m0;
      }
      if (soft) {
#pragma unroll
        for (int k = 0; k < 8; ++k) prob_pair(st, t, k, masked_tag, pb, psum, mx);
        publish(pbuf, 0, pb[0]);
        publish(pbuf, 1, pb[1]);
      }
    } else {
      values(
          prev_stg, prev_pbuf, p0, vf,
          [&](int k) __attribute__((always_inline)) {
            if (k < kStageInstrs - kIn) dma(kIn + k);
            if (soft) {
              prob_pair(st, t, k, masked_tag, pb, psum, mx);
              if ((k & 3) == 3) publish(pbuf, k >> 2, pb[k >> 2]);
            }
          },
          half_tag);
    }
    if (soft) {
      psum = sum_pair(pb, 14, psum);
      l_run += psum;
      mx_run = fmaxf(mx_run, mx * cs);
    }
  };

#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int db = 0; db < 4; ++db) o[hb][db] = f32x16{};
  // The key passes, instantiated separately for the one-node workgroups of group 1.
  auto passes = [&](auto half_tag) __attribute__((always_inline)) {
    for (int attempt = 0; attempt < 2 && t_begin < t_end; ++attempt) {
      if (attempt > 0) {
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
#pragma unroll
          for (int db = 0; db < 4; ++db) o[hb][db] = f32x16{};
      }
      l_run = 0.f;
      mx_run = -INFINITY;

      stage_tile(t_begin, 0);
      if (attempt == 0) {
        // Latent queries of this wave's head block, k-steps [ks0, ks1): all 32 for a node pair;
        // in a one-node workgroup the first kSplitStep - 4 for waves 0, 1 and the rest for
        // waves 2, 3 (each half of the score chain; qc = q0 there).
        constexpr bool kHalf = decltype(half_tag)::value;
        const size_t qrow = ((size_t)s * Q + qc) * kHeads + head;
        const uint16_t* ql = a.q_lat + qrow * kDLat + g * 8;
        const bool lo = !kHalf || wave < 2, hi = !kHalf || wave >= 2;
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) {
          const bool need = ks < kSplitStep - 4 ? lo : hi;
          qf[ks] = need ? *reinterpret_cast<const bf16x8*>(ql + ks * 16) : bf16x8{};
        }
        // Consume every fragment here, so the wait for these loads happens once, before the key
        // loop: otherwise the loop's MFMAs carry waits that also drain the tile prefetch.
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) asm volatile("" : "+v"(qf[ks]));
        if (lo) {  // the rotary k-steps belong to the first half
          const uint16_t* qp = a.q_pe + qrow * kDRope + g * 8;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            *reinterpret_cast<bf16x8*>(smem + kQpeOff + wave * 4096 + ks * 1024 + lane * 16) =
                *reinterpret_cast<const bf16x8*>(qp + ks * 16);
        }
      }
      int t = t_begin;
      // first tile: sets the reference max on the first pass, no value product yet
      if (attempt == 0) {
        if (t < t_mask)
          step(t, Flag<false>{}, Flag<true>{}, Flag<true>{}, half_tag);
        else
          step(t, Flag<true>{}, Flag<true>{}, Flag<true>{}, half_tag);
      } else {  // the second pass keeps the exact max found by the first
        if (t < t_mask)
          step(t, Flag<false>{}, Flag<true>{}, Flag<false>{}, half_tag);
        else
          step(t, Flag<true>{}, Flag<true>{}, Flag<false>{}, half_tag);
      }
      ++t;
      for (; t < t_mask; ++t) step(t, Flag<false>{}, Flag<false>{}, Flag<false>{}, half_tag);
      for (; t < t_end; ++t) step(t, Flag<true>{}, Flag<false>{}, Flag<false>{}, half_tag);
      // last tile's values.  The last step issued its 9 staging instructions against empty
      // resources; out-of-range lanes of an LDS load still write zeros into their stage, which
      // the output transpose areas overlap, so every wave waits for them before the barrier.
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      {
        const int last_stg = (t_end - 1 - t_begin) % kStages, last_pbuf = (t_end - 1 - t_begin) & 1;
        bf16x8 p0[4], vf;
        value_prologue(last_stg, last_pbuf, p0, vf, half_tag);
        values(last_stg, last_pbuf, p0, vf, no_side, half_tag);
      }

      // Was the reference max a safe choice for every head of the workgroup?
      const float mfull = half_max(mx_run);
      const bool redo = mfull != -INFINITY && (mfull > m_ref + kRefHi || mfull < m_ref - kRefLo);
      if (threadIdx.x == 0) redo_s = 0;
      __syncthreads();
      if (attempt == 0 && __builtin_amdgcn_ballot_w64(redo) != 0 && lane == 0) redo_s = 1;
      __syncthreads();
      if (redo_s == 0) break;
      m_ref = mfull == -INFINITY ? 0.f : mfull;
    }

  };
  if (n_nodes == 1)
    passes(Flag<true>{});
  else
    passes(Flag<false>{});

  // ---- finalize: reciprocal denominators of all four head blocks through LDS
  const float lt = half_sum(l_run);
  const float poison = bad_prefix ? __builtin_nanf("") : 0.f;
  // 1 / denominator of every row, once per row (the P buffers are free after the last barrier)
  float* inv_sh = reinterpret_cast<float*>(smem + kPOff);
  if (g == 0) inv_sh[wave * 32 + c32] = (lt > 0.f ? 1.0f / lt : 0.f) + poison;
  const int part_rows = grp == 0 ? a.n_streams * a.n_pairs * 2 * kHeads : a.n_streams * kHeads;
  if (active && g == 0) {
    const float lse_v = (lt > 0.f ? (m_ref + log2f(lt)) * kLn2 : -INFINITY) + poison;
    if (n_split == 1)
      a.lse[((size_t)s * Q + qi) * kHeads + head] = lse_v;
    else
      a.part_lse[grp][(size_t)sp * part_rows + part_row(wave >> 1, head)] = lse_v;
  }
  __syncthreads();
  // Output, one head block at a time through this wave's own LDS area (the key stages are free
  // after the last barrier): the accumulator holds 16-byte runs of 32 rows, the read back hands
  // each lane one 16-byte chunk of a row, so that each store writes two rows' 512-byte segments
  // (this wave's 128 dims) instead of 32-byte pieces of 32 rows.
  unsigned char* tbuf = smem + wave * (32 * kTRow);
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    if ((hb >> 1) >= n_nodes) continue;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float4 v;
        v.x = o[hb][db][4 * i4 + 0];
        v.y = o[hb][db][4 * i4 + 1];
        v.z = o[hb][db][4 * i4 + 2];
        v.w = o[hb][db][4 * i4 + 3];
        *reinterpret_cast<float4*>(tbuf + c32 * kTRow + (32 * db + 8 * i4 + 4 * g) * 4) = v;
      }
    }
    const int h0 = (hb & 1) * 32;
    float* dst = n_split == 1 ? a.out + (((size_t)s * Q + q0 + (hb >> 1)) * kHeads + h0) * kDLat
                              : a.part_out[grp] + ((size_t)sp * part_rows + part_row(hb >> 1, h0)) * kDLat;
    dst += wave * 128 + (lane & 31) * 4;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 2 * j + (lane >> 5);
      const float inv = inv_sh[hb * 32 + r];
      float4 v = *reinterpret_cast<const float4*>(tbuf + r * kTRow + (lane & 31) * 16);
      v.x *= inv;
      v.y *= inv;
      v.z *= inv;
      v.w *= inv;
      // Written once and not read again by this launch: a nontemporal store (measured 0.8%
      // faster for the whole launch than a plain one).
      const F32x4 vv = {v.x, v.y, v.z, v.w};
      __builtin_nontemporal_store(vv, reinterpret_cast<F32x4*>(dst + (size_t)r * kDLat));
    }
  }
}

// Merge of key-range splits by log-sum-exp: lse = log sum_k exp(lse_k),
// out = sum_k exp(lse_k - lse) out_k.  One thread per (partial row, 4 dims), over the split rows
// of both groups in one launch.  The splits are read in chunks of kMergeChunk with every load of
// a chunk in flight, and merged online: the running sums are rescaled when a chunk raises the
// running max.  (A loop with one split per iteration waits out a full memory latency per
// split, which dominated at tens of splits.)  A launch whose groups have at most 4 splits (the
// usual case) uses chunks of 4: half the registers, so more rows' loads are in flight per CU.
template <int kMergeChunk>
__global__ void __launch_bounds__(256) verify_combine_kernel(CombineArgs a) {
  const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  long long row = tid >> 7;
  const int c4 = (int)(tid & 127);
  const int grp = row < a.rows[0] ? 0 : 1;
  if (grp == 1) {
    row -= a.rows[0];
    if (row >= a.rows[1]) return;
  }
  const long long rows = a.rows[grp];
  const int n_splits = a.n_splits[grp];
  const float* part_out = a.part_out[grp];
  const float* part_lse = a.part_lse[grp];
  long long orow;
  if (grp == 0) {
    const int h = (int)(row & (kHeads - 1));
    const int k = (int)((row >> 6) & 1);
    const long long sp_pair = row >> 7;  // s * n_pairs + p
    const long long s = sp_pair / max(a.n_pairs, 1);
    const long long p = sp_pair - s * a.n_pairs;
    orow = (s * a.q_len + 2 * p + k) * kHeads + h;
  } else {
    orow = ((row >> 6) * a.q_len + a.q_len - 1) * kHeads + (row & (kHeads - 1));
  }
  float mx = -INFINITY, den = 0.f;
  float poison = 0.f;  // NaN once any split is NaN (a poisoned stream), whatever the others hold
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < n_splits; k0 += kMergeChunk) {
    float lk[kMergeChunk];
    float4 v[kMergeChunk];
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j) {
      const int k = k0 + j;
      lk[j] = -INFINITY;
      v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (k < n_splits) {
        lk[j] = part_lse[(size_t)k * rows + row];
        v[j] = *reinterpret_cast<const float4*>(part_out + ((size_t)k * rows + row) * kDLat + 4 * c4);
      }
    }
    float cmx = mx;
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j) {
      cmx = fmaxf(cmx, lk[j]);
      if (lk[j] != lk[j]) poison = lk[j];
    }
    if (cmx == -INFINITY) continue;  // nothing but empty splits so far
    const float r = mx == -INFINITY ? 0.f : expf(mx - cmx);
    den *= r;
    acc.x *= r;
    acc.y *= r;
    acc.z *= r;
    acc.w *= r;
#pragma unroll
    for (int j = 0; j < kMergeChunk; ++j) {
      const float w = lk[j] == -INFINITY ? 0.f : expf(lk[j] - cmx);
      den += w;
      acc.x += w * v[j].x;
      acc.y += w * v[j].y;
      acc.z += w * v[j].z;
      acc.w += w * v[j].w;
    }
    mx = cmx;
  }
  const float inv = 1.0f / den + poison;
  acc.x *= inv;
  acc.y *= inv;
  acc.z *= inv;
  acc.w *= inv;
  *reinterpret_cast<float4*>(a.out + (size_t)orow * kDLat + 4 * c4) = acc;
  if (c4 == 0) a.lse[orow] = mx + logf(den) + poison;
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, int wg_total, hipStream_t stream) {
  void* args[] = {const_cast<VerifyArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(verify_attn_kernel), dim3((unsigned)wg_total),
                         dim3(kWGThreads), args, 0, stream);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  const long long threads = (a.rows[0] + a.rows[1]) * 128;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  void* args[] = {const_cast<CombineArgs*>(&a)};
  const int s0 = a.rows[0] ? a.n_splits[0] : 0, s1 = a.rows[1] ? a.n_splits[1] : 0;
  const void* kernel = (s0 > s1 ? s0 : s1) <= 4 ? reinterpret_cast<const void*>(verify_combine_kernel<4>)
                                                : reinterpret_cast<const void*>(verify_combine_kernel<8>);
  return hipLaunchKernel(kernel, dim3(blocks), dim3(256), args, 0, stream);
}

}  // namespace ddtree
