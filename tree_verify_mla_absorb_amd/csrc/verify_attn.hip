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
//   S^T[key, qh] = K[key, 0:576] . Q^T[0:576, qh]          (A = K from LDS, B = Q in VGPRs)
//   O^T[dim, qh] += V^T[dim, key] . P^T[key, qh]            (A = V^T via LDS transpose reads,
//                                                            B = P^T straight from S^T's acc)
//
// Computing S^T (keys as MFMA rows) puts one query-head column in each lane, so the softmax
// statistics are per-lane values plus one cross-half swap, and the accumulator layout of S^T
// is already the B-operand layout the PV product needs (the key order inside the 16-key
// contraction is permuted identically on the V side).
//
// Workgroup = 4 waves over 2 tree nodes x 64 heads.  For the scores, wave w owns node
// (2 * group + w / 2) and heads 32 * (w & 1) .. +31, so the tree mask is wave-uniform: one 64-bit
// ancestor-or-self mask walked from parents[] with a walk bounded by q_len (the bounded-walk
// lesson of "The Microsecond Verdict", section "The Crash That Demanded a Fix").  For the value
// product the waves split the 512 latent dims instead and share the probabilities through LDS.

#include "kernels.h"

#include <math.h>

#include "../../include/ddtree.h"

namespace ddtree {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// LDS layout.
//   latent stages 0/1: 64 rows x 1040 B (1024 B of c_kv + 16 B pad), double-buffered.  Key k of
//       the tile lives in row rho(k), rho swapping the two 2-bit halves of k's low nibble.  With
//       the pad, the 16 rows read by one ds_read_b128 phase land on 16 distinct bank quads and
//       the 4 rows x 64 B read by 32 lanes of a ds_read_b64_tr_b16 land on 4 distinct 16-bank
//       groups; every address is a per-lane base plus an immediate.
//   rotary buffer: chunk-major, [16-byte chunk 8][key 64][16 B], so the 16 keys read by one
//       ds_read_b128 phase are 256 contiguous bytes.  Single-buffered: it is only read by the
//       score product, so the next tile's rows are loaded once every wave is past its scores.
//   P buffer: bf16 probabilities of the tile, [head block 4][16-key slice 4][lane 64][16 B],
//       written by the wave that computed the scores and read by all four waves.
constexpr int kRowBytesGlobal = kDLat * 2;                // 1024 B per c_kv row in HBM
constexpr int kRowStride = kRowBytesGlobal + 16;          // 1040 B per latent row in LDS
constexpr int kLatBytes = kTileKeys * kRowStride;         // 66560 B
constexpr int kRopeRowBytes = kDRope * 2;                 // 128 B
constexpr int kRopeOff = 2 * kLatBytes;
constexpr int kPOff = kRopeOff + kTileKeys * kRopeRowBytes;
constexpr int kPBytes = 4 * 4 * 64 * 16;                  // 16 KiB
constexpr int kSmemBytes = kPOff + kPBytes;               // 157696 B
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

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
// K fragments read ahead of the score MFMA that consumes them (LDS latency ~ 4 MFMAs).
constexpr int kKAhead = 4;

__device__ __forceinline__ int rho(int k) { return (k & ~15) | ((k & 3) << 2) | ((k >> 2) & 3); }

// Raw buffer resource over `bytes` bytes at `base` (stride 0, untyped).
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, unsigned bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  return i32x4{(int)(unsigned)a, (int)((a >> 32) & 0xffffu), (int)bytes, kBufferDword3};
}

// One wave instruction of direct global->LDS staging: lane i's 16 bytes at
// rsrc + soff + voff land at LDS byte lds_addr + 16 i.  Issued from asm so that the compiler
// does not order later LDS reads of the *other* stage behind it; the consumer waits with an
// explicit vmcnt(0) and a workgroup barrier before reading the stage this wrote.
__device__ __forceinline__ void dma16(unsigned lds_addr, i32x4 rsrc, int voff, int soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

// Combine the two lane halves that hold the same head (lanes l and l ^ 32).
__device__ __forceinline__ float half_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float half_sum(float x) { return x + __shfl_xor(x, 32); }

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

// Workgroup = 4 waves, 2 tree nodes x 64 heads = 4 head blocks of 32 query-heads.
//   scores:  wave w computes S^T for head block w (node 2 g + w / 2, heads 32 (w & 1) ..+31)
//            over the tile's 64 keys, turns it into bf16 probabilities and publishes them;
//   values:  wave w accumulates O^T for latent dims 128 w .. 128 w + 127 of all 4 head blocks,
//            so each V^T fragment read from LDS feeds four MFMAs.
__global__ void __attribute__((amdgpu_flat_work_group_size(kWGThreads, kWGThreads),
                               amdgpu_waves_per_eu(1, 1)))
verify_attn_kernel(VerifyArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kSmemBytes];
  __shared__ int redo_s;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c32 = lane & 31;
  const int g = lane >> 5;

  // Group and position of this workgroup.  Workgroup b is dispatched to XCD b % 8; within a
  // group the index is renumbered so that each XCD runs a contiguous run of (stream, node pair,
  // split) units: the workgroups of one stream then share that XCD's L2 while they stream the
  // same key tiles, and the light workgroups of group 1 spread over all XCDs.
  const int grp = (int)blockIdx.x < a.wg_count0 ? 0 : 1;
  const int j = grp == 0 ? (int)blockIdx.x : (int)blockIdx.x - a.wg_count0;
  const int cnt = grp == 0 ? a.wg_count0 : (int)gridDim.x - a.wg_count0;
  const int xcd = j & 7;
  const int per = cnt >> 3, rem = cnt & 7;
  const int logical = xcd * per + min(xcd, rem) + (j >> 3);
  const int n_split = a.splits[grp];
  const int sp = logical % n_split;
  const int unit = logical / n_split;
  const int s = grp == 0 ? unit / max(a.n_pairs, 1) : unit;
  const int pair = grp == 0 ? unit - s * a.n_pairs : 0;
  const int q0 = grp == 0 ? 2 * pair : a.q_len - 1;  // first node of the workgroup
  const int n_nodes = grp == 0 ? 2 : 1;

  const int P = a.prefix_len;
  const int Q = a.q_len;
  const int L = P + Q;
  const int qi = q0 + (wave >> 1);
  const bool active = (wave >> 1) < n_nodes;  // group 1: head blocks 2, 3 compute a copy
  const int qc = active ? qi : q0;
  const int head = (wave & 1) * 32 + c32;
  // row of (node q0 + k, head h) in this group's partial buffers
  auto part_row = [&](int k, int h) { return grp == 0 ? ((s * a.n_pairs + pair) * 2 + k) * kHeads + h : s * kHeads + h; };

  // Ancestor-or-self mask of node qc.  Every step must move to a strictly smaller index, so
  // the walk ends within q_len steps for any input; a malformed entry ends it early.
  uint64_t anc = 0;
  bool bad = false;
  {
    const int32_t* par = a.parents + (size_t)s * Q;
    int node = qc;
    for (int step = 0; step < Q && node >= 0; ++step) {
      anc |= 1ull << node;
      const int pn = par[node];
      if (pn >= node || pn < -1 || (pn == -1 && node != 0)) {
        bad = true;
        node = -1;
      } else {
        node = pn;
      }
    }
  }
  if (bad && active && a.status != nullptr && lane == 0) atomicOr(a.status, DDTREE_STATUS_BAD_PARENTS);

  // Q^T fragments of this wave's head block: lane holds head `head`, dims 16 ks + 8 g .. +7.
  // The 32 latent k-steps stay in VGPRs for the whole key range; the 4 rotary k-steps are
  // re-read (L1/L2 hits) at the start of every tile, which keeps the register file within
  // budget.
  const size_t qrow = ((size_t)s * Q + qc) * kHeads + head;
  bf16x8 qf[32];
  {
    const uint16_t* ql = a.q_lat + qrow * kDLat + g * 8;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(ql + ks * 16);
  }
  const uint16_t* const qp_lane = a.q_pe + qrow * kDRope + g * 8;
  bf16x8 qr[4];
  auto load_qr = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qr[ks] = *reinterpret_cast<const bf16x8*>(qp_lane + ks * 16);
  };

  // Staging of this stream's cache rows.  A latent row is one wave instruction (64 lanes x
  // 16 B); rotary instruction c moves 16-byte chunk c of all 64 rows (lane = key).  Rows past
  // the end of the cache are clamped to the last row: their scores are masked out.
  const i32x4 ckv_rs = buffer_rsrc(a.ckv + (size_t)s * a.kv_rows * kDLat, (unsigned)a.kv_rows * kDLat * 2);
  const i32x4 kpe_rs = buffer_rsrc(a.kpe + (size_t)s * a.kv_rows * kDRope, (unsigned)a.kv_rows * kDRope * 2);
  const unsigned smem_base = (unsigned)(size_t)((__attribute__((address_space(3))) unsigned char*)smem);
  const int lane16 = lane << 4;
  auto load_latent = [&](int t, int stg) __attribute__((always_inline)) {
    const int key0 = t * kTileKeys;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int row = wave * 16 + rr;
      const int key = min(key0 + rho(row), L - 1);  // rho is its own inverse
      dma16(__builtin_amdgcn_readfirstlane(smem_base + stg * kLatBytes + row * kRowStride), ckv_rs, lane16,
            __builtin_amdgcn_readfirstlane(key * kRowBytesGlobal));
    }
  };
  auto load_rope = [&](int t) __attribute__((always_inline)) {
    const int voff = min(t * (kTileKeys * kRopeRowBytes) + (lane16 << 3), (L - 1) * kRopeRowBytes);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = wave * 2 + i;
      dma16(__builtin_amdgcn_readfirstlane(smem_base + kRopeOff + c * 1024), kpe_rs, voff,
            __builtin_amdgcn_readfirstlane(c * 16));
    }
  };

  // Per-lane LDS byte offsets (sub-tile, k-step, slice and block parts are immediates).
  //  K reads: key jt*32 + c32 -> row jt*32 + rho(c32); 16-byte chunk 2 ks + g.
  const int k_off = rho(c32) * kRowStride + (g << 4);
  //  rotary K reads: key jt*32 + c32, chunk 2 ks + g
  const int r_off = kRopeOff + g * 1024 + c32 * 16;
  //  V^T transpose reads.  A ds_read_b64_tr_b16 serves 16 lanes from 4 rows x 4 chunks of 4
  //  bf16: lane (4 r + q) of a 16-lane group points at key r, dims 4q..4q+3 of the group's 16
  //  dims, and output lane j receives dim j of those 4 keys.  For a 16-key slice the two reads
  //  cc = 0, 1 take keys 8cc + 4g + r of the slice (the order in which the S^T accumulator
  //  hands keys to the B operand), which rho maps to rows 4r + 2cc + g of the slice.
  const int r4 = (lane >> 2) & 3;
  const int q4 = lane & 3;
  const int tr_off = (4 * r4 + g) * kRowStride + ((((lane >> 4) & 1) << 1 | (q4 >> 1)) << 4) + ((q4 & 1) << 3) +
                     wave * 256;  // this wave's 128 latent dims
  unsigned char* const p_mine = smem + kPOff + wave * 4096 + lane16;
  const unsigned char* const p_all = smem + kPOff + lane16;

  f32x16 o[4][4];        // [head block][32-dim block]: dims 128 wave + 32 db + 8 (i / 4) + 4 g + i % 4
  float m_ref = 0.f;     // reference max (log2 units) of this lane's head, equal in both halves
  float l_run = 0.f;     // this lane's share of the denominator
  float mx_run = -INFINITY;
  const float cs = a.scale_log2e;
  const int t_begin = sp * a.tiles_per_split[grp];
  const int t_end = min(a.n_tiles, t_begin + a.tiles_per_split[grp]);
  const int t_mask = max(t_begin, min(t_end, P / kTileKeys));  // first tile holding tree keys

  // One 64-key tile held in stage `stg`: scores, probabilities, publish, values.
  auto tile = [&](int t, int stg, auto masked_tag, auto first_tag) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    constexpr bool kFirst = decltype(first_tag)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile t staged; every wave is done with tile t - 1
    const unsigned char* lat = smem + stg * kLatBytes;
    const bool prefetch = t + 1 < t_end;
    load_qr();  // rotary query fragments: consumed after the first 32 latent k-steps

    // ---- per 32-key half: scores S^T (32 keys x 32 heads, K over 576 dims), visibility,
    //      probabilities against the reference max, published as bf16
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      f32x16 st = f32x16{};
      const unsigned char* kp = lat + k_off + jt * 32 * kRowStride;
#pragma unroll
      for (int ks = 0; ks < 32; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kp + ks * 32);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], st, 0, 0, 0);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(smem + r_off + ks * 2048 + jt * 512);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qr[ks], st, 0, 0, 0);
      }
      // Schedule: kKAhead K reads in flight ahead of the MFMA that consumes them.
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kKAhead, 0);
#pragma unroll
      for (int i = 0; i < 36 - kKAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, kKAhead, 0);
      if (jt == 0) {
        // Prefetch the next tile's latent rows into the other stage (nobody reads it now).
        // Issued only after the rotary fragments are consumed, so that the wait for those
        // never waits for the staging as well.
        __builtin_amdgcn_sched_barrier(0);
        if (prefetch) load_latent(t + 1, stg ^ 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      // accumulator entry i holds key 8 (i / 4) + 4 g + i % 4 of the half
      if constexpr (kMasked) {
        const int kb0 = t * kTileKeys + jt * 32 + 4 * g - P;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int rel = kb0 + 8 * (i >> 2) + (i & 3);
          const unsigned sh = (unsigned)min(max(rel, 0), 63);
          const bool vis = (rel < 0) | ((rel < Q) & (unsigned)((anc >> sh) & 1ull));
          st[i] = vis ? st[i] : -INFINITY;
        }
      }
      float mx = st[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, st[i]);
      mx *= cs;
      mx_run = fmaxf(mx_run, mx);
      if constexpr (kFirst) {
        if (jt == 0) {
          const float m0 = half_max(mx);
          m_ref = m0 == -INFINITY ? 0.f : m0;
        }
      }
      float psum = 0.f;
      bf16x8 pb[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(st[i], cs, -m_ref));
        psum += pv;
        pb[i >> 3][i & 7] = (__bf16)pv;
      }
      l_run += psum;
#pragma unroll
      for (int u = 0; u < 2; ++u) *reinterpret_cast<bf16x8*>(p_mine + (jt * 2 + u) * 1024) = pb[u];
    }
    __syncthreads();  // all four head blocks' probabilities published; rotary rows consumed
    if (prefetch) load_rope(t + 1);

    // ---- O^T += V^T P^T: 4 slices of 16 keys, 4 dim blocks x 4 head blocks per slice.
    //      Step k = (slice, dim block); the reads of step k + 1 are issued before the MFMAs of
    //      step k so that LDS latency overlaps the matrix work.
    auto vfrag = [&](int k) __attribute__((always_inline)) -> bf16x8 {
      const int sl = k >> 2, db = k & 3;
      const unsigned char* vp = lat + tr_off + ((sl >> 1) * 32 + (sl & 1) * 16) * kRowStride + db * 64;
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vp);
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 2 * kRowStride));
      return __builtin_bit_cast(bf16x8, s16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
    };
    bf16x8 pf[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) pf[hb] = *reinterpret_cast<const bf16x8*>(p_all + hb * 4096);
    bf16x8 vf = vfrag(0);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int sl = k >> 2, db = k & 3;
      const bf16x8 vcur = vf;
      bf16x8 pcur[4];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) pcur[hb] = pf[hb];
      if (k + 1 < 16) {
        vf = vfrag(k + 1);
        if (((k + 1) & 3) == 0) {
#pragma unroll
          for (int hb = 0; hb < 4; ++hb)
            pf[hb] = *reinterpret_cast<const bf16x8*>(p_all + hb * 4096 + ((k + 1) >> 2) * 1024);
        }
      }
      (void)sl;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        o[hb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vcur, pcur[hb], o[hb][db], 0, 0, 0);
    }
    // Schedule: the reads of step k + 1 (two V^T halves, plus the next slice's four P^T
    // fragments at a slice boundary) are issued before the MFMAs of step k.
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 6, 1);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k < 15) {
        if (((k + 1) & 3) == 0)
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 6, 1);
        else
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 1);
    }
  };

  for (int attempt = 0; attempt < 2; ++attempt) {
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int db = 0; db < 4; ++db) o[hb][db] = f32x16{};
    l_run = 0.f;
    mx_run = -INFINITY;

    load_latent(t_begin, 0);
    load_rope(t_begin);
    int t = t_begin;
    if (attempt == 0) {  // the first 32 keys of the range set the reference max
      if (t < t_mask)
        tile(t, 0, Flag<false>{}, Flag<true>{});
      else
        tile(t, 0, Flag<true>{}, Flag<true>{});
      ++t;
    }
    for (; t < t_mask; ++t) tile(t, (t - t_begin) & 1, Flag<false>{}, Flag<false>{});
    for (; t < t_end; ++t) tile(t, (t - t_begin) & 1, Flag<true>{}, Flag<false>{});

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

  // ---- finalize: denominators of all four head blocks through LDS
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no staging may still be in flight
  const float lt = half_sum(l_run);
  float* l_sh = reinterpret_cast<float*>(smem + kPOff);  // the P buffer is free after the last barrier
  if (g == 0) l_sh[wave * 32 + c32] = lt;
  const int part_rows = grp == 0 ? a.n_streams * a.n_pairs * 2 * kHeads : a.n_streams * kHeads;
  if (active && g == 0) {
    const float lse_v = lt > 0.f ? (m_ref + log2f(lt)) * kLn2 : -INFINITY;
    if (n_split == 1)
      a.lse[((size_t)s * Q + qi) * kHeads + head] = lse_v;
    else
      a.part_lse[grp][(size_t)sp * part_rows + part_row(wave >> 1, head)] = lse_v;
  }
  __syncthreads();
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    if ((hb >> 1) >= n_nodes) continue;
    const float lh = l_sh[hb * 32 + c32];
    const float inv = lh > 0.f ? 1.0f / lh : 0.f;
    const int h = (hb & 1) * 32 + c32;
    float* dst = n_split == 1 ? a.out + (((size_t)s * Q + q0 + (hb >> 1)) * kHeads + h) * kDLat
                              : a.part_out[grp] + ((size_t)sp * part_rows + part_row(hb >> 1, h)) * kDLat;
    dst += wave * 128 + 4 * g;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float4 v;
        v.x = o[hb][db][4 * i4 + 0] * inv;
        v.y = o[hb][db][4 * i4 + 1] * inv;
        v.z = o[hb][db][4 * i4 + 2] * inv;
        v.w = o[hb][db][4 * i4 + 3] * inv;
        *reinterpret_cast<float4*>(dst + 32 * db + 8 * i4) = v;
      }
    }
  }
}

// Merge of key-range splits by log-sum-exp: lse = log sum_k exp(lse_k),
// out = sum_k exp(lse_k - lse) out_k.  One thread per (partial row, 4 dims).
__global__ void __launch_bounds__(256) verify_combine_kernel(CombineArgs a) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  const int row = tid >> 7;
  const int c4 = tid & 127;
  if (row >= a.rows) return;
  int orow;
  if (a.group == 0) {
    const int h = row & (kHeads - 1);
    const int k = (row >> 6) & 1;
    const int sp_pair = row >> 7;  // s * n_pairs + p
    const int s = sp_pair / max(a.n_pairs, 1);
    const int p = sp_pair - s * a.n_pairs;
    orow = (s * a.q_len + 2 * p + k) * kHeads + h;
  } else {
    orow = ((row >> 6) * a.q_len + a.q_len - 1) * kHeads + (row & (kHeads - 1));
  }
  float mx = -INFINITY;
  for (int k = 0; k < a.n_splits; ++k) mx = fmaxf(mx, a.part_lse[(size_t)k * a.rows + row]);
  float den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < a.n_splits; ++k) {
    const float lk = a.part_lse[(size_t)k * a.rows + row];
    const float w = lk == -INFINITY ? 0.f : expf(lk - mx);
    den += w;
    const float4 v = *reinterpret_cast<const float4*>(a.part_out + ((size_t)k * a.rows + row) * kDLat + 4 * c4);
    acc.x += w * v.x;
    acc.y += w * v.y;
    acc.z += w * v.z;
    acc.w += w * v.w;
  }
  const float inv = 1.0f / den;
  acc.x *= inv;
  acc.y *= inv;
  acc.z *= inv;
  acc.w *= inv;
  *reinterpret_cast<float4*>(a.out + (size_t)orow * kDLat + 4 * c4) = acc;
  if (c4 == 0) a.lse[orow] = mx + logf(den);
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, int wg_total, hipStream_t stream) {
  void* args[] = {const_cast<VerifyArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(verify_attn_kernel), dim3((unsigned)wg_total),
                         dim3(kWGThreads), args, 0, stream);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  const long long threads = (long long)a.rows * 128;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  void* args[] = {const_cast<CombineArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(verify_combine_kernel), dim3(blocks), dim3(256),
                         args, 0, stream);
}

}  // namespace ddtree
