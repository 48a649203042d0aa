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
// Workgroup = 4 waves: wave w owns tree query (2 * group + w / 2) and heads 32 * (w & 1) .. +31.
// The tree mask is therefore wave-uniform: one 64-bit ancestor-or-self mask in scalar registers,
// walked from parents[] with a walk bounded by q_len (the bounded-walk lesson of "The
// Microsecond Verdict", section "The Crash That Demanded a Fix").

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

// LDS stage layout (one stage = one 64-key tile):
//   latent part: 64 rows x 1040 B (1024 B of c_kv + 16 B pad).  Key k of the tile lives in
//                row rho(k), rho swapping the two 2-bit halves of k's low nibble.  With the
//                16-byte pad, the 16 rows read by one ds_read_b128 phase land on 16 distinct
//                bank quads and the 4 rows x 64 B read by 32 lanes of a ds_read_b64_tr_b16
//                land on 4 distinct 16-bank groups; every address is a per-lane base plus an
//                immediate.
//   rotary part: 64 rows x 128 B, row = key, 16-byte chunk c stored at slot c ^ ((row>>1)&7).
constexpr int kRowStride = kDLat * 2 + 16;                      // 1040 B
constexpr int kLatBytes = kTileKeys * kRowStride;               // 66560 B
constexpr int kRopeRowBytes = kDRope * 2;                       // 128 B
constexpr int kStageBytes = kLatBytes + kTileKeys * kRopeRowBytes;  // 74752 B
// Scores are exponentiated against a per-head reference max taken from the first 32 keys.
// If the true max ends above ref + kRefHi or below ref - kRefLo (log2 units) the workgroup
// repeats its key range once with the exact max as reference.  Inside the window every
// probability stays in [2^-kRefLo, 2^kRefHi] of the reference, far from fp32/bf16 limits.
constexpr float kRefHi = 64.0f;
constexpr float kRefLo = 32.0f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ int rho(int k) { return (k & ~15) | ((k & 3) << 2) | ((k >> 2) & 3); }
__device__ __forceinline__ int swz_rope(int r) { return (r >> 1) & 7; }

// Combine the two lane halves that hold the same head (lanes l and l ^ 32).
__device__ __forceinline__ float half_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float half_sum(float x) { return x + __shfl_xor(x, 32); }

__global__ void __attribute__((amdgpu_flat_work_group_size(kWGThreads, kWGThreads),
                               amdgpu_waves_per_eu(1, 1)))
verify_attn_kernel(VerifyArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kStageBytes];
  __shared__ int redo_s;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c32 = lane & 31;
  const int g = lane >> 5;

  // Workgroup b is dispatched to XCD b % 8.  Renumber so that each XCD runs a contiguous run
  // of (stream, query group, split) units: the workgroups of one stream then share that XCD's
  // L2 while they stream the same key tiles.
  const int nblk = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int per = nblk >> 3, rem = nblk & 7;
  const int logical = xcd * per + min(xcd, rem) + (blockIdx.x >> 3);
  const int sp = logical % a.n_splits;
  const int unit = logical / a.n_splits;
  const int s = unit / a.n_qgroups;
  const int qg = unit - s * a.n_qgroups;

  const int P = a.prefix_len;
  const int Q = a.q_len;
  const int L = P + Q;
  const int qi = qg * kQueriesPerWG + (wave >> 1);
  const bool active = qi < Q;        // an idle wave (odd q_len) computes a copy of node Q-1
  const int qc = active ? qi : Q - 1;
  const int head = (wave & 1) * 32 + c32;

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

  // Q^T fragments: lane holds head `head`, dims 16 ks + 8 g .. +7 for the 36 k-steps
  // (32 latent + 4 rotary).
  bf16x8 qf[36];
  {
    const size_t qrow = ((size_t)s * Q + qc) * kHeads + head;
    const uint16_t* ql = a.q_lat + qrow * kDLat + g * 8;
    const uint16_t* qp = a.q_pe + qrow * kDRope + g * 8;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(ql + ks * 16);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[32 + ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
  }

  const uint16_t* ckv_s = a.ckv + (size_t)s * a.kv_rows * kDLat;
  const uint16_t* kpe_s = a.kpe + (size_t)s * a.kv_rows * kDRope;
  const int lane16 = lane << 4;

  // Stage key tile t into LDS stage `stg` with direct global->LDS loads.  A latent row is one
  // wave instruction (64 lanes x 16 B); a rotary instruction covers eight rows.  Rows past the
  // end of the cache are clamped to the last row: their scores are masked out.
  auto load_tile = [&](int t, int stg) {
    unsigned char* base = smem + stg * kStageBytes;
    const int key0 = t * kTileKeys;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int row = wave * 16 + rr;
      const int key = min(key0 + rho(row), L - 1);  // rho is its own inverse
      const unsigned char* src = reinterpret_cast<const unsigned char*>(ckv_s + (size_t)key * kDLat) + lane16;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(base + row * kRowStride), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rb = wave * 2 + i;
      const int row = rb * 8 + (lane >> 3);
      const int key = min(key0 + row, L - 1);
      const uint16_t* src = kpe_s + (size_t)key * kDRope + (((lane & 7) ^ swz_rope(row)) << 3);
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(base + kLatBytes + rb * 1024), 16, 0, 0);
    }
  };

  // Per-lane LDS byte offsets (stage-relative; sub-tile, k-step and block parts are immediates).
  //  K reads: key jt*32 + c32 -> row jt*32 + rho(c32); chunk 2 ks + g.
  const int k_off = rho(c32) * kRowStride + (g << 4);
  //  rotary K reads: row jt*32 + c32, chunk (2 ks + g) ^ swz_rope(row)
  int r_off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) r_off[ks] = kLatBytes + c32 * kRopeRowBytes + (((2 * ks + g) ^ swz_rope(c32)) << 4);
  //  V^T transpose reads.  A ds_read_b64_tr_b16 serves 16 lanes from 4 rows x 4 chunks of 4
  //  bf16: lane (4 r + q) of a 16-lane group points at key r, dims 4q..4q+3 of the group's 16
  //  dims, and output lane j receives dim j of those 4 keys.  For PV step u and read cc the 4
  //  keys are 16u + 8cc + 4g + r (the order the S^T accumulator hands to the B operand), which
  //  rho maps to rows 16u + 4r + 2cc + g.
  const int r4 = (lane >> 2) & 3;
  const int q4 = lane & 3;
  const int tr_off = (4 * r4 + g) * kRowStride + ((((lane >> 4) & 1) << 1 | (q4 >> 1)) << 4) + ((q4 & 1) << 3);

  f32x16 o[16];
  float m_ref = 0.f;     // reference max (log2 units), per head, equal in both lane halves
  float l_run = 0.f;     // this lane's share of the denominator
  float mx_run = -INFINITY;
  const float cs = a.scale_log2e;
  const int t_begin = sp * a.tiles_per_split;
  const int t_end = min(a.n_tiles, t_begin + a.tiles_per_split);

  for (int attempt = 0; attempt < 2; ++attempt) {
#pragma unroll
    for (int d = 0; d < 16; ++d) o[d] = f32x16{};
    l_run = 0.f;
    mx_run = -INFINITY;

    load_tile(t_begin, 0);
    for (int t = t_begin; t < t_end; ++t) {
      const int stg = (t - t_begin) & 1;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (t + 1 < t_end) load_tile(t + 1, stg ^ 1);

      const unsigned char* base = smem + stg * kStageBytes;
      const bool masked = (t + 1) * kTileKeys > P;
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        // ---- scores S^T (32 keys x 32 heads) over the 576 dims
        f32x16 st = f32x16{};
        const unsigned char* kp = base + k_off + jt * 32 * kRowStride;
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kp + ks * 32);
          st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], st, 0, 0, 0);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(base + r_off[ks] + jt * 32 * kRopeRowBytes);
          st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[32 + ks], st, 0, 0, 0);
        }

        // ---- visibility: accumulator entry i holds key 8 (i / 4) + 4 g + i % 4 of the sub-tile
        if (masked) {
          const int kb = t * kTileKeys + jt * 32 + 4 * g - P;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int rel = kb + 8 * (i >> 2) + (i & 3);
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
        if (attempt == 0 && t == t_begin && jt == 0) {
          const float m0 = half_max(mx);
          m_ref = m0 == -INFINITY ? 0.f : m0;
        }

        // ---- probabilities against the reference max, bf16 for the PV product
        float psum = 0.f;
        bf16x8 pb[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(st[i], cs, -m_ref));
          psum += pv;
          pb[i >> 3][i & 7] = (__bf16)pv;
        }
        l_run += psum;

        // ---- O^T += V^T P^T over the 32 keys, as two 16-key contractions
        const unsigned char* vp = base + tr_off + jt * 32 * kRowStride;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int d = 0; d < 16; ++d) {
            const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(vp + (16 * u) * kRowStride + d * 64));
            const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(vp + (16 * u + 2) * kRowStride + d * 64));
            const s16x8 v = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v), pb[u], o[d], 0, 0, 0);
          }
        }
      }
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

  if (!active) return;

  // ---- finalize: both lane halves hold partial denominators of the same head
  const float lt = half_sum(l_run);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  const float lse_v = lt > 0.f ? (m_ref + log2f(lt)) * kLn2 : -INFINITY;

  const size_t orow = ((size_t)s * Q + qi) * kHeads + head;
  float* dst;
  float* ldst;
  if (a.n_splits == 1) {
    dst = a.out + orow * kDLat;
    ldst = a.lse + orow;
  } else {
    const size_t prow = (size_t)sp * a.n_streams * Q * kHeads + orow;
    dst = a.part_out + prow * kDLat;
    ldst = a.part_lse + prow;
  }
  // accumulator entry i of block d holds dim 32 d + 8 (i / 4) + 4 g + i % 4
#pragma unroll
  for (int d = 0; d < 16; ++d) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      float4 v;
      v.x = o[d][4 * i4 + 0] * inv;
      v.y = o[d][4 * i4 + 1] * inv;
      v.z = o[d][4 * i4 + 2] * inv;
      v.w = o[d][4 * i4 + 3] * inv;
      *reinterpret_cast<float4*>(dst + 32 * d + 8 * i4 + 4 * g) = v;
    }
  }
  if (g == 0) *ldst = lse_v;
}

// Merge of key-range splits by log-sum-exp: lse = log sum_k exp(lse_k),
// out = sum_k exp(lse_k - lse) out_k.  One thread per (row, 4 dims).
__global__ void __launch_bounds__(256) verify_combine_kernel(CombineArgs a) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  const int row = tid >> 7;
  const int c4 = tid & 127;
  if (row >= a.rows) return;
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
  *reinterpret_cast<float4*>(a.out + (size_t)row * kDLat + 4 * c4) = acc;
  if (c4 == 0) a.lse[row] = mx + logf(den);
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
  const long long blocks = (long long)a.n_streams * a.n_qgroups * a.n_splits;
  void* args[] = {const_cast<VerifyArgs*>(&a)};
  return hipLaunchKernel(reinterpret_cast<const void*>(verify_attn_kernel), dim3((unsigned)blocks),
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
