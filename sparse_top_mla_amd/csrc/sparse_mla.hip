// Sparse top-k MLA attention forward for MI355X (gfx950 / CDNA4).
//
// What is computed (FlashMLA PR #196, "Problem", "Fix", "Correctness notes";
// PR #216, "Summary"; PR #198, "Summary" for the sink): every query row
// attends, with all of its heads sharing one latent KV head, to the KV rows
// its index vector names.  Entries outside [0, K) are masked; the row length
// L (explicit topk_length, else one past the last valid entry found by a tail
// scan) bounds the block loop; positions >= L never address KV; an
// optional per-head sink joins the softmax denominator; a row without keys
// gives out = 0, lse = +inf, max_logits = -inf.
//
// Two kernels share the index, validity, tail-scan and paging routines:
//   * the wide kernel (h_q = 64 or 128, every benchmarked shape): a
//     persistent grid whose workgroups (2 or 4 waves, one wave per SIMD)
//     walk query rows, 32 heads per wave on v_mfma_f32_32x32x16_bf16; see the
//     block comment above it.
//   * the 16-head kernel below (other multiples of 16): one workgroup per
//     (query row, group of up to 64 heads), 16 heads per wave on
//     v_mfma_f32_16x16x32_bf16.
// Common to both:
//   * the row's query slice stays in VGPRs for the whole row (B operand of
//     S^T = K Q^T).
//   * per block (64 keys, or 32 in the 64-head d_qk = 512 layout): the index
//     vector is loaded one entry per lane and the validity of every key
//     becomes a wave ballot.  A block without a
//     valid key is skipped outright (no gather, no MFMA): masked keys add
//     exactly nothing to the softmax, so skipping is exact.
//   * valid KV rows are copied global -> LDS directly (16 B per lane, one
//     1 KiB instruction per row plus the 128 B rope part at d_qk = 576);
//     masked rows become zeros in LDS without touching memory, so a NaN
//     payload behind a masked index never reaches P*V.
//   * P^T is taken straight from the S^T accumulators: the keys of the two
//     MFMA operands are paired in a permuted order that makes each lane's P
//     values exactly the ones it already holds, so P never goes through LDS;
//     V^T is read with ds_read_b64_tr_b16.
//   * every lane owns one head for the whole softmax, so the softmax state
//     and the final 1/denominator are per-lane scalars.
//
// The presence of topk_length, of attn_sink, paging and d_qk are template
// parameters chosen on the host (FlashMLA PR #216, "Why template"): the fixed
// path carries no length load, no tail predicate and no sink code.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>
#include <type_traits>

#include "sparse_mla.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kBlockKeys = 64;    // keys per block (one per lane of a wave)
constexpr int kHeadsPerWave = 16; // MFMA N dimension
constexpr int kDV = 512;          // value width
constexpr int kPage = 64;         // tokens per KV page (decode)
constexpr int kMaxThreads = 512;  // up to 8 waves (h_q = 112 runs 7 in one group)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ds_read_b64_tr_b16: within each 16-lane group, lane i supplies the address
// of 4 consecutive 16-bit values; the 16 addresses describe a 4 x 16 tile
// (row TR_ROW(i), columns 4*TR_COL(i) .. +3) and lane n receives column n of
// the four rows.
#define TR_ROW(i) ((i) >> 2)
#define TR_COL(i) ((i) & 3)

template <int D_QK>
struct Tile {
  static constexpr int kRowBytes = D_QK * 2;        // one KV row in HBM
  static constexpr int kLdsRow = kRowBytes + 16;    // padded LDS row (bank spread)
  static constexpr int kLdsBytes = kBlockKeys * kLdsRow;
  static constexpr int kDSteps = D_QK / 32;         // MFMA K steps over d_qk
  static constexpr int kRopeLanes = (kRowBytes - 1024) / 16;
  static_assert(D_QK == 512 || D_QK == 576, "d_qk");
};

struct FwdArgs {
  const __bf16* q;
  const uint8_t* kv;
  const int32_t* indices;
  const int32_t* topk_length;
  const float* attn_sink;
  const int32_t* block_table;
  const int32_t* cache_seqlens;
  __bf16* out;
  float* lse;
  float* max_logits;      // NULL: not stored (decode)
  int32_t rows;          // query rows (prefill s_q; decode B * s_q)
  int32_t rows_per_seq;  // decode s_q (row r belongs to request r / rows_per_seq)
  int32_t h_q;
  int32_t topk;
  int32_t s_kv;          // prefill validity bound
  int32_t num_blocks;    // decode page pool size
  int32_t mbps;          // decode max_blocks_per_seq
  int32_t head_groups;   // workgroups per row (1 or 2)
  float scale_log2;      // sm_scale * log2(e)
  uint32_t kv_span;      // bytes of the KV table (wide and ring kernels: at most kMaxKvSpan)
  int32_t table_mode;    // 0: kv_span addressing; 1: BIG entries; 2: 64-bit (16-head kernel)
  int32_t splits;        // split decode: key-range splits per row (else 1)
  float* ws_o;           // split decode: [rows][splits][h_q][d_v] partial outputs
  float* ws_stats;       // split decode: [rows][splits][h_q][2] lse and max of each split
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// s_waitcnt vmcnt(0) through the builtin rather than inline assembly, so that
// the compiler's own wait insertion knows every earlier vector-memory load
// has completed (gfx9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15).  Behind an
// inline-asm wait it would still consider, say, the query loads in flight
// and wait for them again inside the block loop, where the count also covers
// the gather copies just issued.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Validity bound K of a row: s_kv for prefill; for paged decode the request's
// cache length, cut to what its block table can address.
__device__ __forceinline__ int row_bound(bool paged, const int32_t* cache_seqlens, int seq,
                                         int s_kv, int mbps) {
  if (!paged) return s_kv;
  const long long cs = cache_seqlens[seq];
  const long long addressable = (long long)mbps * kPage;
  return (int)(cs < addressable ? cs : addressable);
}

// Tail scan (FlashMLA PR #196, "Fix"): one round inspects the trailing 256
// positions of [0, end) with 4 coalesced loads per lane; the loads of the
// first round are issued before the rest of the prologue and consumed after.
struct TailRound {
  int v[4];
};

__device__ __forceinline__ TailRound load_tail_round(const int32_t* idx_row, int end,
                                                     int lane = lane_id()) {
  TailRound t;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int p = end - 256 + e * 64 + lane;
    t.v[e] = p >= 0 ? idx_row[p] : -1;
  }
  return t;
}

// Highest valid position of the round plus one, or 0 if it holds none.
__device__ __forceinline__ int resolve_tail_round(const TailRound& t, int end, int bound) {
#pragma unroll
  for (int e = 3; e >= 0; --e) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(t.v[e] >= 0 && t.v[e] < bound);
    if (m) return end - 256 + e * 64 + (63 - __builtin_clzll(m)) + 1;
  }
  return 0;
}

__device__ __forceinline__ int finish_tail_scan(const TailRound& first, const int32_t* idx_row,
                                                int topk, int bound) {
  int L = resolve_tail_round(first, topk, bound);
  for (int end = topk - 256; L == 0 && end > 0; end -= 256)
    L = resolve_tail_round(load_tail_round(idx_row, end), end, bound);
  return L;
}

__device__ __forceinline__ int clamp_length(int t, int topk) {
  return t < 0 ? 0 : (t > topk ? topk : t);
}

// Copy the block's KV rows into LDS: valid rows by direct global->LDS loads,
// masked rows as zeros (no memory access).  Wave w handles rows w, w+nw, ...
template <int D_QK>
__device__ __forceinline__ void stage_block(LDS_AS uint8_t* lds, const uint8_t* kv, uint64_t mask,
                                            int phys, int wave, int nwaves) {
  using T = Tile<D_QK>;
  const int lane = lane_id();
  for (int j = wave; j < kBlockKeys; j += nwaves) {
    LDS_AS uint8_t* dst = lds + j * T::kLdsRow;
    if ((mask >> j) & 1ull) {
      const int r = __builtin_amdgcn_readlane(phys, j);
      const uint8_t* src = kv + (size_t)(uint32_t)r * T::kRowBytes;
      __builtin_amdgcn_global_load_lds((const void*)(src + lane * 16), (LDS_AS void*)dst, 16, 0, 0);
      if (T::kRopeLanes > 0 && lane < T::kRopeLanes)
        __builtin_amdgcn_global_load_lds((const void*)(src + 1024 + lane * 16),
                                         (LDS_AS void*)(dst + 1024), 16, 0, 0);
    } else {
      *reinterpret_cast<LDS_AS u32x4*>(dst + lane * 16) = u32x4{0u, 0u, 0u, 0u};
      if (T::kRopeLanes > 0 && lane < T::kRopeLanes)
        *reinterpret_cast<LDS_AS u32x4*>(dst + 1024 + lane * 16) = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <int D_QK, bool PAGED, bool DYNAMIC, bool SINK>
__global__ void __launch_bounds__(kMaxThreads) sparse_mla_fwd_kernel(FwdArgs a) {
  using T = Tile<D_QK>;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[T::kLdsBytes];
  LDS_AS uint8_t* lds = (LDS_AS uint8_t*)lds_raw;

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int g = lane >> 4;    // lane group: 4 keys (S^T) / 4 value columns (O^T)
  const int hl = lane & 15;   // head within the wave (S^T / O^T column)

  int row, grp;
  if (a.head_groups == 1) {
    row = blockIdx.x;
    grp = 0;
  } else {  // ids 16*t + u and 16*t + u + 8 share row 8*t + u (same XCD)
    const int t = blockIdx.x >> 4, u = blockIdx.x & 15;
    grp = u >> 3;
    row = t * 8 + (u & 7);
  }
  if (row >= a.rows) return;
  const int seq = row / a.rows_per_seq;
  const int bound = row_bound(PAGED, a.cache_seqlens, seq, a.s_kv, a.mbps);
  const int32_t* idx_row = a.indices + (size_t)row * a.topk;

  TailRound first;
  int tl = 0;
  if (DYNAMIC)
    tl = a.topk_length[row];
  else
    first = load_tail_round(idx_row, a.topk);

  // Query slice of this wave's 16 heads: lane (g, hl) holds q[head hl][32s + 8g .. +8].
  const int head0 = grp * nwaves * kHeadsPerWave + wave * kHeadsPerWave;
  const __bf16* qp = a.q + ((size_t)row * a.h_q + head0 + hl) * D_QK + g * 8;
  bf16x8 qreg[T::kDSteps];
#pragma unroll
  for (int s = 0; s < T::kDSteps; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(qp + s * 32);

  const int L = DYNAMIC ? clamp_length(tl, a.topk) : finish_tail_scan(first, idx_row, a.topk, bound);

  f32x4 acc[kDV / 16];
#pragma unroll
  for (int ct = 0; ct < kDV / 16; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max of the log2-scaled logits
  float l_run = 0.f;        // running sum of exp2(logit - m_run)

  const int nblk = (L + kBlockKeys - 1) / kBlockKeys;
  for (int kb = 0; kb < nblk; ++kb) {
    // a2/a3: index, validity (positions >= L are masked before any use), page.
    const int pos = kb * kBlockKeys + lane;
    const int idx = pos < L ? idx_row[pos] : -1;
    bool ok = idx >= 0 && idx < bound;
    int phys = idx;
    if (PAGED) {
      const int page = ok ? a.block_table[(size_t)seq * a.mbps + (idx >> 6)] : -1;
      ok = ok && page >= 0 && page < a.num_blocks;
      phys = page * kPage + (idx & (kPage - 1));
    }
    const uint64_t mask = __builtin_amdgcn_ballot_w64(ok);
    if (mask == 0) continue;  // identical in every wave of the workgroup

    // a4: gather into LDS.
    __syncthreads();  // every wave is done reading the previous block
    stage_block<D_QK>(lds, a.kv, mask, phys, wave, nwaves);
    wait_vm_all();
    __syncthreads();

    // a5: S^T = K Q^T; lane (g, hl) gets keys kt*16 + 4g + r of head hl.
    f32x4 st[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < T::kDSteps; ++s) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const bf16x8 kfrag = *reinterpret_cast<const LDS_AS bf16x8*>(
            lds + (kt * 16 + hl) * T::kLdsRow + s * 64 + g * 16);
        st[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfrag, qreg[s], st[kt], 0, 0, 0);
      }
    }

    // a6: mask, online softmax in log2 units.
    float rmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const uint32_t bits = (uint32_t)(mask >> (kt * 16 + g * 4)) & 0xFu;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = ((bits >> r) & 1u) ? st[kt][r] * a.scale_log2 : -INFINITY;
        st[kt][r] = x;
        rmax = fmaxf(rmax, x);
      }
    }
    rmax = fmaxf(rmax, __shfl_xor(rmax, 16));
    rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
    const float m_new = fmaxf(m_run, rmax);  // finite: the block has a valid key
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float rsum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(st[kt][r] - m_new);
        st[kt][r] = p;
        rsum += p;
      }
    }
    rsum += __shfl_xor(rsum, 16);
    rsum += __shfl_xor(rsum, 32);
    l_run = l_run * alpha + rsum;
    m_run = m_new;
#pragma unroll
    for (int ct = 0; ct < kDV / 16; ++ct) acc[ct] *= alpha;

    // P^T operand of key step s2: element e <-> key 32*s2 + 16*(e/4) + 4g + e%4.
    bf16x8 pfrag[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int e = 0; e < 8; ++e) pfrag[s2][e] = (__bf16)st[2 * s2 + (e >> 2)][e & 3];

    // a7: O^T += V^T P^T; V^T element e of lane (g, c) is V[same key][c].
#pragma unroll
    for (int ct = 0; ct < kDV / 16; ++ct) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const LDS_AS uint8_t* base =
            lds + (32 * s2 + 4 * g + TR_ROW(hl)) * T::kLdsRow + (ct * 16 + 4 * TR_COL(hl)) * 2;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)base);
        const bf16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(base + 16 * T::kLdsRow));
        const bf16x8 vfrag = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vfrag, pfrag[s2], acc[ct], 0, 0, 0);
      }
    }
  }

  // a8: finalize.  acc[ct][r] = O[head hl][value column ct*16 + 4g + r].
  const int h = head0 + hl;
  float inv = 0.f, lse_v = INFINITY, ml_v = -INFINITY;
  if (l_run > 0.f) {
    float denom = l_run;
    if (SINK) denom += __builtin_amdgcn_exp2f(a.attn_sink[h] * kLog2e - m_run);
    inv = 1.f / denom;
    ml_v = m_run * kLn2;
    lse_v = (m_run + __log2f(l_run)) * kLn2;
  }
  __bf16* op = a.out + ((size_t)row * a.h_q + h) * kDV + g * 4;
#pragma unroll
  for (int ct = 0; ct < kDV / 16; ++ct) {
    const bf16x4 o4 = {(__bf16)(acc[ct][0] * inv), (__bf16)(acc[ct][1] * inv),
                       (__bf16)(acc[ct][2] * inv), (__bf16)(acc[ct][3] * inv)};
    *reinterpret_cast<bf16x4*>(op + ct * 16) = o4;
  }
  if (g == 0) {
    a.lse[(size_t)row * a.h_q + h] = lse_v;
    if (a.max_logits) a.max_logits[(size_t)row * a.h_q + h] = ml_v;
  }
}

// ---------------------------------------------------------------------------
// Wide kernel: 32 heads per wave (h_q a multiple of 32).
//
// LDS read bandwidth (128 B/clk per CU), not the matrix cores, bounds the
// 16-head kernel above: every wave re-reads the whole K and V block for 16
// heads.  Here a wave owns 32 heads, so each K/V byte read from LDS feeds
// twice the MFMA work (v_mfma_f32_32x32x16_bf16 with N = 32 heads), and LDS
// time per block matches MFMA time.  One wave per SIMD: the 32-head O^T
// accumulator (256 fp32 per lane) stays in AGPRs and is touched only by MFMA
// inside the block loop; the query slice stays in VGPRs.
//
// Workgroup: NW waves (one per SIMD of the CUs it occupies) working on blocks
// of BK = 16 NW keys (each wave copies 16 rows of a block), as NW / KS head
// groups of 32 heads times KS key splits:
//   128 heads:             NW = 4, KS = 1, one workgroup per CU, 64-key blocks;
//   64 heads, d_qk = 512:  NW = 2, KS = 1, two workgroups per CU, 32-key blocks;
//   64 heads, d_qk = 576:  NW = 4, KS = 2 (two 2-wave workgroups do not fit the
//                          registers at d_qk = 576): the two waves of a head
//                          group take the lower and upper 32 keys of every
//                          64-key block and merge at the end of the row.
// A wave computes 32 keys x 32 heads per tile in every layout.
//
// Pipeline per block t (two LDS buffers; the loop is unrolled by two so each
// half-iteration reads one buffer and fills the other):
//   wait for block t's rows + barrier
//   rows of block t+1 from the index and page loaded one step earlier; its
//   rope part is copied at once
//   issue the page lookups of block t+2 and the index loads of block t+3
//   S^T, masked softmax, O^T += V^T P^T for block t, with the copies of
//   block t+1's 1 KiB rows issued one at a time between the MFMAs (a wave
//   that issues many copies at once stalls until the memory pipeline drains)
//
// Softmax reference: each head's exp2 reference is the max of its first
// block with a valid key and then stays fixed, so O is never rescaled in the
// loop.  A later logit more than 2^kRefSlack above the reference would
// overflow that scheme; it flags the row, and the workgroup recomputes the
// row once with the true row max as the reference.  P <= 2^kRefSlack is
// representable in bf16 (fp32 exponent range) and the sums stay below 2^90.
// max_logits is the true max.
// ---------------------------------------------------------------------------

typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr float kRefSlack = 64.0f;  // log2 units
constexpr int kWideWaves = 4;       // waves per CU: one per SIMD
constexpr int kMaxSplits = 1024;    // split decode: key-range splits per row

template <int D_QK, int BK = 64>
struct WideTile {
  // LDS block layout: the first 512 columns ("nope" part, also V) of each of
  // the 64 rows in 1 KiB rows, then the remaining d_qk - 512 columns ("rope"
  // part) in 128 B rows.  16-byte chunks are XOR-swizzled within each row so
  // that both MFMA operand reads are bank-conflict free: the K read (16 rows,
  // one chunk column) and the transposed V read (4 rows, 4 adjacent chunks).
  static constexpr int kRowBytes = D_QK * 2;
  static constexpr int kNopeBytes = 1024;
  static constexpr int kRopeBytes = kRowBytes - kNopeBytes;  // 0 or 128
  static constexpr int kRopeBase = BK * kNopeBytes;
  static constexpr int kBufBytes = BK * kRowBytes;
  static constexpr int kDSteps = D_QK / 16;        // 32x32x16 K steps over d_qk
  static constexpr int kRopeLanes = kRopeBytes / 16;
  static_assert(kRopeBytes == 0 || kRopeBytes == 128, "d_qk");
  static_assert(32 * kDV * 2 <= kBufBytes, "a wave's bf16 output tile fits a buffer");
};

// Chunk swizzles: nope rows permute the 16 chunks of each 256 B group by
// r -> 4(r%4) + (r/4)%4; rope rows (8 chunks) by (r/2)%8.
__device__ __forceinline__ int nope_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int rope_swz(int r) { return (r >> 1) & 7; }

struct BlockMeta {
  uint64_t mask;  // bit j: key j of the block is used
  int phys;       // lane j: KV row of key j (prefill index or paged slot)
  bool ok;        // lane j: bit j of mask
};

// Blocks of BK keys: lane j < BK holds position BK blk + j; lanes >= BK
// (BK = 32) hold no key.
template <int BK>
__device__ __forceinline__ int load_index(const int32_t* idx_row, int blk, int topk,
                                          int lane = lane_id()) {
  const int pos = blk * BK + lane;
  return lane < BK && pos < topk ? idx_row[pos] : -1;
}

template <int BK>
__device__ __forceinline__ bool index_ok(int idx, int blk, int L, int bound) {
  const int lane = lane_id();
  const int pos = blk * BK + lane;
  return lane < BK && pos < L && idx >= 0 && idx < bound;
}

template <bool PAGED>
__device__ __forceinline__ int page_lookup(const FwdArgs& a, int seq, bool ok, int idx) {
  if (!PAGED) return 0;
  return ok ? a.block_table[(size_t)seq * a.mbps + (idx >> 6)] : -1;
}

template <bool PAGED>
__device__ __forceinline__ BlockMeta block_meta(const FwdArgs& a, bool ok, int idx, int page) {
  BlockMeta m;
  int phys = idx;
  if (PAGED) {
    ok = ok && page >= 0 && page < a.num_blocks;
    phys = page * kPage + (idx & (kPage - 1));
  }
  m.mask = __builtin_amdgcn_ballot_w64(ok);
  m.phys = phys;
  m.ok = ok;
  return m;
}

// The gather copies KV rows global -> LDS directly (no VGPR round trip).
// Both forms are inline assembly: a direct-to-LDS load the compiler can see
// makes it wait for all outstanding LDS reads (lgkmcnt(0)) before every LDS
// read while the load is in flight, which would serialise the MFMA operand
// stream the loads are interleaved with.  Completion is tracked with the
// explicit vmcnt(0) wait at the top of every pipeline step.  M0 (the LDS
// destination) needs one wait state before the load reads it.  Lane L writes
// LDS bytes [M0 + 16L, M0 + 16L + 16).

// M0 is an operand of both forms ("{m0}"), so the compiler writes it only
// when its value changes; the s_nop is the wait state an LDS DMA needs after
// an M0 write.

// Hides a value from loop-invariant code motion: per-lane offsets that are
// the same in every block (LDS operand offsets summed with the two buffer
// bases) would otherwise each be hoisted into a register of their own.
__device__ __forceinline__ void opaque(int& v) { asm volatile("" : "+v"(v)); }

// A wave-uniform value that the compiler takes as new where this is called:
// what is derived from it is computed there, not hoisted out of the
// enclosing loop (where it would be live across the stage loop and spilled).
__device__ __forceinline__ int fresh_s(int v) {
  asm volatile("" : "+s"(v));
  return v;
}

// The lane index, computed where it is called: lane_id() is a pure builtin
// that the compiler computes once and keeps (or spills) for the whole kernel.
// Values derived from this one are computed per row of the row loop instead
// of being hoisted out of it, where they would hold registers across every
// block.
__device__ __forceinline__ int lane_fresh() {
  int v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
  return v;
}

// The gather reads the KV table through one raw buffer resource
// whose base sits kSpanBias bytes below the table (records: span + bias).
// buffer_load_dwordx4 ... offset:OFF lds reads base + voff + OFF per lane
// and writes LDS bytes [M0 + OFF + 16L, +16) for lane L; the range check
// covers voff + OFF, and an offset outside the records reads nothing and
// writes zeros to LDS, so a masked row is zero-filled without touching
// memory and without a branch or an EXEC change inside the MFMA stream.
typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
constexpr uint32_t kSpanBias = 3 * 1024;  // room for the largest OFF below
constexpr uint32_t kOob = 0xFFFFE000u;    // + lane chunk + OFF: outside, no wrap
constexpr uint32_t kMaxKvSpan = kOob - kSpanBias;

__device__ __forceinline__ u32x4s table_rsrc(const FwdArgs& a) {
  const uint64_t b = (uint64_t)(uintptr_t)a.kv - kSpanBias;
  u32x4s rs;
  rs[0] = __builtin_amdgcn_readfirstlane((uint32_t)b);
  rs[1] = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) & 0xffffu;  // stride 0
  rs[2] = __builtin_amdgcn_readfirstlane(a.kv_span + kSpanBias);
  rs[3] = 0x00020000u;  // 32-bit data format, no swizzle
  return rs;
}

// The same form of resource over one row's query slice (h_q rows of d_qk),
// read by the gather as if it were a KV table with head j at row j.
__device__ __forceinline__ u32x4s query_rsrc(const FwdArgs& a, int row, int row_bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)(a.q + (size_t)row * a.h_q * (row_bytes / 2)) - kSpanBias;
  u32x4s rs;
  rs[0] = __builtin_amdgcn_readfirstlane((uint32_t)b);
  rs[1] = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) & 0xffffu;
  rs[2] = __builtin_amdgcn_readfirstlane((uint32_t)(a.h_q * row_bytes) + kSpanBias);
  rs[3] = 0x00020000u;
  return rs;
}

// Tables above kMaxKvSpan bytes (BIG instances).  A key is then its row's
// byte offset in units of kBigUnit (d_qk * 2 is a multiple; a 32-bit entry
// reaches 512 GiB), or kBigNone for no row, and each copy of a whole row
// reads through a resource rebased on that row: base = row - OFF, where OFF
// is the instruction offset the copy uses, and records OFF + 1 KiB, so the
// copy's lane offsets (below 1 KiB) plus OFF stay inside; a kBigNone row
// gets no records and is zero-filled as a masked row of a small table is.
// The resource is built in scalar registers per copy (shift, 64-bit add,
// select).  A base below 2^48 leaves the stride bits of word 1 clear.
// big_table_rsrc carries the table's address in words 0 and 1.
constexpr uint32_t kBigUnit = 128;
constexpr uint32_t kBigNone = 0xFFFFFFFFu;

__device__ __forceinline__ u32x4s big_table_rsrc(const FwdArgs& a) {
  const uint64_t b = (uint64_t)(uintptr_t)a.kv;
  u32x4s rs;
  rs[0] = __builtin_amdgcn_readfirstlane((uint32_t)b);
  rs[1] = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  rs[2] = 0u;
  rs[3] = 0u;
  return rs;
}

template <int OFF>
__device__ __forceinline__ u32x4s big_row_rsrc(const u32x4s& tb, uint32_t e) {
  const uint64_t b = ((((uint64_t)tb[1]) << 32) | tb[0]) + ((uint64_t)e * kBigUnit) - (uint64_t)OFF;
  u32x4s rs;
  rs[0] = (uint32_t)b;
  rs[1] = (uint32_t)(b >> 32);
  rs[2] = e == kBigNone ? 0u : (uint32_t)(OFF + 1024);
  rs[3] = 0x00020000u;
  return rs;
}

// Zeros for the BIG rope copies of masked rows (a per-lane global copy has
// no records to fall outside of).
__device__ __attribute__((aligned(16))) uint8_t g_zero_chunks[128];

// The BIG rope copy of one lane: 16 bytes at byte `col` of row entry `e`
// (zeros for kBigNone) to LDS [lds + 16 lane, +16).  Inline assembly, as the
// table copies: the compiler would count a builtin LDS copy as a store that
// every later LDS read must wait for.
__device__ __forceinline__ void big_rope_copy(const u32x4s& tb, uint32_t e, uint32_t col,
                                              LDS_AS uint8_t* lds) {
  const uint64_t base = (((uint64_t)tb[1]) << 32) | tb[0];
  const uint64_t src = e == kBigNone ? (uint64_t)(uintptr_t)(g_zero_chunks + (col & 127u))
                                     : base + (uint64_t)e * kBigUnit + col;
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "{m0}"(__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds))
               : "memory");
}

// NOP: the wait state an LDS DMA needs after an M0 write (the compiler writes
// M0 for the operand only when its value changes).
template <int OFF, bool NOP = true>
__device__ __forceinline__ void dma_table16(const u32x4s& rs, uint32_t voff, uint32_t m0v) {
  if (NOP)
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen offset:%2 lds"
                 :
                 : "v"(voff), "s"(rs), "i"(OFF), "{m0}"(__builtin_amdgcn_readfirstlane(m0v))
                 : "memory");
  else
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen offset:%2 lds"
                 :
                 : "v"(voff), "s"(rs), "i"(OFF), "{m0}"(__builtin_amdgcn_readfirstlane(m0v))
                 : "memory");
}

// The copy of one 1 KiB row (nope part) at instruction offset K KiB, lane
// byte `lp` of the row: small tables take `so`, the row's offset moved down
// by K KiB, through the table resource `rs`; BIG tables take `so` as the
// row's entry and `rs` as big_table_rsrc.
template <int K, bool NOP, bool BIG>
__device__ __forceinline__ void copy_row(const u32x4s& rs, uint32_t so, uint32_t lp, uint32_t win) {
  if constexpr (BIG)
    dma_table16<K * 1024, NOP>(big_row_rsrc<K * 1024>(rs, so), lp, win);
  else
    dma_table16<K * 1024, NOP>(rs, lp + so, win);
}

// copy_row with K = s % 4 (s a constant once unrolled); `opens`: M0 was just
// written for this copy.
template <bool BIG>
__device__ __forceinline__ void copy_slot(int s, bool opens, const u32x4s& rs, uint32_t so,
                                          uint32_t lp, uint32_t win) {
  switch (s & 3) {
    case 0: copy_row<0, true, BIG>(rs, so, lp, win); break;
    case 1: opens ? copy_row<1, true, BIG>(rs, so, lp, win) : copy_row<1, false, BIG>(rs, so, lp, win); break;
    case 2: opens ? copy_row<2, true, BIG>(rs, so, lp, win) : copy_row<2, false, BIG>(rs, so, lp, win); break;
    default: opens ? copy_row<3, true, BIG>(rs, so, lp, win) : copy_row<3, false, BIG>(rs, so, lp, win); break;
  }
}

// Nope part (the first 512 columns, also V) of a block, one 1 KiB row per
// call, so that the copies can be spread over the MFMA work of the previous
// block: the issuing wave stalls while the memory pipeline is full, and a
// whole block issued at once would stall it for the full gather time.  Wave w
// copies rows 16w .. 16w + 15; slot s (a constant once the caller's loop is
// unrolled) is row 16w + s.  M0 points at the four-row window 16w + 4(s/4)
// and the instruction offset (s % 4) KiB selects the row within it, so M0
// changes once every four copies (an M0 write costs the issuing wave time).
// The instruction offset is added to the memory address as well, so the
// per-row offsets (one per lane of `offw`, built once per block) are moved
// down by it: a copy is a readlane, two VALU ops and the load.  A masked row,
// or any row of a block past the end of the query row, has offset kOob and
// is zero-filled.  Lane L fills LDS chunk L of the row, so it fetches source
// chunk L ^ swizzle(row); the swizzle depends on the row's low four bits
// only, i.e. on s.  BIG tables: `offw` holds the rows' entries (kBigUnit
// offsets, or kBigNone) and each copy rebases a resource on its row.
template <int D_QK, bool BIG = false>
struct GatherPump {
  using T = WideTile<D_QK>;
  static constexpr int kSlots = 16;  // rows per wave and block
  static_assert(T::kNopeBytes == 1024, "copy_row copies 1 KiB rows");
  u32x4s rsrc;       // table resource, or big_table_rsrc (wave-uniform)
  LDS_AS uint8_t* buf;
  int row0;          // first row of this wave (wave-uniform)
  int offw;          // lane s: source offset of row row0 + s (see row_offsets)
  int lane16;        // 16 * lane
  uint32_t issued;   // slots copied so far (wave-uniform)
  uint32_t win;      // M0 of the current four-row window
  uint32_t so_next;  // offset of the next slot, read one copy ahead

  // Lane j of the result: offset of key j's row for slot j % 4, or kOob
  // (BIG: the row's entry, or kBigNone).
  static __device__ __forceinline__ int row_offsets(const BlockMeta& m) {
    if constexpr (BIG)
      return (int)(m.ok ? (uint32_t)m.phys * (uint32_t)(T::kRowBytes / kBigUnit) : kBigNone);
    const uint32_t off = (uint32_t)m.phys * (uint32_t)T::kRowBytes + kSpanBias -
                         (uint32_t)(lane_id() & 3) * T::kNopeBytes;
    return (int)(m.ok ? off : kOob);
  }
  // The wave's sixteen rows, moved to lanes 0..15.
  static __device__ __forceinline__ int wave_offsets(int offs, int row0) {
    return __shfl(offs, row0 + (lane_id() & (kSlots - 1)));
  }

  // fresh: compute the window here (finish, where slots may be skipped);
  // otherwise slot s % 4 == 0 opens the window and the next three reuse it,
  // so the compiler sees one M0 value per window and writes M0 once.
  // first: the first copy of a run of consecutive slots reads its own
  // offset; every copy reads the next slot's offset ahead, so that the VALU
  // use of a readlane result never follows the readlane directly.
  __device__ __forceinline__ void copy(int s, bool fresh = false, bool first = true) {
    const bool opens = fresh || (s & 3) == 0;
    if (opens) win = (uint32_t)(uintptr_t)(buf + (row0 + (s & ~3)) * T::kNopeBytes);
    const uint32_t so = first ? (uint32_t)__builtin_amdgcn_readlane(offw, s) : so_next;
    if (s + 1 < kSlots) so_next = (uint32_t)__builtin_amdgcn_readlane(offw, s + 1);
    copy_slot<BIG>(s, opens, rsrc, so, (uint32_t)lane16 ^ (uint32_t)(nope_swz(s) << 4), win);
    issued |= 1u << s;
  }
  // Copies every slot in order (a block gathered outside the MFMA stream).
  __device__ __forceinline__ void copy_all() {
#pragma unroll
    for (int s = 0; s < kSlots; ++s) copy(s, false, s == 0);
  }
  // Copies the slots that were not copied in the MFMA stream (all of them for
  // a block whose tiles this wave skipped).
  // LOOP: a run-time loop over the missing slots (usually none: one test
  // instead of sixteen); otherwise unrolled tests.
  template <bool LOOP>
  __device__ __forceinline__ void finish() {
    if (LOOP) {
      for (uint32_t miss = ~issued & ((1u << kSlots) - 1); miss != 0; miss &= miss - 1)
        copy_any(__builtin_ctz(miss));
    } else {
      // A test per four slots, then per slot (tests only; the copies stay
      // one per slot, which is what the register allocation of the 64-head
      // kernel tolerates).
#pragma unroll
      for (int q = 0; q < kSlots; q += 4)
        if (((issued >> q) & 15u) != 15u) {
#pragma unroll
          for (int s = q; s < q + 4; ++s)
            if (!((issued >> s) & 1u)) copy(s, true);
        }
    }
  }
  // copy() for a slot known only at run time (the offset selection branches).
  __device__ __forceinline__ void copy_any(int s) {
    win = (uint32_t)(uintptr_t)(buf + (row0 + (s & ~3)) * T::kNopeBytes);
    const uint32_t so = (uint32_t)__builtin_amdgcn_readlane(offw, s);
    copy_slot<BIG>(s, true, rsrc, so, (uint32_t)lane16 ^ (uint32_t)(nope_swz(s) << 4), win);
  }
};

// Rope part (d_qk = 576) of a block: 8 rows of 128 B per load, wave w of NW
// taking row groups w, w + NW, ...  Lane L handles row jj = 8g + L/8, LDS chunk L%8,
// which holds source chunk (L%8) ^ swizzle(jj); `offs` are the per-key
// offsets of GatherPump::row_offsets (moved down by (jj % 4) KiB, which is
// added back), so masked rows stay outside the records and read zeros.
// BIG: `offs` are entries, and each lane copies from its own row's address.
template <int D_QK, int BK, int NW, bool BIG = false>
__device__ __forceinline__ void stage_rope(LDS_AS uint8_t* buf, const u32x4s& rsrc, int offs,
                                           int wave) {
  using T = WideTile<D_QK, BK>;
  if (T::kRopeLanes == 0) return;
  const int lane = lane_id();
#pragma unroll
  for (int g0 = 0; g0 < BK / 8; g0 += NW) {
    const int g = g0 + wave;
    const int jj = 8 * g + (lane >> 3);
    const uint32_t o = (uint32_t)__shfl(offs, jj);
    const uint32_t col = T::kNopeBytes + (uint32_t)(((lane & 7) ^ rope_swz(jj)) << 4);
    LDS_AS uint8_t* dst = buf + T::kRopeBase + g * 8 * T::kRopeBytes;
    if constexpr (BIG)
      big_rope_copy(rsrc, o, col, dst);
    else
      dma_table16<0>(rsrc, o + (uint32_t)(jj & 3) * T::kNopeBytes + col, (uint32_t)(uintptr_t)dst);
  }
}

// Running softmax state of one lane's head (log2 units); both halves of the
// wave hold identical copies.
struct SoftmaxState {
  float m_ref;  // exp2 reference (fixed once set)
  float l_sum;  // sum of exp2(s - m_ref)
  float m_max;  // true max (max_logits)
  bool overflow;
};

// Max / sum of a value over lanes l and l ^ 32 with v_permlane32_swap (VALU;
// a ds_bpermute shuffle would queue behind outstanding LDS reads).  The swap
// exchanges the upper half of its first operand with the lower half of its
// second, so with both operands holding x every lane ends up with its own
// value and its partner's.  The second copy goes through an identity DPP
// move: given one value twice, the compiler folds the pair into a single
// copy and drops the partner.
__device__ __forceinline__ uint2 pair32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const unsigned v = (unsigned)__builtin_amdgcn_mov_dpp((int)u, 0xE4, 0xF, 0xF, false);
  const auto r = __builtin_amdgcn_permlane32_swap(u, v, false, false);
  return uint2{r[0], r[1]};
}
__device__ __forceinline__ float pair_max32(float x) {
  const uint2 r = pair32(x);
  return fmaxf(__builtin_bit_cast(float, r.x), __builtin_bit_cast(float, r.y));
}
__device__ __forceinline__ float pair_sum32(float x) {
  const uint2 r = pair32(x);
  return __builtin_bit_cast(float, r.x) + __builtin_bit_cast(float, r.y);
}


// v_mfma_f32_32x32x16_bf16 with its accumulator in VGPRs.  The O^T
// accumulator fills the AGPRs, and every MFMA the compiler emits in this
// kernel takes its accumulator from AGPRs, so a compiled S^T chain would
// evict part of O^T to VGPRs and back in every stage (48 moves, each about
// two MFMA-issue cycles with one wave per SIMD).  The compiler does not see
// the timing of these MFMAs: the first of a chain starts after two wait
// states (a VALU write of an operand before it), consecutive ones chain on
// the accumulator without wait states, and the last is followed by 18 wait
// states before anything may read the result (an 8-pass MFMA's result is
// readable by VALU after 11).
__device__ __forceinline__ void mfma_vacc_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vacc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vacc_last(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 1"
               : "+v"(acc)
               : "v"(a), "v"(b));
}

// max of three floats as one v_max3_f32.  fmaxf on values the compiler
// cannot prove canonical (MFMA results) costs a canonicalising v_max_f32 per
// operand first; the scores are never signalling NaNs.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// A wave works on 32-key tiles: keys [r0, r0 + 32) of the block in LDS, with
// validity bits `bits` (bit i <-> key r0 + i).  Every function below that
// issues MFMAs copies one row of the next block's gather (gather slots
// slot0, slot0 + 1, ..., at most NP of them) after every EVERY-th of them.  In the S^T accumulator layout a lane holds keys
// 8(i/4) + 4half + i%4 (i = 0..15) of the tile for its head hl.

// S^T[key][head] = K Q^T of one tile.  Lane (half, hl) reads chunk 2d + half of key row r0 + hl; r0 is a multiple
// of 16, so the swizzle depends on hl only and a lane needs one base offset
// per value of d % 8 (plus 4 for the rope chunks); everything else is an
// immediate offset.  Chunk 2d + half of a row sits at chunk (2d ^ half ^ swz)
// of its 256 B group, so each address is a row base plus (32(d%8) ^ w) with
// one per-lane w; the rope part likewise with its own swizzle.  K fragments
// are read kPrefetch MFMAs ahead.  LFRESH: the lane's addresses are computed
// here per tile (see lane_fresh) instead of once for the kernel; what the
// register allocation of each kernel instance prefers, by measurement.
template <int D_QK, int BK, int EVERY, int NP, bool LFRESH, class Pump, int KP = 0>
__device__ __forceinline__ f32x16 tile_scores(const LDS_AS uint8_t* buf, int r0,
                                              const bf16x8 (&qf)[WideTile<D_QK>::kDSteps],
                                              Pump& pump, int slot0) {
  using T = WideTile<D_QK, BK>;
  // K fragments read ahead: what the register budget allows (KP overrides)
  constexpr int kPrefetch = KP > 0 ? KP : D_QK == 576 ? 3 : 4;
  const int lane = LFRESH ? lane_fresh() : lane_id();
  const int hl = lane & 31, half = lane >> 5;
  int krow = (r0 + hl) * T::kNopeBytes, kw = (half ^ nope_swz(hl)) << 4;
  int rrow = T::kRopeBase + (r0 + hl) * T::kRopeBytes, rw = (half ^ rope_swz(hl)) << 4;
  opaque(krow);
  opaque(kw);
  opaque(rrow);
  opaque(rw);
  auto kaddr = [&](int d) {
    if (d < 32) return buf + krow + (d >> 3) * 256 + ((32 * (d & 7)) ^ kw);
    return buf + rrow + ((32 * (d - 32)) ^ rw);
  };
  f32x16 s;
  bf16x8 kring[kPrefetch];
#pragma unroll
  for (int n = 0; n < kPrefetch; ++n) kring[n] = *reinterpret_cast<const LDS_AS bf16x8*>(kaddr(n));
#pragma unroll
  for (int d = 0; d < T::kDSteps; ++d) {
    const bf16x8 kf = kring[d % kPrefetch];
    if (d + kPrefetch < T::kDSteps)
      kring[d % kPrefetch] = *reinterpret_cast<const LDS_AS bf16x8*>(kaddr(d + kPrefetch));
    // VGPR accumulator: O^T fills the AGPRs (see mfma_vacc)
    if (d == 0)
      mfma_vacc_first(s, kf, qf[d]);
    else if (d == T::kDSteps - 1)
      mfma_vacc_last(s, kf, qf[d]);
    else
      mfma_vacc(s, kf, qf[d]);
    if (d % EVERY == EVERY - 1 && d / EVERY < NP) pump.copy(slot0 + d / EVERY, false, d / EVERY == 0);
    __builtin_amdgcn_sched_barrier(0);  // keep the read-ahead distance
  }
  return s;
}

// Masks the tile (masked logits become -inf) and takes its row max against
// the softmax state; returns the exp2 offset -m_ref (0 while no reference is
// set, when every logit seen is -inf).  The scale is positive, so the max is
// taken on the raw dot products and each probability is
// exp2(fma(s, scale, -m_ref)).  Branch-free: a branch here would split the
// MFMA streams this code is scheduled into.
__device__ __forceinline__ float tile_max(f32x16& s, uint32_t bits, SoftmaxState& st,
                                          float scale_log2) {
  if (bits != 0xffffffffu) {  // wave-uniform: full tiles (almost all) skip the masking
    const uint32_t mlane = bits >> (4 * (lane_id() >> 5));
#pragma unroll
    for (int i = 0; i < 16; ++i)
      s[i] = ((mlane >> (8 * (i >> 2) + (i & 3))) & 1u) ? s[i] : -INFINITY;
  }
  const float m0 = max3_raw(s[0], s[1], s[2]), m1 = max3_raw(s[3], s[4], s[5]);
  const float m2 = max3_raw(s[6], s[7], s[8]), m3 = max3_raw(s[9], s[10], s[11]);
  const float m4 = max3_raw(s[12], s[13], s[14]);
  float rmax = max3_raw(max3_raw(m0, m1, m2), max3_raw(m3, m4, s[15]), -INFINITY);
  const uint2 pr = pair32(rmax);
  // -inf only for a tile without a valid key
  rmax = max_raw(__builtin_bit_cast(float, pr.x), __builtin_bit_cast(float, pr.y)) * scale_log2;
  st.m_max = max_raw(st.m_max, rmax);
  if (st.m_ref == -INFINITY) st.m_ref = rmax;
  st.overflow |= rmax > st.m_ref + kRefSlack;  // this attempt is then discarded
  return st.m_ref == -INFINITY ? 0.f : -st.m_ref;
}

// Probability of logit s (log2 units after scaling) against the reference.
__device__ __forceinline__ float prob(float s, float neg_ref, float scale_log2) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(s, scale_log2, neg_ref));
}

// O^T[c][head] += V^T P^T of one tile, key step u = 0 for every value tile
// first, so that the probabilities of step 1 are computed under the MFMAs of
// step 0.  The P^T operand of step u holds, as element e, key
// 16u + 8(e/4) + 4half + e%4, which is s[8u + e] of this lane.  Lane (16-group grp, i16) reads 8 B of key row r0 + 16u + 4half +
// TR_ROW(i16) (+8 for the upper four keys) at value chunk 4ct + 2(grp&1) +
// TR_COL(i16)/2 with ds_read_b64_tr_b16.  Value chunk 4ct + vc of row vrow
// (+8) sits at chunk (4ct ^ vc ^ swz) of its 256 B group: a row base plus
// (64(ct%4) ^ w) with one w per row half.  MFMA n covers value tile
// ct = n % 16, step u = n / 16.
template <int D_QK, int EVERY, int NP, bool LFRESH, class Pump>
__device__ __forceinline__ void tile_softmax_pv(const LDS_AS uint8_t* buf, int r0, f32x16 s,
                                                uint32_t bits, f32x16 (&acc)[kDV / 32],
                                                SoftmaxState& st, float scale_log2, Pump& pump,
                                                int slot0) {
  using T = WideTile<D_QK>;
  constexpr int kPrefetch = D_QK == 576 ? 3 : 4;  // what the register budget allows
  constexpr int kTiles = kDV / 32;
  const int lane = LFRESH ? lane_fresh() : lane_id();
  const int i16 = lane & 15, cb = (lane >> 4) & 1, half = lane >> 5;
  const int vrow = r0 + 4 * half + TR_ROW(i16);
  const int vc = 2 * cb + (TR_COL(i16) >> 1);
  int row_lo = vrow * T::kNopeBytes + 8 * (TR_COL(i16) & 1);
  int row_hi = row_lo + 8 * T::kNopeBytes;
  int w_lo = (vc ^ nope_swz(vrow)) << 4, w_hi = (vc ^ nope_swz(vrow + 8)) << 4;
  opaque(row_lo);
  opaque(row_hi);
  opaque(w_lo);
  opaque(w_hi);
  auto vaddr = [&](int n, bool upper) {
    const int ct = n % kTiles, u = n / kTiles;
    return buf + (upper ? row_hi : row_lo) + (ct >> 2) * 256 + 16 * u * T::kNopeBytes +
           ((64 * (ct & 3)) ^ (upper ? w_hi : w_lo));
  };
  bf16x4 lo[kPrefetch], hi[kPrefetch];
#pragma unroll
  for (int n = 0; n < kPrefetch; ++n) {
    lo[n] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)vaddr(n, false));
    hi[n] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)vaddr(n, true));
  }
  const float neg_ref = tile_max(s, bits, st, scale_log2);
  float p0[8];
  bf16x8 pf[2];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p0[e] = prob(s[e], neg_ref, scale_log2);
    pf[0][e] = (__bf16)p0[e];
  }
  // Pairwise sums (short dependency chains).
  float rsum = ((p0[0] + p0[1]) + (p0[2] + p0[3])) + ((p0[4] + p0[5]) + (p0[6] + p0[7]));
  // Step 1's probabilities, two per MFMA of step 0 (sched barriers below keep
  // them there).
  float p1[8];
#pragma unroll
  for (int n = 0; n < 2 * kTiles; ++n) {
    const bf16x4 l = lo[n % kPrefetch], h = hi[n % kPrefetch];
    if (n + kPrefetch < 2 * kTiles) {
      lo[n % kPrefetch] =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)vaddr(n + kPrefetch, false));
      hi[n % kPrefetch] =
          __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)vaddr(n + kPrefetch, true));
    }
    const bf16x8 vf = {l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
    acc[n % kTiles] =
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[n / kTiles], acc[n % kTiles], 0, 0, 0);
    if (n < 4) {
      p1[2 * n] = prob(s[8 + 2 * n], neg_ref, scale_log2);
      p1[2 * n + 1] = prob(s[9 + 2 * n], neg_ref, scale_log2);
    } else if (n == 4) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[1][e] = (__bf16)p1[e];
      rsum += ((p1[0] + p1[1]) + (p1[2] + p1[3])) + ((p1[4] + p1[5]) + (p1[6] + p1[7]));
    }
    if (n % EVERY == EVERY - 1 && n / EVERY < NP) pump.copy(slot0 + n / EVERY, false, n / EVERY == 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  st.l_sum += pair_sum32(rsum);
}

// One block with a valid key for one wave: the wave's 32-key tiles among
// keys [koff, koff + BK/KS) (one or two); tiles without a valid key are
// skipped (their gather slots are then copied by GatherPump::finish).  The
// first tile takes every gather slot of the wave, as many under S^T as its
// MFMAs allow at one per EVERY and the rest under P*V, so that the copies
// leave early.
template <int D_QK, int BK, int KS, int EVERY, bool LFRESH, class Pump>
__device__ __forceinline__ void wide_block(const LDS_AS uint8_t* buf, uint64_t mask, int koff,
                                           const bf16x8 (&qf)[WideTile<D_QK>::kDSteps],
                                           f32x16 (&acc)[kDV / 32], SoftmaxState& st,
                                           float scale_log2, Pump& pump) {
  constexpr int kTiles = BK / KS / 32;
  constexpr int kSlots = Pump::kSlots;
  constexpr int kSteps = WideTile<D_QK>::kDSteps;
  constexpr int NS = kSteps / EVERY < kSlots ? kSteps / EVERY : kSlots;  // under S^T
  constexpr int NV = kSlots - NS;                                       // under P*V
  static_assert(NV * EVERY <= 2 * kDV / 32, "gather slots per P*V pass");
#pragma unroll
  for (int kt = 0; kt < kTiles; ++kt) {
    const int r0 = koff + 32 * kt;
    const uint32_t bits = (uint32_t)(mask >> r0);
    if (bits != 0u) {
      const f32x16 s = kt == 0 ? tile_scores<D_QK, BK, EVERY, NS, LFRESH>(buf, r0, qf, pump, 0)
                               : tile_scores<D_QK, BK, EVERY, 0, LFRESH>(buf, r0, qf, pump, 0);
      if (kt == 0)
        tile_softmax_pv<D_QK, EVERY, NV, LFRESH>(buf, r0, s, bits, acc, st, scale_log2, pump, NS);
      else
        tile_softmax_pv<D_QK, EVERY, 0, LFRESH>(buf, r0, s, bits, acc, st, scale_log2, pump, 0);
    }
  }
}

// Look-ahead state of the pipeline at the top of step t: index and page of
// block t+1, index of block t+2.  Every load is consumed only after the next
// step's vmcnt(0) wait, so no wait inside a step covers the gather loads.
struct Ahead {
  int idx1, page1, idx2;
};

template <int D_QK, int NW, int KS, bool PAGED, bool BIG>
struct WidePipe {
  static constexpr int BK = 16 * NW;
  using T = WideTile<D_QK, BK>;
  using Pump = GatherPump<D_QK, BIG>;
  // Per-tile lane addresses: fewer spills and faster in the paged 128-head
  // kernels, slower in the others (measured).
  static constexpr bool LFRESH = PAGED && NW == 4 && KS == 1;
  // The gather of block t+1 leaves in the first tile of block t, one row
  // per kEvery MFMAs (16 rows per wave and block), so that the rows have
  // the rest of the block to land.  Paged rows come from HBM, and there every
  // fourth MFMA keeps the copies' issue cost under the two tiles of a wave's
  // block; every second one suits rows that mostly hit in the caches
  // (prefill) and the single tile of the other layouts.  Measured: both beat
  // spreading the copies over the whole block.
  static constexpr int kEvery = PAGED && NW == 4 && KS == 1 ? 4 : 2;
  // One half-iteration: block t lives in `cur` (already gathered); gather
  // block t+1 into `nxt` while computing block t.
  static __device__ __forceinline__ void step(const FwdArgs& a, const LDS_AS uint8_t* cur,
                                              LDS_AS uint8_t* nxt, int t, int nblk, int L,
                                              int bound, int seq, const int32_t* idx_row,
                                              int wave, int koff, uint64_t& mask_cur, Ahead& ah,
                                              const bf16x8 (&qf)[T::kDSteps],
                                              f32x16 (&acc)[kDV / 32], SoftmaxState& st,
                                              int q_row) {
    wait_vm_all();
    __syncthreads();
    const bool have_nxt = t + 1 < nblk;
    // With a key split (64 heads at d_qk = 576), the last step of a row
    // gathers the query slice of row q_row (64 rows of d_qk: one block
    // buffer) into `nxt` instead, head j as row j.  (Wave-uniform;
    // readfirstlane says so to the compiler, which must keep the selected
    // resource in scalar registers.)
    // (BIG tables: the copies address rows by entry, so the query slice
    // is loaded into registers instead, and q_row is -1.)
    const bool q_nxt =
        KS == 2 && !BIG && __builtin_amdgcn_readfirstlane((int)(!have_nxt && q_row >= 0)) != 0;
    BlockMeta mn = block_meta<PAGED>(a, index_ok<BK>(ah.idx1, t + 1, L, bound), ah.idx1, ah.page1);
    if (q_nxt) mn = BlockMeta{~0ull, lane_id(), true};
    u32x4s rsrc = BIG ? big_table_rsrc(a) : q_nxt ? query_rsrc(a, q_row, T::kRowBytes) : table_rsrc(a);
#pragma unroll
    for (int i = 0; i < 4; ++i) rsrc[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
    const int offs = Pump::row_offsets(mn);
    if (have_nxt || q_nxt) stage_rope<D_QK, BK, NW, BIG>(nxt, rsrc, offs, wave);
    const bool ok2 = index_ok<BK>(ah.idx2, t + 2, L, bound);
    const int page2 = page_lookup<PAGED>(a, seq, ok2, ah.idx2);
    const int idx3 = load_index<BK>(idx_row, t + 3, a.topk);
    // Past the last block (without a query slice to gather) the mask is
    // empty: the copies zero-fill `nxt`, which nothing reads any more.
    const int row0 = Pump::kSlots * wave;
    Pump pump{rsrc, nxt, row0, Pump::wave_offsets(offs, row0), lane_id() * 16, 0u, 0u, 0u};
    const uint64_t wmask = KS == 1 ? mask_cur : ((mask_cur >> koff) & 0xffffffffull);
    if (wmask != 0)
      wide_block<D_QK, BK, KS, kEvery, LFRESH>(cur, mask_cur, koff, qf, acc, st, a.scale_log2,
                                               pump);
    pump.template finish<NW == 4 && KS == 1>();
    mask_cur = mn.mask;
    ah = Ahead{ah.idx2, page2, idx3};
  }
};

// Row of a workgroup's turn k, or -1 once it has none left.  The grid is at
// most what the CUs hold at once (one 4-wave or two 2-wave workgroups per
// CU); positions p = 0, 1, ... go to the workgroups in
// snake order (0..G-1, then G-1..0, ...), so each gets an even share of long
// and short rows.  Prefill takes its rows from the last one down (the rows
// of a causal prefill grow with the row number).
// With key-range splits the units are (row, split) pairs, numbered
// row * splits + split.
__device__ __forceinline__ int turn_row(int units, int k, bool paged) {
  const int G = (int)gridDim.x, b = (int)blockIdx.x;
  const long long p = (long long)k * G + ((k & 1) ? G - 1 - b : b);
  if (p >= units) return -1;
  return paged ? (int)p : units - 1 - (int)p;
}

// What a row needs before its first block: the explicit length (or the last
// round of its index list, for the tail scan) and its first three index
// blocks.
template <bool DYNAMIC>
struct RowHead {
  TailRound first;
  int tl;
  int idx0, idx1, idx2;
};

template <bool DYNAMIC, int BK>
__device__ __forceinline__ RowHead<DYNAMIC> load_row_head(const FwdArgs& a, int row) {
  RowHead<DYNAMIC> h;
  const int lane = lane_fresh();
  const int32_t* idx_row = a.indices + (size_t)row * a.topk;
  h.tl = 0;
  if (DYNAMIC)
    h.tl = a.topk_length[row];
  else
    h.first = load_tail_round(idx_row, a.topk, lane);
  h.idx0 = load_index<BK>(idx_row, 0, a.topk, lane);
  h.idx1 = load_index<BK>(idx_row, 1, a.topk, lane);
  h.idx2 = load_index<BK>(idx_row, 2, a.topk, lane);
  return h;
}

// The MFMA B operand of the row's query slice: lane (half, hl) holds
// elements 16d + 8half .. +7 of head `head` in qf[d].
template <int D_QK>
__device__ __forceinline__ void load_query(bf16x8 (&qf)[WideTile<D_QK>::kDSteps], const FwdArgs& a,
                                           int row, int head, int half) {
  const __bf16* qp = a.q + ((size_t)row * a.h_q + head) * D_QK + half * 8;
#pragma unroll
  for (int d = 0; d < WideTile<D_QK>::kDSteps; ++d)
    qf[d] = *reinterpret_cast<const bf16x8*>(qp + d * 16);
}

// The same operand from a block buffer that the gather filled with the
// row's 64 head rows (head j as row j, laid out like a KV block): head group
// hg reads rows 32hg .. 32hg + 31 the way tile_scores reads key rows.
template <int D_QK, int BK = 64>
__device__ __forceinline__ void load_query_lds(bf16x8 (&qf)[WideTile<D_QK>::kDSteps],
                                               const LDS_AS uint8_t* buf, int hg, int lane) {
  using T = WideTile<D_QK, BK>;
  const int hl = lane & 31, half = lane >> 5;
  const int krow = (32 * hg + hl) * T::kNopeBytes, kw = (half ^ nope_swz(hl)) << 4;
  const int rrow = T::kRopeBase + (32 * hg + hl) * T::kRopeBytes, rw = (half ^ rope_swz(hl)) << 4;
#pragma unroll
  for (int d = 0; d < T::kDSteps; ++d)
    qf[d] = *reinterpret_cast<const LDS_AS bf16x8*>(
        d < 32 ? buf + krow + (d >> 3) * 256 + ((32 * (d & 7)) ^ kw)
               : buf + rrow + ((32 * (d - 32)) ^ rw));
}

// Split decode's partial outputs: unit u (row * splits + split) stores the
// fp32 output of head group g (32 heads x 512 values) as the tile at
// split_tile(u, g, h_q / 32): 64 chunks of 1 KiB, chunk 4 ct + j holding
// acc[ct][4 j .. 4 j + 3] of lane L at floats 4 L .. 4 L + 3, i.e. head
// 32 g + L % 32 at columns 32 ct + 8 j + 4 (L / 32) .. + 3 (the MFMA
// accumulator layout).  Each store instruction then writes 1 KiB
// contiguous, straight from the accumulators.
__device__ __forceinline__ size_t split_tile(size_t unit, int g, int groups) {
  return (unit * (size_t)groups + (size_t)g) * (32 * kDV);
}

// SPLIT (paged decode without a key split): a unit is a (row, split) pair
// covering blocks [split * nblk / splits, (split + 1) * nblk / splits) of the
// row; it writes its partial output normalised by its own sum, with its lse
// and max, to the workspace, and split_combine_kernel merges the splits.
// BIG: a KV table above kMaxKvSpan bytes (copies rebased per row).
template <int D_QK, int NW, int KS, bool PAGED, bool DYNAMIC, bool SINK, bool SPLIT = false,
          bool BIG = false>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
sparse_mla_fwd_wide_kernel(FwdArgs a) {
  static_assert(!SPLIT || (PAGED && KS == 1), "split decode: paged, without a key split");
  constexpr int BK = 16 * NW;  // keys per block: 16 rows per wave
  constexpr int G = NW / KS;   // head groups of 32
  using T = WideTile<D_QK, BK>;
  __shared__ __attribute__((aligned(16))) uint8_t buf0_raw[T::kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t buf1_raw[T::kBufBytes];
  LDS_AS uint8_t* buf0 = (LDS_AS uint8_t*)buf0_raw;
  LDS_AS uint8_t* buf1 = (LDS_AS uint8_t*)buf1_raw;

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hg = wave % G, ks = wave / G;  // head group, key split
  const int hl = lane & 31, half = lane >> 5;
  const int koff = ks * (BK / KS);

  const int head = hg * 32 + hl;
  // The per-head sinks sit in LDS for the epilogues: a global load there
  // would be counted behind the next row's query loads and wait for them.
  __shared__ float sink_lds[SINK ? G * 32 : 1];
  if (SINK && (int)threadIdx.x < G * 32) sink_lds[threadIdx.x] = a.attn_sink[threadIdx.x];
  // (The first barrier of the row loop comes before the first epilogue.)

  // The workgroup's rows (persistent grid), each started while the previous
  // row's epilogue runs: its length, first indices and query slice are
  // loaded before that epilogue.
  const int units = SPLIT ? a.rows * a.splits : a.rows;
  int turn = 0;
  int unit = turn_row(units, turn, PAGED);
  bf16x8 qf[T::kDSteps];
  load_query<D_QK>(qf, a, SPLIT ? unit / a.splits : unit, head, half);
  for (;;) {
  const int row = SPLIT ? unit / a.splits : unit;
  const RowHead<DYNAMIC> rh = load_row_head<DYNAMIC, BK>(a, row);
  const int seq = row / a.rows_per_seq;
  const int bound = row_bound(PAGED, a.cache_seqlens, seq, a.s_kv, a.mbps);
  const int32_t* idx_row = a.indices + (size_t)row * a.topk;
  const int L = DYNAMIC ? clamp_length(rh.tl, a.topk) : finish_tail_scan(rh.first, idx_row, a.topk, bound);
  const int nblk_row = (L + BK - 1) / BK;
  // The unit's blocks [t0, nblk): the whole row, or the split's share.
  const int split = SPLIT ? unit % a.splits : 0;
  const int t0 = SPLIT ? (int)((long long)split * nblk_row / a.splits) : 0;
  const int nblk = SPLIT ? (int)((long long)(split + 1) * nblk_row / a.splits) : nblk_row;
  // Kept for a recompute: loading them again there would make the compiler
  // wait for every outstanding load (the query rows included) at the join.
  const int idx0 = SPLIT ? load_index<BK>(idx_row, t0, a.topk) : rh.idx0;
  const int idx1 = SPLIT ? load_index<BK>(idx_row, t0 + 1, a.topk) : rh.idx1;
  const int idx2 = SPLIT ? load_index<BK>(idx_row, t0 + 2, a.topk) : rh.idx2;
  const int next_unit = turn_row(units, ++turn, PAGED);
  const int next = next_unit < 0 ? -1 : SPLIT ? next_unit / a.splits : next_unit;
  // With a key split, the next row's query slice fits one block buffer, and
  // the last block step gathers it there (contiguous 1 KiB rows; loaded
  // straight into the MFMA operand layout, each load would touch 32 head
  // rows).
  const int q_row = KS == 2 && !BIG && nblk > t0 ? next : -1;

  f32x16 acc[kDV / 32];
  SoftmaxState st;
  float m_preset = -INFINITY;
  for (int attempt = 0; attempt < 2; ++attempt) {
#pragma unroll
    for (int ct = 0; ct < kDV / 32; ++ct) acc[ct] = f32x16{};
    st = SoftmaxState{m_preset, 0.f, -INFINITY, false};
    if (nblk > t0) {
      const bool ok0 = index_ok<BK>(idx0, t0, L, bound);
      const bool ok1 = index_ok<BK>(idx1, t0 + 1, L, bound);
      const int pg0 = page_lookup<PAGED>(a, seq, ok0, idx0);
      const int pg1 = page_lookup<PAGED>(a, seq, ok1, idx1);
      const BlockMeta m0 = block_meta<PAGED>(a, ok0, idx0, pg0);
      uint64_t mask_cur = m0.mask;
      Ahead ah{idx1, pg1, idx2};
      __syncthreads();  // a previous attempt or row may still read the buffers
      {
        using Pump = GatherPump<D_QK, BIG>;
        const u32x4s rsrc = BIG ? big_table_rsrc(a) : table_rsrc(a);
        const int offs = Pump::row_offsets(m0);
        const int row0 = Pump::kSlots * wave;
        stage_rope<D_QK, BK, NW, BIG>(buf0, rsrc, offs, wave);
        Pump{rsrc, buf0, row0, Pump::wave_offsets(offs, row0), lane_id() * 16, 0u, 0u, 0u}
            .copy_all();
      }
      using P = WidePipe<D_QK, NW, KS, PAGED, BIG>;
      for (int t = t0; t < nblk; t += 2) {
        P::step(a, buf0, buf1, t, nblk, L, bound, seq, idx_row, wave, koff, mask_cur, ah, qf, acc,
                st, q_row);
        if (t + 1 < nblk)
          P::step(a, buf1, buf0, t + 1, nblk, L, bound, seq, idx_row, wave, koff, mask_cur, ah, qf,
                  acc, st, q_row);
      }
      // The last step's zero-fill copies may still be landing in a buffer
      // that the next attempt or the epilogue writes.
      wait_vm_all();
    }
    // Workgroup-uniform: recompute once if any head outgrew its reference.
    if (!__syncthreads_or(st.overflow) || attempt == 1) break;
    m_preset = st.m_max;
  }

  // Lane values for the rest of the row (see lane_fresh), then the next
  // row's query slice: from the last block's buffer (read before the
  // epilogue reuses the buffers: the barrier there follows the reads), or
  // loaded now to land under this row's epilogue.
  const int lane = lane_fresh(), hl = lane & 31, half = lane >> 5, head = hg * 32 + hl;
  const float sink = SINK ? sink_lds[head] : 0.f;
  if (q_row >= 0)
    load_query_lds<D_QK>(qf, (nblk - 1 - t0) & 1 ? buf0 : buf1, hg, lane);
  else if (next >= 0)
    load_query<D_QK>(qf, a, next, head, half);

  // Combine, normalise, store.  acc[ct][i] = O[head][c = 32ct + 8(i/4) + 4half + i%4].
  float m_fin = st.m_ref, l_fin = st.l_sum, mx_fin = st.m_max, a_self = 1.f;
  LDS_AS float* part = (LDS_AS float*)(hg == 0 ? buf0 : buf1);
  if (KS == 2) {
    __shared__ float stats_raw[2 * 2 * 32 * 3];
    LDS_AS float* sx = (LDS_AS float*)stats_raw + hg * (2 * 32 * 3);
    __syncthreads();  // every wave is done with the block buffers
    if (half == 0) {
      sx[(ks * 32 + hl) * 3 + 0] = st.m_ref;
      sx[(ks * 32 + hl) * 3 + 1] = st.l_sum;
      sx[(ks * 32 + hl) * 3 + 2] = st.m_max;
    }
    __syncthreads();
    const int other = (1 - ks) * 32 + hl;
    const float mo = sx[other * 3 + 0], lo = sx[other * 3 + 1], xo = sx[other * 3 + 2];
    const float m = fmaxf(st.m_ref, mo);
    float a_other = 0.f;
    a_self = 0.f;
    if (m != -INFINITY) {
      a_self = __builtin_amdgcn_exp2f(st.m_ref - m);
      a_other = __builtin_amdgcn_exp2f(mo - m);
    }
    l_fin = a_self * st.l_sum + a_other * lo;
    m_fin = m;
    mx_fin = fmaxf(st.m_max, xo);
  }
  float scale = 0.f, lse_v = INFINITY, ml_v = -INFINITY;
  if (l_fin > 0.f) {
    float denom = l_fin;
    if (SINK) denom += __builtin_amdgcn_exp2f(sink * kLog2e - m_fin);
    scale = a_self / denom;
    ml_v = mx_fin * kLn2;
    lse_v = (m_fin + __log2f(l_fin)) * kLn2;
  }
  if constexpr (SPLIT) {
    // The split's output normalised by its own sum (the sink joins once, in
    // the merge), 16 B per lane and value group straight from the
    // accumulator layout; an empty split has lse = -inf (no contribution).
    const size_t u = (size_t)unit * a.h_q + head;
    const float inv = l_fin > 0.f ? 1.f / l_fin : 0.f;
    float* o = a.ws_o + split_tile(unit, hg, a.h_q / 32) + 4 * lane;
#pragma unroll
    for (int ct = 0; ct < kDV / 32; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        // non-temporal: the merge kernel reads the partials once
        __builtin_nontemporal_store(
            f32x4{acc[ct][4 * j] * inv, acc[ct][4 * j + 1] * inv, acc[ct][4 * j + 2] * inv,
                  acc[ct][4 * j + 3] * inv},
            reinterpret_cast<f32x4*>(o + (4 * ct + j) * 256));
    if (half == 0) {
      a.ws_stats[2 * u] = l_fin > 0.f ? lse_v : -INFINITY;
      a.ws_stats[2 * u + 1] = ml_v;
    }
  } else {
  if (half == 0 && (KS == 1 || ks == 0)) {
    a.lse[(size_t)row * a.h_q + head] = lse_v;
    if (a.max_logits) a.max_logits[(size_t)row * a.h_q + head] = ml_v;
  }
  if (KS == 2) {
    // Each wave of a head group finishes one half of the value columns
    // (wave ks: columns 256ks .. 256ks + 255, i.e. ct in [8ks, 8ks + 8)).  It
    // hands its scaled partial of the other half to the partner through the
    // partner's 32 KiB region of the group's block buffer, adds the partner's
    // partial of its own half, stages the bf16 result in its own region (only
    // this wave reads it) and stores 512 B half rows.
    // The half is a compile-time constant in each branch (acc is indexed
    // with it and must stay in registers).
    auto finish_half = [&](auto ks_c) {
    constexpr int K = decltype(ks_c)::value;
    constexpr int kHalf = kDV / 64;  // value tiles per half
    LDS_AS float* mine = part + K * (32 * kDV / 2);
    LDS_AS float* theirs = part + (1 - K) * (32 * kDV / 2);
#pragma unroll
    for (int c = 0; c < kHalf; ++c) {
      const int ct = (1 - K) * kHalf + c;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<LDS_AS f32x4*>(theirs + ((c * 4 + j) * 64 + lane) * 4) =
            f32x4{acc[ct][4 * j] * scale, acc[ct][4 * j + 1] * scale, acc[ct][4 * j + 2] * scale,
                  acc[ct][4 * j + 3] * scale};
    }
    __syncthreads();
    // Rounded to bf16 as they are combined (the next row's query slice may
    // be in flight into half of the registers).
    bf16x4 o[kHalf][4];
#pragma unroll
    for (int c = 0; c < kHalf; ++c) {
      const int ct = K * kHalf + c;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 v = f32x4{acc[ct][4 * j] * scale, acc[ct][4 * j + 1] * scale,
                              acc[ct][4 * j + 2] * scale, acc[ct][4 * j + 3] * scale} +
                        *reinterpret_cast<const LDS_AS f32x4*>(mine + ((c * 4 + j) * 64 + lane) * 4);
        o[c][j] = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
      }
      __builtin_amdgcn_sched_barrier(0);  // one value tile of partials in flight at a time
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // partials read before the tile overwrites them
    // Half row h (512 B) at h * 512; its chunk c (16 B) sits at chunk c ^ h.
    LDS_AS uint8_t* tile = (LDS_AS uint8_t*)mine;
#pragma unroll
    for (int c = 0; c < kHalf; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<LDS_AS bf16x4*>(tile + hl * kDV + (((4 * c + j) ^ hl) << 4) + 8 * half) =
            o[c][j];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the tile is complete for every lane
    const int hsub = lane >> 5, chunk = lane & 31;
    uint8_t* obase = reinterpret_cast<uint8_t*>(a.out + ((size_t)row * a.h_q + hg * 32) * kDV) +
                     K * kDV + chunk * 16;
#pragma unroll 4
    for (int k = 0; k < 16; ++k) {
      const int h = 2 * k + hsub;
      const u32x4 v = *reinterpret_cast<const LDS_AS u32x4*>(tile + h * kDV + ((chunk ^ h) << 4));
      *reinterpret_cast<u32x4*>(obase + (size_t)h * (kDV * 2)) = v;
    }
    };
    if (ks == 0)
      finish_half(std::integral_constant<int, 0>{});
    else
      finish_half(std::integral_constant<int, 1>{});
  } else {
    // The output goes through LDS so that every global store writes one
    // head's whole 1 KiB row: stored straight from the accumulator layout, a
    // store instruction would touch 32 rows with 16 bytes each.  The wave's
    // bf16 tile takes 32 KiB of a block buffer that no wave reads any more
    // (two tiles per buffer of a 64-key block, one per buffer of a 32-key
    // block).  Chunk c (16 B) of head row h sits at chunk c ^ h of the row.
    constexpr int kTileBytes = 32 * kDV * 2, kPer = T::kBufBytes / kTileBytes;
    LDS_AS uint8_t* tile = (wave / kPer == 0 ? buf0 : buf1) + (wave % kPer) * kTileBytes;
#pragma unroll
    for (int ct = 0; ct < kDV / 32; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x4 o4 = {(__bf16)(acc[ct][4 * j] * scale), (__bf16)(acc[ct][4 * j + 1] * scale),
                           (__bf16)(acc[ct][4 * j + 2] * scale), (__bf16)(acc[ct][4 * j + 3] * scale)};
        *reinterpret_cast<LDS_AS bf16x4*>(tile + hl * (kDV * 2) + (((4 * ct + j) ^ hl) << 4) + 8 * half) = o4;
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the tile is complete for every lane
    uint8_t* orow = reinterpret_cast<uint8_t*>(a.out + ((size_t)row * a.h_q + hg * 32) * kDV) + lane * 16;
#pragma unroll 4
    for (int h = 0; h < 32; ++h) {
      const u32x4 v = *reinterpret_cast<const LDS_AS u32x4*>(tile + h * (kDV * 2) + ((lane ^ h) << 4));
      *reinterpret_cast<u32x4*>(orow + (size_t)h * (kDV * 2)) = v;
    }
  }
  }
  if (next_unit < 0) break;
  unit = next_unit;
  }
}

// ---------------------------------------------------------------------------
// Ring kernel: 128 heads (4 waves of 32), rows of at most kRingMaxTopk index
// positions.  A persistent grid as the wide kernel's, one workgroup per CU.
//
// Row prologue:
//   * the row's query slice (128 head rows of d_qk) is copied global -> LDS
//     into the ring's buffers (head j as row j) while the index vector is
//     read; each wave then reads its 32 heads in the MFMA operand layout;
//   * the row's keys are compacted: every index position below the length
//     (explicit topk_length, else the whole vector) is tested for validity
//     (and paged through the block table), and the table offsets of the valid
//     keys are written, in position order, to a list in LDS.  Masked keys add
//     exactly nothing to the softmax, so dropping them is exact; the derived
//     length of the pages' tail scan needs no scan here, since the positions
//     past it are invalid anyway.
// Stage loop: the compacted keys stream through a ring of kRingStages LDS
// stages of 32 keys (one 32 x 32 MFMA tile per wave).  While stage t is
// computed, stages t+1 .. t+kRingStages-1 are in flight: about 110 KB per CU
// at d_qk = 576.  For a random-row gather the bytes in flight per CU, not the
// bytes moved, set the rate the memory system attains (measured on MI355X
// with the decode rows of 1152 B: about 2.8 TB/s with 37 KB in flight per CU,
// 4.0 TB/s with 74 KB, 5.4 TB/s with 147 KB), and a double buffer keeps at
// most one block in flight.  No other vector-memory access runs inside the
// loop and every step issues exactly kGather copies per wave, so the wait for
// stage t is vmcnt((kRingStages - 2) * kGather): the copies of the stages
// issued after it may stay in flight.  Copies for stages past the end of the
// list read nothing and zero-fill their buffer.
// ---------------------------------------------------------------------------

constexpr int kRingStages = 4;       // LDS stages of the gather ring
constexpr int kRingKeys = 32;        // keys per stage: one tile per wave
constexpr int kRingMaxTopk = 2048;   // index positions per row (the key list lives in LDS)

// The row prologue's division of the waves.  Unsplit (every wave copies a
// quarter of the query slice, then reads a quarter of the positions), a wave
// waits for its index and block-table loads behind its query copies: the
// memory counter completes in issue order.  Split (paged decode rows), two
// waves copy the query slice while the other two read the index vector and
// the block table and compact the keys, so the two latencies overlap.
template <bool WAVE_SPLIT>
struct RingPrologue {
  static constexpr bool kSplit = WAVE_SPLIT;
  static constexpr int kQWaves = WAVE_SPLIT ? 2 : kWideWaves;     // query-copy waves
  static constexpr int kListWaves = WAVE_SPLIT ? 2 : kWideWaves;  // the last kListWaves waves
  static constexpr int kChunks = kRingMaxTopk / (kListWaves * 64);  // 64-position chunks per wave
};

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding: vmcnt
// bits 3:0 and 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15: no wait on those).
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// A barrier that waits for LDS accesses but not for vector-memory loads
// (__syncthreads() would also wait for every copy in flight).
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The copies of one stage's nope rows (the first 1 KiB of each row), 8 rows
// per wave: wave w copies rows 8w .. 8w + 7 of the 32-row stage, with M0 on
// the four-row windows 8w and 8w + 4 and the row selected by the instruction
// offset, as GatherPump does for 16 rows.  The rows' chunk swizzle depends on
// the row's low four bits, 8(w % 2) + s: `lane16w` holds 16 * lane with the
// wave's half of the pattern XORed in, the slot's half is a constant.  BIG
// tables: `offw` holds entries and `rsrc` is big_table_rsrc (see copy_row).
template <int D_QK, bool BIG = false>
struct RingPump {
  using T = WideTile<D_QK, kRingKeys>;
  static constexpr int kSlots = kRingKeys / kWideWaves;  // rows per wave and stage
  static_assert(T::kNopeBytes == 1024, "copy_row copies 1 KiB rows");
  u32x4s rsrc;       // table resource (wave-uniform)
  LDS_AS uint8_t* buf;
  int row0;          // 8 * wave
  int offw;          // lane s < 8: source offset of row row0 + s, moved down by (s % 4) KiB, or kOob
  int lane16w;
  uint32_t win;
  uint32_t so_next;

  __device__ __forceinline__ void copy(int s, bool fresh = false, bool first = true) {
    const bool opens = fresh || (s & 3) == 0;
    if (opens) win = (uint32_t)(uintptr_t)(buf + (row0 + (s & ~3)) * T::kNopeBytes);
    const uint32_t so = first ? (uint32_t)__builtin_amdgcn_readlane(offw, s) : so_next;
    if (s + 1 < kSlots) so_next = (uint32_t)__builtin_amdgcn_readlane(offw, s + 1);
    copy_slot<BIG>(s, opens, rsrc, so, (uint32_t)lane16w ^ (uint32_t)(nope_swz(s) << 4), win);
  }
  __device__ __forceinline__ void copy_all() {
#pragma unroll
    for (int s = 0; s < kSlots; ++s) copy(s, false, s == 0);
  }
};

// The rope part (d_qk = 576) of a 32-key stage, one copy per wave: lane L
// copies chunk L % 8 of row jj = 8 wave + L / 8 (LDS chunk L % 8 holds source
// chunk (L % 8) ^ swizzle(jj)).  `o` is row jj's offset as ring_lane_offset
// gives it for this lane (moved down by (L % 4) KiB; kOob for no row; BIG:
// the row's entry, or kBigNone).
template <int D_QK, bool BIG = false>
__device__ __forceinline__ void ring_rope(LDS_AS uint8_t* buf, const u32x4s& rsrc, int o, int wave,
                                          int lane) {
  using T = WideTile<D_QK, kRingKeys>;
  if (T::kRopeLanes == 0) return;
  const int jj = 8 * wave + (lane >> 3);
  const uint32_t col = T::kNopeBytes + (uint32_t)(((lane & 7) ^ rope_swz(jj)) << 4);
  LDS_AS uint8_t* dst = buf + T::kRopeBase + wave * 8 * T::kRopeBytes;
  if constexpr (BIG)
    big_rope_copy(rsrc, (uint32_t)o, col, dst);
  else
    dma_table16<0>(rsrc, (uint32_t)o + (uint32_t)(lane & 3) * T::kNopeBytes + col,
                   (uint32_t)(uintptr_t)dst);
}

// The list entries one wave needs for the copies of one stage, read ahead
// of their use: lane L holds the entry of row 8 wave + L / 8 (its rope copy)
// and of row 8 wave + L % 8 (its RingPump).  The reads are volatile and
// unconditional (of a clamped entry): the compiler would otherwise sink them
// into a branch on the position and wait for them right away.  The offsets
// themselves are formed where they are used (`rope`, `pump`: moved down by
// (L % 4) KiB, or kOob past the end of the list of n keys; BIG: the entry,
// or kBigNone).
struct RingOffs {
  uint32_t rope_raw, pump_raw;
  int stage;

  static __device__ __forceinline__ uint32_t entry(const LDS_AS uint32_t* keys, int p) {
    return *reinterpret_cast<const volatile LDS_AS uint32_t*>(
        keys + (p < kRingMaxTopk ? p : kRingMaxTopk - 1));
  }
  static __device__ __forceinline__ RingOffs read(const LDS_AS uint32_t* keys, int stage, int wave,
                                                  int lane) {
    const int p0 = stage * kRingKeys + 8 * wave;
    return RingOffs{entry(keys, p0 + (lane >> 3)), entry(keys, p0 + (lane & 7)), stage};
  }
  template <bool BIG>
  __device__ __forceinline__ int rope(int n, int wave, int lane) const {
    const int p = stage * kRingKeys + 8 * wave + (lane >> 3);
    if constexpr (BIG) return p < n ? (int)rope_raw : (int)kBigNone;
    return p < n ? (int)(rope_raw - (uint32_t)(lane & 3) * 1024u) : (int)kOob;
  }
  template <bool BIG>
  __device__ __forceinline__ int pump(int n, int wave, int lane) const {
    const int p = stage * kRingKeys + 8 * wave + (lane & 7);
    if constexpr (BIG) return p < n ? (int)pump_raw : (int)kBigNone;
    return p < n ? (int)(pump_raw - (uint32_t)(lane & 3) * 1024u) : (int)kOob;
  }
};

// All copies of one stage (rope part, then the nope rows) from `rsrc` into
// buffer `buf`, outside the MFMA stream.
template <int D_QK, bool BIG>
__device__ __forceinline__ void ring_copy_stage(LDS_AS uint8_t* buf, const u32x4s& rsrc,
                                                const LDS_AS uint32_t* keys, int n, int stage,
                                                int wave, int lane) {
  const RingOffs o = RingOffs::read(keys, stage, wave, lane);
  ring_rope<D_QK, BIG>(buf, rsrc, o.template rope<BIG>(n, wave, lane), wave, lane);
  RingPump<D_QK, BIG>{rsrc, buf, 8 * wave, o.template pump<BIG>(n, wave, lane),
                      (lane * 16) ^ ((wave & 1) << 5), 0u, 0u}
      .copy_all();
}

// S^T = K Q^T of a ring stage (32 keys at row 0 of `buf`), as tile_scores
// with r0 = 0 but with the accumulator in VGPRs (mfma_vacc); the pump's nope
// copies go after every fourth MFMA.
template <int D_QK, int KP, bool LFRESH, class Pump, class Hook>
__device__ __forceinline__ f32x16 ring_scores(const LDS_AS uint8_t* buf,
                                              const bf16x8 (&qf)[WideTile<D_QK>::kDSteps],
                                              Pump& pump, Hook&& hook) {
  using T = WideTile<D_QK, kRingKeys>;
  constexpr int kSteps = T::kDSteps;
  constexpr int kSlots = Pump::kSlots;
  const int lane = LFRESH ? lane_fresh() : lane_id();
  const int hl = lane & 31, half = lane >> 5;
  int krow = hl * T::kNopeBytes, kw = (half ^ nope_swz(hl)) << 4;
  int rrow = T::kRopeBase + hl * T::kRopeBytes, rw = (half ^ rope_swz(hl)) << 4;
  opaque(krow);
  opaque(kw);
  opaque(rrow);
  opaque(rw);
  auto kaddr = [&](int d) {
    if (d < 32) return buf + krow + (d >> 3) * 256 + ((32 * (d & 7)) ^ kw);
    return buf + rrow + ((32 * (d - 32)) ^ rw);
  };
  f32x16 s;
  bf16x8 kring[KP];
#pragma unroll
  for (int n = 0; n < KP; ++n) kring[n] = *reinterpret_cast<const LDS_AS bf16x8*>(kaddr(n));
#pragma unroll
  for (int d = 0; d < kSteps; ++d) {
    const bf16x8 kf = kring[d % KP];
    if (d + KP < kSteps)
      kring[d % KP] = *reinterpret_cast<const LDS_AS bf16x8*>(kaddr(d + KP));
    if (d == 0)
      mfma_vacc_first(s, kf, qf[d]);
    else if (d == kSteps - 1)
      mfma_vacc_last(s, kf, qf[d]);
    else
      mfma_vacc(s, kf, qf[d]);
    if (d % 4 == 3 && d / 4 < kSlots) pump.copy(d / 4, false, d == 3);
    hook(d);
    __builtin_amdgcn_sched_barrier(0);  // keep the read-ahead distance
  }
  return s;
}

// The V^T operand stream of P*V over a 32-key stage (row 0 of `vbuf`), as in
// tile_softmax_pv: value tile ct = n % 16 and key step u = n / 16 for MFMA n.
// Lane (16-group g, i16) reads 8 B of key row 16u + 4 half + TR_ROW(i16)
// (+8 for the upper four keys) at value chunk 4 ct + 2 (g & 1) + TR_COL(i16) / 2
// with ds_read_b64_tr_b16.  The first kPrefetch operands can be read ahead
// (inside the S^T chain), so that the first P*V MFMA does not wait on LDS.
template <int D_QK>
struct RingV {
  using T = WideTile<D_QK, kRingKeys>;
  static constexpr int kPrefetch = 3;
  static constexpr int kTiles = kDV / 32;
  const LDS_AS uint8_t* vbuf;
  int row_lo, row_hi, w_lo, w_hi;
  bf16x4 lo[kPrefetch], hi[kPrefetch];

  __device__ __forceinline__ void init(const LDS_AS uint8_t* vb, int lane) {
    vbuf = vb;
    const int i16 = lane & 15, cb = (lane >> 4) & 1, half = lane >> 5;
    const int vrow = 4 * half + TR_ROW(i16);
    const int vc = 2 * cb + (TR_COL(i16) >> 1);
    row_lo = vrow * T::kNopeBytes + 8 * (TR_COL(i16) & 1);
    row_hi = row_lo + 8 * T::kNopeBytes;
    w_lo = (vc ^ nope_swz(vrow)) << 4;
    w_hi = (vc ^ nope_swz(vrow + 8)) << 4;
    opaque(row_lo);
    opaque(row_hi);
    opaque(w_lo);
    opaque(w_hi);
  }
  __device__ __forceinline__ const LDS_AS uint8_t* addr(int n, bool upper) const {
    const int ct = n % kTiles, u = n / kTiles;
    return vbuf + (upper ? row_hi : row_lo) + (ct >> 2) * 256 + 16 * u * T::kNopeBytes +
           ((64 * (ct & 3)) ^ (upper ? w_hi : w_lo));
  }
  __device__ __forceinline__ void read(int n) {
    lo[n % kPrefetch] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)addr(n, false));
    hi[n % kPrefetch] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)addr(n, true));
  }
  __device__ __forceinline__ void prefetch() {
#pragma unroll
    for (int n = 0; n < kPrefetch; ++n) read(n);
  }
};

// O^T += V^T P^T over the 32 keys of the previous stage (buffer `vbuf`, its
// probabilities `pprev`), with the softmax of the current stage's scores `s`
// scheduled between those MFMAs: its masked max, its probabilities (into
// `pnext`, the P^T operands of the next call) and their sum.  The softmax
// reference is fixed, so O is never rescaled and the two are independent.
// DO_PV / DO_SM leave out one half (the first and the last stage of a row);
// MASK = false skips the masking of a stage whose 32 keys are all used.
// Operand layouts as in tile_softmax_pv (r0 = 0): value tile ct = n % 16 and
// key step u = n / 16 for MFMA n; pnext[u][e] = P of s[8u + e].
template <int D_QK, bool DO_PV, bool DO_SM, bool MASK = true>
__device__ __forceinline__ void ring_pv_softmax(RingV<D_QK>& v, const bf16x8 (&pprev)[2],
                                                f32x16 (&acc)[kDV / 32], f32x16 s,
                                                uint32_t bits, SoftmaxState& st,
                                                float scale_log2, bf16x8 (&pnext)[2]) {
  constexpr int kPrefetch = RingV<D_QK>::kPrefetch;
  constexpr int kTiles = kDV / 32;
  const int half = lane_id() >> 5;
  float rmax = -INFINITY, neg_ref = 0.f, rsum = 0.f;
  // Softmax work placed after MFMA n: 0 mask, 1 local max, 2 lane-pair max and
  // reference, 3..10 two probabilities each, 11 the sum.
  auto sm_piece = [&](int n) {
    if (n == 0) {
      if (MASK) {
        const uint32_t mlane = bits >> (4 * half);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[i] = ((mlane >> (8 * (i >> 2) + (i & 3))) & 1u) ? s[i] : -INFINITY;
      }
    } else if (n == 1) {
      const float m0 = max3_raw(s[0], s[1], s[2]), m1 = max3_raw(s[3], s[4], s[5]);
      const float m2 = max3_raw(s[6], s[7], s[8]), m3 = max3_raw(s[9], s[10], s[11]);
      const float m4 = max3_raw(s[12], s[13], s[14]);
      rmax = max3_raw(max3_raw(m0, m1, m2), max3_raw(m3, m4, s[15]), -INFINITY);
    } else if (n == 2) {
      const uint2 r = pair32(rmax);
      // -inf only for a stage without a key
      rmax = max_raw(__builtin_bit_cast(float, r.x), __builtin_bit_cast(float, r.y)) * scale_log2;
      st.m_max = max_raw(st.m_max, rmax);
      if (st.m_ref == -INFINITY) st.m_ref = rmax;
      st.overflow |= rmax > st.m_ref + kRefSlack;  // this attempt is then discarded
      neg_ref = st.m_ref == -INFINITY ? 0.f : -st.m_ref;
    } else if (n >= 3 && n < 11) {
      const int e = 2 * (n - 3);
      const float p0 = prob(s[e], neg_ref, scale_log2), p1 = prob(s[e + 1], neg_ref, scale_log2);
      pnext[e >> 3][e & 7] = (__bf16)p0;
      pnext[e >> 3][(e & 7) + 1] = (__bf16)p1;
      rsum = n == 3 ? p0 + p1 : rsum + (p0 + p1);
    } else if (n == 11) {
      st.l_sum += pair_sum32(rsum);
    }
  };
#pragma unroll
  for (int n = 0; n < 2 * kTiles; ++n) {
    if (DO_PV) {
      const bf16x4 l = v.lo[n % kPrefetch], h = v.hi[n % kPrefetch];
      if (n + kPrefetch < 2 * kTiles) v.read(n + kPrefetch);
      const bf16x8 vf = {l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
      acc[n % kTiles] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pprev[n / kTiles], acc[n % kTiles], 0, 0, 0);
    }
    if (DO_SM) sm_piece(n);
    if (DO_PV) __builtin_amdgcn_sched_barrier(0);
  }
}

// SPLIT (split decode): a unit is a (row, split) pair that takes the row's
// index blocks [split * n / S, (split + 1) * n / S) of 64 positions, n =
// ceil(L / 64) for the row length L (S splits; at most kRingMaxTopk
// positions per unit), the partition the wide kernel's split units use, so
// that derived and explicit lengths give the same units; it writes its
// output normalised by its own sum, with its lse and max, to the workspace;
// split_combine_kernel merges the splits.
template <int D_QK, bool PAGED, bool DYNAMIC, bool SINK, bool BIG, bool SPLIT = false>
__global__ void __launch_bounds__(kWideWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
sparse_mla_fwd_ring_kernel(FwdArgs a) {
  constexpr int NW = kWideWaves, BK = kRingKeys, NS = kRingStages;
  using T = WideTile<D_QK, BK>;
  constexpr int kRopeCopies = T::kRopeBytes ? BK / 8 / NW : 0;
  static_assert(T::kRopeBytes == 0 || BK / 8 == NW, "one rope copy per wave and stage");
  constexpr int kGather = RingPump<D_QK>::kSlots + kRopeCopies;  // copies per wave and stage
  // Stages resident: the one whose S^T is computed and the one whose P*V
  // is; kAhead = NS - 2 stages are in flight.
  constexpr int kAhead = NS - 2;
  constexpr int kKRead = D_QK == 576 ? 4 : 5;  // K fragments read ahead
  constexpr int kHeads = NW * 32;
  static_assert(kHeads * T::kRowBytes <= NS * T::kBufBytes, "the query slice fits the ring");
  // LFRESH: per-tile lane addresses (what the paged 128-head wide kernel prefers).
  constexpr bool LFRESH = false;
  __shared__ __attribute__((aligned(16))) uint8_t ring_raw[NS * T::kBufBytes];
  __shared__ __attribute__((aligned(16))) uint32_t keys_raw[kRingMaxTopk];
  __shared__ int counts_raw[NW];
  __shared__ float sink_lds[SINK ? kHeads : 1];
  __shared__ uint32_t rsrc_raw[4];
  LDS_AS uint8_t* ring = (LDS_AS uint8_t*)ring_raw;
  LDS_AS uint32_t* keys = (LDS_AS uint32_t*)keys_raw;
  LDS_AS int* counts = (LDS_AS int*)counts_raw;
  using PRO = RingPrologue<PAGED && !SPLIT>;

  const int wave_k = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (SINK && (int)threadIdx.x < kHeads) sink_lds[threadIdx.x] = a.attn_sink[threadIdx.x];
  // The table's resource, read from LDS where a row needs it: kept in
  // registers across the stage loop it is spilled, and each reload waits for
  // every copy in flight.
  if (threadIdx.x == 0) {
    const u32x4s r = BIG ? big_table_rsrc(a) : table_rsrc(a);
#pragma unroll
    for (int i = 0; i < 4; ++i) ((LDS_AS uint32_t*)rsrc_raw)[i] = r[i];
  }

  bf16x8 qf[T::kDSteps];
  int turn = 0;
  const int units = SPLIT ? a.rows * a.splits : a.rows;
  for (int unit = turn_row(units, turn, PAGED); unit >= 0; unit = turn_row(units, ++turn, PAGED)) {
    const int row = SPLIT ? unit / a.splits : unit;
    const int lane = lane_fresh();
    const int wave = fresh_s(wave_k);
    const int seq = row / a.rows_per_seq;
    // The previous row's epilogue has read the ring (and the sinks are staged).
    __syncthreads();
    const int lw = wave - (NW - PRO::kListWaves);  // list wave, or < 0
    if (!PRO::kSplit || wave < PRO::kQWaves) {
      // Query slice into the ring: head h is row h % 32 of stage buffer
      // h / 32, in row groups of 8 per stage; wave w copies groups w + j
      // kQWaves.
      const u32x4s rsrc = query_rsrc(a, row, T::kRowBytes);
      const int heads = lane & 31;  // lane j: head 32 st + j, offset moved down by (j % 4) KiB
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        LDS_AS uint8_t* buf = ring + st * T::kBufBytes;
        const int o = (int)((uint32_t)(st * 32 + heads) * (uint32_t)T::kRowBytes + kSpanBias -
                            (uint32_t)(lane & 3) * 1024u);
#pragma unroll
        for (int j = 0; j < NW / PRO::kQWaves; ++j) {
          const int g = PRO::kSplit ? wave + j * PRO::kQWaves : wave;
          stage_rope<D_QK, BK, NW>(buf, rsrc, o, g);
          RingPump<D_QK>{rsrc, buf, 8 * g, __shfl(o, 8 * g + (lane & 7)),
                         (lane * 16) ^ ((g & 1) << 5), 0u, 0u}
              .copy_all();
        }
      }
    }
    constexpr int KC = PRO::kChunks;
    uint64_t mk[KC];
    uint32_t offv[KC];
    if (!PRO::kSplit || lw >= 0) {
      const int bound = row_bound(PAGED, a.cache_seqlens, seq, a.s_kv, a.mbps);
      const int32_t* idx_row = a.indices + (size_t)row * a.topk;
      // Positions examined: below the explicit length, else the whole vector
      // (a split unit: its blocks' positions [lo, scan) below the row length).
      int lo = 0, scan = DYNAMIC ? clamp_length(a.topk_length[row], a.topk) : a.topk;
      if constexpr (SPLIT) {
        const int L = DYNAMIC ? scan
                              : finish_tail_scan(load_tail_round(idx_row, a.topk, lane), idx_row,
                                                 a.topk, bound);
        const int nblk = (L + 63) / 64, split = unit % a.splits;
        lo = (int)((long long)split * nblk / a.splits) * 64;
        const int hi = (int)((long long)(split + 1) * nblk / a.splits) * 64;
        scan = hi < L ? hi : L;
        scan = scan > lo ? scan : lo;
      }
      // Compaction: list wave v examines positions [lo + v per, lo + (v + 1) per).
      const int per = ((scan - lo + 64 * PRO::kListWaves - 1) / (64 * PRO::kListWaves)) * 64;
      const int p0 = lo + lw * per;
      int idxv[KC];
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const int pos = p0 + 64 * k + lane;
        idxv[k] = 64 * k < per && pos < scan ? idx_row[pos] : -1;
      }
      int pgv[KC];
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const bool ok = idxv[k] >= 0 && idxv[k] < bound;
        pgv[k] = page_lookup<PAGED>(a, seq, ok, idxv[k]);
      }
      int cnt = 0;
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const bool ok = idxv[k] >= 0 && idxv[k] < bound;
        const BlockMeta m = block_meta<PAGED>(a, ok, idxv[k], pgv[k]);
        mk[k] = m.mask;
        offv[k] = BIG ? (uint32_t)m.phys * (uint32_t)(T::kRowBytes / kBigUnit)
                      : (uint32_t)m.phys * (uint32_t)T::kRowBytes + kSpanBias;
        cnt += __builtin_popcountll(m.mask);
      }
      if constexpr (PRO::kListWaves == 2) {
        // The valid keys' table offsets in position order, written before
        // the barrier (held across it, they would be spilled): list wave 0
        // from the start of the list, list wave 1 (whose start depends on
        // wave 0's count) against the end of the list area, moved below.
        int base = lw == 0 ? 0 : kRingMaxTopk - cnt;
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          const uint64_t m = mk[k];
          const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          if ((m >> lane) & 1ull) keys[base + below] = offv[k];
          base += __builtin_popcountll(m);
        }
      }
      if (lane == 0) counts[lw] = cnt;
    }
    wait_vm_all();  // this wave's query copies have landed
    __syncthreads();
    int n = 0, base = 0;
#pragma unroll
    for (int w = 0; w < PRO::kListWaves; ++w) {
      const int c = counts[w];
      base += w < lw ? c : 0;
      n += c;
    }
    if constexpr (PRO::kListWaves == 2) {
      if (lw == 1) {
        // All reads before any write: the two ranges may overlap.
        const int c1 = n - base;
        uint32_t e[KC];
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          const int i = 64 * k + lane;
          e[k] = i < c1 ? keys[kRingMaxTopk - c1 + i] : 0u;
        }
#pragma unroll
        for (int k = 0; k < KC; ++k) {
          const int i = 64 * k + lane;
          if (i < c1) keys[base + i] = e[k];
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const uint64_t m = mk[k];
        const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if ((m >> lane) & 1ull) keys[base + below] = offv[k];
        base += __builtin_popcountll(m);
      }
    }
    __syncthreads();  // the key list and every wave's query rows are in LDS
    load_query_lds<D_QK, BK>(qf, ring + wave * T::kBufBytes, 0, lane);
    const int nst = (n + BK - 1) / BK;

    f32x16 acc[kDV / 32];
    SoftmaxState st;
    float m_preset = -INFINITY;
    for (int attempt = 0; attempt < 2; ++attempt) {
#pragma unroll
      for (int ct = 0; ct < kDV / 32; ++ct) acc[ct] = f32x16{};
      st = SoftmaxState{m_preset, 0.f, -INFINITY, false};
      __syncthreads();  // the query rows (or a previous attempt's stages) have been read
      u32x4s rsrc;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        rsrc[i] = __builtin_amdgcn_readfirstlane(((const volatile LDS_AS uint32_t*)rsrc_raw)[i]);
      const int wave_a = fresh_s(wave);
#pragma unroll
      for (int t = 0; t < kAhead; ++t)
        ring_copy_stage<D_QK, BIG>(ring + t * T::kBufBytes, rsrc, keys, n, t, wave_a, lane_id());
      // Step t: wait for stage t (stage t+1 stays in flight), issue stage
      // t + kAhead into the buffer of stage t - 2 (its rope part now, its
      // nope rows under the S^T MFMAs), S^T of stage t, then P*V of stage
      // t-1 with the softmax of stage t between its MFMAs.  The first step
      // has no P*V; the last stage's P*V follows the loop.
      bf16x8 pprev[2];
      // The list entries of the stage a step gathers are read one step
      // earlier (no LDS wait at the top of the step).
      RingOffs offs = RingOffs::read(keys, kAhead, wave_a, lane_id());
      auto step = [&](int t, auto first, auto masked) {
        __builtin_amdgcn_s_waitcnt(vmcnt_only((kAhead - 1) * kGather));
        barrier_lds();
        const int lane_t = lane_id();
        LDS_AS uint8_t* cur = ring + (t % NS) * T::kBufBytes;
        LDS_AS uint8_t* prev = ring + ((t + NS - 1) % NS) * T::kBufBytes;
        LDS_AS uint8_t* nxt = ring + ((t + kAhead) % NS) * T::kBufBytes;
        const int rope_off = offs.template rope<BIG>(n, wave, lane_t);
        RingPump<D_QK, BIG> pump{rsrc, nxt, 8 * wave, offs.template pump<BIG>(n, wave, lane_t),
                                 (lane_t * 16) ^ ((wave & 1) << 5), 0u, 0u};
        offs = RingOffs::read(keys, t + kAhead + 1, wave, lane_t);
        const int rem = n - t * BK;
        const uint32_t bits = rem >= BK ? 0xffffffffu : (1u << rem) - 1u;
        // Inside the S^T chain: the rope copy of stage t + kAhead, and the
        // first V^T operands of stage t - 1 before its last MFMAs.
        RingV<D_QK> v;
        auto hook = [&](int d) {
          if (d == 1) ring_rope<D_QK, BIG>(nxt, rsrc, rope_off, wave, lane_t);
          if (!decltype(first)::value && d == T::kDSteps - 4) {
            v.init(prev, lane_t);
            v.prefetch();
          }
        };
        const f32x16 s = ring_scores<D_QK, kKRead, LFRESH>(cur, qf, pump, hook);
        bf16x8 pnext[2];
        ring_pv_softmax<D_QK, !decltype(first)::value, true, decltype(masked)::value>(
            v, pprev, acc, s, bits, st, a.scale_log2, pnext);
        pprev[0] = pnext[0];
        pprev[1] = pnext[1];
      };
      if (nst > 0) {
        // Only the last stage can hold fewer than 32 keys.
        if (nst == 1) {
          step(0, std::true_type{}, std::true_type{});
        } else {
          step(0, std::true_type{}, std::false_type{});
          for (int t = 1; t < nst - 1; ++t) step(t, std::false_type{}, std::false_type{});
          step(nst - 1, std::false_type{}, std::true_type{});
        }
        RingV<D_QK> v;
        v.init(ring + ((nst - 1) % NS) * T::kBufBytes, lane_fresh());
        v.prefetch();
        bf16x8 none[2];
        ring_pv_softmax<D_QK, true, false>(v, pprev, acc, f32x16{}, 0u, st, a.scale_log2, none);
      }
      // The zero-fill copies of the stages past the end may still be landing.
      wait_vm_all();
      if (!__syncthreads_or(st.overflow) || attempt == 1) break;
      m_preset = st.m_max;
    }

    const int lane_e = lane_fresh(), hl = lane_e & 31, half = lane_e >> 5, head = wave * 32 + hl;
    if constexpr (SPLIT) {
      // The unit's output normalised by its own sum (the sink joins once,
      // in the merge); an empty unit has lse = -inf (no contribution).
      // Stored in the accumulator layout (split_tile): 1 KiB per store
      // instruction.
      const size_t u = (size_t)unit * a.h_q + head;
      const float inv = st.l_sum > 0.f ? 1.f / st.l_sum : 0.f;
      float* obase = a.ws_o + split_tile(unit, wave, a.h_q / 32) + 4 * lane_e;
#pragma unroll
      for (int ct = 0; ct < kDV / 32; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          // non-temporal: the merge kernel reads the partials once
          __builtin_nontemporal_store(
              f32x4{acc[ct][4 * j] * inv, acc[ct][4 * j + 1] * inv, acc[ct][4 * j + 2] * inv,
                    acc[ct][4 * j + 3] * inv},
              reinterpret_cast<f32x4*>(obase + (4 * ct + j) * 256));
      if (half == 0) {
        a.ws_stats[2 * u] = st.l_sum > 0.f ? (st.m_ref + __log2f(st.l_sum)) * kLn2 : -INFINITY;
        a.ws_stats[2 * u + 1] = st.l_sum > 0.f ? st.m_max * kLn2 : -INFINITY;
      }
      continue;
    }
    // Normalise and store, as the wide kernel without a key split does: the
    // wave's bf16 tile is staged in its own ring buffer (no wave reads the
    // ring any more: the barrier above follows the last stage).
    float scale = 0.f, lse_v = INFINITY, ml_v = -INFINITY;
    if (st.l_sum > 0.f) {
      float denom = st.l_sum;
      if (SINK) denom += __builtin_amdgcn_exp2f(sink_lds[head] * kLog2e - st.m_ref);
      scale = 1.f / denom;
      ml_v = st.m_max * kLn2;
      lse_v = (st.m_ref + __log2f(st.l_sum)) * kLn2;
    }
    if (half == 0) {
      a.lse[(size_t)row * a.h_q + head] = lse_v;
      if (a.max_logits) a.max_logits[(size_t)row * a.h_q + head] = ml_v;
    }
    LDS_AS uint8_t* tile = ring + wave * T::kBufBytes;
#pragma unroll
    for (int ct = 0; ct < kDV / 32; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x4 o4 = {(__bf16)(acc[ct][4 * j] * scale), (__bf16)(acc[ct][4 * j + 1] * scale),
                           (__bf16)(acc[ct][4 * j + 2] * scale), (__bf16)(acc[ct][4 * j + 3] * scale)};
        *reinterpret_cast<LDS_AS bf16x4*>(tile + hl * (kDV * 2) + (((4 * ct + j) ^ hl) << 4) + 8 * half) = o4;
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the tile is complete for every lane
    uint8_t* orow = reinterpret_cast<uint8_t*>(a.out + ((size_t)row * a.h_q + wave * 32) * kDV) + lane_e * 16;
#pragma unroll 4
    for (int h = 0; h < 32; ++h) {
      const u32x4 v = *reinterpret_cast<const LDS_AS u32x4*>(tile + h * (kDV * 2) + ((lane_e ^ h) << 4));
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(orow + (size_t)h * (kDV * 2)));
    }
  }
}

// Merge of the splits of split decode.  The split lses give lse =
// logsumexp over the splits, each split's output enters with weight
// exp(lse_s - lse), and an empty split (lse_s = -inf) contributes nothing;
// the sink joins the denominator once, after the merge; a row whose splits
// are all empty gives out = 0, lse = +inf, max_logits = -inf.
// One wave per (row, group of 32 heads, 32 value columns ct): the partials
// are stored in the attention kernels' accumulator layout (split_tile), so
// lane (half, j32) reads 16 B chunks j = 0..3 of its tile, values of head
// 32 g + j32 at columns 32 ct + 8 j + 4 half .. + 3.  The splits are read
// eight at a time, every load of a round issued before any is used (a loop
// over single splits waits one memory latency per split).  Rounds past the
// last split re-read that split with weight 0 (it is finite), so the sums
// keep the split order.
template <bool SINK>
__global__ void __launch_bounds__(256) split_combine_kernel(FwdArgs a) {
  const int groups = a.h_q / 32;
  const long long w = (long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (w >= (long long)a.rows * groups * (kDV / 32)) return;
  const int ct = (int)(w % (kDV / 32));
  const int g = (int)((w / (kDV / 32)) % groups), row = (int)(w / (kDV / 32) / groups);
  const int lane = lane_id(), j32 = lane & 31, half = lane >> 5, head = g * 32 + j32;
  const int S = a.splits;
  const float* st = a.ws_stats + ((size_t)row * S * a.h_q + head) * 2;
  const size_t sstride = (size_t)a.h_q * 2;  // between the splits of one head
  constexpr int R = 8;                       // splits per round
  const float* o = a.ws_o + split_tile((size_t)row * S, g, groups) + (size_t)ct * 4 * 256 + 4 * lane;
  const size_t ostride = (size_t)groups * 32 * kDV;  // between the splits' tiles
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  float lse_v = INFINITY, ml_v = -INFINITY;
  auto add_round = [&](int s0, float lse) {
    f32x4 v[R][4];
    float wg[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int s = s0 + j < S ? s0 + j : S - 1;
      wg[j] = st[s * sstride];
#pragma unroll
      for (int c = 0; c < 4; ++c) v[j][c] = *reinterpret_cast<const f32x4*>(o + s * ostride + c * 256);
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float wgt = s0 + j < S ? expf(wg[j] - lse) : 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * c + e] += wgt * v[j][c][e];
    }
  };
  if (S <= R) {
    // One round: every statistic and partial loaded before any is used.
    f32x4 v[R][4];
    float l8[R], x8[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int s = j < S ? j : S - 1;
      l8[j] = st[s * sstride];
      x8[j] = st[s * sstride + 1];
#pragma unroll
      for (int c = 0; c < 4; ++c) v[j][c] = *reinterpret_cast<const f32x4*>(o + s * ostride + c * 256);
    }
    float m = -INFINITY, mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      m = fmaxf(m, l8[j]);
      mx = fmaxf(mx, x8[j]);
    }
    if (m != -INFINITY) {
      float z = 0.f;
#pragma unroll
      for (int j = 0; j < R; ++j)
        if (j < S) z += expf(l8[j] - m);
      const float lse = m + logf(z);
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const float wgt = j < S ? expf(l8[j] - lse) : 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * c + e] += wgt * v[j][c][e];
      }
      lse_v = lse;
      ml_v = mx;
    }
  } else {
    // Rounds of R splits: the maxima, the sum, then the weighted partials.
    float m = -INFINITY, mx = -INFINITY;
    for (int s0 = 0; s0 < S; s0 += R) {
      float l8[R], x8[R];
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const int s = s0 + j < S ? s0 + j : S - 1;
        l8[j] = st[s * sstride];
        x8[j] = st[s * sstride + 1];
      }
#pragma unroll
      for (int j = 0; j < R; ++j) {
        m = fmaxf(m, l8[j]);
        mx = fmaxf(mx, x8[j]);
      }
    }
    if (m != -INFINITY) {
      float z = 0.f;
      for (int s0 = 0; s0 < S; s0 += R) {
        float e8[R];
#pragma unroll
        for (int j = 0; j < R; ++j) e8[j] = st[(s0 + j < S ? s0 + j : S - 1) * sstride];
#pragma unroll
        for (int j = 0; j < R; ++j)
          if (s0 + j < S) z += expf(e8[j] - m);  // exp(-inf) = 0
      }
      const float lse = m + logf(z);
      for (int s0 = 0; s0 < S; s0 += R) add_round(s0, lse);
      lse_v = lse;
      ml_v = mx;
    }
  }
  if (lse_v != INFINITY) {
    float f = 1.f;
    if (SINK) f = 1.f / (1.f + expf(a.attn_sink[head] - lse_v));
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] *= f;
  }
  __bf16* orow = a.out + ((size_t)row * a.h_q + head) * kDV + 32 * ct + 4 * half;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    *reinterpret_cast<bf16x4*>(orow + 8 * c) =
        bf16x4{(__bf16)acc[4 * c], (__bf16)acc[4 * c + 1], (__bf16)acc[4 * c + 2],
               (__bf16)acc[4 * c + 3]};
  if (ct == 0 && half == 0) {
    a.lse[(size_t)row * a.h_q + head] = lse_v;
    if (a.max_logits) a.max_logits[(size_t)row * a.h_q + head] = ml_v;
  }
}

// Row lengths from the same routines the attention kernels use; one wave per row.
__global__ void __launch_bounds__(256) row_lengths_kernel(const int32_t* indices,
                                                          const int32_t* topk_length,
                                                          const int32_t* cache_seqlens, int rows,
                                                          int rows_per_seq, int topk, int s_kv,
                                                          int mbps, int32_t* row_len) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  int L;
  if (topk_length != nullptr) {
    L = clamp_length(topk_length[row], topk);
  } else {
    const int bound = row_bound(cache_seqlens != nullptr, cache_seqlens, row / rows_per_seq, s_kv, mbps);
    const int32_t* idx_row = indices + (size_t)row * topk;
    L = finish_tail_scan(load_tail_round(idx_row, topk), idx_row, topk, bound);
  }
  if (lane_id() == 0) row_len[row] = L;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

thread_local std::string g_last_error;

smla_status fail(smla_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

smla_status check_common(int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t d_v, int32_t topk,
                         float sm_scale) {
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale))
    return fail(SMLA_ERR_UNSUPPORTED, "sm_scale=%g (must be positive and finite)", (double)sm_scale);
  if (h_q <= 0 || topk <= 0 || d_qk <= 0 || d_v <= 0)
    return fail(SMLA_ERR_BAD_SHAPE, "non-positive size (h_q=%d topk=%d d_qk=%d d_v=%d)", h_q, topk,
                d_qk, d_v);
  if (d_v > d_qk) return fail(SMLA_ERR_BAD_SHAPE, "d_v=%d exceeds d_qk=%d", d_v, d_qk);
  if (h_kv != 1) return fail(SMLA_ERR_UNSUPPORTED, "h_kv=%d (only 1 is supported)", h_kv);
  if (d_qk != 512 && d_qk != 576)
    return fail(SMLA_ERR_UNSUPPORTED, "d_qk=%d (supported: 512, 576)", d_qk);
  if (d_v != kDV) return fail(SMLA_ERR_UNSUPPORTED, "d_v=%d (supported: 512)", d_v);
  if (h_q % kHeadsPerWave != 0 || h_q > 128)
    return fail(SMLA_ERR_UNSUPPORTED, "h_q=%d (supported: multiples of 16 up to 128)", h_q);
  return SMLA_OK;
}

// The attention kernel the last forward or decode call on this thread
// launched (for tests and tools).
thread_local const char* g_last_kernel = "";

template <int D_QK, bool PAGED, bool DYNAMIC, bool SINK>
smla_status launch_fwd(const FwdArgs& args, hipStream_t stream) {
  const int waves_total = args.h_q / kHeadsPerWave;
  const int nwaves = waves_total / args.head_groups;
  const int grid = args.head_groups == 1 ? args.rows : ((args.rows + 7) / 8) * 16;
  hipLaunchKernelGGL((sparse_mla_fwd_kernel<D_QK, PAGED, DYNAMIC, SINK>), dim3(grid),
                     dim3(nwaves * 64), 0, stream, args);
  g_last_kernel = "heads16";
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SMLA_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

// Compute units of the current device (cached per device), or -1.
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev >= 0 && dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return -1;
  if (dev >= 0 && dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int D_QK, int NW, int KS, bool PAGED, bool DYNAMIC, bool SINK, bool BIG>
smla_status launch_wide(const FwdArgs& args, hipStream_t stream) {
  if (args.h_q != 32 * NW / KS)
    return fail(SMLA_ERR_UNSUPPORTED, "wide kernel with %d waves and %d key splits needs h_q=%d",
                NW, KS, 32 * NW / KS);
  const int cus = cu_count();
  if (cus <= 0) return fail(SMLA_ERR_LAUNCH, "cannot read the device's compute-unit count");
  // As many workgroups as the CUs hold at once (one wave per SIMD), each
  // looping over rows.
  const long long slots = (long long)cus * (kWideWaves / NW);
  const int grid = args.rows < slots ? args.rows : (int)slots;
  hipLaunchKernelGGL((sparse_mla_fwd_wide_kernel<D_QK, NW, KS, PAGED, DYNAMIC, SINK, false, BIG>),
                     dim3(grid), dim3(NW * 64), 0, stream, args);
  g_last_kernel = BIG ? "wide_big" : "wide";
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SMLA_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

template <int D_QK, bool PAGED, bool DYNAMIC, bool SINK, bool BIG>
smla_status launch_ring(const FwdArgs& args, hipStream_t stream) {
  const int cus = cu_count();
  if (cus <= 0) return fail(SMLA_ERR_LAUNCH, "cannot read the device's compute-unit count");
  const int grid = args.rows < cus ? args.rows : cus;  // one workgroup per CU (LDS)
  hipLaunchKernelGGL((sparse_mla_fwd_ring_kernel<D_QK, PAGED, DYNAMIC, SINK, BIG>), dim3(grid),
                     dim3(kWideWaves * 64), 0, stream, args);
  g_last_kernel = BIG ? "ring_big" : "ring";
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SMLA_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

// 128 heads and rows of at most kRingMaxTopk positions: the ring kernel.
template <bool PAGED, bool BIG>
smla_status dispatch_ring(int d_qk, FwdArgs& args, hipStream_t stream) {
  const bool dyn = args.topk_length != nullptr;
  const bool sink = args.attn_sink != nullptr;
  args.head_groups = 1;
#define SMLA_RING(D, DYN, SNK)                                 \
  if (d_qk == D && dyn == DYN && sink == SNK)                  \
    return launch_ring<D, PAGED, DYN, SNK, BIG>(args, stream);
  SMLA_RING(512, false, false)
  SMLA_RING(512, false, true)
  SMLA_RING(512, true, false)
  SMLA_RING(512, true, true)
  SMLA_RING(576, false, false)
  SMLA_RING(576, false, true)
  SMLA_RING(576, true, false)
  SMLA_RING(576, true, true)
#undef SMLA_RING
  return fail(SMLA_ERR_UNSUPPORTED, "no ring kernel instance for d_qk=%d", d_qk);
}

template <bool PAGED, bool BIG>
smla_status dispatch_wide(int d_qk, FwdArgs& args, hipStream_t stream) {
  // 128 heads: 4 waves; 64 heads at d_qk = 512: 2 waves (two workgroups per
  // CU, 32-key blocks); 64 heads at d_qk = 576: 4 waves as 2 head groups x 2
  // key splits (a 2-wave kernel at d_qk = 576 does not fit the registers).
  const int nw = args.h_q == 64 && d_qk == 512 ? 2 : 4;
  const int ks = args.h_q == 64 && d_qk == 576 ? 2 : 1;
  const bool dyn = args.topk_length != nullptr;
  const bool sink = args.attn_sink != nullptr;
  args.head_groups = 1;
#define SMLA_WIDE(D, W, K, DYN, SNK)                                     \
  if (d_qk == D && nw == W && ks == K && dyn == DYN && sink == SNK)      \
    return launch_wide<D, W, K, PAGED, DYN, SNK, BIG>(args, stream);
  SMLA_WIDE(512, 4, 1, false, false)
  SMLA_WIDE(512, 4, 1, false, true)
  SMLA_WIDE(512, 4, 1, true, false)
  SMLA_WIDE(512, 4, 1, true, true)
  SMLA_WIDE(512, 2, 1, false, false)
  SMLA_WIDE(512, 2, 1, false, true)
  SMLA_WIDE(512, 2, 1, true, false)
  SMLA_WIDE(512, 2, 1, true, true)
  SMLA_WIDE(576, 4, 1, false, false)
  SMLA_WIDE(576, 4, 1, false, true)
  SMLA_WIDE(576, 4, 1, true, false)
  SMLA_WIDE(576, 4, 1, true, true)
  SMLA_WIDE(576, 4, 2, false, false)
  SMLA_WIDE(576, 4, 2, false, true)
  SMLA_WIDE(576, 4, 2, true, false)
  SMLA_WIDE(576, 4, 2, true, true)
#undef SMLA_WIDE
  return fail(SMLA_ERR_UNSUPPORTED, "no wide kernel instance for d_qk=%d", d_qk);
}

// Split decode: the wide kernel over (row, split) units writing partials to
// the workspace, then the merge.  Only layouts without a key split (128
// heads, or 64 heads at d_qk = 512).
template <int D_QK, int NW, bool DYNAMIC, bool SINK, bool BIG>
smla_status launch_split(const FwdArgs& args, hipStream_t stream) {
  const int cus = cu_count();
  if (cus <= 0) return fail(SMLA_ERR_LAUNCH, "cannot read the device's compute-unit count");
  const long long units = (long long)args.rows * args.splits;
  const long long slots = (long long)cus * (kWideWaves / NW);
  const int grid = (int)(units < slots ? units : slots);
  hipLaunchKernelGGL((sparse_mla_fwd_wide_kernel<D_QK, NW, 1, true, DYNAMIC, SINK, true, BIG>),
                     dim3(grid), dim3(NW * 64), 0, stream, args);
  g_last_kernel = BIG ? "split_big" : "split";
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SMLA_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  const long long waves = (long long)args.rows * (args.h_q / 32) * (kDV / 32);
  // One wave per workgroup: the (row, head group, column tile) waves spread
  // over every CU.
  hipLaunchKernelGGL((split_combine_kernel<SINK>), dim3((unsigned)waves), dim3(64), 0, stream,
                     args);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(SMLA_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

// Split decode at 128 heads with at most kRingMaxTopk positions per unit:
// the ring kernel over (row, split) units, then the merge.
template <int D_QK, bool DYNAMIC, bool SINK, bool BIG>
smla_status launch_ring_split(const FwdArgs& args, hipStream_t stream) {
  const int cus = cu_count();
  if (cus <= 0) return fail(SMLA_ERR_LAUNCH, "cannot read the device's compute-unit count");
  const long long units = (long long)args.rows * args.splits;
  const int grid = (int)(units < cus ? units : cus);
  hipLaunchKernelGGL((sparse_mla_fwd_ring_kernel<D_QK, true, DYNAMIC, SINK, BIG, true>), dim3(grid),
                     dim3(kWideWaves * 64), 0, stream, args);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SMLA_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  g_last_kernel = BIG ? "ring_split_big" : "ring_split";
  const long long waves = (long long)args.rows * (args.h_q / 32) * (kDV / 32);
  // One wave per workgroup: the (row, head group, column tile) waves spread
  // over every CU.
  hipLaunchKernelGGL((split_combine_kernel<SINK>), dim3((unsigned)waves), dim3(64), 0, stream,
                     args);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(SMLA_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

smla_status dispatch_split(int d_qk, FwdArgs& args, hipStream_t stream) {
  if (!(args.h_q == 128 || (args.h_q == 64 && d_qk == 512)))
    return fail(SMLA_ERR_UNSUPPORTED,
                "split decode supports h_q=128, or h_q=64 at d_qk=512 (got h_q=%d, d_qk=%d)",
                args.h_q, d_qk);
  if (args.table_mode == 2)
    return fail(SMLA_ERR_UNSUPPORTED, "split decode: KV pool rows beyond 32-bit row entries");
  const int nw = args.h_q / 32;
  const bool dyn = args.topk_length != nullptr;
  const bool sink = args.attn_sink != nullptr;
  const bool big = args.table_mode == 1;
  // (A unit then takes at most ceil(ceil(topk / 64) / splits) blocks of 64.)
  if (args.h_q == 128 && (args.topk + 63) / 64 <= (kRingMaxTopk / 64) * args.splits) {
#define SMLA_RSPLIT(D, DYN, SNK)                                          \
    if (d_qk == D && dyn == DYN && sink == SNK)                         \
      return big ? launch_ring_split<D, DYN, SNK, true>(args, stream)   \
                 : launch_ring_split<D, DYN, SNK, false>(args, stream);
    SMLA_RSPLIT(512, false, false)
    SMLA_RSPLIT(512, false, true)
    SMLA_RSPLIT(512, true, false)
    SMLA_RSPLIT(512, true, true)
    SMLA_RSPLIT(576, false, false)
    SMLA_RSPLIT(576, false, true)
    SMLA_RSPLIT(576, true, false)
    SMLA_RSPLIT(576, true, true)
#undef SMLA_RSPLIT
  }
#define SMLA_SPLIT(D, W, DYN, SNK)                              \
  if (d_qk == D && nw == W && dyn == DYN && sink == SNK)        \
    return big ? launch_split<D, W, DYN, SNK, true>(args, stream) \
               : launch_split<D, W, DYN, SNK, false>(args, stream);
  SMLA_SPLIT(512, 4, false, false)
  SMLA_SPLIT(512, 4, false, true)
  SMLA_SPLIT(512, 4, true, false)
  SMLA_SPLIT(512, 4, true, true)
  SMLA_SPLIT(512, 2, false, false)
  SMLA_SPLIT(512, 2, false, true)
  SMLA_SPLIT(512, 2, true, false)
  SMLA_SPLIT(512, 2, true, true)
  SMLA_SPLIT(576, 4, false, false)
  SMLA_SPLIT(576, 4, false, true)
  SMLA_SPLIT(576, 4, true, false)
  SMLA_SPLIT(576, 4, true, true)
#undef SMLA_SPLIT
  return fail(SMLA_ERR_UNSUPPORTED, "no split decode instance for d_qk=%d", d_qk);
}

// Table addressing of the wide and ring kernels for a KV table of `rows`
// rows: 32-bit byte offsets (kv_span) up to kMaxKvSpan bytes; above that,
// BIG entries while every row's entry stays below kBigNone (tables up to
// about 550 GB at d_qk = 576); beyond, the 16-head kernel's 64-bit
// addresses.
void set_table(FwdArgs& args, uint64_t rows, int d_qk) {
  const uint64_t bytes = rows * (uint64_t)d_qk * 2u;
  args.kv_span = bytes <= kMaxKvSpan ? (uint32_t)bytes : 0xFFFFFFFFu;
  args.table_mode = bytes <= kMaxKvSpan                                        ? 0
                    : rows * (uint64_t)(d_qk * 2 / kBigUnit) < (uint64_t)kBigNone ? 1
                                                                                : 2;
}

template <bool PAGED>
smla_status dispatch_fwd(int d_qk, FwdArgs& args, hipStream_t stream) {
  // The ring kernel takes 128 heads with rows of at most kRingMaxTopk
  // positions, the wide kernel 64 and 128 heads (see dispatch_wide); both
  // address the KV table as set_table decided.
  const bool big = args.table_mode == 1;
  if (args.table_mode != 2 && args.h_q == 128 && args.topk <= kRingMaxTopk)
    return big ? dispatch_ring<PAGED, true>(d_qk, args, stream)
               : dispatch_ring<PAGED, false>(d_qk, args, stream);
  if (args.table_mode != 2 && (args.h_q == 64 || args.h_q == 128))
    return big ? dispatch_wide<PAGED, true>(d_qk, args, stream)
               : dispatch_wide<PAGED, false>(d_qk, args, stream);
  const int waves_total = args.h_q / kHeadsPerWave;
  args.head_groups = (waves_total > 4 && waves_total % 2 == 0) ? 2 : 1;
  const bool dyn = args.topk_length != nullptr;
  const bool sink = args.attn_sink != nullptr;
#define SMLA_CASE(D, DYN, SNK)                                                     \
  if (d_qk == D && dyn == DYN && sink == SNK) return launch_fwd<D, PAGED, DYN, SNK>(args, stream);
  SMLA_CASE(512, false, false)
  SMLA_CASE(512, false, true)
  SMLA_CASE(512, true, false)
  SMLA_CASE(512, true, true)
  SMLA_CASE(576, false, false)
  SMLA_CASE(576, false, true)
  SMLA_CASE(576, true, false)
  SMLA_CASE(576, true, true)
#undef SMLA_CASE
  return fail(SMLA_ERR_UNSUPPORTED, "no kernel instance for d_qk=%d", d_qk);
}

}  // namespace

extern "C" smla_status sparse_mla_fwd(const void* q, const void* kv, const int32_t* indices,
                                      const int32_t* topk_length, const float* attn_sink,
                                      int32_t s_q, int32_t s_kv, int32_t h_q, int32_t h_kv,
                                      int32_t d_qk, int32_t d_v, int32_t topk, float sm_scale,
                                      void* out, float* lse, float* max_logits,
                                      smla_stream_t stream) {
  g_last_error.clear();
  g_last_kernel = "";
  if (s_q < 0 || s_kv < 0) return fail(SMLA_ERR_BAD_SHAPE, "negative s_q=%d or s_kv=%d", s_q, s_kv);
  smla_status st = check_common(h_q, h_kv, d_qk, d_v, topk, sm_scale);
  if (st != SMLA_OK) return st;
  if (s_q == 0) return SMLA_OK;
  if (!q || (!kv && s_kv > 0) || !indices || !out || !lse || !max_logits)
    return fail(SMLA_ERR_NULL_ARG,
                "sparse_mla_fwd: q, kv (unless s_kv = 0), indices, out, lse and max_logits are required");
  FwdArgs args{};
  args.q = static_cast<const __bf16*>(q);
  args.kv = static_cast<const uint8_t*>(kv);
  args.indices = indices;
  args.topk_length = topk_length;
  args.attn_sink = attn_sink;
  args.out = static_cast<__bf16*>(out);
  args.lse = lse;
  args.max_logits = max_logits;
  args.rows = s_q;
  args.rows_per_seq = 1;
  args.h_q = h_q;
  args.topk = topk;
  args.s_kv = s_kv;
  args.scale_log2 = sm_scale * kLog2e;
  set_table(args, (uint64_t)s_kv, d_qk);
  return dispatch_fwd<false>(d_qk, args, static_cast<hipStream_t>(stream));
}

// Validation and arguments shared by both decode entry points; rows = 0 for
// an empty batch.
smla_status decode_args(const char* who, const void* q, const void* kv_cache,
                        const int32_t* block_table, const int32_t* cache_seqlens,
                        const int32_t* indices, const int32_t* topk_length, const float* attn_sink,
                        int32_t B, int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk,
                        int32_t d_v, int32_t topk, int32_t num_blocks, int32_t page_size,
                        int32_t max_blocks_per_seq, float sm_scale, void* out, float* lse,
                        float* max_logits, FwdArgs& args) {
  args = FwdArgs{};
  if (B < 0 || s_q <= 0 || num_blocks < 0 || max_blocks_per_seq <= 0)
    return fail(SMLA_ERR_BAD_SHAPE, "bad sizes (B=%d s_q=%d num_blocks=%d max_blocks_per_seq=%d)",
                B, s_q, num_blocks, max_blocks_per_seq);
  smla_status st = check_common(h_q, h_kv, d_qk, d_v, topk, sm_scale);
  if (st != SMLA_OK) return st;
  if (page_size != kPage) return fail(SMLA_ERR_UNSUPPORTED, "page_size=%d (supported: 64)", page_size);
  if ((long long)num_blocks * kPage > 0x7fffffffLL)
    return fail(SMLA_ERR_UNSUPPORTED, "num_blocks=%d exceeds 2^31 tokens", num_blocks);
  if ((long long)B * s_q > 0x7fffffffLL) return fail(SMLA_ERR_BAD_SHAPE, "B*s_q overflows int32");
  if (B == 0) return SMLA_OK;
  if (!q || (!kv_cache && num_blocks > 0) || !block_table || !cache_seqlens || !indices || !out ||
      !lse)
    return fail(SMLA_ERR_NULL_ARG,
                "%s: q, kv_cache (unless num_blocks = 0), block_table, cache_seqlens, indices, "
                "out and lse are required", who);
  args.q = static_cast<const __bf16*>(q);
  args.kv = static_cast<const uint8_t*>(kv_cache);
  args.indices = indices;
  args.topk_length = topk_length;
  args.attn_sink = attn_sink;
  args.block_table = block_table;
  args.cache_seqlens = cache_seqlens;
  args.out = static_cast<__bf16*>(out);
  args.lse = lse;
  args.max_logits = max_logits;
  args.rows = B * s_q;
  args.rows_per_seq = s_q;
  args.h_q = h_q;
  args.topk = topk;
  args.num_blocks = num_blocks;
  args.mbps = max_blocks_per_seq;
  args.scale_log2 = sm_scale * kLog2e;
  set_table(args, (uint64_t)num_blocks * kPage, d_qk);
  args.splits = 1;
  return SMLA_OK;
}

extern "C" smla_status sparse_mla_decode_fwd(
    const void* q, const void* kv_cache, const int32_t* block_table, const int32_t* cache_seqlens,
    const int32_t* indices, const int32_t* topk_length, const float* attn_sink, int32_t B,
    int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t d_v, int32_t topk,
    int32_t num_blocks, int32_t page_size, int32_t max_blocks_per_seq, float sm_scale, void* out,
    float* lse, float* max_logits, smla_stream_t stream) {
  g_last_error.clear();
  g_last_kernel = "";
  FwdArgs args;
  const smla_status st = decode_args("sparse_mla_decode_fwd", q, kv_cache, block_table,
                                     cache_seqlens, indices, topk_length, attn_sink, B, s_q, h_q,
                                     h_kv, d_qk, d_v, topk, num_blocks, page_size,
                                     max_blocks_per_seq, sm_scale, out, lse, max_logits, args);
  if (st != SMLA_OK || args.rows == 0) return st;
  return dispatch_fwd<true>(d_qk, args, static_cast<hipStream_t>(stream));
}

extern "C" size_t sparse_mla_decode_split_workspace_bytes(int32_t B, int32_t s_q, int32_t h_q,
                                                          int32_t d_v, int32_t num_splits) {
  if (B <= 0 || s_q <= 0 || h_q <= 0 || d_v <= 0 || num_splits <= 1) return 0;
  return (size_t)B * (size_t)s_q * (size_t)num_splits * (size_t)h_q * ((size_t)d_v + 2) *
         sizeof(float);
}

extern "C" smla_status sparse_mla_decode_fwd_split(
    const void* q, const void* kv_cache, const int32_t* block_table, const int32_t* cache_seqlens,
    const int32_t* indices, const int32_t* topk_length, const float* attn_sink, int32_t B,
    int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t d_v, int32_t topk,
    int32_t num_blocks, int32_t page_size, int32_t max_blocks_per_seq, float sm_scale,
    int32_t num_splits, void* workspace, size_t workspace_bytes, void* out, float* lse,
    float* max_logits, smla_stream_t stream) {
  g_last_error.clear();
  g_last_kernel = "";
  FwdArgs args;
  smla_status st = decode_args("sparse_mla_decode_fwd_split", q, kv_cache, block_table,
                               cache_seqlens, indices, topk_length, attn_sink, B, s_q, h_q, h_kv,
                               d_qk, d_v, topk, num_blocks, page_size, max_blocks_per_seq, sm_scale,
                               out, lse, max_logits, args);
  if (st != SMLA_OK) return st;
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(SMLA_ERR_BAD_SHAPE, "num_splits=%d (1 .. %d)", num_splits, kMaxSplits);
  if ((long long)B * s_q * num_splits > 0x7fffffffLL)
    return fail(SMLA_ERR_BAD_SHAPE, "B*s_q*num_splits overflows int32");
  if ((long long)B * s_q * h_q > 0x7fffffffLL)  // the merge's grid: one wave per (row, head)
    return fail(SMLA_ERR_BAD_SHAPE, "B*s_q*h_q overflows int32");
  if (args.rows == 0) return SMLA_OK;
  if (num_splits == 1) return dispatch_fwd<true>(d_qk, args, static_cast<hipStream_t>(stream));
  const size_t need = sparse_mla_decode_split_workspace_bytes(B, s_q, h_q, d_v, num_splits);
  if (!workspace) return fail(SMLA_ERR_NULL_ARG, "sparse_mla_decode_fwd_split: workspace is required");
  if (workspace_bytes < need)
    return fail(SMLA_ERR_BAD_SHAPE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  if (((uintptr_t)workspace & 15u) != 0)
    return fail(SMLA_ERR_BAD_SHAPE, "workspace must be 16-byte aligned");
  args.splits = num_splits;
  args.ws_o = static_cast<float*>(workspace);
  args.ws_stats = args.ws_o + (size_t)args.rows * num_splits * h_q * kDV;
  return dispatch_split(d_qk, args, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// Split decode without allocation: the partials live in a static device
// array instead of a caller-owned workspace.  Each GPU the library runs on
// holds its own copy of the array until the process ends; in host code the
// array's name is only a stand-in, so its device address is looked up once
// per device (with that device current) and kept.
// ---------------------------------------------------------------------------

namespace {

// 256 (row, split) units at 128 heads: (512 + 2) fp32 per unit and head.
constexpr size_t kNoAllocScratchBytes = (size_t)256 * 128 * (kDV + 2) * sizeof(float);

__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, or nullptr (the
// error text is set).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    fail(SMLA_ERR_LAUNCH, "cannot identify the current device");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      fail(SMLA_ERR_LAUNCH, "hipGetSymbolAddress of the scratch array failed: %s",
           hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" size_t sparse_mla_decode_split_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

extern "C" smla_status sparse_mla_decode_fwd_split_noalloc(
    const void* q, const void* kv_cache, const int32_t* block_table, const int32_t* cache_seqlens,
    const int32_t* indices, const int32_t* topk_length, const float* attn_sink, int32_t B,
    int32_t s_q, int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t d_v, int32_t topk,
    int32_t num_blocks, int32_t page_size, int32_t max_blocks_per_seq, float sm_scale,
    int32_t num_splits, void* out, float* lse, float* max_logits, smla_stream_t stream) {
  g_last_error.clear();
  g_last_kernel = "";
  FwdArgs args;
  smla_status st = decode_args("sparse_mla_decode_fwd_split_noalloc", q, kv_cache, block_table,
                               cache_seqlens, indices, topk_length, attn_sink, B, s_q, h_q, h_kv,
                               d_qk, d_v, topk, num_blocks, page_size, max_blocks_per_seq, sm_scale,
                               out, lse, max_logits, args);
  if (st != SMLA_OK) return st;
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(SMLA_ERR_BAD_SHAPE, "num_splits=%d (1 .. %d)", num_splits, kMaxSplits);
  if ((long long)B * s_q * num_splits > 0x7fffffffLL)
    return fail(SMLA_ERR_BAD_SHAPE, "B*s_q*num_splits overflows int32");
  if ((long long)B * s_q * h_q > 0x7fffffffLL)
    return fail(SMLA_ERR_BAD_SHAPE, "B*s_q*h_q overflows int32");
  const size_t need = sparse_mla_decode_split_workspace_bytes(B, s_q, h_q, d_v, num_splits);
  if (need > kNoAllocScratchBytes)
    return fail(SMLA_ERR_BAD_SHAPE,
                "the partials of %d x %d rows x %d splits x %d heads take %zu bytes; the static "
                "scratch array holds %zu (use sparse_mla_decode_fwd_split with a workspace)",
                B, s_q, num_splits, h_q, need, kNoAllocScratchBytes);
  if (args.rows == 0) return SMLA_OK;
  if (num_splits == 1) return dispatch_fwd<true>(d_qk, args, static_cast<hipStream_t>(stream));
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return SMLA_ERR_LAUNCH;
  args.splits = num_splits;
  args.ws_o = static_cast<float*>(ws);
  args.ws_stats = args.ws_o + (size_t)args.rows * num_splits * h_q * kDV;
  return dispatch_split(d_qk, args, static_cast<hipStream_t>(stream));
}

extern "C" smla_status sparse_mla_row_lengths(const int32_t* indices, const int32_t* topk_length,
                                              const int32_t* cache_seqlens, int32_t rows,
                                              int32_t rows_per_seq, int32_t topk, int32_t s_kv,
                                              int32_t max_blocks_per_seq, int32_t* row_len,
                                              smla_stream_t stream) {
  g_last_error.clear();
  g_last_kernel = "";
  if (rows < 0 || topk <= 0 || rows_per_seq <= 0 || s_kv < 0)
    return fail(SMLA_ERR_BAD_SHAPE, "bad sizes (rows=%d topk=%d rows_per_seq=%d s_kv=%d)", rows,
                topk, rows_per_seq, s_kv);
  if (cache_seqlens != nullptr && max_blocks_per_seq <= 0)
    return fail(SMLA_ERR_BAD_SHAPE, "max_blocks_per_seq=%d with cache_seqlens", max_blocks_per_seq);
  if (rows == 0) return SMLA_OK;
  if (!indices || !row_len)
    return fail(SMLA_ERR_NULL_ARG, "sparse_mla_row_lengths: indices and row_len are required");
  hipLaunchKernelGGL(row_lengths_kernel, dim3((rows + 3) / 4), dim3(256), 0,
                     static_cast<hipStream_t>(stream), indices, topk_length, cache_seqlens, rows,
                     rows_per_seq, topk, s_kv, max_blocks_per_seq, row_len);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SMLA_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

extern "C" const char* sparse_mla_last_error(void) { return g_last_error.c_str(); }

extern "C" const char* sparse_mla_last_kernel(void) { return g_last_kernel; }

// Error reporting for the library's other translation units (the backward).
__attribute__((visibility("hidden"))) smla_status smla_report(smla_status s, const char* msg) {
  g_last_error = msg;
  return s;
}
__attribute__((visibility("hidden"))) void smla_clear_error() { g_last_error.clear(); }
__attribute__((visibility("hidden"))) void smla_set_last_kernel(const char* name) {
  g_last_kernel = name;
}
