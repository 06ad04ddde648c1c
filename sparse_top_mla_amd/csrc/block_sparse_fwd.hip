// Block-sparse attention forward, non-absorbed MLA shape, for MI355X
// (gfx950 / CDNA4).
//
// What is computed (FlashMLA PR #198, "Summary", item 3: each query block
// attends only the key blocks it selects, O(s * selected) work; "Benchmarks":
// 192/128 heads, and a full-causal selection reproduces dense attention):
// one sequence of s tokens, q [s][h_q][192], k [s][h_kv][192],
// v [s][h_kv][128]; query head h reads KV head h / (h_q / h_kv).  Row i
// attends the keys of every block id listed for its query block
// (i / q_block) in the CSR selection, each listing once, ids outside
// [0, ceil(s / k_block)) ignored, and with `causal` only keys j <= i.  A row
// without keys gives out = 0, lse = +inf.
//
// Layout of work: one workgroup per (ROWS query rows, query head), waves of
// 32 rows: ROWS = 256 (8 waves) when the query block is a multiple of 256,
// else 128 (4 waves) or 64 (2 waves); a larger group shares each K and V
// tile between more rows.  Work items are numbered head-major (neighbouring
// items share a head and their key tiles), and the launch hands each XCD a
// contiguous range of them: workgroups are dispatched to the 8 XCDs in turn,
// so workgroup L runs item (L % 8) * ceil(N / 8) + L / 8, and the items that
// read the same K and V tiles meet in one XCD's L2.  The key blocks of the
// query block are walked in 64-key tiles (a tile wholly after the
// workgroup's last row is skipped under `causal`):
//   K and V of the tile go to LDS (padded rows; keys past the block or s as
//   zeros); the next tile's K and V are loaded into registers while this
//   one is computed;
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16, the wave's 32 query rows'
//   slice in registers as the B operand, so lanes j and j + 32 own row j and
//   keep its online-softmax state (running max, sum);
//   O^T += V^T P^T with V^T read by ds_read_b64_tr_b16 and P^T taken straight
//   from the S^T accumulators (the key order of both operands is permuted
//   alike).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <type_traits>

#include "sparse_mla.h"

__attribute__((visibility("hidden"))) smla_status smla_report(smla_status s, const char* msg);
__attribute__((visibility("hidden"))) void smla_clear_error();

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kDQK = 192;
constexpr int kDV = 128;
constexpr int kTile = 64;       // keys per tile
constexpr int kKRow = 2 * kDQK + 16;   // padded LDS row of K
constexpr int kVRow = 2 * kDV + 16;    // padded LDS row of V
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct BsArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  __bf16* out;
  float* lse;
  int32_t s, h_q, h_kv, q_block, k_block, n_kblocks;
  int32_t n_sub;       // ROWS-row groups of the sequence
  int32_t per_xcd;     // work items per XCD range, ceil(n_sub * h_q / 8)
  float scale_log2;
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Moves (e, t0, kend) to the tile after the current one (t0 < 0: to the
// first tile of the list from entry e on): the next 64 keys of the current
// block, else the first tile of the next listed block id in range.  Under
// CAUSAL a tile starting after row_last ends its block.  Returns false at the
// end of the list.  Every thread computes the same answer.
template <bool CAUSAL>
__device__ __forceinline__ bool next_tile(const BsArgs& a, int e_end, int row_last, int& e, int& t0,
                                          int& kend) {
  if (t0 >= 0) {
    t0 += kTile;
    if (t0 < kend && !(CAUSAL && t0 > row_last)) return true;
    ++e;
  }
  for (; e < e_end; ++e) {
    // A scalar load (the index is wave-uniform and the list read-only): a
    // vector load would make the wait for it cover the tile copies in flight.
    const int b = ((const __attribute__((address_space(4))) int32_t*)(uintptr_t)a.col_idx)[e];
    if (b < 0 || b >= a.n_kblocks) continue;
    t0 = b * a.k_block;
    kend = min(t0 + a.k_block, a.s);
    if (CAUSAL && t0 > row_last) continue;
    return true;
  }
  return false;
}

// One thread's share of a tile's K (64 rows x 24 chunks) and V (64 x 16)
// in 16-byte chunks, for THREADS threads; keys at or past kend read as zeros.
template <int THREADS>
struct TileRegs {
  static constexpr int kK = kTile * 24 / THREADS, kV = kTile * 16 / THREADS;
  u32x4 k[kK], v[kV];
};

template <int THREADS>
__device__ __forceinline__ void load_tile(const BsArgs& a, int kvh, int t0, int kend, int tid,
                                          TileRegs<THREADS>& r) {
#pragma unroll
  for (int i = 0; i < TileRegs<THREADS>::kK; ++i) {
    const int c = tid + THREADS * i, j = c / 24, ch = c % 24;
    r.k[i] = t0 + j < kend ? *reinterpret_cast<const u32x4*>(
                                 a.k + ((size_t)(t0 + j) * a.h_kv + kvh) * kDQK + ch * 8)
                           : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < TileRegs<THREADS>::kV; ++i) {
    const int c = tid + THREADS * i, j = c / 16, ch = c % 16;
    r.v[i] = t0 + j < kend ? *reinterpret_cast<const u32x4*>(
                                 a.v + ((size_t)(t0 + j) * a.h_kv + kvh) * kDV + ch * 8)
                           : u32x4{0u, 0u, 0u, 0u};
  }
}

template <int THREADS>
__device__ __forceinline__ void store_tile(LDS_AS uint8_t* ks, LDS_AS uint8_t* vs, int tid,
                                           const TileRegs<THREADS>& r) {
#pragma unroll
  for (int i = 0; i < TileRegs<THREADS>::kK; ++i) {
    const int c = tid + THREADS * i;
    *reinterpret_cast<LDS_AS u32x4*>(ks + (c / 24) * kKRow + (c % 24) * 16) = r.k[i];
  }
#pragma unroll
  for (int i = 0; i < TileRegs<THREADS>::kV; ++i) {
    const int c = tid + THREADS * i;
    *reinterpret_cast<LDS_AS u32x4*>(vs + (c / 16) * kVRow + (c % 16) * 16) = r.v[i];
  }
}

// 32 query rows per wave on v_mfma_f32_32x32x16_bf16: each K or V fragment
// read from LDS serves 32 rows, half the LDS reads per FLOP of 16-row waves
// on the 16x16 shape, at the registers of one row group.  ROWS = 128 (4
// waves, two per SIMD) or 64 (2 waves, whose tile prefetch takes twice the
// registers per thread: one per SIMD) rows per workgroup.
//   S^T (32 keys x 32 rows) = K Q^T per 32-key half of the 64-key tile: lane
//   (half, j) holds row j and keys 8 (i / 4) + 4 half + i % 4 in s[i].
//   P^T operand of key step u (16 keys): element e is key
//   16 u + 8 (e / 4) + 4 half + e % 4, i.e. s[8 (u % 2) + e] of half u / 2;
//   the V^T operand reads its key rows in the same order (ds_read_b64_tr_b16:
//   lane (16-group g, i16) takes 8 B of key row 16 u + 4 half + TR_ROW(i16),
//   and +8 for the upper four keys, at value chunk 4 ct + 2 (g % 2) +
//   TR_COL(i16) / 2).
//   O^T (32 value columns x 32 rows) per value tile ct: lane (half, j) holds
//   row j, columns 32 ct + 8 (i / 4) + 4 half + i % 4.
template <bool CAUSAL, int ROWS>
__global__ void __launch_bounds__(ROWS * 2)
    __attribute__((amdgpu_waves_per_eu(ROWS == 64 ? 1 : 2, ROWS == 64 ? 1 : 2)))
    block_sparse_fwd_kernel(BsArgs a) {
  constexpr int kRows = ROWS;
  constexpr int kThreads = ROWS * 2;  // 32 rows per wave
  constexpr int kSteps16 = kDQK / 16;  // 32x32x16 K steps over d_qk
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[kTile * (kKRow + kVRow)];
  LDS_AS uint8_t* ks = (LDS_AS uint8_t*)lds_raw;
  LDS_AS uint8_t* vs = ks + kTile * kKRow;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j32 = lane & 31, half = lane >> 5;
  const int item = (int)(blockIdx.x % 8u) * a.per_xcd + (int)(blockIdx.x / 8u);
  if (item >= a.n_sub * a.h_q) return;  // padding of the last XCD range (whole workgroup)
  const int head = item / a.n_sub;
  const int kvh = head / (a.h_q / a.h_kv);
  const int row0 = (item % a.n_sub) * kRows;
  const int row = row0 + wave * 32 + j32;          // this lane's query row
  const int row_last = min(row0 + kRows, a.s) - 1;  // last row of the workgroup

  bf16x8 qf[kSteps16];
  {
    const __bf16* qp = a.q + ((size_t)row * a.h_q + head) * kDQK + half * 8;
#pragma unroll
    for (int s = 0; s < kSteps16; ++s)
      qf[s] = row < a.s ? *reinterpret_cast<const bf16x8*>(qp + s * 16) : bf16x8{};
  }
  // V^T read: key row offset and chunk byte of this lane (see above).
  const int i16 = lane & 15, cb = (lane >> 4) & 1;
  const int vrow = 4 * half + (i16 >> 2);
  const int vcol = (2 * cb + ((i16 & 3) >> 1)) * 16 + 8 * (i16 & 1);

  f32x16 acc[kDV / 32];
#pragma unroll
  for (int ct = 0; ct < kDV / 32; ++ct) acc[ct] = f32x16{};
  float m_run = -INFINITY;  // running max of the log2-scaled logits
  float l_run = 0.f;        // running sum of exp2(logit - m_run)

  const int qb = row0 / a.q_block;
  const int e_end = a.row_ptr[qb + 1];
  int e = a.row_ptr[qb], t0 = -1, kend = 0;
  bool have = next_tile<CAUSAL>(a, e_end, row_last, e, t0, kend);
  TileRegs<kThreads> regs;
  if (have) load_tile(a, kvh, t0, kend, tid, regs);
  while (have) {
    __syncthreads();  // the previous tile's readers are done
    store_tile(ks, vs, tid, regs);
    __syncthreads();
    const int key_end = kend;
    const int tile0 = t0;
    have = next_tile<CAUSAL>(a, e_end, row_last, e, t0, kend);
    if (have) load_tile(a, kvh, t0, kend, tid, regs);  // in flight during this tile

    f32x16 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      st[kt] = f32x16{};
#pragma unroll
      for (int s = 0; s < kSteps16; ++s) {
        const bf16x8 kf = *reinterpret_cast<const LDS_AS bf16x8*>(ks + (kt * 32 + j32) * kKRow +
                                                                  s * 32 + half * 16);
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st[kt], 0, 0, 0);
      }
    }

    // Mask (keys past the block or the sequence; with CAUSAL keys after the
    // row), then the online softmax in log2 units; a row's 64 logits sit in
    // lanes j and j + 32.
    float rmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = tile0 + 32 * kt + 8 * (i >> 2) + 4 * half + (i & 3);
        const bool ok = key < key_end && (!CAUSAL || key <= row);
        const float x = ok ? st[kt][i] * a.scale_log2 : -INFINITY;
        st[kt][i] = x;
        rmax = fmaxf(rmax, x);
      }
    rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
    const float m_new = fmaxf(m_run, rmax);
    // A row with no key yet keeps m = -inf: nothing to add, nothing to scale.
    const bool live = m_new != -INFINITY;
    const float alpha = live ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
    float rsum = 0.f;
    bf16x8 pf[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = live ? __builtin_amdgcn_exp2f(st[kt][i] - m_new) : 0.f;
        rsum += p;
        pf[2 * kt + (i >> 3)][i & 7] = (__bf16)p;
      }
    rsum += __shfl_xor(rsum, 32);
    l_run = l_run * alpha + rsum;
    m_run = m_new;
#pragma unroll
    for (int ct = 0; ct < kDV / 32; ++ct) acc[ct] *= alpha;

    // O^T += V^T P^T.
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int ct = 0; ct < kDV / 32; ++ct) {
        const LDS_AS uint8_t* p = vs + (16 * u + vrow) * kVRow + ct * 64 + vcol;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p);
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p + 8 * kVRow));
        const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[u], acc[ct], 0, 0, 0);
      }
  }

  if (row >= a.s) return;
  float inv = 0.f, lse_v = INFINITY;
  if (l_run > 0.f) {
    inv = 1.f / l_run;
    lse_v = (m_run + __log2f(l_run)) * kLn2;
  }
  __bf16* op = a.out + ((size_t)row * a.h_q + head) * kDV + 4 * half;
#pragma unroll
  for (int ct = 0; ct < kDV / 32; ++ct)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bf16x4 o4 = {(__bf16)(acc[ct][4 * k] * inv), (__bf16)(acc[ct][4 * k + 1] * inv),
                         (__bf16)(acc[ct][4 * k + 2] * inv), (__bf16)(acc[ct][4 * k + 3] * inv)};
      *reinterpret_cast<bf16x4*>(op + 32 * ct + 8 * k) = o4;
    }
  if (half == 0) a.lse[(size_t)row * a.h_q + head] = lse_v;
}

// ---------------------------------------------------------------------------
// 256-row workgroups with a 3-stage LDS ring filled by LDS DMA
// ---------------------------------------------------------------------------
// The tiles reach LDS by buffer loads in direct-to-LDS mode: 1 KiB per
// instruction, per-lane source offsets, and keys past the tile and pad
// chunks outside the buffer's records, so they zero-fill without a branch.
// No register staging and no LDS stores; one barrier per tile (the step
// loop below says which tiles are in flight).  Each wave copies rows
// 8w .. 8w + 7 of K (4 copies of 2 rows) and of V (2 copies of 4 rows).
// LDS stage layout: 64 K rows of 512 B (24 data chunks of 16 B, 8 pad
// chunks; chunk c of row r at c ^ (r % 16): a data chunk may land in the pad
// range and the other way round), then 64 V rows of 256 B (chunk c of row r
// at c ^ 4 (r % 4)).  The S^T reads (32 rows, one chunk column) and the V^T
// reads (4 rows and 2 chunks per 16-lane group) are free of bank conflicts:
// SQ_LDS_BANK_CONFLICT reads 0, against 37% of the LDS cycles with the K
// swizzle c ^ (r % 8), which took 2% more time.  The buffer resources sit 3 KiB
// below the tensors (the instruction offset of a copy, up to 3 KiB, moves
// the memory address as well as the LDS one).
constexpr int kKRowD = 512, kVRowD = 256;
constexpr int kStageD = kTile * (kKRowD + kVRowD);  // 48 KiB
constexpr int kRingD = 3;
constexpr uint32_t kBiasD = 3 * 1024;
constexpr uint32_t kOobD = 0xFFFFE000u;  // + lane chunk + offset: outside, no wrap
constexpr uint64_t kMaxDmaBytes = kOobD - kBiasD;  // K or V tensor bytes the resources reach

typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4s dma_rsrc(const void* p, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)p - kBiasD;
  u32x4s rs;
  rs[0] = __builtin_amdgcn_readfirstlane((uint32_t)b);
  rs[1] = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) & 0xffffu;  // stride 0
  rs[2] = __builtin_amdgcn_readfirstlane(bytes + kBiasD);
  rs[3] = 0x00020000u;  // 32-bit data format, no swizzle
  return rs;
}

// One 1 KiB copy: LDS [m0 + OFF + 16 lane, +16) <- records + voff + OFF.
template <int OFF>
__device__ __forceinline__ void dma16(const u32x4s& rs, uint32_t voff, uint32_t m0) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen offset:%2 lds"
               :
               : "v"(voff), "s"(rs), "i"(OFF), "{m0}"(__builtin_amdgcn_readfirstlane(m0))
               : "memory");
}

template <bool CAUSAL>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
block_sparse_fwd_ring_kernel(BsArgs a) {
  constexpr int kRows = 256;
  constexpr int kSteps16 = kDQK / 16;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[kRingD * kStageD];
  LDS_AS uint8_t* lds = (LDS_AS uint8_t*)lds_raw;

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j32 = lane & 31, half = lane >> 5;
  const int item = (int)(blockIdx.x % 8u) * a.per_xcd + (int)(blockIdx.x / 8u);
  if (item >= a.n_sub * a.h_q) return;  // padding of the last XCD range (whole workgroup)
  const int head = item / a.n_sub;
  const int kvh = head / (a.h_q / a.h_kv);
  const int row0 = (item % a.n_sub) * kRows;
  const int row = row0 + wave * 32 + j32;          // this lane's query row
  const int row_last = min(row0 + kRows, a.s) - 1;  // last row of the workgroup

  // V^T read: lane (16-group g, i16) takes key rows 4 half + i16 / 4 (+ 16 u,
  // + 8) at chunk 4 ct + 2 (g % 2) + (i16 % 4) / 2, byte 8 (i16 % 2); the
  // swizzle term 4 (row % 4) is 4 ((i16 / 4) % 4) for all of them.
  const int i16 = lane & 15, cb = (lane >> 4) & 1;
  const int vrow = 4 * half + (i16 >> 2);
  const int vchunk = 2 * cb + ((i16 & 3) >> 1), vswz = 4 * ((i16 >> 2) & 3), vbyte = 8 * (i16 & 1);

  // Copy constants of this lane (rows relative to the tile start).
  const u32x4s rk = dma_rsrc(a.k, (uint32_t)((uint64_t)a.s * a.h_kv * (kDQK * 2)));
  const u32x4s rv = dma_rsrc(a.v, (uint32_t)((uint64_t)a.s * a.h_kv * (kDV * 2)));
  const uint32_t kstride = (uint32_t)a.h_kv * (kDQK * 2), vstride = (uint32_t)a.h_kv * (kDV * 2);
  // Copies of one tile (t0: first key, nk: keys, 0 for a zero-fill) into stage st.
  auto issue = [&](int st, int t0, int nk) {
    const uint32_t kb = (uint32_t)(uintptr_t)(lds + st * kStageD + 8 * wave * kKRowD);
    const uint32_t vb = (uint32_t)(uintptr_t)(lds + st * kStageD + kTile * kKRowD + 8 * wave * kVRowD);
    const int ln = lane_id();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 8 * wave + 2 * k + (ln >> 5);
      const int c = (ln & 31) ^ ((8 * wave + 2 * k + (ln >> 5)) & 15);
      const uint32_t off = (uint32_t)(t0 + r) * kstride + (uint32_t)kvh * (kDQK * 2) +
                           (uint32_t)c * 16u + kBiasD - (uint32_t)k * 1024u;
      const uint32_t voff = r < nk && c < 24 ? off : kOobD;
      switch (k) {
        case 0: dma16<0>(rk, voff, kb); break;
        case 1: dma16<1024>(rk, voff, kb); break;
        case 2: dma16<2048>(rk, voff, kb); break;
        default: dma16<3072>(rk, voff, kb); break;
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int r = 8 * wave + 4 * k + (ln >> 4);
      const int c = (ln & 15) ^ (4 * ((ln >> 4) & 3));
      const uint32_t off = (uint32_t)(t0 + r) * vstride + (uint32_t)kvh * (kDV * 2) +
                           (uint32_t)c * 16u + kBiasD - (uint32_t)k * 1024u;
      const uint32_t voff = r < nk ? off : kOobD;
      if (k == 0) dma16<0>(rv, voff, vb);
      else dma16<1024>(rv, voff, vb);
    }
  };

  f32x16 acc[kDV / 32];
#pragma unroll
  for (int ct = 0; ct < kDV / 32; ++ct) acc[ct] = f32x16{};
  float m_run = -INFINITY;  // reference of the log2-scaled logits (see the lazy rescale)
  float l_run = 0.f;        // sum of exp2(logit - m_run)

  const int qb = row0 / a.q_block;
  const int e_end = a.row_ptr[qb + 1];
  int e = a.row_ptr[qb], t0 = -1, kend = 0;
  // Tile i sits in stage i % 3.  Step i waits for tile i (issued in step
  // i - 1); the barrier then also says that tile i - 2's stage is free (its
  // P*V ran in step i - 1), and tile i + 1 goes there.  Then S^T of tile i,
  // and P*V of tile i - 1 with tile i's softmax placed between its MFMAs
  // (the two are independent: the rescale that tile i may call for is
  // applied to O after the P*V of tile i - 1).
  bool h0 = next_tile<CAUSAL>(a, e_end, row_last, e, t0, kend);
  int t0_0 = t0, n_0 = h0 ? min(kTile, kend - t0) : 0;
  if (h0) issue(0, t0_0, n_0);
  // The query slice lands with the first tile; the wait is the compiler's
  // own, so it knows nothing is in flight inside the loop.
  bf16x8 qf[kSteps16];
  {
    const __bf16* qp = a.q + ((size_t)row * a.h_q + head) * kDQK + half * 8;
#pragma unroll
    for (int s = 0; s < kSteps16; ++s)
      qf[s] = row < a.s ? *reinterpret_cast<const bf16x8*>(qp + s * 16) : bf16x8{};
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // The lane pair max / sum over lanes j and j + 32 (v_permlane32_swap).
  auto pair = [](float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const unsigned v = (unsigned)__builtin_amdgcn_mov_dpp((int)u, 0xE4, 0xF, 0xF, false);
    const auto r = __builtin_amdgcn_permlane32_swap(u, v, false, false);
    return uint2{r[0], r[1]};
  };
  bf16x8 pprev[4];  // P^T operands of the previous tile
  int st = 0;
  auto step = [&](auto do_pv) {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int cur = st, nxt = st == 2 ? 0 : st + 1, prv = st == 0 ? 2 : st - 1;
    const bool h1 = next_tile<CAUSAL>(a, e_end, row_last, e, t0, kend);
    const int t0_1 = t0, n_1 = h1 ? min(kTile, kend - t0) : 0;
    if (h1) issue(nxt, t0_1, n_1);

    const LDS_AS uint8_t* ks = lds + cur * kStageD;
    const LDS_AS uint8_t* vs = lds + prv * kStageD + kTile * kKRowD;  // tile i - 1's V
    const int tile0 = t0_0, key_end = t0_0 + n_0;
    // S^T as two interleaved chains (the tile's two 32-key halves), each
    // step's K fragments read one step ahead of its MFMAs.
    f32x16 sc[2] = {f32x16{}, f32x16{}};
    {
      auto rd = [&](int s, int kt) {
        return *reinterpret_cast<const LDS_AS bf16x8*>(
            ks + (kt * 32 + j32) * kKRowD + (((2 * s + half) ^ (j32 & 15)) << 4));
      };
      bf16x8 kr[2] = {rd(0, 0), rd(0, 1)};
#pragma unroll
      for (int s = 0; s < kSteps16; ++s) {
        const bf16x8 k0 = kr[0], k1 = kr[1];
        if (s + 1 < kSteps16) { kr[0] = rd(s + 1, 0); kr[1] = rd(s + 1, 1); }
        sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[s], sc[0], 0, 0, 0);
        sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[s], sc[1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Tile i's softmax, in pieces: mask (keys past the tile; with CAUSAL keys
    // after the row; a tile wholly inside both bounds for every row of the
    // workgroup needs none), the max of the raw logits (the scale is
    // positive), the lazy-rescale decision (the reference moves only when a
    // logit exceeds it by more than 8 in log2 units, so P stays below 2^8),
    // then P with the scale folded into the exponent, and the sum.
    const bool full = tile0 + kTile <= key_end && (!CAUSAL || tile0 + kTile - 1 <= row0);
    float rmax = -INFINITY, alpha = 1.f, neg = 0.f, rsum = 0.f;
    bool grow = false;
    bf16x8 pf[4];
    auto sm_piece = [&](int n) {
      if (n < 2) {
        if (!full) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = tile0 + 32 * n + 8 * (i >> 2) + 4 * half + (i & 3);
            const bool ok = key < key_end && (!CAUSAL || key <= row);
            sc[n][i] = ok ? sc[n][i] : -INFINITY;
          }
        }
      } else if (n == 2) {
        float m = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) m = fmaxf(m, sc[kt][i]);
        rmax = m;
      } else if (n == 3) {
        const uint2 r = pair(rmax);
        rmax = fmaxf(__builtin_bit_cast(float, r.x), __builtin_bit_cast(float, r.y)) * a.scale_log2;
        grow = rmax > m_run + 8.f;  // m_run = -inf: any key grows it
        if (grow) {
          alpha = __builtin_amdgcn_exp2f(m_run - rmax);
          m_run = rmax;
        }
        // a row without a key so far has only -inf logits: exp2 gives 0
        neg = m_run != -INFINITY ? -m_run : 0.f;
      } else if (n < 12) {
        const int q = n - 4;  // values 4q .. 4q + 3
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = 4 * q + i, kt = v >> 4, ii = v & 15;
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kt][ii], a.scale_log2, neg));
          rsum += p;
          pf[2 * kt + (ii >> 3)][ii & 7] = (__bf16)p;
        }
      } else if (n == 12) {
        const uint2 r = pair(rsum);
        rsum = __builtin_bit_cast(float, r.x) + __builtin_bit_cast(float, r.y);
      }
    };
    // V^T fragment of P*V product n, read one product ahead.
    auto vread = [&](int n) {
      const int u = n >> 2, ct = n & 3;
      const LDS_AS uint8_t* p =
          vs + (16 * u + vrow) * kVRowD + (((4 * ct + vchunk) ^ vswz) << 4) + vbyte;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p);
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p + 8 * kVRowD));
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    bf16x8 vnext{};
    if constexpr (decltype(do_pv)::value) vnext = vread(0);
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      if constexpr (decltype(do_pv)::value) {
        // O^T += V^T P^T of tile i - 1: key step u = n / 4, value tile ct = n % 4
        const int u = n >> 2, ct = n & 3;
        const bf16x8 vf = vnext;
        if (n + 1 < 16) vnext = vread(n + 1);
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pprev[u], acc[ct], 0, 0, 0);
      }
      sm_piece(n);
      __builtin_amdgcn_sched_barrier(0);
    }
    // The rescale tile i called for, after tile i - 1's P*V (a wave-uniform
    // branch: rare once the reference has settled).
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int ct = 0; ct < kDV / 32; ++ct) acc[ct] *= alpha;
    }
    l_run = l_run * alpha + rsum;
#pragma unroll
    for (int u = 0; u < 4; ++u) pprev[u] = pf[u];
    h0 = h1;
    t0_0 = t0_1;
    n_0 = n_1;
    st = nxt;
  };
  if (h0) {
    step(std::false_type{});
    while (h0) step(std::true_type{});
    // P*V of the last tile (stage st - 1).
    __syncthreads();
    const LDS_AS uint8_t* vs = lds + (st == 0 ? 2 : st - 1) * kStageD + kTile * kKRowD;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int ct = 0; ct < kDV / 32; ++ct) {
        const LDS_AS uint8_t* p =
            vs + (16 * u + vrow) * kVRowD + (((4 * ct + vchunk) ^ vswz) << 4) + vbyte;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p);
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p + 8 * kVRowD));
        const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pprev[u], acc[ct], 0, 0, 0);
      }
  }

  if (row >= a.s) return;
  float inv = 0.f, lse_v = INFINITY;
  if (l_run > 0.f) {
    inv = 1.f / l_run;
    lse_v = (m_run + __log2f(l_run)) * kLn2;
  }
  __bf16* op = a.out + ((size_t)row * a.h_q + head) * kDV + 4 * half;
#pragma unroll
  for (int ct = 0; ct < kDV / 32; ++ct)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bf16x4 o4 = {(__bf16)(acc[ct][4 * k] * inv), (__bf16)(acc[ct][4 * k + 1] * inv),
                         (__bf16)(acc[ct][4 * k + 2] * inv), (__bf16)(acc[ct][4 * k + 3] * inv)};
      *reinterpret_cast<bf16x4*>(op + 32 * ct + 8 * k) = o4;
    }
  if (half == 0) a.lse[(size_t)row * a.h_q + head] = lse_v;
}

// host side

smla_status bs_fail(smla_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
smla_status bs_fail(smla_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return smla_report(s, buf);
}

}  // namespace

extern "C" smla_status sparse_mla_block_sparse_fwd(const void* q, const void* k, const void* v,
                                                   const int32_t* q2k_row_ptr,
                                                   const int32_t* q2k_col_idx, int32_t s,
                                                   int32_t h_q, int32_t h_kv, int32_t d_qk,
                                                   int32_t d_v, int32_t q_block, int32_t k_block,
                                                   int32_t causal, float sm_scale, void* out,
                                                   float* lse, smla_stream_t stream) {
  smla_clear_error();
  if (s < 0 || h_q <= 0 || h_kv <= 0)
    return bs_fail(SMLA_ERR_BAD_SHAPE, "bad sizes (s=%d h_q=%d h_kv=%d)", s, h_q, h_kv);
  if (h_q % h_kv != 0)
    return bs_fail(SMLA_ERR_BAD_SHAPE, "h_q=%d is not a multiple of h_kv=%d", h_q, h_kv);
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale))
    return bs_fail(SMLA_ERR_UNSUPPORTED, "sm_scale=%g (must be positive and finite)", (double)sm_scale);
  if (d_qk != kDQK || d_v != kDV)
    return bs_fail(SMLA_ERR_UNSUPPORTED, "d_qk=%d d_v=%d (supported: 192 / 128)", d_qk, d_v);
  if (q_block <= 0 || q_block % 64 != 0 || k_block <= 0 || k_block % kTile != 0)
    return bs_fail(SMLA_ERR_UNSUPPORTED, "q_block=%d k_block=%d (supported: multiples of 64)", q_block,
                   k_block);
  if (causal != 0 && causal != 1) return bs_fail(SMLA_ERR_BAD_SHAPE, "causal=%d (0 or 1)", causal);
  if (s == 0) return SMLA_OK;
  if (!q || !k || !v || !q2k_row_ptr || !out || !lse)
    return bs_fail(SMLA_ERR_NULL_ARG,
                   "sparse_mla_block_sparse_fwd: q, k, v, q2k_row_ptr, out and lse are required");
  BsArgs args{};
  args.q = static_cast<const __bf16*>(q);
  args.k = static_cast<const __bf16*>(k);
  args.v = static_cast<const __bf16*>(v);
  args.row_ptr = q2k_row_ptr;
  args.col_idx = q2k_col_idx;
  args.out = static_cast<__bf16*>(out);
  args.lse = lse;
  args.s = s;
  args.h_q = h_q;
  args.h_kv = h_kv;
  args.q_block = q_block;
  args.k_block = k_block;
  args.n_kblocks = (int32_t)(((int64_t)s + k_block - 1) / k_block);
  args.scale_log2 = sm_scale * kLog2e;
  const int rows = q_block % 256 == 0 ? 256 : q_block % 128 == 0 ? 128 : 64;
  args.n_sub = (s + rows - 1) / rows;
  const int64_t items = (int64_t)args.n_sub * h_q;
  if (items > 0x7fffffffLL - 8)
    return bs_fail(SMLA_ERR_UNSUPPORTED, "s=%d with h_q=%d gives too many work items", s, h_q);
  args.per_xcd = (int32_t)((items + 7) / 8);
  const dim3 grid((unsigned)(8 * args.per_xcd));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 block((unsigned)(rows * 2));
  const bool dma = (uint64_t)s * h_kv * (kDQK * 2) <= kMaxDmaBytes;
  if (rows == 256 && dma) {
    if (causal)
      hipLaunchKernelGGL((block_sparse_fwd_ring_kernel<true>), grid, block, 0, st, args);
    else
      hipLaunchKernelGGL((block_sparse_fwd_ring_kernel<false>), grid, block, 0, st, args);
  } else if (rows == 256) {
    if (causal)
      hipLaunchKernelGGL((block_sparse_fwd_kernel<true, 256>), grid, block, 0, st, args);
    else
      hipLaunchKernelGGL((block_sparse_fwd_kernel<false, 256>), grid, block, 0, st, args);
  } else if (rows == 128) {
    if (causal)
      hipLaunchKernelGGL((block_sparse_fwd_kernel<true, 128>), grid, block, 0, st, args);
    else
      hipLaunchKernelGGL((block_sparse_fwd_kernel<false, 128>), grid, block, 0, st, args);
  } else {
    if (causal)
      hipLaunchKernelGGL((block_sparse_fwd_kernel<true, 64>), grid, block, 0, st, args);
    else
      hipLaunchKernelGGL((block_sparse_fwd_kernel<false, 64>), grid, block, 0, st, args);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return bs_fail(SMLA_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}
