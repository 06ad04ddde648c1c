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
// 16 rows: ROWS = 128 (8 waves) when the query block is a multiple of 128,
// else 64 (4 waves); the larger group shares each K and V tile between
// twice the rows.  Work items are numbered head-major (neighbouring items share
// a head and their key tiles), and the launch hands each XCD a contiguous
// range of them: workgroups are dispatched to the 8 XCDs in turn, so
// workgroup L runs item (L % 8) * ceil(N / 8) + L / 8, and the items that
// read the same K and V tiles meet in one XCD's L2.  The key blocks of the
// query block are walked in 64-key tiles (a tile wholly after the
// workgroup's last row is skipped under `causal`):
//   K and V of the tile go to LDS (padded rows; keys past the block or s as
//   zeros); the next tile's K and V are loaded into registers while this
//   one is computed;
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16, the query rows' slice in
//   registers as the B operand, so each lane owns one query row and keeps
//   its online-softmax state (running max, sum) as scalars;
//   O^T += V^T P^T with V^T read by ds_read_b64_tr_b16 and P^T taken straight
//   from the S^T accumulators (the key order of both operands is permuted
//   alike).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "sparse_mla.h"

__attribute__((visibility("hidden"))) smla_status smla_report(smla_status s, const char* msg);
__attribute__((visibility("hidden"))) void smla_clear_error();

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kDQK = 192;
constexpr int kDV = 128;
constexpr int kTile = 64;       // keys per tile
constexpr int kKRow = 2 * kDQK + 16;   // padded LDS row of K
constexpr int kVRow = 2 * kDV + 16;    // padded LDS row of V
constexpr int kSteps = kDQK / 32;      // MFMA K steps over d_qk
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

// ds_read_b64_tr_b16: in each 16-lane group, lane i gives the address of four
// consecutive 16-bit values at row (i >> 2), columns 4 (i & 3) .. +3 of a
// 4 x 16 tile, and lane n receives column n of the four rows.
__device__ __forceinline__ bf16x8 tr_pair(const LDS_AS uint8_t* tile, int row_bytes, int r0,
                                          int c0, int g, int i) {
  const LDS_AS uint8_t* p = tile + (r0 + 4 * g + (i >> 2)) * row_bytes + (c0 + 4 * (i & 3)) * 2;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p + 16 * row_bytes));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

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
    const int b = a.col_idx[e];
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

// ROWS = 128: 4 waves per SIMD (two workgroups per CU, at most 128 registers;
// a few spills, measured about 12% faster than one workgroup at 170); ROWS =
// 64: 2 waves per SIMD.
template <bool CAUSAL, int ROWS>
__global__ void __launch_bounds__(ROWS * 4)
    __attribute__((amdgpu_waves_per_eu(ROWS / 32, ROWS / 32))) block_sparse_fwd_kernel(BsArgs a) {
  constexpr int kRows = ROWS;
  constexpr int kThreads = ROWS * 4;  // 16 rows per wave
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[kTile * (kKRow + kVRow)];
  LDS_AS uint8_t* ks = (LDS_AS uint8_t*)lds_raw;
  LDS_AS uint8_t* vs = ks + kTile * kKRow;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int hl = lane & 15;
  const int item = (int)(blockIdx.x % 8u) * a.per_xcd + (int)(blockIdx.x / 8u);
  if (item >= a.n_sub * a.h_q) return;  // padding of the last XCD range (whole workgroup)
  const int head = item / a.n_sub;
  const int kvh = head / (a.h_q / a.h_kv);
  const int row0 = (item % a.n_sub) * kRows;
  const int row = row0 + wave * 16 + hl;           // this lane's query row
  const int row_last = min(row0 + kRows, a.s) - 1;  // last row of the workgroup

  bf16x8 qf[kSteps];
  {
    const __bf16* qp = a.q + ((size_t)row * a.h_q + head) * kDQK + g * 8;
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
      qf[s] = row < a.s ? *reinterpret_cast<const bf16x8*>(qp + s * 32) : bf16x8{};
  }

  f32x4 acc[kDV / 16];
#pragma unroll
  for (int ct = 0; ct < kDV / 16; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max of the log2-scaled logits
  float l_run = 0.f;        // running sum of exp2(logit - m_run)

  const int qb = row0 / a.q_block;
  const int e_end = a.row_ptr[qb + 1];
  int e = a.row_ptr[qb], t0 = -1, kend = 0;
  bool have = next_tile<CAUSAL>(a, e_end, row_last, e, t0, kend);
  TileRegs<kThreads> regs;
  if (have) load_tile(a, kvh, t0, kend, tid, regs);
  while (have) {
    {
      __syncthreads();  // the previous tile's readers are done
      store_tile(ks, vs, tid, regs);
      __syncthreads();
      const int key_end = kend;
      const int tile0 = t0;
      have = next_tile<CAUSAL>(a, e_end, row_last, e, t0, kend);
      if (have) load_tile(a, kvh, t0, kend, tid, regs);  // in flight during this tile

      // S^T: lane (g, hl) gets keys 16 kt + 4g + r of row `row`.
      f32x4 st[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const bf16x8 kf =
              *reinterpret_cast<const LDS_AS bf16x8*>(ks + (kt * 16 + hl) * kKRow + s * 64 + g * 16);
          st[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], st[kt], 0, 0, 0);
        }
      }

      // Mask (keys past the block or the sequence; with CAUSAL keys after
      // the row), then the online softmax in log2 units.
      float rmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = tile0 + kt * 16 + 4 * g + r;
          const bool ok = key < key_end && (!CAUSAL || key <= row);
          const float x = ok ? st[kt][r] * a.scale_log2 : -INFINITY;
          st[kt][r] = x;
          rmax = fmaxf(rmax, x);
        }
      rmax = fmaxf(rmax, __shfl_xor(rmax, 16));
      rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
      const float m_new = fmaxf(m_run, rmax);
      // A row with no key yet keeps m = -inf: nothing to add, nothing to scale.
      const bool live = m_new != -INFINITY;
      const float alpha = live ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      float rsum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = live ? __builtin_amdgcn_exp2f(st[kt][r] - m_new) : 0.f;
          st[kt][r] = p;
          rsum += p;
        }
      rsum += __shfl_xor(rsum, 16);
      rsum += __shfl_xor(rsum, 32);
      l_run = l_run * alpha + rsum;
      m_run = m_new;
#pragma unroll
      for (int ct = 0; ct < kDV / 16; ++ct) acc[ct] *= alpha;

      // P^T operand of key step s2: element e <-> key 32 s2 + 16 (e / 4) + 4g + e % 4.
      bf16x8 pf[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[s2][e] = (__bf16)st[2 * s2 + (e >> 2)][e & 3];

      // O^T += V^T P^T.
#pragma unroll
      for (int ct = 0; ct < kDV / 16; ++ct)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_pair(vs, kVRow, 32 * s2, ct * 16, g, hl),
                                                            pf[s2], acc[ct], 0, 0, 0);
    }
  }

  if (row >= a.s) return;
  // acc[ct][r] = O[row][16 ct + 4g + r] * l_run.
  float inv = 0.f, lse_v = INFINITY;
  if (l_run > 0.f) {
    inv = 1.f / l_run;
    lse_v = (m_run + __log2f(l_run)) * kLn2;
  }
  __bf16* op = a.out + ((size_t)row * a.h_q + head) * kDV + g * 4;
#pragma unroll
  for (int ct = 0; ct < kDV / 16; ++ct) {
    const bf16x4 o4 = {(__bf16)(acc[ct][0] * inv), (__bf16)(acc[ct][1] * inv),
                       (__bf16)(acc[ct][2] * inv), (__bf16)(acc[ct][3] * inv)};
    *reinterpret_cast<bf16x4*>(op + ct * 16) = o4;
  }
  if (g == 0) a.lse[(size_t)row * a.h_q + head] = lse_v;
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
  const int rows = q_block % 128 == 0 ? 128 : 64;
  args.n_sub = (s + rows - 1) / rows;
  const int64_t items = (int64_t)args.n_sub * h_q;
  if (items > 0x7fffffffLL - 8)
    return bs_fail(SMLA_ERR_UNSUPPORTED, "s=%d with h_q=%d gives too many work items", s, h_q);
  args.per_xcd = (int32_t)((items + 7) / 8);
  const dim3 grid((unsigned)(8 * args.per_xcd));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 block((unsigned)(rows * 4));
  if (rows == 128) {
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
