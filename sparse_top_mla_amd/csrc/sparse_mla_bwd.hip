// Sparse top-k MLA attention backward for MI355X (gfx950 / CDNA4).
//
// What is computed (FlashMLA PR #198, "Summary", item 1: the sparse MLA
// backward runs from the forward's saved out and lse, and scatters the key and
// value gradients into an fp32 accumulator over the KV rows; the forward's
// definition is PR #196, "Problem"): for query row i, head h and each key
// occurrence j of the row (the forward's keys: valid entries before the row
// length),
//   p      = exp(s_j - lse')       s_j = sm_scale q_h . k_j, lse' = the row's
//                                  softmax normaliser (lse in natural log, or
//                                  base 2; with a sink, lse and the sink
//                                  logit combined)
//   delta  = dout_h . out_h        (over the d_v value columns)
//   ds     = sm_scale p (dout_h . v_j - delta)
//   dq_h  += ds k_j                dkv[idx_j] += ds q_h  (all d_qk columns)
//                                  dkv[idx_j] += p dout_h (value columns)
// and, with a sink, d_sink[h] -= exp(sink[h] - lse') delta, once per row.
//
// Three kernels share the work (h_q = 64, the shape the pages give for this
// operation; four waves, one per SIMD, in each):
//
// The row pass (sparse_mla_bwd_kernel), one workgroup per query row, 16 heads
// per wave.  Per block of 32 keys, gathered into LDS while the block before
// is computed (masked rows as zeros):
//   S^T = K Q^T and dP^T = V dO^T on v_mfma_f32_16x16x32_bf16 (each lane owns
//   one head, so lse' and delta are per-lane scalars);
//   P and dS in registers; dS^T and P^T also go to LDS as bf16;
//   dKV[32 keys x d_qk] = dS^T Q (+ P^T dO on the value columns), the d_qk
//   columns split over the four waves, contracted over all 64 heads, then
//   added to the fp32 accumulator with global_atomic_add_f32;
//   dQ^T += K^T dS^T with K^T read by ds_read_b64_tr_b16 and dS^T taken from
//   the registers (the key order of both operands is permuted alike).
// Those atomic adds, one per valid (row, key) pair and d_qk column, bound it.
//
// Where the selections are dense enough, the scatter is replaced: the dq
// pass (sparse_mla_bwd_dq_kernel) is the row pass without it, and the
// key-outer pass (sparse_mla_bwd_dkv_kernel) sums dK + dV per block of 64 KV
// rows over the query rows that name them, in registers, with one atomic add
// per element of the block.  Rows that name a key twice still scatter.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "sparse_mla.h"

// Error reporting shared with the forward's host code (same library).
__attribute__((visibility("hidden"))) smla_status smla_report(smla_status s, const char* msg);
__attribute__((visibility("hidden"))) void smla_clear_error();
__attribute__((visibility("hidden"))) void smla_set_last_kernel(const char* name);

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kHeads = 64;       // h_q
constexpr int kWaves = 4;        // 16 heads each
constexpr int kDV = 512;         // value width
constexpr int kBK = 32;          // keys per block
constexpr int kRowAhead = 2;     // S / dP steps whose LDS operands are read ahead
constexpr int kDqAhead = 4;      // dQ products whose K^T operands are read ahead
constexpr float kLog2e = 1.4426950408889634f;

// Padded LDS row of `bytes` of bf16: 16 bytes of pad, or 32 for a 1 KiB row,
// so that consecutive rows start 36 or 8 banks apart and neither the 16-byte
// row reads nor the ds_read_b64_tr_b16 reads (4 rows x 32 bytes per 16 lanes)
// meet in a bank.
constexpr int padded_row(int bytes) { return bytes + (bytes == 1024 ? 32 : 16); }

// ds_read_b64_tr_b16: in each 16-lane group, lane i gives the address of four
// consecutive 16-bit values at row (i >> 2), columns 4 (i & 3) .. +3 of a
// 4 x 16 tile, and lane n receives column n of the four rows.
__device__ __forceinline__ int tr_row(int i) { return i >> 2; }
__device__ __forceinline__ int tr_col(int i) { return i & 3; }

struct BwdArgs {
  const __bf16* q;          // [s_q][64][D]
  const __bf16* kv;         // [s_kv][D]
  const __bf16* out;        // [s_q][64][512]
  const __bf16* dout;       // [s_q][64][512]
  const int32_t* indices;   // [s_q][topk]
  const int32_t* row_len;   // [s_q]
  const float* lse;         // [s_q][64]
  const float* attn_sink;   // [64] or null
  __bf16* dq;               // [s_q][64][D]
  float* dkv_acc;           // [s_kv][D], zeroed before the launch
  float* d_sink;            // [64] or null, zeroed before the launch
  float* stats_out;         // [s_q][128] or null: per head the row's normaliser in
                            // log2 units (0..63), then dout . out (64..127)
  const int32_t* dup;       // [s_q]: 1 where the row names a key twice (key-outer mode)
  int32_t key_outer;        // 1: dkv comes from the key-outer pass, except rows with dup
  int32_t dup_only;         // 1: only rows with dup run (their dq again, and their scatter)
  int32_t s_q, s_kv, topk;
  float scale;              // sm_scale
  float lse_to_log2;        // log2(e) for natural-log lse, 1 for base-2 lse
};

template <int D>
struct BwdTile {
  static constexpr int kRow = padded_row(2 * D);   // padded LDS row (query head or KV row)
  static constexpr int kQBytes = kHeads * kRow;
  static constexpr int kKBytes = kBK * kRow;
  static constexpr int kSRow = 2 * kHeads + 16;    // padded LDS row of dS^T / P^T (one key)
  static constexpr int kSBytes = kBK * kSRow;
  static constexpr int kLds = kQBytes + 2 * kKBytes + 2 * kSBytes;
  static constexpr int kDSteps = D / 32;           // MFMA K steps over d_qk
  static constexpr int kVSteps = kDV / 32;         // ... over d_v
  static constexpr int kTiles = D / 16;            // 16-column tiles of a KV row
  static constexpr int kWaveTiles = kTiles / kWaves;  // dKV column tiles per wave
  static constexpr int kDoRow = padded_row(2 * kDV);  // padded LDS row of the staged dO
  static_assert(kHeads * kDoRow <= kQBytes + kKBytes, "dO staging fits");
  static_assert(kTiles % kWaves == 0, "column split");
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// LDS [lds + 16 lane, +16) <- this lane's 16 bytes at src, by LDS DMA.  The
// compiler does not count it: the kernel waits for it with vmcnt itself.
__device__ __forceinline__ void lds_dma16(const void* src, LDS_AS uint8_t* lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "{m0}"(__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds))
               : "memory");
}


__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Eight bf16 of a transposed 4+4-row pair: rows r0 + 4g + (0..3) and
// r0 + 16 + 4g + (0..3) of `base`'s tile, column c0 + (lane & 15).
__device__ __forceinline__ bf16x8 tr_pair(const LDS_AS uint8_t* tile, int row_bytes, int r0,
                                          int c0, int g, int i) {
  const LDS_AS uint8_t* p = tile + (r0 + 4 * g + tr_row(i)) * row_bytes + (c0 + 4 * tr_col(i)) * 2;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p + 16 * row_bytes));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Eight bf16 of one LDS row at elements e0 + 4g + (0..3) and e0 + 16 + 4g + (0..3):
// the same permuted order as tr_pair, read along a row.
__device__ __forceinline__ bf16x8 row_pair(const LDS_AS uint8_t* row, int e0, int g) {
  const bf16x4 lo = *reinterpret_cast<const LDS_AS bf16x4*>(row + (e0 + 4 * g) * 2);
  const bf16x4 hi = *reinterpret_cast<const LDS_AS bf16x4*>(row + (e0 + 16 + 4 * g) * 2);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <int D, bool SINK>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
sparse_mla_bwd_kernel(BwdArgs a) {
  using T = BwdTile<D>;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[T::kLds];
  LDS_AS uint8_t* qs = (LDS_AS uint8_t*)lds_raw;     // query rows [64][kRow]
  LDS_AS uint8_t* ks0 = qs + T::kQBytes;               // KV blocks [2][32][kRow]
  LDS_AS uint8_t* dst = ks0 + 2 * T::kKBytes;          // dS^T [32 keys][kSRow]
  LDS_AS uint8_t* pst = dst + T::kSBytes;              // P^T  [32 keys][kSRow]

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int hl = lane & 15;
  const int head = wave * 16 + hl;
  const int row = blockIdx.x;
  const size_t rh = (size_t)row * kHeads + head;
  if (a.dup_only && a.dup[row] == 0) return;  // the whole workgroup
  // Whether this row scatters its own dkv (the same in every wave).
  const bool scatter = a.key_outer == 0 || a.dup[row] != 0;

  // dO in registers: fragments of dP^T's B operand (own head) ...
  const __bf16* dop = a.dout + rh * kDV + g * 8;
  const __bf16* op = a.out + rh * kDV + g * 8;
  bf16x8 dor[T::kVSteps];
  float delta = 0.f;
#pragma unroll
  for (int s = 0; s < T::kVSteps; ++s) {
    dor[s] = *reinterpret_cast<const bf16x8*>(dop + s * 32);
    const bf16x8 o8 = *reinterpret_cast<const bf16x8*>(op + s * 32);
#pragma unroll
    for (int e = 0; e < 8; ++e) delta += (float)dor[s][e] * (float)o8[e];
  }
  delta += __shfl_xor(delta, 16);
  delta += __shfl_xor(delta, 32);

  // ... and of dV's B operand (all 64 heads, this wave's value columns),
  // read transposed from a staged copy of the row's dO (rows that scatter).
  bf16x8 dov[2][T::kWaveTiles];
  const int ct0 = wave * T::kWaveTiles;
  if (scatter) {
    const __bf16* drow = a.dout + (size_t)row * kHeads * kDV;
    for (int c = tid; c < kHeads * (kDV / 8); c += kWaves * 64) {
      const int h = c / (kDV / 8), ch = c % (kDV / 8);
      *reinterpret_cast<LDS_AS u32x4*>(qs + h * T::kDoRow + ch * 16) =
          *reinterpret_cast<const u32x4*>(drow + h * kDV + ch * 8);
    }
    __syncthreads();
#pragma unroll
    for (int hs = 0; hs < 2; ++hs)
#pragma unroll
      for (int c = 0; c < T::kWaveTiles; ++c) {
        const int ct = ct0 + c < kDV / 16 ? ct0 + c : 0;  // unused past the value columns
        dov[hs][c] = tr_pair(qs, T::kDoRow, 32 * hs, ct * 16, g, hl);
      }
    __syncthreads();
  }

  // Query rows into LDS.
  {
    const __bf16* qrow = a.q + (size_t)row * kHeads * D;
    for (int c = tid; c < kHeads * (D / 8); c += kWaves * 64) {
      const int h = c / (D / 8), ch = c % (D / 8);
      *reinterpret_cast<LDS_AS u32x4*>(qs + h * T::kRow + ch * 16) =
          *reinterpret_cast<const u32x4*>(qrow + h * D + ch * 8);
    }
  }

  // The row's normaliser in log2 units.
  float l2 = a.lse[rh] * a.lse_to_log2;
  float sk2 = 0.f;
  if (SINK) {
    sk2 = a.attn_sink[head] * kLog2e;
    if (!__builtin_isinf(l2)) {
      const float m = fmaxf(l2, sk2);
      l2 = m + __log2f(__builtin_amdgcn_exp2f(l2 - m) + __builtin_amdgcn_exp2f(sk2 - m));
    }
  }
  const float scale_log2 = a.scale * kLog2e;
  if (a.stats_out != nullptr && g == 0) {
    a.stats_out[(size_t)row * 2 * kHeads + head] = l2;
    a.stats_out[(size_t)row * 2 * kHeads + kHeads + head] = delta;
  }

  f32x4 dqa[T::kTiles];
#pragma unroll
  for (int ct = 0; ct < T::kTiles; ++ct) dqa[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int L = a.row_len[row];
  const int32_t* idx_row = a.indices + (size_t)row * a.topk;
  const int nblk = (L + kBK - 1) / kBK;
  // Block kb's KV rows go to buffer kb % 2 by LDS DMA while block kb - 1 is
  // computed (masked rows as zeros); lane j < 32 holds position 32 kb + j.
  auto load_idx = [&](int kb) {
    const int pos = kb * kBK + lane;
    return (kb < nblk && lane < kBK && pos < L) ? idx_row[pos] : -1;
  };
  auto gather = [&](int idx, uint64_t mask, LDS_AS uint8_t* kbuf) {
    for (int j = wave; j < kBK; j += kWaves) {
      LDS_AS uint8_t* d = kbuf + j * T::kRow;
      if ((mask >> j) & 1ull) {
        const uint8_t* src = reinterpret_cast<const uint8_t*>(a.kv) +
                             (size_t)(uint32_t)__builtin_amdgcn_readlane(idx, j) * (2 * D);
        lds_dma16(src + lane * 16, d);
        if (D > kDV && lane < (2 * D - 2 * kDV) / 16) lds_dma16(src + 2 * kDV + lane * 16, d + 2 * kDV);
      } else {
        *reinterpret_cast<LDS_AS u32x4*>(d + lane * 16) = u32x4{0u, 0u, 0u, 0u};
        if (D > kDV && lane < (2 * D - 2 * kDV) / 16)
          *reinterpret_cast<LDS_AS u32x4*>(d + 2 * kDV + lane * 16) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto valid_mask = [&](int idx) { return __builtin_amdgcn_ballot_w64(idx >= 0 && idx < a.s_kv); };
  int idx_nxt = load_idx(0);
  uint64_t mask_nxt = valid_mask(idx_nxt);
  if (nblk > 0) gather(idx_nxt, mask_nxt, ks0);
  int idx_far = load_idx(1);
  for (int kb = 0; kb < nblk; ++kb) {
    const int idx = idx_nxt;
    const uint64_t mask = mask_nxt;
    LDS_AS uint8_t* ks = ks0 + (kb & 1) * T::kKBytes;
    wait_vm_all();    // block kb's copies (and the previous block's atomics)
    __syncthreads();  // ... of every wave; block kb - 1's readers are done
    idx_nxt = idx_far;
    mask_nxt = valid_mask(idx_nxt);
    if (kb + 1 < nblk) gather(idx_nxt, mask_nxt, ks0 + ((kb + 1) & 1) * T::kKBytes);
    idx_far = load_idx(kb + 2);

    // S^T and dP^T: lane (g, hl) holds keys 16 kt + 4g + r of head `head`.
    f32x4 st[2], dpt[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dpt[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // The step's three LDS operands (query slice, two key rows) are read
    // kRowAhead steps ahead of its products.
    {
      auto rd = [&](int s, int k) {  // k = 0: query; 1, 2: key rows kt = k - 1
        const LDS_AS uint8_t* p = k == 0 ? qs + head * T::kRow : ks + ((k - 1) * 16 + hl) * T::kRow;
        return *reinterpret_cast<const LDS_AS bf16x8*>(p + s * 64 + g * 16);
      };
      bf16x8 buf[kRowAhead][3];
#pragma unroll
      for (int s = 0; s < kRowAhead; ++s)
#pragma unroll
        for (int k = 0; k < 3; ++k) buf[s][k] = rd(s, k);
#pragma unroll
      for (int s = 0; s < T::kDSteps; ++s) {
        const bf16x8 qf = buf[s % kRowAhead][0];
        const bf16x8 kf0 = buf[s % kRowAhead][1];
        const bf16x8 kf1 = buf[s % kRowAhead][2];
        if (s + kRowAhead < T::kDSteps)
#pragma unroll
          for (int k = 0; k < 3; ++k) buf[s % kRowAhead][k] = rd(s + kRowAhead, k);
        st[0] = mfma(kf0, qf, st[0]);
        st[1] = mfma(kf1, qf, st[1]);
        if (s < T::kVSteps) {
          dpt[0] = mfma(kf0, dor[s], dpt[0]);
          dpt[1] = mfma(kf1, dor[s], dpt[1]);
        }
        __builtin_amdgcn_sched_barrier(0);  // keeps the read-ahead distance
      }
    }

    // P and dS (scaled by sm_scale); masked keys get 0.
    bf16x8 dsf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kt * 16 + 4 * g + r;
        const bool valid = (mask >> key) & 1ull;
        const float p = valid ? __builtin_amdgcn_exp2f(st[kt][r] * scale_log2 - l2) : 0.f;
        const float ds = a.scale * p * (dpt[kt][r] - delta);
        dsf[kt * 4 + r] = (__bf16)ds;
        if (scatter) {
          *reinterpret_cast<LDS_AS __bf16*>(dst + key * T::kSRow + head * 2) = (__bf16)ds;
          *reinterpret_cast<LDS_AS __bf16*>(pst + key * T::kSRow + head * 2) = (__bf16)p;
        }
      }

    if (scatter) __syncthreads();  // dS^T and P^T of every wave are in LDS

    // dKV of this wave's columns: element e of both operands is head
    // 32 hs + 16 (e / 4) + 4g + e % 4.
    if (scatter)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x4 acc[T::kWaveTiles];
#pragma unroll
      for (int c = 0; c < T::kWaveTiles; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        const bf16x8 af = row_pair(dst + (kt * 16 + hl) * T::kSRow, 32 * hs, g);
        const bf16x8 pf = row_pair(pst + (kt * 16 + hl) * T::kSRow, 32 * hs, g);
#pragma unroll
        for (int c = 0; c < T::kWaveTiles; ++c) {
          acc[c] = mfma(af, tr_pair(qs, T::kRow, 32 * hs, (ct0 + c) * 16, g, hl), acc[c]);
          if (ct0 + c < kDV / 16) acc[c] = mfma(pf, dov[hs][c], acc[c]);
        }
      }
      // acc[c][r] is dKV[key 16 kt + 4g + r][column 16 (ct0 + c) + hl].
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kt * 16 + 4 * g + r;
        const int kidx = __shfl(idx, key);
        if ((mask >> key) & 1ull) {
          float* drow = a.dkv_acc + (size_t)(uint32_t)kidx * D + ct0 * 16 + hl;
#pragma unroll
          for (int c = 0; c < T::kWaveTiles; ++c) unsafeAtomicAdd(drow + c * 16, acc[c][r]);
        }
      }
    }

    // dQ^T += K^T dS^T, after the atomic adds so that they drain behind it
    // (the next block's loads wait for them): element e of both operands is
    // key 16 (e / 4) + 4g + e % 4.
    {
      bf16x8 kt_op[kDqAhead];
#pragma unroll
      for (int ct = 0; ct < kDqAhead; ++ct) kt_op[ct] = tr_pair(ks, T::kRow, 0, ct * 16, g, hl);
#pragma unroll
      for (int ct = 0; ct < T::kTiles; ++ct) {
        const bf16x8 cur = kt_op[ct % kDqAhead];
        if (ct + kDqAhead < T::kTiles)
          kt_op[ct % kDqAhead] = tr_pair(ks, T::kRow, 0, (ct + kDqAhead) * 16, g, hl);
        dqa[ct] = mfma(cur, dsf, dqa[ct]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // dq[row][head][16 ct + 4g + r] = dqa[ct][r].
  __bf16* dqp = a.dq + rh * D + g * 4;
#pragma unroll
  for (int ct = 0; ct < T::kTiles; ++ct) {
    const bf16x4 v = {(__bf16)dqa[ct][0], (__bf16)dqa[ct][1], (__bf16)dqa[ct][2],
                      (__bf16)dqa[ct][3]};
    *reinterpret_cast<bf16x4*>(dqp + ct * 16) = v;
  }
  if (SINK && a.d_sink != nullptr && !a.dup_only && g == 0 && !__builtin_isinf(l2))
    unsafeAtomicAdd(a.d_sink + head, -__builtin_amdgcn_exp2f(sk2 - l2) * delta);
}

// ---------------------------------------------------------------------------
// dq pass of key-outer calls
// ---------------------------------------------------------------------------
// The row pass without the scatter (rows that name a key twice run the row
// pass above afterwards, alone): the query slice stays in registers, so LDS
// holds four 32-key KV blocks and the row's index list, and each block's
// rows are gathered three blocks ahead.  Masked rows copy a row of zeros,
// so every block takes the same number of copies and the waits count them.

constexpr int kDqBufs = 4;          // KV blocks in LDS
constexpr int kDqMaxTopk = 3072;    // the row's index list in LDS

template <int D>
struct DqTile {
  static constexpr int kRow = padded_row(2 * D);   // padded LDS row of a KV row
  static constexpr int kKBytes = kBK * kRow;
  static constexpr int kLds = kDqBufs * kKBytes + kDqMaxTopk * 4;
  static constexpr int kDSteps = D / 32;           // 16x16x32 steps over d_qk
  static constexpr int kVSteps = kDV / 32;         // ... over d_v
  static constexpr int kTiles = D / 16;            // 16-column tiles of a KV row
  static constexpr int kCopies = (kBK / kWaves) * (D > kDV ? 2 : 1);  // per wave and block
  static_assert(kLds <= 160 * 1024, "LDS budget");
  static_assert(2 * kCopies < 64, "vmcnt range");
};

__device__ __attribute__((aligned(16))) const uint8_t g_zero_kv_row[2 * 576] = {};

template <int D, bool SINK>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
sparse_mla_bwd_dq_kernel(BwdArgs a) {
  using T = DqTile<D>;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[T::kLds];
  LDS_AS uint8_t* kbuf = (LDS_AS uint8_t*)lds_raw;                          // [4][32][kRow]
  LDS_AS int32_t* idx_l = (LDS_AS int32_t*)(kbuf + kDqBufs * T::kKBytes);  // the row's indices

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int hl = lane & 15;
  const int head = wave * 16 + hl;
  const int row = blockIdx.x;
  const size_t rh = (size_t)row * kHeads + head;

  // dO (B operand of dP^T) and the query slice (of S^T) in registers, for
  // this lane's head: columns 32 s + 8 g .. +7.
  const __bf16* dop = a.dout + rh * kDV + g * 8;
  const __bf16* op = a.out + rh * kDV + g * 8;
  bf16x8 dor[T::kVSteps];
  float delta = 0.f;
#pragma unroll
  for (int s = 0; s < T::kVSteps; ++s) {
    dor[s] = *reinterpret_cast<const bf16x8*>(dop + s * 32);
    const bf16x8 o8 = *reinterpret_cast<const bf16x8*>(op + s * 32);
#pragma unroll
    for (int e = 0; e < 8; ++e) delta += (float)dor[s][e] * (float)o8[e];
  }
  delta += __shfl_xor(delta, 16);
  delta += __shfl_xor(delta, 32);
  bf16x8 qr[T::kDSteps];
  {
    const __bf16* qp = a.q + rh * D + g * 8;
#pragma unroll
    for (int s = 0; s < T::kDSteps; ++s) qr[s] = *reinterpret_cast<const bf16x8*>(qp + s * 32);
  }

  float l2 = a.lse[rh] * a.lse_to_log2;
  float sk2 = 0.f;
  if (SINK) {
    sk2 = a.attn_sink[head] * kLog2e;
    if (!__builtin_isinf(l2)) {
      const float m = fmaxf(l2, sk2);
      l2 = m + __log2f(__builtin_amdgcn_exp2f(l2 - m) + __builtin_amdgcn_exp2f(sk2 - m));
    }
  }
  const float scale_log2 = a.scale * kLog2e;
  if (a.stats_out != nullptr && g == 0) {
    a.stats_out[(size_t)row * 2 * kHeads + head] = l2;
    a.stats_out[(size_t)row * 2 * kHeads + kHeads + head] = delta;
  }

  const int L = a.row_len[row];
  const int nblk = (L + kBK - 1) / kBK;
  {
    const int32_t* idx_row = a.indices + (size_t)row * a.topk;
    for (int p = tid; p < nblk * kBK; p += kWaves * 64) idx_l[p] = p < L ? idx_row[p] : -1;
  }
  f32x4 dqa[T::kTiles];
#pragma unroll
  for (int ct = 0; ct < T::kTiles; ++ct) dqa[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Every load above has landed: the loop has none the compiler would wait for.
  wait_vm<0>();
  __syncthreads();

  // Rows wave + 4 i of block kb into buffer kb % 4 (their indices read in
  // one LDS access, lane i holding row wave + 4 i's).
  auto gather = [&](int kb) {
    LDS_AS uint8_t* buf = kbuf + (kb % kDqBufs) * T::kKBytes;
    const int mine = idx_l[kb * kBK + wave + kWaves * (lane & (kBK / kWaves - 1))];
#pragma unroll
    for (int i = 0; i < kBK / kWaves; ++i) {
      const int j = wave + kWaves * i;
      const int e = __builtin_amdgcn_readlane(mine, i);
      const uint8_t* src = e >= 0 && e < a.s_kv
                               ? reinterpret_cast<const uint8_t*>(a.kv) + (size_t)(uint32_t)e * (2 * D)
                               : g_zero_kv_row;
      lds_dma16(src + lane * 16, buf + j * T::kRow);
      if (D > kDV && lane < (2 * D - 2 * kDV) / 16)
        lds_dma16(src + 2 * kDV + lane * 16, buf + j * T::kRow + 2 * kDV);
    }
  };
  for (int kb = 0; kb < nblk && kb < kDqBufs - 1; ++kb) gather(kb);

  for (int kb = 0; kb < nblk; ++kb) {
    // Block kb's copies are done once at most the later blocks' are pending.
    const int later = min(nblk - 1 - kb, kDqBufs - 2);
    if (later >= 2) wait_vm<2 * T::kCopies>();
    else if (later == 1) wait_vm<T::kCopies>();
    else wait_vm<0>();
    __syncthreads();  // ... in every wave; block kb - 1's readers are done
    if (kb + kDqBufs - 1 < nblk) gather(kb + kDqBufs - 1);
    const LDS_AS uint8_t* ks = kbuf + (kb % kDqBufs) * T::kKBytes;
    const int idx = lane < kBK ? idx_l[kb * kBK + lane] : -1;
    const uint64_t mask = __builtin_amdgcn_ballot_w64(idx >= 0 && idx < a.s_kv);

    // S^T and dP^T: lane (g, hl) holds keys 16 kt + 4g + r of head `head`;
    // the two key rows of a step are read kRowAhead steps ahead.
    f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    f32x4 dpt[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    {
      auto rd = [&](int s, int kt) {
        return *reinterpret_cast<const LDS_AS bf16x8*>(ks + (kt * 16 + hl) * T::kRow + s * 64 + g * 16);
      };
      bf16x8 buf[kRowAhead][2];
#pragma unroll
      for (int s = 0; s < kRowAhead; ++s) {
        buf[s][0] = rd(s, 0);
        buf[s][1] = rd(s, 1);
      }
#pragma unroll
      for (int s = 0; s < T::kDSteps; ++s) {
        const bf16x8 kf0 = buf[s % kRowAhead][0], kf1 = buf[s % kRowAhead][1];
        if (s + kRowAhead < T::kDSteps) {
          buf[s % kRowAhead][0] = rd(s + kRowAhead, 0);
          buf[s % kRowAhead][1] = rd(s + kRowAhead, 1);
        }
        st[0] = mfma(kf0, qr[s], st[0]);
        st[1] = mfma(kf1, qr[s], st[1]);
        if (s < T::kVSteps) {
          dpt[0] = mfma(kf0, dor[s], dpt[0]);
          dpt[1] = mfma(kf1, dor[s], dpt[1]);
        }
        __builtin_amdgcn_sched_barrier(0);  // keeps the read-ahead distance
      }
    }

    // dS (scaled by sm_scale); masked keys get 0.
    bf16x8 dsf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kt * 16 + 4 * g + r;
        const bool valid = (mask >> key) & 1ull;
        const float p = valid ? __builtin_amdgcn_exp2f(st[kt][r] * scale_log2 - l2) : 0.f;
        dsf[kt * 4 + r] = (__bf16)(a.scale * p * (dpt[kt][r] - delta));
      }

    // dQ^T += K^T dS^T: element e of both operands is key 16 (e / 4) + 4g + e % 4.
    {
      bf16x8 kt_op[kDqAhead];
#pragma unroll
      for (int ct = 0; ct < kDqAhead; ++ct) kt_op[ct] = tr_pair(ks, T::kRow, 0, ct * 16, g, hl);
#pragma unroll
      for (int ct = 0; ct < T::kTiles; ++ct) {
        const bf16x8 cur = kt_op[ct % kDqAhead];
        if (ct + kDqAhead < T::kTiles)
          kt_op[ct % kDqAhead] = tr_pair(ks, T::kRow, 0, (ct + kDqAhead) * 16, g, hl);
        dqa[ct] = mfma(cur, dsf, dqa[ct]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // dq[row][head][16 ct + 4g + r] = dqa[ct][r].
  __bf16* dqp = a.dq + rh * D + g * 4;
#pragma unroll
  for (int ct = 0; ct < T::kTiles; ++ct) {
    const bf16x4 v = {(__bf16)dqa[ct][0], (__bf16)dqa[ct][1], (__bf16)dqa[ct][2],
                      (__bf16)dqa[ct][3]};
    *reinterpret_cast<bf16x4*>(dqp + ct * 16) = v;
  }
  if (SINK && a.d_sink != nullptr && g == 0 && !__builtin_isinf(l2))
    unsafeAtomicAdd(a.d_sink + head, -__builtin_amdgcn_exp2f(sk2 - l2) * delta);
}

// ---------------------------------------------------------------------------
// Key-outer dkv pass
// ---------------------------------------------------------------------------
// When a call's selections are dense enough (the KV table is at most a few
// times the row width), dkv is summed per block of 64 KV rows instead of
// scattered per (row, key) pair: a workgroup owns one key block and a chunk
// of query rows, recomputes P and dS for every row of the chunk that names a
// key of the block (all 64 heads at once), and keeps the block's dK + dV in
// its accumulator registers; one atomic add per element of the block and
// chunk moves it to the fp32 accumulator.  A row that names one key twice is
// left to the row pass (its per-occurrence scatter), so the mask below can be
// a plain bitmap.

constexpr int kKoKeys = 64;       // keys per block
constexpr int kAhead = 4;         // LDS operand reads in flight per S / dP chain
constexpr int kKoMaxRows = 128;   // query rows per chunk, at most
constexpr int kKoMaxKv = 16384;   // widest KV table with a bitmap in LDS

// Row bitmap of the keys each row names (valid entries before its length),
// and whether the row names a key twice.  One workgroup per query row.
__global__ void __launch_bounds__(256) bwd_mask_kernel(const int32_t* indices, const int32_t* row_len,
                                                       int32_t topk, int32_t s_kv, int32_t nw,
                                                       uint32_t* bits, int32_t* dup) {
  __shared__ uint32_t words[kKoMaxKv / 32];
  __shared__ int any_dup;
  const int row = blockIdx.x;
  for (int w = threadIdx.x; w < nw; w += 256) words[w] = 0u;
  if (threadIdx.x == 0) any_dup = 0;
  __syncthreads();
  const int L = row_len[row];
  const int32_t* ir = indices + (size_t)row * topk;
  bool twice = false;
  for (int p = threadIdx.x; p < L; p += 256) {
    const int j = ir[p];
    if (j >= 0 && j < s_kv) {
      const uint32_t bit = 1u << (j & 31);
      twice |= (atomicOr(&words[j >> 5], bit) & bit) != 0u;
    }
  }
  if (twice) any_dup = 1;
  __syncthreads();
  uint32_t* out = bits + (size_t)row * nw;
  for (int w = threadIdx.x; w < nw; w += 256) out[w] = words[w];
  if (threadIdx.x == 0) dup[row] = any_dup;
}

struct DkvArgs {
  const __bf16* q;          // [s_q][64][D]
  const __bf16* kv;         // [s_kv][D]
  const __bf16* dout;       // [s_q][64][512]
  const uint32_t* bits;     // [s_q][nw]
  const int32_t* dup;       // [s_q]
  const float* stats;       // [s_q][128]: the row pass's normaliser in log2 units, then delta
  float* dkv_acc;           // [s_kv][D]
  int32_t s_q, s_kv, nw, n_kb, chunk_rows, n_chunks;
  float scale, scale_log2;
};

template <int D>
struct KoTile {
  static constexpr int kQRow = padded_row(2 * D);      // padded LDS row of a query head
  static constexpr int kDoRow = padded_row(2 * kDV);   // ... of a dout head
  static constexpr int kSRow = 2 * kKoKeys + 16;       // ... of dS / P (one head, 64 keys)
  static constexpr int kQBytes = kHeads * kQRow;
  static constexpr int kDoBytes = kHeads * kDoRow;
  static constexpr int kSBytes = kHeads * kSRow;
  static constexpr int kStatBytes = 2 * kHeads * 4;   // a row's normalisers and deltas
  static constexpr int kLds = kQBytes + kDoBytes + 2 * kSBytes + kStatBytes + kKoMaxRows * 12 + 16;
  static constexpr int kSteps = D / 16;                // 32x32x16 steps over d_qk
  static constexpr int kVSteps = kDV / 16;             // ... over d_v
  // A wave's dkv tiles, for both 32-key halves of the block: value tiles
  // 4w .. 4w + 3 and, at d576, waves 0 and 1 the rope tiles 16 and 17.
  static constexpr int kWaveCols = D > kDV ? 5 : 4;
  static constexpr int kQCopies = (kHeads / kWaves) * (D > kDV ? 2 : 1);  // per wave and row
  static_assert(kLds <= 160 * 1024, "LDS budget");
  static_assert(kQCopies < 64, "vmcnt range");
};

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// B operand of a 32x32x16 product read down the rows of an LDS tile: lane
// (half, j) receives rows r0 + 8 half + (0..7) of column c0 + j, by two
// ds_read_b64_tr_b16 over 4 x 16 sub-tiles.
__device__ __forceinline__ bf16x8 tr_col8(const LDS_AS uint8_t* tile, int row_bytes, int r0, int c0,
                                          int lane) {
  const int grp = lane >> 4, i = lane & 15;
  const LDS_AS uint8_t* p = tile + (r0 + 8 * (grp >> 1) + (i >> 2)) * row_bytes +
                            (c0 + 16 * (grp & 1) + 4 * (i & 3)) * 2;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(p + 4 * row_bytes));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}


// One workgroup per (row chunk, key block).  Wave w
// computes S^T and dP^T for keys 32 (w / 2) .. +31 and heads 32 (w % 2) ..
// +31 (its K fragments stay in registers for the whole chunk), and owns the
// dkv tiles of a quarter of the value columns (and at d576 half of the rope
// columns) for all 64 keys.
// Each row's query heads, dout heads and statistics reach LDS by DMA in two
// parts, so that each overlaps products of the row before:
//   top of row t: dout_t and stats_t in LDS, q_t in flight;
//   dP^T (dout_t); wait for q_t; S^T (q_t); P, dS to LDS;
//   dV += P^T dout_t; barrier; dout and stats of the next row in flight;
//   dK += dS^T q_t; barrier; the next row's q in flight; wait for its dout.
template <int D>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
sparse_mla_bwd_dkv_kernel(DkvArgs a) {
  using T = KoTile<D>;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[T::kLds];
  LDS_AS uint8_t* qs = (LDS_AS uint8_t*)lds_raw;     // query heads [64][kQRow]
  LDS_AS uint8_t* dos = qs + T::kQBytes;              // dout heads [64][kDoRow]
  LDS_AS uint8_t* dss = dos + T::kDoBytes;            // dS [64 heads][kSRow]
  LDS_AS uint8_t* pss = dss + T::kSBytes;             // P  [64 heads][kSRow]
  LDS_AS uint8_t* sts = pss + T::kSBytes;             // l2[64], delta[64] of the row
  LDS_AS uint64_t* rsel = (LDS_AS uint64_t*)(sts + T::kStatBytes);  // their key masks
  LDS_AS int32_t* rlist = (LDS_AS int32_t*)(rsel + kKoMaxRows);      // rows of the chunk
  LDS_AS int32_t* wcnt = rlist + kKoMaxRows;          // per-wave row counts

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j32 = lane & 31, half = lane >> 5;
  // Workgroup i runs on XCD i % 8 (round-robin dispatch).  Chunks, heaviest
  // (last) first, are dealt to the XCDs in snake order, and each XCD walks
  // the key blocks of its chunks in turn: the workgroups that read one row's
  // q and dout at about the same time share an L2.
  const int xcd = (int)(blockIdx.x % 8u), k = (int)(blockIdx.x / 8u);
  const int round = k / a.n_kb, kb = k % a.n_kb;
  const int j = 8 * round + ((round & 1) ? 7 - xcd : xcd);
  if (j >= a.n_chunks) return;
  const int chunk = a.n_chunks - 1 - j;
  const int r0 = chunk * a.chunk_rows;
  const int key0 = kb * kKoKeys;
  const int w0 = 2 * kb;

  // The chunk's rows that name a key of the block, in order, with their
  // masks of the block's keys.
  {
    const int t = r0 + tid;
    uint64_t sel = 0;
    if (tid < a.chunk_rows && t < a.s_q && a.dup[t] == 0) {
      const uint32_t* b = a.bits + (size_t)t * a.nw;
      sel = (uint64_t)b[w0] | ((uint64_t)(w0 + 1 < a.nw ? b[w0 + 1] : 0u) << 32);
    }
    const bool present = sel != 0;
    const uint64_t m = __builtin_amdgcn_ballot_w64(present);
    if (lane == 0) wcnt[wave] = __builtin_popcountll(m);
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wcnt[w];
    if (present) {
      const int at = base + __builtin_popcountll(m & ((1ull << lane) - 1ull));
      rlist[at] = t;
      rsel[at] = sel;
    }
    __syncthreads();
  }
  const int n_rows = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
  if (n_rows == 0) return;

  // DMA of a row's parts: this wave's 16 heads of dout (and wave 0: the
  // statistics), then of q.
  // (copy i of 16 per wave: head wave + 4 i; the statistics with copy 15).
  auto issue_dout_one = [&](int t, int i) {
    const int h = wave + kWaves * i;
    const uint8_t* src = reinterpret_cast<const uint8_t*>(a.dout + (size_t)t * kHeads * kDV);
    lds_dma16(src + h * 2 * kDV + lane * 16, dos + h * T::kDoRow);
    if (i == kHeads / kWaves - 1 && wave == 0 && lane < T::kStatBytes / 16)
      lds_dma16(reinterpret_cast<const uint8_t*>(a.stats + (size_t)t * 2 * kHeads) + lane * 16, sts);
  };
  auto issue_dout = [&](int t) {
#pragma unroll
    for (int i = 0; i < kHeads / kWaves; ++i) issue_dout_one(t, i);
  };
  auto issue_q = [&](int t) {
    const uint8_t* src = reinterpret_cast<const uint8_t*>(a.q + (size_t)t * kHeads * D);
#pragma unroll
    for (int i = 0; i < kHeads / kWaves; ++i) {
      const int h = wave + kWaves * i;
      lds_dma16(src + h * 2 * D + lane * 16, qs + h * T::kQRow);
      if (D > kDV && lane < (2 * D - 2 * kDV) / 16)
        lds_dma16(src + h * 2 * D + 2 * kDV + lane * 16, qs + h * T::kQRow + 2 * kDV);
    }
  };

  const int kh = wave >> 1, hh = wave & 1;
  // K fragments (A operand of S^T and, over the first d_v columns, of dP^T):
  // key 32 kh + j32, columns 16 s + 8 half .. +7.  A key past the table reads
  // row 0 instead: no row names it, so its P and dS are set to 0.
  bf16x8 kf[T::kSteps];
  {
    const int key = key0 + 32 * kh + j32;
    const __bf16* kp = a.kv + (size_t)(key < a.s_kv ? key : 0) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < T::kSteps; ++s) kf[s] = *reinterpret_cast<const bf16x8*>(kp + 16 * s);
  }
  // The wave's dkv column tiles (both key halves): value tiles 4w .. 4w + 3,
  // then at d576 the rope tile 16 + w for waves 0 and 1 (`has_rope`).
  auto tile_col = [&](int c) { return c < 4 ? 4 * wave + c : kDV / 32 + (wave & 1); };
  const bool has_rope = D > kDV && wave < 2;
  f32x16 acc[2][T::kWaveCols];
#pragma unroll
  for (int c = 0; c < T::kWaveCols; ++c) acc[0][c] = acc[1][c] = f32x16{};

  const int head = 32 * hh + j32;
  int t = __builtin_amdgcn_readfirstlane(rlist[0]);
  issue_dout(t);
  issue_q(t);
  // Everything, the K fragments included: the loop then has no load the
  // compiler would wait for.
  wait_vm<0>();
  __syncthreads();
  for (int v = 0; v < n_rows; ++v) {
    const uint64_t sel = rsel[v];
    const float l2 = *reinterpret_cast<const LDS_AS float*>(sts + 4 * head);
    const float dl = *reinterpret_cast<const LDS_AS float*>(sts + 4 * (kHeads + head));

    // dP^T, then S^T: element i is key 32 kh + 8 (i / 4) + 4 half + i % 4 of
    // the block, head `head`.
    f32x16 dpt = f32x16{}, st = f32x16{};
    const LDS_AS uint8_t* drow = dos + head * T::kDoRow + 16 * half;
    // The B operands are read kAhead steps ahead of their products.
    {
      bf16x8 bq[kAhead];
#pragma unroll
      for (int s = 0; s < kAhead; ++s) bq[s] = *reinterpret_cast<const LDS_AS bf16x8*>(drow + 32 * s);
#pragma unroll
      for (int s = 0; s < T::kVSteps; ++s) {
        const bf16x8 cur = bq[s % kAhead];
        if (s + kAhead < T::kVSteps)
          bq[s % kAhead] = *reinterpret_cast<const LDS_AS bf16x8*>(drow + 32 * (s + kAhead));
        dpt = mfma32(kf[s], cur, dpt);
        __builtin_amdgcn_sched_barrier(0);  // keeps the read-ahead distance
      }
    }
    wait_vm<0>();  // this wave's q copies
    __syncthreads();
    const LDS_AS uint8_t* qrow = qs + head * T::kQRow + 16 * half;
    {
      bf16x8 bq[kAhead];
#pragma unroll
      for (int s = 0; s < kAhead; ++s) bq[s] = *reinterpret_cast<const LDS_AS bf16x8*>(qrow + 32 * s);
#pragma unroll
      for (int s = 0; s < T::kSteps; ++s) {
        const bf16x8 cur = bq[s % kAhead];
        if (s + kAhead < T::kSteps)
          bq[s % kAhead] = *reinterpret_cast<const LDS_AS bf16x8*>(qrow + 32 * (s + kAhead));
        st = mfma32(kf[s], cur, st);
        __builtin_amdgcn_sched_barrier(0);  // keeps the read-ahead distance
      }
    }
    // dS and P go to LDS as [head][key]: the lane's four consecutive keys
    // 32 kh + 8 g + 4 half .. +3 in one 8-byte store.
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 d4, p4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * g + r;
        const int key = 32 * kh + 8 * g + 4 * half + r;
        const bool on = (sel >> key) & 1ull;
        const float p = on ? __builtin_amdgcn_exp2f(st[i] * a.scale_log2 - l2) : 0.f;
        const float ds = on ? a.scale * p * (dpt[i] - dl) : 0.f;
        d4[r] = (__bf16)ds;
        p4[r] = (__bf16)p;
      }
      const int off = head * T::kSRow + (32 * kh + 8 * g + 4 * half) * 2;
      *reinterpret_cast<LDS_AS bf16x4*>(dss + off) = d4;
      *reinterpret_cast<LDS_AS bf16x4*>(pss + off) = p4;
    }
    __syncthreads();  // dS and P of the block are in LDS

    // dkv[32 keys x 32 columns] += P^T dO on the value columns, then dS^T Q,
    // contracted over the 64 heads in four steps of 16, for both key halves:
    // each B operand (read kAhead reads ahead) serves two products.  Read n
    // of a phase is head step n / C and tile n % C.
    bf16x8 af[2][4], pf[2][4];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int hs = 0; hs < 4; ++hs) {
        af[k2][hs] = tr_col8(dss, T::kSRow, 16 * hs, 32 * k2, lane);
        pf[k2][hs] = tr_col8(pss, T::kSRow, 16 * hs, 32 * k2, lane);
      }
    {
      constexpr int C = 4, N = 4 * C;
      auto bop = [&](int n) { return tr_col8(dos, T::kDoRow, 16 * (n / C), 32 * tile_col(n % C), lane); };
      bf16x8 bq[kAhead];
#pragma unroll
      for (int n = 0; n < kAhead; ++n) bq[n] = bop(n);
#pragma unroll
      for (int n = 0; n < N; ++n) {
        const bf16x8 cur = bq[n % kAhead];
        if (n + kAhead < N) bq[n % kAhead] = bop(n + kAhead);
        acc[0][n % C] = mfma32(pf[0][n / C], cur, acc[0][n % C]);
        acc[1][n % C] = mfma32(pf[1][n / C], cur, acc[1][n % C]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const bool more = v + 1 < n_rows;
    const int tn = more ? __builtin_amdgcn_readfirstlane(rlist[v + 1]) : t;
    __syncthreads();  // dout and stats are free
    {
      // The next row's dout copies go out one per B read, under the MFMAs.
      constexpr int C = T::kWaveCols, N = 4 * C;
      static_assert(N >= kHeads / kWaves, "one copy per read");
      auto bop = [&](int n) { return tr_col8(qs, T::kQRow, 16 * (n / C), 32 * tile_col(n % C), lane); };
      bf16x8 bq[kAhead];
#pragma unroll
      for (int n = 0; n < kAhead; ++n) bq[n] = bop(n);
#pragma unroll
      for (int n = 0; n < N; ++n) {
        const bf16x8 cur = bq[n % kAhead];
        if (n + kAhead < N) bq[n % kAhead] = bop(n + kAhead);
        if (n % C < 4 || has_rope) {
          acc[0][n % C] = mfma32(af[0][n / C], cur, acc[0][n % C]);
          acc[1][n % C] = mfma32(af[1][n / C], cur, acc[1][n % C]);
        }
        if (n < kHeads / kWaves && more) issue_dout_one(tn, n);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();  // q, dS^T and P^T are free
    if (more) {
      issue_q(tn);
      wait_vm<T::kQCopies>();  // the next row's dout and stats
      __syncthreads();
    }
    t = tn;
  }

  // acc[k2][c][i] is dkv[key0 + 32 k2 + 8 (i / 4) + 4 half + i % 4][32 tile_col(c) + j32].
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key0 + 32 * k2 + 8 * (i >> 2) + 4 * half + (i & 3);
      if (key < a.s_kv) {
        float* drow = a.dkv_acc + (size_t)key * D + j32;
#pragma unroll
        for (int c = 0; c < T::kWaveCols; ++c)
          if (c < 4 || has_rope) unsafeAtomicAdd(drow + 32 * tile_col(c), acc[k2][c][i]);
      }
    }
}

// Zero fill (also the fp32 accumulators before a launch).
__global__ void __launch_bounds__(256) bwd_zero_kernel(float* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = 0.f;
}

// dkv = bf16(dkv_acc), four values per thread step.
__global__ void __launch_bounds__(256) bwd_convert_kernel(const float* acc, __bf16* dkv, size_t n4) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const f32x4 v = reinterpret_cast<const f32x4*>(acc)[i];
    reinterpret_cast<bf16x4*>(dkv)[i] = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  }
}

// host side

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

smla_status bwd_fail(smla_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
smla_status bwd_fail(smla_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return smla_report(s, buf);
}

smla_status launched() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return bwd_fail(SMLA_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
  return SMLA_OK;
}

int grid_for(size_t n) {
  const size_t g = (n + 255) / 256;
  return (int)(g < 4096 ? (g > 0 ? g : 1) : 4096);
}

// Shapes whose key-outer buffers the workspace holds: the row bitmaps fit
// LDS and stay under 32 MB.
bool key_outer_eligible(int32_t s_q, int32_t s_kv) {
  return s_kv > 0 && s_kv <= kKoMaxKv && (size_t)s_q * (size_t)s_kv <= ((size_t)1 << 28);
}

// The key-outer pass runs where the KV table is at most 4 row widths.  It
// visits every (row, 64-key block) pair with a named key.  Measured on the
// T = 4096 shape: a visit takes about 24 ns of the device, a pair's scatter
// 1.8 ns, and the row pass without the scatter 0.36 ns per pair; with keys
// drawn uniformly that breaks even near 3.8 row widths, and local selections
// (causal rows visit only the blocks below them) favour the key-outer pass
// further out.
constexpr int kKoWidths = 4;
constexpr int kKoChunk = 128;  // query rows per key-outer workgroup

struct BwdWorkspace {
  float* acc;        // [s_kv][d_qk] fp32 dkv accumulator
  int32_t* row_len;  // [s_q]
  float* stats;      // [s_q][128] (key-outer shapes)
  int32_t* dup;      // [s_q]
  uint32_t* bits;    // [s_q][nw]
  int32_t nw;
  size_t bytes;
};

BwdWorkspace workspace_layout(void* base, int32_t s_q, int32_t s_kv, int32_t d_qk) {
  BwdWorkspace w{};
  uint8_t* p = static_cast<uint8_t*>(base);
  size_t off = 0;
  auto take = [&](size_t n) {
    uint8_t* at = p ? p + off : nullptr;
    off += align_up(n);
    return at;
  };
  w.acc = reinterpret_cast<float*>(take((size_t)s_kv * (size_t)d_qk * sizeof(float)));
  w.row_len = reinterpret_cast<int32_t*>(take((size_t)s_q * sizeof(int32_t)));
  if (key_outer_eligible(s_q, s_kv)) {
    w.nw = (s_kv + 31) / 32;
    w.stats = reinterpret_cast<float*>(take((size_t)s_q * 2 * kHeads * sizeof(float)));
    w.dup = reinterpret_cast<int32_t*>(take((size_t)s_q * sizeof(int32_t)));
    w.bits = reinterpret_cast<uint32_t*>(take((size_t)s_q * w.nw * sizeof(uint32_t)));
  }
  w.bytes = off;
  return w;
}

}  // namespace

extern "C" size_t sparse_mla_bwd_workspace_bytes(int32_t s_q, int32_t s_kv, int32_t d_qk) {
  if (s_q < 0 || s_kv < 0 || d_qk <= 0) return 0;
  return workspace_layout(nullptr, s_q, s_kv, d_qk).bytes;
}

extern "C" smla_status sparse_mla_bwd(const void* q, const void* kv, const void* out,
                                      const void* dout, const int32_t* indices,
                                      const int32_t* topk_length, const float* lse,
                                      const float* attn_sink, int32_t s_q, int32_t s_kv,
                                      int32_t h_q, int32_t h_kv, int32_t d_qk, int32_t d_v,
                                      int32_t topk, float sm_scale, int32_t lse_base2,
                                      void* workspace, size_t workspace_bytes, void* dq, void* dkv,
                                      float* d_sink, smla_stream_t stream) {
  smla_clear_error();
  smla_set_last_kernel("");
  if (s_q < 0 || s_kv < 0 || topk <= 0)
    return bwd_fail(SMLA_ERR_BAD_SHAPE, "bad sizes (s_q=%d s_kv=%d topk=%d)", s_q, s_kv, topk);
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale))
    return bwd_fail(SMLA_ERR_UNSUPPORTED, "sm_scale=%g (must be positive and finite)", (double)sm_scale);
  if (h_q != kHeads) return bwd_fail(SMLA_ERR_UNSUPPORTED, "h_q=%d (supported: 64)", h_q);
  if (h_kv != 1) return bwd_fail(SMLA_ERR_UNSUPPORTED, "h_kv=%d (only 1 is supported)", h_kv);
  if (d_qk != 512 && d_qk != 576)
    return bwd_fail(SMLA_ERR_UNSUPPORTED, "d_qk=%d (supported: 512, 576)", d_qk);
  if (d_v != kDV) return bwd_fail(SMLA_ERR_UNSUPPORTED, "d_v=%d (supported: 512)", d_v);
  if (lse_base2 != 0 && lse_base2 != 1)
    return bwd_fail(SMLA_ERR_BAD_SHAPE, "lse_base2=%d (0 or 1)", lse_base2);
  if (d_sink != nullptr && attn_sink == nullptr)
    return bwd_fail(SMLA_ERR_NULL_ARG, "d_sink needs attn_sink");
  const size_t need = sparse_mla_bwd_workspace_bytes(s_q, s_kv, d_qk);
  if (need > 0 && workspace == nullptr)
    return bwd_fail(SMLA_ERR_NULL_ARG, "workspace of %zu bytes needed (got null)", need);
  if (workspace_bytes < need)
    return bwd_fail(SMLA_ERR_BAD_SHAPE, "workspace of %zu bytes needed (got %zu)", need,
                    workspace_bytes);
  if (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0)
    return bwd_fail(SMLA_ERR_BAD_SHAPE, "workspace must be 16-byte aligned");
  if ((s_kv > 0 && (!kv || !dkv)) || (s_q > 0 && (!q || !out || !dout || !indices || !lse || !dq)))
    return bwd_fail(SMLA_ERR_NULL_ARG,
                    "sparse_mla_bwd: q, out, dout, indices, lse, dq (s_q > 0) and kv, dkv "
                    "(s_kv > 0) are required");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const BwdWorkspace ws = workspace_layout(workspace, s_q, s_kv, d_qk);
  float* acc = ws.acc;
  int32_t* row_len = ws.row_len;
  const bool key_outer = s_q > 0 && key_outer_eligible(s_q, s_kv) &&
                         (size_t)s_kv <= (size_t)kKoWidths * (size_t)topk;
  const size_t n_acc = (size_t)s_kv * d_qk;
  if (n_acc > 0) {
    hipLaunchKernelGGL(bwd_zero_kernel, dim3(grid_for(n_acc)), dim3(256), 0, st, acc, n_acc);
    if (smla_status e = launched()) return e;
  }
  if (d_sink != nullptr) {
    hipLaunchKernelGGL(bwd_zero_kernel, dim3(1), dim3(256), 0, st, d_sink, (size_t)kHeads);
    if (smla_status e = launched()) return e;
  }
  if (s_q > 0) {
    if (smla_status e = sparse_mla_row_lengths(indices, topk_length, nullptr, s_q, 1, topk, s_kv, 0,
                                               row_len, stream))
      return e;
    if (key_outer) {
      hipLaunchKernelGGL(bwd_mask_kernel, dim3(s_q), dim3(256), 0, st, indices, row_len, topk, s_kv,
                         ws.nw, ws.bits, ws.dup);
      if (smla_status e = launched()) return e;
    }
    BwdArgs args{};
    args.q = static_cast<const __bf16*>(q);
    args.kv = static_cast<const __bf16*>(kv);
    args.out = static_cast<const __bf16*>(out);
    args.dout = static_cast<const __bf16*>(dout);
    args.indices = indices;
    args.row_len = row_len;
    args.lse = lse;
    args.attn_sink = attn_sink;
    args.dq = static_cast<__bf16*>(dq);
    args.dkv_acc = acc;
    args.d_sink = d_sink;
    args.s_q = s_q;
    args.s_kv = s_kv;
    args.topk = topk;
    args.scale = sm_scale;
    args.lse_to_log2 = lse_base2 ? 1.f : kLog2e;
    if (key_outer) {
      args.stats_out = ws.stats;
      args.dup = ws.dup;
      args.key_outer = 1;
    }
    const bool sink = attn_sink != nullptr;
    auto row_pass = [&](const BwdArgs& ra) {
      if (d_qk == 576) {
        if (sink)
          hipLaunchKernelGGL((sparse_mla_bwd_kernel<576, true>), dim3(s_q), dim3(256), 0, st, ra);
        else
          hipLaunchKernelGGL((sparse_mla_bwd_kernel<576, false>), dim3(s_q), dim3(256), 0, st, ra);
      } else {
        if (sink)
          hipLaunchKernelGGL((sparse_mla_bwd_kernel<512, true>), dim3(s_q), dim3(256), 0, st, ra);
        else
          hipLaunchKernelGGL((sparse_mla_bwd_kernel<512, false>), dim3(s_q), dim3(256), 0, st, ra);
      }
      return launched();
    };
    if (key_outer && topk <= kDqMaxTopk) {
      // dq, d_sink and the statistics for every row, then the rows that name
      // a key twice again through the row pass, for their scatter.
      if (d_qk == 576) {
        if (sink)
          hipLaunchKernelGGL((sparse_mla_bwd_dq_kernel<576, true>), dim3(s_q), dim3(256), 0, st, args);
        else
          hipLaunchKernelGGL((sparse_mla_bwd_dq_kernel<576, false>), dim3(s_q), dim3(256), 0, st, args);
      } else {
        if (sink)
          hipLaunchKernelGGL((sparse_mla_bwd_dq_kernel<512, true>), dim3(s_q), dim3(256), 0, st, args);
        else
          hipLaunchKernelGGL((sparse_mla_bwd_dq_kernel<512, false>), dim3(s_q), dim3(256), 0, st, args);
      }
      if (smla_status e = launched()) return e;
      BwdArgs dup_args = args;
      dup_args.stats_out = nullptr;
      dup_args.dup_only = 1;
      if (smla_status e = row_pass(dup_args)) return e;
    } else {
      if (smla_status e = row_pass(args)) return e;
    }
    if (key_outer) {
      DkvArgs k{};
      k.q = args.q;
      k.kv = args.kv;
      k.dout = args.dout;
      k.bits = ws.bits;
      k.dup = ws.dup;
      k.stats = ws.stats;
      k.dkv_acc = acc;
      k.s_q = s_q;
      k.s_kv = s_kv;
      k.nw = ws.nw;
      k.n_kb = (s_kv + kKoKeys - 1) / kKoKeys;
      // At least 8 chunks, one per XCD, where the rows allow.
      k.chunk_rows = std::min(kKoChunk, std::max(1, (s_q + 7) / 8));
      k.n_chunks = (s_q + k.chunk_rows - 1) / k.chunk_rows;
      k.scale = sm_scale;
      k.scale_log2 = sm_scale * kLog2e;
      const dim3 grid((unsigned)(8 * k.n_kb * ((k.n_chunks + 7) / 8)));
      if (d_qk == 576)
        hipLaunchKernelGGL((sparse_mla_bwd_dkv_kernel<576>), grid, dim3(256), 0, st, k);
      else
        hipLaunchKernelGGL((sparse_mla_bwd_dkv_kernel<512>), grid, dim3(256), 0, st, k);
      if (smla_status e = launched()) return e;
    }
  }
  if (n_acc > 0) {
    hipLaunchKernelGGL(bwd_convert_kernel, dim3(grid_for(n_acc / 4)), dim3(256), 0, st, acc,
                       static_cast<__bf16*>(dkv), n_acc / 4);
    if (smla_status e = launched()) return e;
  }
  // After the row-length entry point, which resets the name.
  smla_set_last_kernel(s_q == 0 ? "" : key_outer ? "bwd_key_outer" : "bwd_scatter");
  return SMLA_OK;
}
