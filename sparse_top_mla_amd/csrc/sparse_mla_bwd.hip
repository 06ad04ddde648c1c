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
// Layout of work: one workgroup per query row, four waves, 16 heads per wave
// (h_q = 64, the shape the pages give for this operation).  Per block of 32
// keys:
//   gather the KV rows into LDS (masked rows as zeros);
//   S^T = K Q^T and dP^T = V dO^T on v_mfma_f32_16x16x32_bf16 (each lane owns
//   one head, so lse' and delta are per-lane scalars);
//   P and dS in registers; dS^T and P^T also go to LDS as bf16;
//   dKV[32 keys x d_qk] = dS^T Q (+ P^T dO on the value columns), the d_qk
//   columns split over the four waves, contracted over all 64 heads, then
//   added to the fp32 accumulator with global_atomic_add_f32;
//   dQ^T += K^T dS^T with K^T read by ds_read_b64_tr_b16 and dS^T taken from
//   the registers (the key order of both operands is permuted alike).
// The atomic adds bound the kernel: one fp32 add per valid (row, key) pair
// and d_qk column.
// The query rows stay in LDS for the whole row; dO stays in registers (its
// B-operand fragments for both products).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "sparse_mla.h"

// Error reporting shared with the forward's host code (same library).
__attribute__((visibility("hidden"))) smla_status smla_report(smla_status s, const char* msg);
__attribute__((visibility("hidden"))) void smla_clear_error();

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kHeads = 64;       // h_q
constexpr int kWaves = 4;        // 16 heads each
constexpr int kDV = 512;         // value width
constexpr int kBK = 32;          // keys per block
constexpr float kLog2e = 1.4426950408889634f;

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
  int32_t s_q, s_kv, topk;
  float scale;              // sm_scale
  float lse_to_log2;        // log2(e) for natural-log lse, 1 for base-2 lse
};

template <int D>
struct BwdTile {
  static constexpr int kRow = 2 * D + 16;          // padded LDS row (query head or KV row)
  static constexpr int kQBytes = kHeads * kRow;
  static constexpr int kKBytes = kBK * kRow;
  static constexpr int kSRow = 2 * kHeads + 16;    // padded LDS row of dS^T / P^T (one key)
  static constexpr int kSBytes = kBK * kSRow;
  static constexpr int kLds = kQBytes + kKBytes + 2 * kSBytes;
  static constexpr int kDSteps = D / 32;           // MFMA K steps over d_qk
  static constexpr int kVSteps = kDV / 32;         // ... over d_v
  static constexpr int kTiles = D / 16;            // 16-column tiles of a KV row
  static constexpr int kWaveTiles = kTiles / kWaves;  // dKV column tiles per wave
  static constexpr int kDoRow = 2 * kDV + 16;      // padded LDS row of the staged dO
  static_assert(kHeads * kDoRow <= kQBytes + kKBytes, "dO staging fits");
  static_assert(kTiles % kWaves == 0, "column split");
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

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
  LDS_AS uint8_t* ks = qs + T::kQBytes;                // KV block [32][kRow]
  LDS_AS uint8_t* dst = ks + T::kKBytes;               // dS^T [32 keys][kSRow]
  LDS_AS uint8_t* pst = dst + T::kSBytes;              // P^T  [32 keys][kSRow]

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int hl = lane & 15;
  const int head = wave * 16 + hl;
  const int row = blockIdx.x;
  const size_t rh = (size_t)row * kHeads + head;

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
  // read transposed from a staged copy of the row's dO.
  {
    const __bf16* drow = a.dout + (size_t)row * kHeads * kDV;
    for (int c = tid; c < kHeads * (kDV / 8); c += kWaves * 64) {
      const int h = c / (kDV / 8), ch = c % (kDV / 8);
      *reinterpret_cast<LDS_AS u32x4*>(qs + h * T::kDoRow + ch * 16) =
          *reinterpret_cast<const u32x4*>(drow + h * kDV + ch * 8);
    }
  }
  __syncthreads();
  bf16x8 dov[2][T::kWaveTiles];
  const int ct0 = wave * T::kWaveTiles;
#pragma unroll
  for (int hs = 0; hs < 2; ++hs)
#pragma unroll
    for (int c = 0; c < T::kWaveTiles; ++c) {
      const int ct = ct0 + c < kDV / 16 ? ct0 + c : 0;  // unused past the value columns
      dov[hs][c] = tr_pair(qs, T::kDoRow, 32 * hs, ct * 16, g, hl);
    }
  __syncthreads();

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

  f32x4 dqa[T::kTiles];
#pragma unroll
  for (int ct = 0; ct < T::kTiles; ++ct) dqa[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int L = a.row_len[row];
  const int32_t* idx_row = a.indices + (size_t)row * a.topk;
  const int nblk = (L + kBK - 1) / kBK;
  for (int kb = 0; kb < nblk; ++kb) {
    const int pos = kb * kBK + lane;
    const int idx = (lane < kBK && pos < L) ? idx_row[pos] : -1;
    const bool ok = idx >= 0 && idx < a.s_kv;
    const uint64_t mask = __builtin_amdgcn_ballot_w64(ok);
    if (mask == 0) continue;  // the same in every wave

    __syncthreads();  // the previous block's readers of ks / dst / pst are done
    for (int j = wave; j < kBK; j += kWaves) {
      LDS_AS uint8_t* d = ks + j * T::kRow;
      if ((mask >> j) & 1ull) {
        const uint8_t* src = reinterpret_cast<const uint8_t*>(a.kv) +
                             (size_t)(uint32_t)__builtin_amdgcn_readlane(idx, j) * (2 * D);
        __builtin_amdgcn_global_load_lds((const void*)(src + lane * 16), (LDS_AS void*)d, 16, 0, 0);
        if (D > kDV && lane < (2 * D - 2 * kDV) / 16)
          __builtin_amdgcn_global_load_lds((const void*)(src + 2 * kDV + lane * 16),
                                           (LDS_AS void*)(d + 2 * kDV), 16, 0, 0);
      } else {
        *reinterpret_cast<LDS_AS u32x4*>(d + lane * 16) = u32x4{0u, 0u, 0u, 0u};
        if (D > kDV && lane < (2 * D - 2 * kDV) / 16)
          *reinterpret_cast<LDS_AS u32x4*>(d + 2 * kDV + lane * 16) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    wait_vm_all();
    __syncthreads();

    // S^T and dP^T: lane (g, hl) holds keys 16 kt + 4g + r of head `head`.
    f32x4 st[2], dpt[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      st[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dpt[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < T::kDSteps; ++s) {
      const bf16x8 qf = *reinterpret_cast<const LDS_AS bf16x8*>(qs + head * T::kRow + s * 64 + g * 16);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 kf =
            *reinterpret_cast<const LDS_AS bf16x8*>(ks + (kt * 16 + hl) * T::kRow + s * 64 + g * 16);
        st[kt] = mfma(kf, qf, st[kt]);
        if (s < T::kVSteps) dpt[kt] = mfma(kf, dor[s], dpt[kt]);
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
        *reinterpret_cast<LDS_AS __bf16*>(dst + key * T::kSRow + head * 2) = (__bf16)ds;
        *reinterpret_cast<LDS_AS __bf16*>(pst + key * T::kSRow + head * 2) = (__bf16)p;
      }

    __syncthreads();  // dS^T and P^T of every wave are in LDS

    // dKV of this wave's columns: element e of both operands is head
    // 32 hs + 16 (e / 4) + 4g + e % 4.
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
#pragma unroll
    for (int ct = 0; ct < T::kTiles; ++ct)
      dqa[ct] = mfma(tr_pair(ks, T::kRow, 0, ct * 16, g, hl), dsf, dqa[ct]);
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

}  // namespace

extern "C" size_t sparse_mla_bwd_workspace_bytes(int32_t s_q, int32_t s_kv, int32_t d_qk) {
  if (s_q < 0 || s_kv < 0 || d_qk <= 0) return 0;
  return align_up((size_t)s_kv * (size_t)d_qk * sizeof(float)) + align_up((size_t)s_q * sizeof(int32_t));
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
  float* acc = static_cast<float*>(workspace);
  int32_t* row_len = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) +
                                                align_up((size_t)s_kv * d_qk * sizeof(float)));
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
    const bool sink = attn_sink != nullptr;
    if (d_qk == 576) {
      if (sink)
        hipLaunchKernelGGL((sparse_mla_bwd_kernel<576, true>), dim3(s_q), dim3(256), 0, st, args);
      else
        hipLaunchKernelGGL((sparse_mla_bwd_kernel<576, false>), dim3(s_q), dim3(256), 0, st, args);
    } else {
      if (sink)
        hipLaunchKernelGGL((sparse_mla_bwd_kernel<512, true>), dim3(s_q), dim3(256), 0, st, args);
      else
        hipLaunchKernelGGL((sparse_mla_bwd_kernel<512, false>), dim3(s_q), dim3(256), 0, st, args);
    }
    if (smla_status e = launched()) return e;
  }
  if (n_acc > 0) {
    hipLaunchKernelGGL(bwd_convert_kernel, dim3(grid_for(n_acc / 4)), dim3(256), 0, st, acc,
                       static_cast<__bf16*>(dkv), n_acc / 4);
    if (smla_status e = launched()) return e;
  }
  return SMLA_OK;
}
