// Attainable-peak probe for the benchmark (not part of the attention path).
//
// smla_probe_mfma runs back-to-back v_mfma_f32_32x32x16_bf16 on every SIMD:
// each wave keeps four independent accumulator chains, two waves per SIMD,
// so the matrix cores never wait on a result.  The host divides the FLOPs
// (2 * 32 * 32 * 16 per MFMA) by the measured time to get the dense bf16
// MFMA rate this device attains at its running clock.
//
// smla_probe_stream_read reads a buffer once (16 B per lane, four loads in
// flight per lane, grid-stride) and writes one word per thread: the HBM rate
// a read-dominated kernel can attain (the decode gathers are about 95%
// reads), beside the read+write rate of a device copy.
//
// smla_probe_atomic_add adds 1.0 to fp32 words of a [rows][576] accumulator
// with global_atomic_add_f32 (no return), in the backward's scatter pattern:
// per wave instruction, four hashed rows x 16 consecutive words, nine
// instructions per row group covering a wave's quarter of the 576 columns.
// The host divides the adds by the time: the fp32 atomic-add rate this device
// sustains, the floor of a kernel whose reduction is an atomic scatter.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;

__global__ void __launch_bounds__(512) mfma_loop(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
    b[e] = (__bf16)(0.002f * (float)((lane * 3 + e) & 7));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) acc[k] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kChains; ++k)
      acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) stream_read(const u32x4* __restrict__ p, size_t n16,
                                                   uint32_t* __restrict__ out) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= p[i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

constexpr int kAtomCols = 576;

__global__ void __launch_bounds__(256) atomic_scatter(float* acc, uint32_t rows, int iters) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, hl = lane & 15;
  const uint32_t seed = blockIdx.x * 977u + wave * 131u + 13u;
  for (int it = 0; it < iters; ++it) {
    const uint32_t row = mix32(seed + 4u * it + g) % rows;
    float* p = acc + (size_t)row * kAtomCols + wave * (kAtomCols / 4) + hl;
#pragma unroll
    for (int c = 0; c < kAtomCols / 64; ++c)
      __hip_atomic_fetch_add(p + 16 * c, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

extern "C" {

// Atomic scatter into `acc` ([rows][576] fp32, rows > 0) with `blocks`
// workgroups of 256 threads, each thread issuing iters * 9 adds of 1.0.
// Returns 0 or the HIP error code of the launch.
int smla_probe_atomic_add(float* acc, int rows, int blocks, int iters, void* stream) {
  if (!acc || rows <= 0 || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(atomic_scatter, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), acc, (uint32_t)rows, iters);
  return (int)hipGetLastError();
}

// fp32 adds one atomic-probe launch issues.
long long smla_probe_atomic_count(int blocks, int iters) {
  return (long long)blocks * 256 * iters * (kAtomCols / 64);
}

// Reads `bytes` (a multiple of 16) from `src` with `blocks` workgroups of 256
// threads; `out` holds blocks * 256 words.  Returns 0 or the HIP error code.
int smla_probe_stream_read(const void* src, size_t bytes, uint32_t* out, int blocks,
                           void* stream) {
  if (!src || !out || blocks <= 0 || bytes % 16 != 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, out);
  return (int)hipGetLastError();
}

// Launches `blocks` workgroups of 512 threads (8 waves), each wave issuing
// iters * 4 MFMAs; `out` holds blocks * 512 floats.  Returns 0 on success,
// else the HIP error code of the launch.
int smla_probe_mfma(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(512), 0, static_cast<hipStream_t>(stream), out,
                     iters);
  return (int)hipGetLastError();
}

// MFMAs one launch issues.
long long smla_probe_mfma_count(int blocks, int iters) {
  return (long long)blocks * 8 * iters * kChains;
}

}  // extern "C"
