// Measurement kernels (not part of the forward pass): the achievable peaks of the GPU that
// the kernels' roofline fractions are also reported against.
//   k_peak_copy: a plain streaming copy, 16-byte loads and stores, grid-stride (bytes
//                read plus bytes written per second);
//   k_peak_read: a streaming read, 16-byte non-temporal loads, sixteen in flight per
//                thread (the reference for kernels that mostly read: weights and KV
//                cache);
//   k_peak_mfma: independent chains of v_mfma_f32_32x32x16_bf16 on register operands, no
//                memory traffic (the matrix-core reference for bf16 work).
#include "common.h"
#include "kernels.h"

namespace ember {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256) k_peak_copy(const u32x4_t* __restrict__ src,
                                                   u32x4_t* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src[i];
}

// a streaming read: each block takes 64 KB segments in turn (sixteen 16-byte loads per
// thread, all in flight before any is used), every chunk folded into one word per thread
// (written, so the loads cannot be dropped)
__global__ void __launch_bounds__(256) k_peak_read(const u32x4_t* __restrict__ src, size_t n,
                                                   uint32_t* __restrict__ out) {
  constexpr int U = 16;
  const size_t nseg = n / (256 * U);
  uint32_t acc = 0;
  for (size_t sg = blockIdx.x; sg < nseg; sg += gridDim.x) {
    const u32x4_t* p = src + sg * 256 * U + threadIdx.x;
    u32x4_t v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) v[j] = ld_stream(p + 256 * j);
#pragma unroll
    for (int j = 0; j < U; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// sixteen independent accumulators per wave (as a 128 x 128 wave tile holds): with four,
// the loop measured ~15 % below what the GEMM inner loop reaches
constexpr int kMfmaChains = 16;

__global__ void __launch_bounds__(256) k_peak_mfma(float* out, int n_iter) {
  const uint32_t t = threadIdx.x + blockIdx.x * 256u;
  // small distinct operands (bf16 bit patterns of values near 1) so no value overflows
  u32x4_t av, bv;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    av[j] = 0x3F803F80u + ((t + j) & 7u);
    bv[j] = 0x3F803F80u + ((t >> 3) & 7u);
  }
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av), b = __builtin_bit_cast(bf16x8_t, bv);
  f32x16_t acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  for (int i = 0; i < n_iter; ++i) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  out[t] = s;
}

}  // namespace

void launch_peak_copy(const void* src, void* dst, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 16;
  hipLaunchKernelGGL(k_peak_copy, dim3(256 * 16), dim3(256), 0, st, (const u32x4_t*)src,
                     (u32x4_t*)dst, n);
}

void launch_peak_read(const void* src, size_t bytes, uint32_t* out, hipStream_t st) {
  hipLaunchKernelGGL(k_peak_read, dim3(kPeakReadBlocks), dim3(256), 0, st, (const u32x4_t*)src,
                     bytes / 16, out);
}

double launch_peak_mfma(float* out, hipStream_t st) {
  // few, long waves (one 256-accumulator wave per SIMD at a time): wave start-up and the
  // final sums stay small against ~8k MFMAs per wave
  constexpr int kBlocks = kPeakMfmaBlocks, kIter = 512;
  hipLaunchKernelGGL(k_peak_mfma, dim3(kBlocks), dim3(256), 0, st, out, kIter);
  // flops: every wave issues kIter * chains MFMAs of 2 * 32 * 32 * 16
  return (double)kBlocks * 4 * kIter * kMfmaChains * 2.0 * 32 * 32 * 16;
}

}  // namespace ember
