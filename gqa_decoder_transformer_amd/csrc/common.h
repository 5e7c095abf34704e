// Device helpers shared by the gfx950 kernels: bf16 conversions, wave64 reductions,
// vector types for 16-byte loads and the MFMA operand types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define EMBER_DEV __device__ __forceinline__

typedef uint16_t bf16_t;                                        // raw bf16 bits
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));     // MFMA A/B operand
typedef float f32x4_t __attribute__((ext_vector_type(4)));       // MFMA 16x16 accumulator
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));    // 16-byte load unit

constexpr int kWave = 64;

// bf16 -> f32 is exact: the stored 16 bits become the high half of the f32 word
// ("ember scripts/reference_forward.py", load_safetensors, BF16 branch).
// 16-byte load of data read once per launch (weights of a decode projection, the KV
// cache in decode attention), marked non-temporal: streaming reads with the hint measured
// 6.6-6.8 TB/s against 5.8-6.2 without it
EMBER_DEV u32x4_t ld_stream(const void* p) { return __builtin_nontemporal_load((const u32x4_t*)p); }
EMBER_DEV float4 ld_stream_f4(const void* p) { return __builtin_bit_cast(float4, ld_stream(p)); }
EMBER_DEV float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
EMBER_DEV float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
EMBER_DEV float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

// IEEE binary16 bits -> f32 (exact).
EMBER_DEV float f16_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// f32 -> bf16, round to nearest, ties to even (finite inputs).
EMBER_DEV uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Split x = hi + lo with hi = bf16(x), lo = bf16(x - hi); |x - hi - lo| <= 2^-17 |x|.
EMBER_DEV void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_rne(x);
  lo = f32_to_bf16_rne(x - bf16_to_f32(hi));
}

// Split x = x0 + x1 + x2 into three bf16 planes, each the nearest bf16 of what the
// previous ones leave; |x - x0 - x1 - x2| <= 2^-25 |x| (finite x).
EMBER_DEV void split3_bf16(float x, uint32_t& x0, uint32_t& x1, uint32_t& x2) {
  x0 = f32_to_bf16_rne(x);
  const float r = x - bf16_to_f32(x0);
  x1 = f32_to_bf16_rne(r);
  x2 = f32_to_bf16_rne(r - bf16_to_f32(x1));
}

template <typename T>
EMBER_DEV T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <typename T>
EMBER_DEV T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// DPP lane moves (gfx9 encodings): quad_perm [1,0,3,2] = 0xB1 (xor 1), [2,3,0,1] = 0x4E
// (xor 2); row_ror:4 = 0x124 and row_ror:8 = 0x128 rotate within a 16-lane row.
template <int CTRL>
EMBER_DEV float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned 16-lane row; every lane of the row receives the row's sum.
EMBER_DEV float row16_sum(float v) {
  v += dpp_move<0xB1>(v);
  v += dpp_move<0x4E>(v);
  v += dpp_move<0x124>(v);
  v += dpp_move<0x128>(v);
  return v;
}

// Wave sum with a wave-uniform result: row sums by DPP, then the four rows combined
// through v_readlane in a fixed order.
EMBER_DEV float wave_sum_uniform(float v) {
  v = row16_sum(v);
  const int b = __float_as_int(v);
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}

// Sum over aligned groups of `WIDTH` lanes (power of two <= 64); every lane of a group
// receives the group's sum.
template <int WIDTH>
EMBER_DEV float group_sum(float v) {
  if (WIDTH >= 2) v += dpp_move<0xB1>(v);
  if (WIDTH >= 4) v += dpp_move<0x4E>(v);
  if (WIDTH == 8) v += dpp_move<0x141>(v);     // row_half_mirror: the other quad of the 8
  if (WIDTH >= 16) {
    v += dpp_move<0x124>(v);
    v += dpp_move<0x128>(v);
  }
  if (WIDTH >= 32) v += __shfl_xor(v, 16);
  if (WIDTH >= 64) v += __shfl_xor(v, 32);
  return v;
}

// Block-wide sum for blockDim.x <= 1024; `red` holds >= 16 floats of shared memory.
EMBER_DEV float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int nw = (blockDim.x + kWave - 1) / kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nw; ++i) s += red[i];   // same order in every thread
  return s;
}

// Order-preserving map of an f32 to u32 (larger float -> larger key); -0.0 is folded
// onto +0.0 first so the two zeros tie.
EMBER_DEV uint32_t ordered_key(float v) {
  v = v + 0.0f;
  uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Argmax key: value in the high word, complemented index in the low word, so the max
// key is the max value with the lowest index.
EMBER_DEV unsigned long long argmax_key(float v, uint32_t idx) {
  return ((unsigned long long)ordered_key(v) << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}

EMBER_DEV unsigned long long wave_max_u64(unsigned long long k) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long other = __shfl_xor(k, o);
    k = other > k ? other : k;
  }
  return k;
}

EMBER_DEV float silu(float z) { return z / (1.0f + expf(-z)); }
