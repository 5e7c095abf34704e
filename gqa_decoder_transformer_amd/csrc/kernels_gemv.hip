// Decode GEMV: y[n] = sum_k W[n, k] x[k] for one token, streaming W from HBM
// once with 16-byte coalesced loads (bf16 weights widened to f32 in registers, f32 FMA).
//
// Latency is what limits these kernels at decode sizes (a dependent global round trip
// costs ~1 us on this part), so every thread issues ALL of its weight loads first --
// they depend on nothing the previous kernel wrote -- and only then stages the input
// vector in LDS: RMS-normalised on the fly (RMSNorm fused into the consumer GEMV) or
// combined from split-K attention partials (combine fused into the O projection).
//
// Two layouts of the work:
//  * row per wave  (K <= 64 * U * E): a wave owns RPW outputs, lane l reads 16-byte
//    chunks l + 64 t of each row, wave-shuffle reduction;
//  * row per block (longer K): the whole block owns RPW outputs, thread t reads chunks
//    t + 256 t', partial sums reduced through LDS in a fixed order.
// Epilogues: store (+bias), residual add, SiLU*up (gate/up rows interleaved in blocks of
// 16), logits with a fused block argmax (value, then lowest index).
#include "common.h"
#include "kernels.h"

namespace ember {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <typename WT> struct WTraits;
template <> struct WTraits<uint16_t> {
  static constexpr int E = 8;   // elements per 16-byte chunk
  static EMBER_DEV void widen(const u32x4_t& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(v[i]); f[2 * i + 1] = bf16_hi(v[i]); }
  }
};
template <> struct WTraits<float> {
  static constexpr int E = 4;
  static EMBER_DEV void widen(const u32x4_t& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
};

// packed row of gate/up output n: rows are interleaved in blocks of 16 (16 gate rows,
// then the 16 matching up rows).
EMBER_DEV int gu_row(int n, int up) { return (n >> 4) * 32 + (up ? 16 : 0) + (n & 15); }

// Stage the (normalised or combined) input vector into LDS xs[K]. `cw` is LDS scratch
// of 3 * NH * nsplit floats for the attention combine.
EMBER_DEV void stage_input(const GemvArgs& a, float* xs, float* cw, float* red) {
  const int K = a.K;
  if (a.x) {
    if (a.norm_w) {
      float ss = 0.f;
      for (int k = threadIdx.x; k < K; k += blockDim.x) {
        const float v = a.x[k];
        xs[k] = v;
        ss += v * v;
      }
      ss = block_sum(ss, red);
      const float rms = sqrtf(ss / (float)K + a.eps);
      for (int k = threadIdx.x; k < K; k += blockDim.x) xs[k] = xs[k] / rms * a.norm_w[k];
    } else {
      for (int k = threadIdx.x; k < K; k += blockDim.x) xs[k] = a.x[k];
    }
  } else {
    // split-K attention combine: att_h = sum_j acc_hj * (e^{m_hj - M_h} / L_h),
    // M_h = max_j m_hj, L_h = sum_j l_hj e^{m_hj - M_h}
    const int HD = a.part_hd, NH = a.part_heads, ns = a.part_nsplit;
    const int S = *a.d_pos + 1;
    int chunk = (S + ns - 1) / ns;
    if (chunk < a.part_chunk_min) chunk = a.part_chunk_min;
    const int nv = (S + chunk - 1) / chunk;
    const int stride = HD + 2;
    float* sm = cw;
    float* sl = cw + NH * ns;
    float* sw = cw + 2 * NH * ns;
    for (int e = threadIdx.x; e < NH * nv; e += blockDim.x) {
      const int h = e / nv, j = e % nv;
      const float* ph = a.part + ((size_t)h * ns + j) * stride;
      sm[e] = ph[0];
      sl[e] = ph[1];
    }
    __syncthreads();
    for (int h = threadIdx.x; h < NH; h += blockDim.x) {
      float M = -INFINITY;
      for (int j = 0; j < nv; ++j) M = fmaxf(M, sm[h * nv + j]);
      float L = 0.f;
      for (int j = 0; j < nv; ++j) {
        const float mj = sm[h * nv + j];
        const float w = (mj == -INFINITY) ? 0.f : expf(mj - M);
        sw[h * nv + j] = w;
        L += sl[h * nv + j] * w;
      }
      const float inv = L > 0.f ? 1.f / L : 0.f;
      for (int j = 0; j < nv; ++j) sw[h * nv + j] *= inv;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < NH * HD; e += blockDim.x) {
      const int h = e / HD, d = e % HD;
      const float* ph = a.part + (size_t)h * ns * stride + 2 + d;
      float acc = 0.f;
      for (int j = 0; j < nv; ++j) acc = fmaf(ph[(size_t)j * stride], sw[h * nv + j], acc);
      xs[e] = acc;
    }
  }
  __syncthreads();
}

// BLOCK_ROW = false: a wave owns RPW outputs; true: the block owns RPW outputs.
template <typename WT, int EPI, int RPW, int U, bool BLOCK_ROW>
__global__ void __launch_bounds__(kThreads) k_gemv(GemvArgs a) {
  extern __shared__ float xs[];                       // [K] (+ combine scratch)
  __shared__ float red[16];
  __shared__ float wred[kWaves][4];                   // BLOCK_ROW partial sums
  __shared__ unsigned long long best[kWaves];

  constexpr int E = WTraits<WT>::E;
  constexpr int RU = (EPI == GEMV_SILU) ? 2 : 1;     // weight rows per output unit
  constexpr int NR = RPW * RU;
  static_assert(!BLOCK_ROW || NR <= 4, "BLOCK_ROW partials");
  constexpr int STRIDE = BLOCK_ROW ? kThreads : kWave;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int tix = BLOCK_ROW ? (int)threadIdx.x : lane;
  const int K = a.K;
  const int nch = K / E;
  const int n0 = BLOCK_ROW ? blockIdx.x * RPW : (blockIdx.x * kWaves + wave) * RPW;

  const WT* rows[NR];
#pragma unroll
  for (int u = 0; u < RPW; ++u) {
    int n = n0 + u;
    if (n >= a.N) n = a.N - 1;                        // clamp: duplicate work, not stored
#pragma unroll
    for (int r = 0; r < RU; ++r) {
      const int row = (EPI == GEMV_SILU) ? gu_row(n, r) : n;
      rows[u * RU + r] = (const WT*)a.W + (size_t)row * K;
    }
  }

  // 1) weight loads of the first batch, before anything that depends on the input
  u32x4_t wv[U][NR];
#pragma unroll
  for (int t = 0; t < U; ++t) {
    const int c = tix + t * STRIDE;
#pragma unroll
    for (int r = 0; r < NR; ++r)
      wv[t][r] = c < nch ? *(const u32x4_t*)(rows[r] + (size_t)c * E) : u32x4_t{0, 0, 0, 0};
  }
  // 2) input vector -> LDS (norm or attention combine) while the loads are in flight
  stage_input(a, xs, xs + K, red);

  float acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.f;

  for (int c0 = 0; c0 < nch; c0 += STRIDE * U) {
    if (c0 > 0) {
#pragma unroll
      for (int t = 0; t < U; ++t) {
        const int c = c0 + tix + t * STRIDE;
#pragma unroll
        for (int r = 0; r < NR; ++r)
          wv[t][r] = c < nch ? *(const u32x4_t*)(rows[r] + (size_t)c * E) : u32x4_t{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int t = 0; t < U; ++t) {
      const int c = c0 + tix + t * STRIDE;
      if (c >= nch) break;
      float xv[E];
#pragma unroll
      for (int e = 0; e < E; ++e) xv[e] = xs[c * E + e];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float wf[E];
        WTraits<WT>::widen(wv[t][r], wf);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[r] = fmaf(wf[e], xv[e], acc[r]);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = wave_sum_uniform(acc[r]);

  if (BLOCK_ROW) {
    // fixed-order sum of the 4 waves' partials (identical result in every thread)
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r) wred[wave][r] = acc[r];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = (wred[0][r] + wred[1][r]) + (wred[2][r] + wred[3][r]);
  }
  const bool writer = BLOCK_ROW ? threadIdx.x == 0 : lane == 0;

  unsigned long long bk = 0;
#pragma unroll
  for (int u = 0; u < RPW; ++u) {
    const int n = n0 + u;
    if (n >= a.N) continue;
    float* yp = a.y + n;
    if (EPI == GEMV_STORE) {
      if (writer) *yp = acc[u] + (a.bias ? a.bias[n] : 0.f);
    } else if (EPI == GEMV_RESID) {
      if (writer) *yp += acc[u];
    } else if (EPI == GEMV_SILU) {
      if (writer) *yp = silu(acc[2 * u]) * acc[2 * u + 1];
    } else {
      const float v = acc[u];
      if (writer) {
        *yp = v;
        if (v != v) atomicOr(&a.flags[kFlagNaN], 1);
      }
      const unsigned long long key = argmax_key(v, (uint32_t)n);
      bk = key > bk ? key : bk;
    }
  }
  if (EPI == GEMV_LOGITS) {
    if (BLOCK_ROW) {
      if (threadIdx.x == 0) a.argmax_part[blockIdx.x] = bk;
    } else {
      if (lane == 0) best[wave] = bk;
      __syncthreads();
      if (threadIdx.x == 0) {
        unsigned long long k = best[0];
        for (int w = 1; w < kWaves; ++w) k = best[w] > k ? best[w] : k;
        a.argmax_part[blockIdx.x] = k;
      }
    }
  }
}

struct Shape {
  bool block_row;
  int rpw, u;
};

// Work layout: every load of a thread issued in one round when the row fits.
Shape pick(int N, int K, bool bf16, int epi) {
  const int E = bf16 ? 8 : 4;
  const int nch = K / E;
  Shape s;
  if (nch <= kWave * 4) {
    s.block_row = false;
    s.u = nch <= kWave * 2 ? 2 : 4;
    s.rpw = (N >= 4096 && epi != GEMV_SILU) ? 4 : (N >= 4096 ? 2 : 1);
    if (epi == GEMV_SILU && s.u == 4) s.rpw = 1;
  } else {
    s.block_row = true;
    s.u = 4;
    s.rpw = N >= 8192 ? 2 : 1;
    if (epi == GEMV_SILU) s.rpw = 1;
  }
  return s;
}

template <typename WT, int EPI, int RPW, int U, bool BR>
void launch_one(const GemvArgs& a, hipStream_t st) {
  size_t shmem = (size_t)a.K * sizeof(float);
  if (!a.x) shmem += (size_t)3 * a.part_heads * a.part_nsplit * sizeof(float);
  const int per_block = BR ? RPW : kWaves * RPW;
  const int blocks = (a.N + per_block - 1) / per_block;
  hipLaunchKernelGGL((k_gemv<WT, EPI, RPW, U, BR>), dim3(blocks), dim3(kThreads), shmem, st, a);
}

template <typename WT, int EPI>
void launch_t(const GemvArgs& a, hipStream_t st) {
  const Shape s = pick(a.N, a.K, sizeof(WT) == 2, EPI);
  if (s.block_row) {
    if (s.rpw == 2) launch_one<WT, EPI, 2, 4, true>(a, st);
    else launch_one<WT, EPI, 1, 4, true>(a, st);
  } else if (s.u == 2) {
    if (s.rpw == 4) launch_one<WT, EPI, 4, 2, false>(a, st);
    else if (s.rpw == 2) launch_one<WT, EPI, 2, 2, false>(a, st);
    else launch_one<WT, EPI, 1, 2, false>(a, st);
  } else {
    if (s.rpw == 4) launch_one<WT, EPI, 4, 4, false>(a, st);
    else if (s.rpw == 2) launch_one<WT, EPI, 2, 4, false>(a, st);
    else launch_one<WT, EPI, 1, 4, false>(a, st);
  }
}

}  // namespace

int gemv_num_blocks(int N, int epi, int K, bool bf16) {
  const Shape s = pick(N, K, bf16, epi);
  const int per_block = s.block_row ? s.rpw : kWaves * s.rpw;
  return (N + per_block - 1) / per_block;
}

void launch_gemv(const GemvArgs& a, int epi, hipStream_t st) {
  if (a.M != 1 || a.N <= 0) return;     // one token per launch
#define EMBER_GEMV_CASE(E)                                               \
  case E:                                                                \
    if (a.w_bf16) launch_t<uint16_t, E>(a, st);                          \
    else launch_t<float, E>(a, st);                                      \
    break;
  switch (epi) {
    EMBER_GEMV_CASE(GEMV_STORE)
    EMBER_GEMV_CASE(GEMV_RESID)
    EMBER_GEMV_CASE(GEMV_SILU)
    EMBER_GEMV_CASE(GEMV_LOGITS)
    default: break;
  }
#undef EMBER_GEMV_CASE
}

}  // namespace ember
