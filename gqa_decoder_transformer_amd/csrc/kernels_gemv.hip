// Decode GEMV: y[m, n] = sum_k W[n, k] x[m, k] for M <= 2 tokens, streaming W from HBM
// once with 16-byte coalesced loads (bf16 weights widened to f32 in registers, f32 FMA).
//
// The input vector is staged in LDS once per block, either RMS-normalised on the fly
// (RMSNorm fused into the consumer GEMV) or combined from split-K attention partials
// (the attention combine fused into the O projection). Each wave owns RPW outputs; each
// lane owns 16-byte chunks c = lane + 64 t of the weight rows, with U chunks per row in
// flight before the FMAs. Epilogues: store (+bias), residual add, SiLU*up (gate/up rows
// interleaved in blocks of 16), logits with a fused block argmax.
#include "common.h"
#include "kernels.h"

namespace ember {

namespace {

constexpr int kMaxM = 2;
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

// Stage the (normalised or combined) input rows into LDS xs[M][K].
EMBER_DEV void stage_input(const GemvArgs& a, float* xs, float* red) {
  const int K = a.K;
  if (a.x) {
    for (int m = 0; m < a.M; ++m) {
      const float* xr = a.x + (size_t)m * K;
      float inv_scale = 1.f;
      if (a.norm_w) {
        float ss = 0.f;
        for (int k = threadIdx.x; k < K; k += blockDim.x) ss += xr[k] * xr[k];
        ss = block_sum(ss, red);
        inv_scale = sqrtf(ss / (float)K + a.eps);
        for (int k = threadIdx.x; k < K; k += blockDim.x) xs[m * K + k] = xr[k] / inv_scale * a.norm_w[k];
      } else {
        for (int k = threadIdx.x; k < K; k += blockDim.x) xs[m * K + k] = xr[k];
      }
    }
  } else {
    // split-K attention combine: out = sum_j acc_j e^{m_j - M} / sum_j l_j e^{m_j - M}
    const int HD = a.part_hd, NH = a.part_heads, ns = a.part_nsplit;
    const int S = *a.d_pos + 1;
    int chunk = (S + ns - 1) / ns;
    if (chunk < a.part_chunk_min) chunk = a.part_chunk_min;
    const int nvalid = (S + chunk - 1) / chunk;
    const int stride = HD + 2;
    for (int m = 0; m < a.M; ++m) {
      for (int e = threadIdx.x; e < NH * HD; e += blockDim.x) {
        const int h = e / HD, d = e % HD;
        const float* ph = a.part + (((size_t)m * NH + h) * ns) * stride;
        float mx = -INFINITY;
        for (int j = 0; j < nvalid; ++j) mx = fmaxf(mx, ph[(size_t)j * stride]);
        float L = 0.f, acc = 0.f;
        if (mx != -INFINITY) {
          for (int j = 0; j < nvalid; ++j) {
            const float mj = ph[(size_t)j * stride];
            const float wj = (mj == -INFINITY) ? 0.f : expf(mj - mx);
            L += ph[(size_t)j * stride + 1] * wj;
            acc += ph[(size_t)j * stride + 2 + d] * wj;
          }
        }
        xs[m * K + e] = L > 0.f ? acc / L : 0.f;
      }
    }
  }
  __syncthreads();
}

template <typename WT, int EPI, int RPW, int U>
__global__ void __launch_bounds__(kThreads) k_gemv(GemvArgs a) {
  extern __shared__ float xs[];                       // [M][K]
  __shared__ float red[16];
  __shared__ unsigned long long best[kWaves];
  stage_input(a, xs, red);

  constexpr int E = WTraits<WT>::E;
  constexpr int RU = (EPI == GEMV_SILU) ? 2 : 1;     // weight rows per output unit
  constexpr int NR = RPW * RU;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int K = a.K, M = a.M;
  const int nch = K / E;
  const int n0 = (blockIdx.x * kWaves + wave) * RPW;

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

  float acc[kMaxM][NR];
#pragma unroll
  for (int m = 0; m < kMaxM; ++m)
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[m][r] = 0.f;

  for (int c0 = lane; c0 < nch; c0 += kWave * U) {
    u32x4_t wv[U][NR];
#pragma unroll
    for (int t = 0; t < U; ++t) {
      const int c = c0 + t * kWave;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (c < nch) wv[t][r] = *(const u32x4_t*)(rows[r] + (size_t)c * E);
        else wv[t][r] = u32x4_t{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int t = 0; t < U; ++t) {
      const int c = c0 + t * kWave;
      if (c >= nch) break;
      float xv[kMaxM][E];
#pragma unroll
      for (int m = 0; m < kMaxM; ++m) {
        if (m < M) {
#pragma unroll
          for (int e = 0; e < E; ++e) xv[m][e] = xs[m * K + c * E + e];
        }
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float wf[E];
        WTraits<WT>::widen(wv[t][r], wf);
#pragma unroll
        for (int m = 0; m < kMaxM; ++m) {
          if (m < M) {
#pragma unroll
            for (int e = 0; e < E; ++e) acc[m][r] = fmaf(wf[e], xv[m][e], acc[m][r]);
          }
        }
      }
    }
  }

#pragma unroll
  for (int m = 0; m < kMaxM; ++m)
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[m][r] = wave_sum(acc[m][r]);

  for (int m = 0; m < M; ++m) {
    unsigned long long bk = 0;
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      const int n = n0 + u;
      if (n >= a.N) continue;
      float* yp = a.y + (size_t)m * a.ldy + n;
      if (EPI == GEMV_STORE) {
        if (lane == 0) *yp = acc[m][u] + (a.bias ? a.bias[n] : 0.f);
      } else if (EPI == GEMV_RESID) {
        if (lane == 0) *yp += acc[m][u];
      } else if (EPI == GEMV_SILU) {
        if (lane == 0) *yp = silu(acc[m][2 * u]) * acc[m][2 * u + 1];
      } else {
        const float v = acc[m][u];
        if (lane == 0) {
          *yp = v;
          if (v != v) atomicOr(&a.flags[kFlagNaN], 1);
        }
        const unsigned long long key = argmax_key(v, (uint32_t)n);
        bk = key > bk ? key : bk;
      }
    }
    if (EPI == GEMV_LOGITS) {
      if (lane == 0) best[wave] = bk;
      __syncthreads();
      if (threadIdx.x == 0) {
        unsigned long long k = best[0];
        for (int w = 1; w < kWaves; ++w) k = best[w] > k ? best[w] : k;
        a.argmax_part[(size_t)m * gridDim.x + blockIdx.x] = k;
      }
      __syncthreads();
    }
  }
}

template <typename WT, int EPI>
void launch_t(const GemvArgs& a, int rpw, hipStream_t st) {
  const size_t shmem = (size_t)a.M * a.K * sizeof(float);
  if (rpw == 4) {
    const int blocks = (a.N + kWaves * 4 - 1) / (kWaves * 4);
    hipLaunchKernelGGL((k_gemv<WT, EPI, 4, 2>), dim3(blocks), dim3(kThreads), shmem, st, a);
  } else {
    const int blocks = (a.N + kWaves - 1) / kWaves;
    hipLaunchKernelGGL((k_gemv<WT, EPI, 1, 4>), dim3(blocks), dim3(kThreads), shmem, st, a);
  }
}

int pick_rpw(int N, int epi) {
  (void)epi;
  return N >= 4096 ? 4 : 1;
}

}  // namespace

int gemv_num_blocks(int N, int epi, int K) {
  (void)K;
  const int rpw = pick_rpw(N, epi);
  return (N + kWaves * rpw - 1) / (kWaves * rpw);
}

void launch_gemv(const GemvArgs& a, int epi, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return;
  const int rpw = pick_rpw(a.N, epi);
#define EMBER_GEMV_CASE(E)                                               \
  case E:                                                                \
    if (a.w_bf16) launch_t<uint16_t, E>(a, rpw, st);                     \
    else launch_t<float, E>(a, rpw, st);                                 \
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
