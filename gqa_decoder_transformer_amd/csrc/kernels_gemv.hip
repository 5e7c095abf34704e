// Decode GEMV: y[n] = sum_k W[n, k] x[k] for one token, streaming W from HBM once with
// 16-byte coalesced loads (bf16 weights widened to f32 in registers, f32 FMA; q8_0
// weights as bytes plus one f16 scale per 32, dequantised in registers: see chunk_dot).
//
// At decode sizes these kernels are bound by how early and how many weight bytes are in
// flight, so nothing is staged through LDS:
//  * row per wave  (K <= 128 chunks of 16 bytes): lane l owns the chunks c = l + 64 t of
//    its wave's rows. It first requests the matching input elements x[E c .. E c + E)
//    (and norm weights; they come from L2), then every weight load of its row group, so
//    the input arrives first and the RMSNorm (the wave's lanes cover all of K: sum(x^2),
//    one reciprocal of the RMS) is done while the weights are in flight. All loads are
//    branch-free (clamped chunk indices; a clamped chunk meets x = 0; a spare wave past
//    the last row group reloads it), which keeps the compiler's waits counted. Each
//    output is reduced with DPP row sums + readlane (no block barrier).
//  * row per block (up to 1024 chunks): thread t owns chunks t + 256 u; one block-wide
//    sum of squares for the norm; per row group the four waves' partials meet in LDS.
//  * the output projection of a one-row decode step can take its input as the decode
//    attention's split partials (no combine launch): row per wave rebuilds it once per
//    block into LDS (<= 4 splits); row per block with one chunk per thread combines the
//    thread's head in registers (<= 8 splits), eight output rows per block so the
//    partials are read by few blocks.
//  * longer K: a block per output looping over K (shapes past the two layouts above).
// Epilogues: store (+bias), residual add, SiLU*up (gate/up rows interleaved in blocks of
// 32, see gu_row), logits with an argmax partial (value, then lowest index) per wave or block.
#include "common.h"
#include "kernels.h"

namespace ember {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

struct Q8 {};                   // q8 weights: the byte plane (q + 128) and f16 scales
template <typename WT> struct WTraits;
template <> struct WTraits<uint16_t> {
  using Elem = uint16_t;
  static constexpr int E = 8;   // elements per 16-byte chunk
  static constexpr bool kQ8 = false;
  static EMBER_DEV void widen(const u32x4_t& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(v[i]); f[2 * i + 1] = bf16_hi(v[i]); }
  }
};
template <> struct WTraits<float> {
  using Elem = float;
  static constexpr int E = 4;
  static constexpr bool kQ8 = false;
  static EMBER_DEV void widen(const u32x4_t& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
};
template <> struct WTraits<Q8> {
  using Elem = uint8_t;
  static constexpr int E = 16;  // half a q8_0 block per chunk
  static constexpr bool kQ8 = true;
};

// acc plus one chunk's contribution. bf16 / f32: the widened weights times x, one FMA
// each. q8: d * (sum_e b_e x_e - 128 sum_e x_e) with b_e = q_e + 128 (a byte converts to
// f32 in one instruction), sx = sum_e x_e and d the block's scale (f16 bits in sc).
template <typename WT>
EMBER_DEV float chunk_dot(const u32x4_t& w, const float* x, float sx, uint32_t sc, float acc) {
  constexpr int E = WTraits<WT>::E;
  if constexpr (WTraits<WT>::kQ8) {
    float p = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) p = fmaf((float)((w[e / 4] >> (8 * (e % 4))) & 0xFFu), x[e], p);
    p = fmaf(-128.f, sx, p);
    return fmaf(f16_to_f32(sc), p, acc);
  } else {
    float wf[E];
    WTraits<WT>::widen(w, wf);
#pragma unroll
    for (int e = 0; e < E; ++e) acc = fmaf(wf[e], x[e], acc);
    return acc;
  }
}

// scale of chunk c (16 values, half a block) of weight row `row` (q8 only)
template <typename WT>
EMBER_DEV uint32_t chunk_scale(const GemvArgs& a, int row, int c) {
  if constexpr (WTraits<WT>::kQ8) return a.w_scale[(size_t)row * (a.K / kQ8Block) + (c >> 1)];
  else return 0u;
}


template <int EPI>
EMBER_DEV int weight_row(int n, int r) { return EPI == GEMV_SILU ? gu_row(n, r) : n; }

// Input elements x[E c .. E c + E) of chunk c as f32 (c clamped into range: the loads are
// branch-free so they issue right behind the weight loads; `valid` zeroes a clamped chunk).
template <int E>
EMBER_DEV void load_chunk_f32(const float* p, int c, bool valid, float* out) {
  const float4* q = (const float4*)(p + (size_t)c * E);
#pragma unroll
  for (int i = 0; i < E / 4; ++i) {
    const float4 v = q[i];
    out[4 * i + 0] = valid ? v.x : 0.f;
    out[4 * i + 1] = valid ? v.y : 0.f;
    out[4 * i + 2] = valid ? v.z : 0.f;
    out[4 * i + 3] = valid ? v.w : 0.f;
  }
}

// The input vector rebuilt from decode-attention split partials (see GemvArgs::xpart),
// once per block into LDS (xs, 1024 entries): thread t takes elements t + 256 u (u < 4;
// K <= 1024). Splits at or past the number that hold keys are excluded by select (their
// memory may hold anything). part_load loads the partials; part_finish combines them
// into the LDS copy.
struct PartIn {
  float m[4][4], l[4][4], ac[4][4];     // [element u][split j]
};
EMBER_DEV void part_load(const GemvArgs& a, PartIn& p) {
  const int stride = a.xp_hd + 2;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int k = min((int)threadIdx.x + kThreads * u, a.K - 1);
    const int h = k / a.xp_hd, d = k % a.xp_hd;
    const float* ph = a.xpart + (size_t)h * a.xp_nsplit * stride;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float* pj = ph + (size_t)min(j, a.xp_nsplit - 1) * stride;
      p.m[u][j] = pj[0];
      p.l[u][j] = pj[1];
      p.ac[u][j] = pj[2 + d];
    }
  }
}
EMBER_DEV void part_finish(const GemvArgs& a, const PartIn& p, int S, float* xs) {
  int chunk = (S + a.xp_nsplit - 1) / a.xp_nsplit;
  if (chunk < a.xp_chunk_min) chunk = a.xp_chunk_min;
  const int nv = (S + chunk - 1) / chunk;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) M = j < nv ? fmaxf(M, p.m[u][j]) : M;
    float L = 0.f, x = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float w = (j < nv && p.m[u][j] != -INFINITY) ? expf(p.m[u][j] - M) : 0.f;
      L = j < nv ? fmaf(p.l[u][j], w, L) : L;
      x = j < nv ? fmaf(p.ac[u][j], w, x) : x;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    // unconditional: xs holds 4 x 256 entries and entries past K are never read (a guarded
    // store let the compiler sink its loads behind the weight loads)
    xs[threadIdx.x + kThreads * u] = x * inv;
  }
}

// Epilogue of one output unit n (value(s) already reduced).
template <int EPI>
EMBER_DEV void epilogue(const GemvArgs& a, int n, const float* v, bool writer,
                        unsigned long long& best) {
  float* yp = a.y + n;
  if (EPI == GEMV_STORE) {
    if (writer) *yp = v[0] + (a.bias ? a.bias[n] : 0.f);
  } else if (EPI == GEMV_RESID) {
    if (writer) *yp += v[0];
  } else if (EPI == GEMV_SILU) {
    if (writer) *yp = silu(v[0]) * v[1];
  } else {
    if (writer) {
      *yp = v[0];
      if (v[0] != v[0]) atomicOr(&a.flags[kFlagNaN], 1);
    }
    const unsigned long long key = argmax_key(v[0], (uint32_t)n);
    best = key > best ? key : best;
  }
}

// ---------------------------------------------------------------- row per wave
template <typename WT, int EPI, int RPW, int U, bool XP>
__global__ void __launch_bounds__(kThreads) k_gemv_wave(GemvArgs a) {
  constexpr int E = WTraits<WT>::E;
  constexpr int RU = (EPI == GEMV_SILU) ? 2 : 1;
  constexpr int NR = RPW * RU;
  const int lane = threadIdx.x % kWave;
  const int gw = blockIdx.x * kWaves + threadIdx.x / kWave;   // global wave index
  const int nwaves = gridDim.x * kWaves;
  const int K = a.K, nch = K / E;
  const int ngroups = (a.N + RPW - 1) / RPW;

  auto load_group = [&](int grp, u32x4_t (&w)[U][NR], uint32_t (&sc)[U][NR]) {
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      int n = grp * RPW + u;
      n = n < a.N ? n : a.N - 1;                      // clamp: duplicate, never stored
#pragma unroll
      for (int r = 0; r < RU; ++r) {
        const int wr = weight_row<EPI>(n, r);
        const auto* row = (const typename WTraits<WT>::Elem*)a.W + (size_t)wr * K;
#pragma unroll
        for (int t = 0; t < U; ++t) {
          const int c = min(lane + kWave * t, nch - 1);   // clamped chunk: x is 0 there
          w[t][u * RU + r] = ld_stream(row + (size_t)c * E);
          sc[t][u * RU + r] = chunk_scale<WT>(a, wr, c);
        }
      }
    }
  };

  // this lane's input elements (and norm weights) are requested first: they come from L2
  // and are normalised while the weights are still in flight
  float xv[U][E], nv[U][E];
  u32x4_t wa[U][NR];
  uint32_t sca[U][NR];
  int grp = gw;
  if constexpr (XP) {
    // input rebuilt from attention partials: loads first, then the weights, then the
    // block combines into LDS and every wave reads its chunks from there
    __shared__ float xs[kWave * 2 * 8];
    const int S = *a.xp_pos + 1;
    PartIn pin;
    part_load(a, pin);
    load_group(min(grp, ngroups - 1), wa, sca);
    __builtin_amdgcn_sched_barrier(0);              // every weight load issued before any wait
    part_finish(a, pin, S, xs);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < U; ++t) {
      const int c = lane + kWave * t;
      load_chunk_f32<E>(xs, min(c, nch - 1), c < nch, xv[t]);
    }
  } else {
#pragma unroll
    for (int t = 0; t < U; ++t) {
      const int c = lane + kWave * t;
      load_chunk_f32<E>(a.x, min(c, nch - 1), c < nch, xv[t]);
      if (a.norm_w) load_chunk_f32<E>(a.norm_w, min(c, nch - 1), c < nch, nv[t]);
    }
    load_group(min(grp, ngroups - 1), wa, sca);     // unconditional: a spare wave reloads
  }

  float ss = 0.f;
#pragma unroll
  for (int t = 0; t < U; ++t)
#pragma unroll
    for (int e = 0; e < E; ++e) ss += xv[t][e] * xv[t][e];
  if (a.norm_w) {
    ss = wave_sum_uniform(ss);
    const float inv_rms = 1.0f / sqrtf(ss / (float)K + a.eps);
#pragma unroll
    for (int t = 0; t < U; ++t)
#pragma unroll
      for (int e = 0; e < E; ++e) xv[t][e] = xv[t][e] * inv_rms * nv[t][e];
  }
  float sx[U];
#pragma unroll
  for (int t = 0; t < U; ++t) {
    sx[t] = 0.f;
    if constexpr (WTraits<WT>::kQ8)
#pragma unroll
      for (int e = 0; e < E; ++e) sx[t] += xv[t][e];
  }

  unsigned long long best = 0;
  auto compute = [&](int g, const u32x4_t (&w)[U][NR], const uint32_t (&sc)[U][NR]) {
    float acc[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = 0.f;
#pragma unroll
    for (int t = 0; t < U; ++t)
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = chunk_dot<WT>(w[t][r], xv[t], sx[t], sc[t][r], acc[r]);
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = wave_sum_uniform(acc[r]);
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      const int n = g * RPW + u;
      if (n < a.N) epilogue<EPI>(a, n, acc + u * RU, lane == 0, best);
    }
  };
  while (grp < ngroups) {
    compute(grp, wa, sca);
    grp += nwaves;
    if (grp < ngroups) load_group(grp, wa, sca);
  }
  if (EPI == GEMV_LOGITS && lane == 0) a.argmax_part[gw] = best;
}

// ---------------------------------------------------------------- row per block
constexpr int kBlockParts = 8;   // attention splits the row-per-block layout can take
constexpr int kBlockPartRows = 8; // output rows per block when it rebuilds its input

template <typename WT, int EPI, int RPW, int U, bool XP>
__global__ void __launch_bounds__(kThreads) k_gemv_block(GemvArgs a) {
  constexpr int E = WTraits<WT>::E;
  constexpr int RU = (EPI == GEMV_SILU) ? 2 : 1;
  constexpr int NR = RPW * RU;
  __shared__ float red[16];
  __shared__ float wred[2][kWaves][NR];            // double-buffered: one barrier per group
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int K = a.K, nch = K / E;
  const int ngroups = (a.N + RPW - 1) / RPW;

  auto load_group = [&](int grp, u32x4_t (&w)[U][NR], uint32_t (&sc)[U][NR]) {
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      int n = grp * RPW + u;
      n = n < a.N ? n : a.N - 1;
#pragma unroll
      for (int r = 0; r < RU; ++r) {
        const int wr = weight_row<EPI>(n, r);
        const auto* row = (const typename WTraits<WT>::Elem*)a.W + (size_t)wr * K;
#pragma unroll
        for (int t = 0; t < U; ++t) {
          const int c = min((int)threadIdx.x + kThreads * t, nch - 1);
          w[t][u * RU + r] = ld_stream(row + (size_t)c * E);
          sc[t][u * RU + r] = chunk_scale<WT>(a, wr, c);
        }
      }
    }
  };

  float xv[U][E], nv[U][E];
  u32x4_t wa[U][NR];
  uint32_t sca[U][NR];
  int grp = blockIdx.x;
  if constexpr (XP) {
    // input rebuilt from the attention partials, once per block (a block covers
    // kBlockPartRows output rows): the thread's one chunk lies inside one head, so it
    // combines that head's splits for its E elements in registers (partials requested
    // first, then the weights; splits at or past the number that hold keys are excluded
    // by select: their memory may hold anything)
    static_assert(U == 1 && !WTraits<WT>::kQ8, "one bf16 / f32 chunk per thread");
    const int c = min((int)threadIdx.x, nch - 1);
    const int k0 = c * E, h = k0 / a.xp_hd, d0 = k0 % a.xp_hd;
    const int stride = a.xp_hd + 2;
    const float* ph = a.xpart + (size_t)h * a.xp_nsplit * stride;
    float mj[kBlockParts], lj[kBlockParts], aj[kBlockParts][E];
#pragma unroll
    for (int j = 0; j < kBlockParts; ++j) {
      const float* pj = ph + (size_t)min(j, a.xp_nsplit - 1) * stride;
      mj[j] = pj[0];
      lj[j] = pj[1];
#pragma unroll
      for (int e = 0; e < E; e += 2) {
        const float2 v = *(const float2*)(pj + 2 + d0 + e);
        aj[j][e] = v.x;
        aj[j][e + 1] = v.y;
      }
    }
    load_group(min(grp, ngroups - 1), wa, sca);
    __builtin_amdgcn_sched_barrier(0);              // every weight load issued before any wait
    const int S = *a.xp_pos + 1;
    int chunk = (S + a.xp_nsplit - 1) / a.xp_nsplit;
    if (chunk < a.xp_chunk_min) chunk = a.xp_chunk_min;
    const int nvs = (S + chunk - 1) / chunk;
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < kBlockParts; ++j) M = j < nvs ? fmaxf(M, mj[j]) : M;
    float L = 0.f, xs[E];
#pragma unroll
    for (int e = 0; e < E; ++e) xs[e] = 0.f;
#pragma unroll
    for (int j = 0; j < kBlockParts; ++j) {
      const float w = (j < nvs && mj[j] != -INFINITY) ? expf(mj[j] - M) : 0.f;
      L = j < nvs ? fmaf(lj[j], w, L) : L;
#pragma unroll
      for (int e = 0; e < E; ++e) xs[e] = j < nvs ? fmaf(aj[j][e], w, xs[e]) : xs[e];
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const bool valid = (int)threadIdx.x < nch;
#pragma unroll
    for (int e = 0; e < E; ++e) xv[0][e] = valid ? xs[e] * inv : 0.f;
  } else {
#pragma unroll
    for (int t = 0; t < U; ++t) {
      const int c = threadIdx.x + kThreads * t;
      load_chunk_f32<E>(a.x, min(c, nch - 1), c < nch, xv[t]);
      if (a.norm_w) load_chunk_f32<E>(a.norm_w, min(c, nch - 1), c < nch, nv[t]);
    }
    load_group(min(grp, ngroups - 1), wa, sca);
  }

  float ss = 0.f;
#pragma unroll
  for (int t = 0; t < U; ++t)
#pragma unroll
    for (int e = 0; e < E; ++e) ss += xv[t][e] * xv[t][e];
  if (!XP && a.norm_w) {
    ss = block_sum(ss, red);
    const float inv_rms = 1.0f / sqrtf(ss / (float)K + a.eps);
#pragma unroll
    for (int t = 0; t < U; ++t)
#pragma unroll
      for (int e = 0; e < E; ++e) xv[t][e] = xv[t][e] * inv_rms * nv[t][e];
  }
  float sx[U];
#pragma unroll
  for (int t = 0; t < U; ++t) {
    sx[t] = 0.f;
    if constexpr (WTraits<WT>::kQ8)
#pragma unroll
      for (int e = 0; e < E; ++e) sx[t] += xv[t][e];
  }

  unsigned long long best = 0;
  int parity = 0;
  auto compute = [&](int g, const u32x4_t (&w)[U][NR], const uint32_t (&sc)[U][NR]) {
    float acc[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = 0.f;
#pragma unroll
    for (int t = 0; t < U; ++t)
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[r] = chunk_dot<WT>(w[t][r], xv[t], sx[t], sc[t][r], acc[r]);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      acc[r] = wave_sum_uniform(acc[r]);
      if (lane == 0) wred[parity][wave][r] = acc[r];
    }
    __syncthreads();                                  // (double-buffered: one barrier per group)
#pragma unroll
    for (int r = 0; r < NR; ++r)
      acc[r] = (wred[parity][0][r] + wred[parity][1][r]) + (wred[parity][2][r] + wred[parity][3][r]);
    parity ^= 1;
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      const int n = g * RPW + u;
      if (n < a.N) epilogue<EPI>(a, n, acc + u * RU, threadIdx.x == 0, best);
    }
  };
  while (grp < ngroups) {
    compute(grp, wa, sca);
    grp += (int)gridDim.x;
    if (grp < ngroups) load_group(grp, wa, sca);
  }
  if (EPI == GEMV_LOGITS && threadIdx.x == 0) a.argmax_part[blockIdx.x] = best;
}

// ---------------------------------------------------------------- long K
// K beyond 1024 chunks (1024 x 16 bytes): one block per output unit at a time, looping
// over K; the norm's sum of squares takes its own pass over the input. Only shapes past
// the limits of the two kernels above use it.
template <typename WT, int EPI>
__global__ void __launch_bounds__(kThreads) k_gemv_long(GemvArgs a) {
  constexpr int E = WTraits<WT>::E;
  constexpr int RU = (EPI == GEMV_SILU) ? 2 : 1;
  __shared__ float red[16];
  const int K = a.K, nch = K / E;
  float inv_rms = 1.f;
  if (a.norm_w) {
    float ss = 0.f;
    for (int c = threadIdx.x; c < nch; c += kThreads) {
      float xv[E];
      load_chunk_f32<E>(a.x, c, true, xv);
#pragma unroll
      for (int e = 0; e < E; ++e) ss += xv[e] * xv[e];
    }
    ss = block_sum(ss, red);
    inv_rms = 1.0f / sqrtf(ss / (float)K + a.eps);
  }
  unsigned long long best = 0;
  for (int n = blockIdx.x; n < a.N; n += gridDim.x) {          // block-uniform
    float acc[RU];
#pragma unroll
    for (int r = 0; r < RU; ++r) acc[r] = 0.f;
    for (int c = threadIdx.x; c < nch; c += kThreads) {
      float xv[E];
      load_chunk_f32<E>(a.x, c, true, xv);
      if (a.norm_w) {
        float nv[E];
        load_chunk_f32<E>(a.norm_w, c, true, nv);
#pragma unroll
        for (int e = 0; e < E; ++e) xv[e] = xv[e] * inv_rms * nv[e];
      }
      float sx = 0.f;
      if constexpr (WTraits<WT>::kQ8)
#pragma unroll
        for (int e = 0; e < E; ++e) sx += xv[e];
#pragma unroll
      for (int r = 0; r < RU; ++r) {
        const int wr = weight_row<EPI>(n, r);
        const auto* row = (const typename WTraits<WT>::Elem*)a.W + (size_t)wr * K;
        acc[r] = chunk_dot<WT>(ld_stream(row + (size_t)c * E), xv, sx,
                               chunk_scale<WT>(a, wr, c), acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < RU; ++r) acc[r] = block_sum(acc[r], red);
    epilogue<EPI>(a, n, acc, threadIdx.x == 0, best);
  }
  if (EPI == GEMV_LOGITS && threadIdx.x == 0) a.argmax_part[blockIdx.x] = best;
}

enum ShapeKind { SHAPE_WAVE, SHAPE_BLOCK, SHAPE_LONG };
struct Shape {
  ShapeKind kind;
  int rpw, u, blocks;
};

// Work layout, from graph-timed sweeps over weights streamed from HBM: many waves with few
// loads each beat few waves with many loads (each row group costs a reduction and an
// epilogue after its last weight byte lands). Row per wave (one output unit, one or two
// 16-byte loads per lane per row) while 128 chunks cover K; row per block up to 1024
// chunks (two output units per block once the grid would pass 1024 blocks); a K loop
// beyond. The logits GEMV keeps larger row groups (8 rows): it loops over 128k+ rows and
// its per-group argmax favours fewer groups (with four loads per lane per row, groups of 8
// instead of 4 took the 1B LM head from 91 to 88 us).
Shape pick(int N, int K, int wk, int epi) {
  const int E = wk == WK_Q8 ? 16 : (wk == WK_BF16 ? 8 : 4);
  const int nch = K / E;
  const int ru = epi == GEMV_SILU ? 2 : 1;
  Shape s;
  if (nch > kThreads * 4) {
    s.kind = SHAPE_LONG;
    s.rpw = 1;
    s.u = 0;
    s.blocks = N < 2048 ? N : 2048;
    return s;
  }
  if (epi == GEMV_LOGITS) {
    if (nch <= kWave * 4) {
      s.kind = SHAPE_WAVE;
      s.u = nch <= kWave ? 1 : (nch <= kWave * 2 ? 2 : 4);
      s.rpw = 8 / ru;
      const int groups = (N + s.rpw - 1) / s.rpw;
      const int waves = groups < 8192 ? groups : 8192;
      s.blocks = (waves + kWaves - 1) / kWaves;
    } else {
      s.kind = SHAPE_BLOCK;
      s.u = (nch + kThreads - 1) / kThreads <= 2 ? 2 : 4;
      s.rpw = s.u == 2 ? 4 / ru : 2 / ru;
      const int groups = (N + s.rpw - 1) / s.rpw;
      s.blocks = groups < 2048 ? groups : 2048;
    }
    return s;
  }
  if (nch <= kWave * 2) {
    s.kind = SHAPE_WAVE;
    s.u = nch <= kWave ? 1 : 2;
    s.rpw = 1;
    const int waves = N < 8192 ? N : 8192;
    s.blocks = (waves + kWaves - 1) / kWaves;
  } else {
    s.kind = SHAPE_BLOCK;
    s.u = (nch + kThreads - 1) / kThreads;            // 1 .. 4
    s.rpw = (s.u >= 3 && N > 1024) ? 2 : 1;
    const int groups = (N + s.rpw - 1) / s.rpw;
    s.blocks = groups < 2048 ? groups : 2048;
  }
  return s;
}

// the input rebuilt from attention partials is built only for the residual epilogue (the
// output projection) in the row-per-wave layout; other instances keep their register budget
template <typename WT, int EPI, int RPW, int U>
void launch_wave(const GemvArgs& a, int blocks, hipStream_t st) {
  if (EPI == GEMV_RESID && a.xpart)
    hipLaunchKernelGGL((k_gemv_wave<WT, EPI, RPW, U, EPI == GEMV_RESID>), dim3(blocks), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((k_gemv_wave<WT, EPI, RPW, U, false>), dim3(blocks), dim3(kThreads), 0, st, a);
}
template <typename WT, int EPI, int RPW, int U>
void launch_block(const GemvArgs& a, int blocks, hipStream_t st) {
  if constexpr (EPI == GEMV_RESID && U == 1 && !WTraits<WT>::kQ8) {
    if (a.xpart) {                  // kBlockPartRows rows per block: one rebuild serves them
      const int pb = (a.N + kBlockPartRows - 1) / kBlockPartRows;
      hipLaunchKernelGGL((k_gemv_block<WT, EPI, kBlockPartRows, U, true>), dim3(pb), dim3(kThreads), 0,
                         st, a);
      return;
    }
  }
  hipLaunchKernelGGL((k_gemv_block<WT, EPI, RPW, U, false>), dim3(blocks), dim3(kThreads), 0, st, a);
}

template <typename WT> constexpr int kind_of() {
  return WTraits<WT>::kQ8 ? WK_Q8 : (WTraits<WT>::E == 8 ? WK_BF16 : WK_F32);
}

template <typename WT, int EPI>
void launch_t(const GemvArgs& a, hipStream_t st) {
  const Shape s = pick(a.N, a.K, kind_of<WT>(), EPI);
  constexpr int RU = EPI == GEMV_SILU ? 2 : 1;
  if (s.kind == SHAPE_LONG) {
    hipLaunchKernelGGL((k_gemv_long<WT, EPI>), dim3(s.blocks), dim3(kThreads), 0, st, a);
  } else if constexpr (EPI == GEMV_LOGITS) {
    if (s.kind == SHAPE_BLOCK) {
      if (s.u == 2) launch_block<WT, EPI, 4 / RU, 2>(a, s.blocks, st);
      else launch_block<WT, EPI, 2 / RU, 4>(a, s.blocks, st);
    } else if (s.u == 1) {
      launch_wave<WT, EPI, 8 / RU, 1>(a, s.blocks, st);
    } else if (s.u == 2) {
      launch_wave<WT, EPI, 8 / RU, 2>(a, s.blocks, st);
    } else {
      launch_wave<WT, EPI, 8 / RU, 4>(a, s.blocks, st);
    }
  } else if (s.kind == SHAPE_WAVE) {
    if (s.u == 1) launch_wave<WT, EPI, 1, 1>(a, s.blocks, st);
    else launch_wave<WT, EPI, 1, 2>(a, s.blocks, st);
  } else {
    switch (s.u * 4 + s.rpw) {
      case 1 * 4 + 1: launch_block<WT, EPI, 1, 1>(a, s.blocks, st); break;
      case 2 * 4 + 1: launch_block<WT, EPI, 1, 2>(a, s.blocks, st); break;
      case 3 * 4 + 1: launch_block<WT, EPI, 1, 3>(a, s.blocks, st); break;
      case 3 * 4 + 2: launch_block<WT, EPI, 2, 3>(a, s.blocks, st); break;
      case 4 * 4 + 1: launch_block<WT, EPI, 1, 4>(a, s.blocks, st); break;
      default: launch_block<WT, EPI, 2, 4>(a, s.blocks, st); break;
    }
  }
}

}  // namespace

int gemv_num_blocks(int N, int epi, int K, int wk) {
  const Shape s = pick(N, K, wk, epi);
  return s.kind == SHAPE_WAVE ? s.blocks * kWaves : s.blocks;   // argmax partials written
}

// row per wave: the rebuilt input lives in a 1024-entry LDS copy (K <= 1024, 4 splits);
// row per block: one bf16 / f32 chunk per thread combined in registers (8 splits)
int gemv_parts_max(int N, int K, int wk) {
  const Shape s = pick(N, K, wk, GEMV_RESID);
  if (s.kind == SHAPE_WAVE) return K <= 1024 ? 4 : 0;
  if (s.kind == SHAPE_BLOCK && s.u == 1 && wk != WK_Q8) return kBlockParts;
  return 0;
}

void launch_gemv(const GemvArgs& a, int epi, hipStream_t st) {
  if (a.M != 1 || a.N <= 0 || (!a.x && !a.xpart)) {          // one token, an input required
    report_unlaunched("decode GEMV: one token with an input");
    return;
  }
  const int wk = a.w_scale ? WK_Q8 : (a.w_bf16 ? WK_BF16 : WK_F32);
  if (wk == WK_Q8 && a.K % kQ8Block) {                        // q8 rows are whole blocks
    report_unlaunched("decode GEMV: q8_0 rows of whole blocks");
    return;
  }
  if (a.xpart && (epi != GEMV_RESID || a.xp_nsplit < 1 ||
                  a.xp_nsplit > gemv_parts_max(a.N, a.K, wk))) {
    report_unlaunched("decode GEMV: attention splits as input");   // callers check gemv_parts_max
    return;
  }
#define EMBER_GEMV_CASE(E)                                               \
  case E:                                                                \
    if (wk == WK_Q8) launch_t<Q8, E>(a, st);                             \
    else if (wk == WK_BF16) launch_t<uint16_t, E>(a, st);                \
    else launch_t<float, E>(a, st);                                      \
    break;
  switch (epi) {
    EMBER_GEMV_CASE(GEMV_STORE)
    EMBER_GEMV_CASE(GEMV_RESID)
    EMBER_GEMV_CASE(GEMV_SILU)
    EMBER_GEMV_CASE(GEMV_LOGITS)
    default: report_unlaunched("decode GEMV: epilogue"); break;
  }
#undef EMBER_GEMV_CASE
}

}  // namespace ember
