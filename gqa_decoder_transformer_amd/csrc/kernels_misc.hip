// Small row-wise kernels of the forward pass: embedding gather, RMSNorm, the QKV
// epilogue (per-head q/k norm, RoPE, KV-cache store), argmax, the classification head,
// logits conversion and decode-step staging.
#include "common.h"
#include "kernels.h"

namespace ember {

// ------------------------------------------------------------------ embedding gather
// x = E[id] widened to f32 ("ember scripts/reference_forward.py", forward: embed[tok]).
// Row `id` of the embedding widened to f32: bf16 and f32 exactly; q8 as (byte - 128) * d
// with d the block's f16 scale (an exact f32 product, "ember internals", q8_0 blocks).
EMBER_DEV void embed_row(const void* E, int wk, const uint16_t* e_scale, int id, int H, float* xr) {
  if (wk == WK_BF16) {
    const uint16_t* er = (const uint16_t*)E + (size_t)id * H;
    for (int i = threadIdx.x; i < H; i += blockDim.x) xr[i] = bf16_to_f32(er[i]);
  } else if (wk == WK_Q8) {
    const uint8_t* er = (const uint8_t*)E + (size_t)id * H;
    const uint16_t* sr = e_scale + (size_t)id * (H / kQ8Block);
    for (int i = threadIdx.x; i < H; i += blockDim.x)
      xr[i] = (float)((int)er[i] - 128) * f16_to_f32(sr[i / kQ8Block]);
  } else {
    const float* er = (const float*)E + (size_t)id * H;
    for (int i = threadIdx.x; i < H; i += blockDim.x) xr[i] = er[i];
  }
}

__global__ void __launch_bounds__(256) k_embed(const int32_t* ids, const void* E, int wk,
                                               const uint16_t* e_scale, float* x, int H, int V,
                                               int* flags) {
  const int m = blockIdx.x;
  int id = ids[m];
  if (id < 0 || id >= V) {
    if (threadIdx.x == 0) atomicOr(&flags[kFlagBadToken], 1);
    id = 0;
  }
  embed_row(E, wk, e_scale, id, H, x + (size_t)m * H);
}

void launch_embed(const int32_t* ids, const void* E, int e_wk, const uint16_t* e_scale, float* x,
                  int M, int H, int V, int* flags, hipStream_t st) {
  if (M <= 0) return;
  hipLaunchKernelGGL(k_embed, dim3(M), dim3(256), 0, st, ids, E, e_wk, e_scale, x, H, V, flags);
}

// ------------------------------------------------------------------ q8_0 planes
// One thread per block: 34 source bytes (scale, then 32 int8) -> 32 bytes of q + 128 in
// the byte plane (q xor 0x80) and the scale's bits in the scale plane.
__global__ void __launch_bounds__(256) k_q8_unpack(const uint8_t* src, int N, int K, uint8_t* dst_q,
                                                   uint16_t* dst_s, int dst_row0, int gu) {
  const int nb = K / kQ8Block;
  const long long i = threadIdx.x + (long long)blockIdx.x * blockDim.x;
  if (i >= (long long)N * nb) return;
  const int n = (int)(i / nb), b = (int)(i % nb);
  const int d = gu < 0 ? dst_row0 + n : gu_row(n, gu);
  const uint8_t* blk = src + (size_t)i * kQ8BlockBytes;
  dst_s[(size_t)d * nb + b] = (uint16_t)(blk[0] | (blk[1] << 8));
  uint8_t* q = dst_q + (size_t)d * K + (size_t)b * kQ8Block;
#pragma unroll
  for (int j = 0; j < kQ8Block; ++j) q[j] = blk[2 + j] ^ 0x80u;
}

void launch_q8_unpack(const uint8_t* src, int N, int K, uint8_t* dst_q, uint16_t* dst_s,
                      int dst_row0, int gu, hipStream_t st) {
  const long long n = (long long)N * (K / kQ8Block);
  if (n <= 0) return;
  hipLaunchKernelGGL(k_q8_unpack, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, N, K,
                     dst_q, dst_s, dst_row0, gu);
}

// One thread per 16 bytes of the byte plane: 16 values (byte - 128) * d.
__global__ void __launch_bounds__(256) k_q8_dequant(const uint8_t* q, const uint16_t* s, int N, int K,
                                                    void* dst, int mode) {
  const long long i = threadIdx.x + (long long)blockIdx.x * blockDim.x;
  const long long nch = (long long)N * K / 16;
  if (i >= nch) return;
  const long long e0 = i * 16;
  const int n = (int)(e0 / K), k0 = (int)(e0 % K);
  const float d = f16_to_f32(s[(size_t)n * (K / kQ8Block) + k0 / kQ8Block]);
  const u32x4_t w = *(const u32x4_t*)(q + e0);
  float v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = (float)((int)((w[j / 4] >> (8 * (j % 4))) & 0xFFu) - 128) * d;
  if (mode == Q8_TO_BF16 || mode == Q8_TO_BF16_PAIR) {
    uint32_t h[16], l[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) split_bf16(v[j], h[j], l[j]);
    u32x4_t o0, o1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o0[j] = h[2 * j] | (h[2 * j + 1] << 16);
      o1[j] = h[8 + 2 * j] | (h[8 + 2 * j + 1] << 16);
    }
    u32x4_t* o = (u32x4_t*)((uint16_t*)dst + e0);
    o[0] = o0;
    o[1] = o1;
    if (mode == Q8_TO_BF16_PAIR) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o0[j] = l[2 * j] | (l[2 * j + 1] << 16);
        o1[j] = l[8 + 2 * j] | (l[8 + 2 * j + 1] << 16);
      }
      u32x4_t* ol = (u32x4_t*)((uint16_t*)dst + (size_t)N * K + e0);
      ol[0] = o0;
      ol[1] = o1;
    }
  } else {
    float4* o = (float4*)((float*)dst + e0);
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
  }
}

void launch_q8_dequant(const uint8_t* q, const uint16_t* s, int N, int K, void* dst, int mode,
                       hipStream_t st) {
  const long long n = (long long)N * K / 16;
  if (n <= 0) return;
  hipLaunchKernelGGL(k_q8_dequant, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, q, s, N, K,
                     dst, mode);
}

// ------------------------------------------------------------------ RMSNorm
// y = x / sqrt(mean(x^2) + eps) * w (operation order of "ember scripts/
// reference_forward.py", rmsnorm). Sum of squares accumulated in f32 per thread, then a
// fixed-order block reduction.
__global__ void __launch_bounds__(256) k_rmsnorm(const float* x, const float* w, float eps, int H,
                                                 int row_step, int row_off, float* out_f32,
                                                 uint16_t* hi, uint16_t* lo, uint16_t* x2,
                                                 int ld_plane) {
  __shared__ float red[16];
  const int r = blockIdx.x;
  const float* xr = x + ((size_t)r * row_step + row_off) * H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += blockDim.x) ss += xr[i] * xr[i];
  ss = block_sum(ss, red);
  const float rms = sqrtf(ss / (float)H + eps);
  for (int i = threadIdx.x; i < H; i += blockDim.x) {
    const float y = xr[i] / rms * w[i];
    if (out_f32) out_f32[(size_t)r * H + i] = y;
    if (hi) {
      uint32_t h, l, t = 0;
      if (x2) split3_bf16(y, h, l, t);
      else split_bf16(y, h, l);
      hi[(size_t)r * ld_plane + i] = (uint16_t)h;
      if (lo) lo[(size_t)r * ld_plane + i] = (uint16_t)l;
      if (x2) x2[(size_t)r * ld_plane + i] = (uint16_t)t;
    }
  }
}

// Vector form for H a multiple of 4 and at most 4096: each thread keeps its NV groups of
// four elements in registers (one read of the row), 16-byte loads and stores, 8-byte
// stores of the bf16 planes. With nsplit > 0 (rows 0..R-1 in order) the residual add of a
// split-K GEMM comes first: x += sum of its partial planes [nsplit][R][H], summed in plane
// order as the split-K reduce sums them, and the new row is written back to x.
template <int NV>
__global__ void __launch_bounds__(256) k_rmsnorm_v(float* x, const float* w, float eps, int H,
                                                   int row_step, int row_off, float* out_f32,
                                                   uint16_t* hi, uint16_t* lo, uint16_t* x2,
                                                   int ld_plane, const float* part, int nsplit) {
  __shared__ float red[16];
  const int r = blockIdx.x;
  const int H4 = H / 4;
  float4* xr = (float4*)(x + ((size_t)r * row_step + row_off) * H);
  float4 v[NV];
  // the residual add of a deferred split-K GEMM: every load of the row and of its planes
  // issued before the first add (one latency, not one per plane or per group; the plane
  // count is uniform, so the guards are scalar branches)
  float4 pv[NV][kMaxDeferredPlanes];
  const size_t plane = (size_t)gridDim.x * H4;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int i = threadIdx.x + 256 * j;
    v[j] = i < H4 ? ld_stream_f4(xr + i) : make_float4(0.f, 0.f, 0.f, 0.f);   // read once
    if (nsplit > 0 && i < H4) {
      const float4* pp = (const float4*)part + (size_t)r * H4 + i;
#pragma unroll
      for (int s = 0; s < kMaxDeferredPlanes; ++s)
        if (s < nsplit) pv[j][s] = ld_stream_f4(pp + s * plane);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int i = threadIdx.x + 256 * j;
    if (nsplit > 0 && i < H4) {
      float4 acc = pv[j][0];
#pragma unroll
      for (int s = 1; s < kMaxDeferredPlanes; ++s)
        if (s < nsplit) { acc.x += pv[j][s].x; acc.y += pv[j][s].y; acc.z += pv[j][s].z; acc.w += pv[j][s].w; }
      v[j] = make_float4(v[j].x + acc.x, v[j].y + acc.y, v[j].z + acc.z, v[j].w + acc.w);
      xr[i] = v[j];
    }
    // explicit FMAs: the order of the sum of squares does not depend on how the
    // compiler chooses to contract x*x + y*y
    ss = fmaf(v[j].x, v[j].x, ss);
    ss = fmaf(v[j].y, v[j].y, ss);
    ss = fmaf(v[j].z, v[j].z, ss);
    ss = fmaf(v[j].w, v[j].w, ss);
  }
  ss = block_sum(ss, red);
  const float rms = sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int i = threadIdx.x + 256 * j;
    if (i >= H4) continue;
    const float4 wv = ((const float4*)w)[i];
    float y[4] = {v[j].x / rms * wv.x, v[j].y / rms * wv.y, v[j].z / rms * wv.z,
                  v[j].w / rms * wv.w};
    if (out_f32) ((float4*)(out_f32 + (size_t)r * H))[i] = make_float4(y[0], y[1], y[2], y[3]);
    if (hi) {
      uint32_t h[4], l[4], t[4];
      if (x2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) split3_bf16(y[e], h[e], l[e], t[e]);
        ((uint2*)(x2 + (size_t)r * ld_plane))[i] = make_uint2(t[0] | (t[1] << 16), t[2] | (t[3] << 16));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) split_bf16(y[e], h[e], l[e]);
      }
      ((uint2*)(hi + (size_t)r * ld_plane))[i] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      if (lo)
        ((uint2*)(lo + (size_t)r * ld_plane))[i] = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
    }
  }
}

bool rmsnorm_adds_partials(int H, int ld_plane) {
  return H % 4 == 0 && ld_plane % 4 == 0 && (H / 4 + 255) / 256 <= 4;
}

void launch_rmsnorm(const float* x, const float* w, float eps, int R, int H, int row_step,
                    int row_off, float* out_f32, uint16_t* hi, uint16_t* lo, int ld_plane,
                    hipStream_t st, uint16_t* x2, const float* part, int nsplit) {
  if (R <= 0) return;
  const int nv = (H / 4 + 255) / 256;
  if (nsplit > 0 && (!part || row_step != 1 || row_off != 0 || nsplit > kMaxDeferredPlanes ||
                     !rmsnorm_adds_partials(H, ld_plane))) {
    report_unlaunched("RMSNorm: residual partial planes in a form that cannot add them");
    return;
  }
  // the residual add writes x (only with nsplit > 0)
  float* xm = const_cast<float*>(x);
  if (H % 4 == 0 && (!hi || ld_plane % 4 == 0) && nv <= 4) {
    switch (nv) {
      case 1: hipLaunchKernelGGL(k_rmsnorm_v<1>, dim3(R), dim3(256), 0, st, xm, w, eps, H, row_step, row_off, out_f32, hi, lo, x2, ld_plane, part, nsplit); return;
      case 2: hipLaunchKernelGGL(k_rmsnorm_v<2>, dim3(R), dim3(256), 0, st, xm, w, eps, H, row_step, row_off, out_f32, hi, lo, x2, ld_plane, part, nsplit); return;
      case 3: hipLaunchKernelGGL(k_rmsnorm_v<3>, dim3(R), dim3(256), 0, st, xm, w, eps, H, row_step, row_off, out_f32, hi, lo, x2, ld_plane, part, nsplit); return;
      default: hipLaunchKernelGGL(k_rmsnorm_v<4>, dim3(R), dim3(256), 0, st, xm, w, eps, H, row_step, row_off, out_f32, hi, lo, x2, ld_plane, part, nsplit); return;
    }
  }
  hipLaunchKernelGGL(k_rmsnorm, dim3(R), dim3(256), 0, st, x, w, eps, H, row_step, row_off,
                     out_f32, hi, lo, x2, ld_plane);
}

// ------------------------------------------------------------------ QKV epilogue
// One thread per two adjacent rotated pairs (i, i + HD/2) and (i + 1, i + 1 + HD/2) of a
// head (rotate-half RoPE: "ember scripts/reference_forward.py", rope; 8-byte loads and
// stores), grid (tokens, pair blocks); the HD/4 threads of a head sit in adjacent lanes of
// one wave, so the optional per-head RMSNorm over HD ("PII-Tracer serving/
// reference_forward.py", forward: q_norm / k_norm before RoPE) is a lane-group sum. Value
// heads pass through. K and V are stored at the token's explicit position (ember internals
// page, "cursor semantics"). Every thread issues its loads at once (a wave looping over
// heads waited for one round trip per head).
template <int HALF>
__global__ void __launch_bounds__(256) k_qkv_post(QkvPostArgs a) {
  constexpr int HD = 2 * HALF, TPH = HALF / 2;      // two adjacent pairs per thread
  const int m = blockIdx.x;
  const int pidx = blockIdx.y * 256 + threadIdx.x;
  const bool live = pidx < (a.NH + 2 * a.NKV) * TPH;    // whole heads live or dead
  const int h = pidx / TPH, i = 2 * (pidx % TPH);       // pairs (i, i + HALF), (i + 1, ..)
  const int start = a.d_pos ? *a.d_pos : a.start_pos;
  const int b = a.b0 + m / a.tokens_per_row;
  const int p = start + m % a.tokens_per_row;
  const bool is_q = h < a.NH, is_v = h >= a.NH + a.NKV;
  const int N = (a.NH + 2 * a.NKV) * HD;
  float2 x0 = make_float2(0.f, 0.f), x1 = make_float2(0.f, 0.f);
  if (a.splits > 0) {                 // split-K planes summed in order, then the bias
    const float* src = a.partial + (size_t)m * N + (size_t)h * HD;
    const size_t plane = (size_t)a.M * N;
    if (live) {
      x0 = *(const float2*)(src + i);
      x1 = *(const float2*)(src + i + HALF);
      for (int s = 1; s < a.splits; ++s) {
        const float2 u0 = *(const float2*)(src + s * plane + i);
        const float2 u1 = *(const float2*)(src + s * plane + i + HALF);
        x0.x += u0.x; x0.y += u0.y;
        x1.x += u1.x; x1.y += u1.y;
      }
      if (a.bias) {
        const float2 b0 = *(const float2*)(a.bias + h * HD + i);
        const float2 b1 = *(const float2*)(a.bias + h * HD + i + HALF);
        x0.x += b0.x; x0.y += b0.y;
        x1.x += b1.x; x1.y += b1.y;
      }
    }
  } else if (live) {
    const float* src = a.qkv + (size_t)m * N + (size_t)h * HD;
    x0 = *(const float2*)(src + i);
    x1 = *(const float2*)(src + i + HALF);
  }
  float2 c = make_float2(0.f, 0.f), sn = make_float2(0.f, 0.f);
  if (live && !is_v) {
    c = *(const float2*)(a.cos_t + (size_t)p * HALF + i);
    sn = *(const float2*)(a.sin_t + (size_t)p * HALF + i);
  }
  if (a.q_norm) {                    // q and k norms come together
    const float ss = group_sum<TPH>(x0.x * x0.x + x0.y * x0.y + x1.x * x1.x + x1.y * x1.y);
    if (live && !is_v) {
      const float* nw = is_q ? a.q_norm : a.k_norm;
      const float rms = sqrtf(ss / (float)HD + a.eps);
      const float2 w0 = *(const float2*)(nw + i), w1 = *(const float2*)(nw + i + HALF);
      x0.x = x0.x / rms * w0.x; x0.y = x0.y / rms * w0.y;
      x1.x = x1.x / rms * w1.x; x1.y = x1.y / rms * w1.y;
    }
  }
  if (!live) return;
  float2 y0 = x0, y1 = x1;
  if (!is_v) {
    y0 = make_float2(x0.x * c.x - x1.x * sn.x, x0.y * c.y - x1.y * sn.y);
    y1 = make_float2(x1.x * c.x + x0.x * sn.x, x1.y * c.y + x0.y * sn.y);
  }
  if (is_q) {
    float* dst = a.q_out + (size_t)m * a.NH * HD + (size_t)h * HD;
    *(float2*)(dst + i) = y0;
    *(float2*)(dst + i + HALF) = y1;
    return;
  }
  const int kvh = is_v ? h - a.NH - a.NKV : h - a.NH;
  const size_t off = (((size_t)b * a.NKV + kvh) * a.max_seq + p) * HD;
  void* cache = is_v ? a.v_cache : a.k_cache;
  if (a.kv_bf16) {
    *(uint32_t*)((uint16_t*)cache + off + i) = f32_to_bf16_rne(y0.x) | (f32_to_bf16_rne(y0.y) << 16);
    *(uint32_t*)((uint16_t*)cache + off + i + HALF) =
        f32_to_bf16_rne(y1.x) | (f32_to_bf16_rne(y1.y) << 16);
  } else {
    *(float2*)((float*)cache + off + i) = y0;
    *(float2*)((float*)cache + off + i + HALF) = y1;
  }
}

void launch_qkv_post(const QkvPostArgs& a, hipStream_t st) {
  if (a.M <= 0) return;
  const dim3 grid(a.M, ((a.NH + 2 * a.NKV) * (a.HD / 4) + 255) / 256);
  switch (a.HD) {
    case 8: hipLaunchKernelGGL(k_qkv_post<4>, grid, dim3(256), 0, st, a); break;
    case 16: hipLaunchKernelGGL(k_qkv_post<8>, grid, dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL(k_qkv_post<16>, grid, dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL(k_qkv_post<32>, grid, dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL(k_qkv_post<64>, grid, dim3(256), 0, st, a); break;
    default: report_unlaunched("QKV post-processing: head_dim"); break;
  }
}

// ------------------------------------------------------------------ argmax
// Greedy choice: lowest index of the maximum ("ember scripts/reference_forward.py",
// np.argmax in the decode loop). Keys order by value, then by lowest index.
// One block of 1024 threads per row; each thread takes 8 partials per pass, all loads
// issued before the first comparison (indices clamped: a repeated partial cannot change
// a maximum).
constexpr int kArgThreads = 1024;
__global__ void __launch_bounds__(kArgThreads) k_argmax_reduce(const unsigned long long* part,
                                                               int nparts, int32_t* next) {
  __shared__ unsigned long long red[kArgThreads / kWave];
  const int r = blockIdx.x;
  const unsigned long long* pr = part + (size_t)r * nparts;
  unsigned long long k = 0;
  for (int i0 = 0; i0 < nparts; i0 += 8 * kArgThreads) {
    unsigned long long v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = pr[min(i0 + (int)threadIdx.x + kArgThreads * u, nparts - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) k = v[u] > k ? v[u] : k;
  }
  k = wave_max_u64(k);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = k;
  __syncthreads();
  if (threadIdx.x == 0) {
    k = red[0];
    for (int i = 1; i < kArgThreads / kWave; ++i) k = red[i] > k ? red[i] : k;
    next[r] = (int32_t)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
  }
}

void launch_argmax_reduce(const unsigned long long* part, int nparts, int R, int32_t* next,
                          hipStream_t st) {
  if (R <= 0 || nparts <= 0) return;
  hipLaunchKernelGGL(k_argmax_reduce, dim3(R), dim3(kArgThreads), 0, st, part, nparts, next);
}

// One block of 1024 threads per row of logits, four 16-byte loads in flight per thread
// when the rows are 16-byte aligned (else four 4-byte loads); the key keeps the lowest
// index of equal maxima whatever the visiting order.
constexpr int kArgRowThreads = 1024;
__global__ void __launch_bounds__(kArgRowThreads) k_argmax_rows(const float* logits, int n,
                                                                long long ld, int32_t* next,
                                                                int* flags, int vec) {
  __shared__ unsigned long long red[kArgRowThreads / kWave];
  const int r = blockIdx.x;
  const float* row = logits + (size_t)r * ld;
  unsigned long long k = 0;
  bool nan = false;
  auto take = [&](float v, int i) {
    nan |= (v != v);
    const unsigned long long key = argmax_key(v, (uint32_t)i);
    k = key > k ? key : k;
  };
  int done = 0;
  if (vec) {
    const int n4 = n / 4;
    const float4* r4 = (const float4*)row;
    for (int i0 = 0; i0 < n4; i0 += 4 * kArgRowThreads) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = r4[min(i0 + (int)threadIdx.x + kArgRowThreads * u, n4 - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + (int)threadIdx.x + kArgRowThreads * u;
        if (i < n4) {
          take(v[u].x, 4 * i);
          take(v[u].y, 4 * i + 1);
          take(v[u].z, 4 * i + 2);
          take(v[u].w, 4 * i + 3);
        }
      }
    }
    done = 4 * n4;
  }
  for (int i0 = done; i0 < n; i0 += 4 * kArgRowThreads) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = row[min(i0 + (int)threadIdx.x + kArgRowThreads * u, n - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + (int)threadIdx.x + kArgRowThreads * u;
      if (i < n) take(v[u], i);
    }
  }
  if (nan) atomicOr(&flags[kFlagNaN], 1);
  k = wave_max_u64(k);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = k;
  __syncthreads();
  if (threadIdx.x == 0) {
    k = red[0];
    for (int i = 1; i < kArgRowThreads / kWave; ++i) k = red[i] > k ? red[i] : k;
    next[r] = (int32_t)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
  }
}

void launch_argmax_rows(const float* logits, int R, int n, long long ld, int32_t* next, int* flags,
                        hipStream_t st) {
  if (R <= 0 || n <= 0) return;
  const int vec = ld % 4 == 0 && ((uintptr_t)logits & 15) == 0;
  hipLaunchKernelGGL(k_argmax_rows, dim3(R), dim3(kArgRowThreads), 0, st, logits, n, ld, next, flags,
                     vec);
}

// ------------------------------------------------------------------ classification head
// logits = Wc h + bc per token ("PII-Tracer serving/reference_forward.py", token head),
// one wave per (token, class); then the per-token argmax.
__global__ void __launch_bounds__(256) k_cls_head(const float* h, const void* W, int w_bf16,
                                                  const float* b, int M, int H, int C, float* out,
                                                  int32_t* next) {
  const int m = blockIdx.x;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  __shared__ float vals[64];
  const float* hr = h + (size_t)m * H;
  for (int c = wave; c < C; c += blockDim.x / kWave) {
    float acc = 0.f;
    for (int k = lane; k < H; k += kWave) {
      const float wv = w_bf16 ? bf16_to_f32(((const uint16_t*)W)[(size_t)c * H + k])
                              : ((const float*)W)[(size_t)c * H + k];
      acc += wv * hr[k];
    }
    acc = wave_sum(acc);
    if (lane == 0) {
      const float v = acc + (b ? b[c] : 0.f);
      vals[c] = v;
      if (out) out[(size_t)m * C + c] = v;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && next) {
    int best = 0;
    for (int c = 1; c < C; ++c) if (ordered_key(vals[c]) > ordered_key(vals[best])) best = c;
    next[m] = best;
  }
}

void launch_cls_head(const float* h, const void* W, bool w_bf16, const float* b, int M, int H,
                     int C, float* out, int32_t* next, hipStream_t st) {
  if (M <= 0) return;
  hipLaunchKernelGGL(k_cls_head, dim3(M), dim3(256), 0, st, h, W, (int)w_bf16, b, M, H, C, out,
                     next);
}

// ------------------------------------------------------------------ conversions, staging
__global__ void k_convert_logits(const float* src, int n, long long ld, void* dst, int to_bf16) {
  const int r = blockIdx.y;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const float v = src[(size_t)r * ld + i];
    if (to_bf16) ((uint16_t*)dst)[(size_t)r * n + i] = (uint16_t)f32_to_bf16_rne(v);
    else ((float*)dst)[(size_t)r * n + i] = v;
  }
}

void launch_convert_logits(const float* src, int R, int n, long long ld, void* dst, bool to_bf16,
                           hipStream_t st) {
  if (R <= 0 || n <= 0) return;
  int gx = (n + 255) / 256;
  if (gx > 512) gx = 512;
  hipLaunchKernelGGL(k_convert_logits, dim3(gx, R), dim3(256), 0, st, src, n, ld, dst,
                     (int)to_bf16);
}

// Per decode step: the position, the embedding rows of the step's ids (x = E[id] widened
// to f32, out-of-range ids flagged and replaced by 0), and the RoPE row of the position
// (cos, sin) copied to a fixed place so that the step's kernels can read it without
// first reading the position. Block r embeds row r; block 0 also writes the position and
// the RoPE row.
__global__ void __launch_bounds__(256) k_step_begin(StepBeginArgs a) {
  const int r = blockIdx.x;
  const int pos = a.ragged ? a.row_pos[r] : a.pos;
  if (threadIdx.x == 0) {
    if (!a.ragged) a.row_pos[r] = pos;
    if (r == 0) *a.d_pos = pos;
  }
  float* rc = a.rope_cur + (size_t)r * 2 * a.half;
  for (int i = threadIdx.x; i < a.half; i += blockDim.x) {
    rc[i] = a.cos_t[(size_t)pos * a.half + i];
    rc[a.half + i] = a.sin_t[(size_t)pos * a.half + i];
  }
  int id = a.ids[r];
  if (id < 0 || id >= a.V) {
    if (threadIdx.x == 0) atomicOr(&a.flags[kFlagBadToken], 1);
    id = 0;
  }
  embed_row(a.E, a.e_wk, a.e_scale, id, a.H, a.x + (size_t)r * a.H);
}

void launch_step_begin(const StepBeginArgs& a, hipStream_t st) {
  if (a.R <= 0) return;
  hipLaunchKernelGGL(k_step_begin, dim3(a.R), dim3(256), 0, st, a);
}

__global__ void __launch_bounds__(256) k_copy_rows(const float* src, int row_step, int row_off, int H,
                                                   float* dst, long long dst_stride) {
  const int r = blockIdx.x;
  const float* s = src + ((size_t)r * row_step + row_off) * H;
  float* d = dst + (size_t)r * dst_stride;
  for (int i = threadIdx.x; i < H; i += blockDim.x) d[i] = s[i];
}

void launch_copy_rows(const float* src, int R, int row_step, int row_off, int H, float* dst,
                      long long dst_stride, hipStream_t st) {
  if (R <= 0) return;
  hipLaunchKernelGGL(k_copy_rows, dim3(R), dim3(256), 0, st, src, row_step, row_off, H, dst,
                     dst_stride);
}

// ------------------------------------------------------------------ mean-pooled head
// The sequence score of "PII-Tracer serving/reference_forward.py" (forward, sensitivity
// head): the final-normed states summed over the row's tokens (column sums, token order,
// accumulated across passes of one row), then mean and dot product.
__global__ void __launch_bounds__(256) k_pool_accum(const float* h, int tpr, int H, float* acc,
                                                    int first) {
  const int r = blockIdx.y;
  const int d = blockIdx.x * blockDim.x + threadIdx.x;
  if (d >= H) return;
  const float* hr = h + (size_t)r * tpr * H + d;
  float s = first ? 0.f : acc[(size_t)r * H + d];
  for (int t = 0; t < tpr; ++t) s += hr[(size_t)t * H];
  acc[(size_t)r * H + d] = s;
}

void launch_pool_accum(const float* h, int R, int tpr, int H, float* acc, bool first,
                       hipStream_t st) {
  if (R <= 0 || tpr <= 0) return;
  hipLaunchKernelGGL(k_pool_accum, dim3((H + 255) / 256, R), dim3(256), 0, st, h, tpr, H, acc,
                     (int)first);
}

__global__ void __launch_bounds__(256) k_pool_head(const float* acc, int H, int T, const float* w,
                                                   const float* b, float* out) {
  __shared__ float red[16];
  const int r = blockIdx.x;
  float s = 0.f;
  for (int d = threadIdx.x; d < H; d += blockDim.x) s += (acc[(size_t)r * H + d] / (float)T) * w[d];
  s = block_sum(s, red);
  if (threadIdx.x == 0) out[r] = s + b[0];
}

void launch_pool_head(const float* acc, int R, int H, int T, const float* w, const float* b,
                      float* out, hipStream_t st) {
  if (R <= 0) return;
  hipLaunchKernelGGL(k_pool_head, dim3(R), dim3(256), 0, st, acc, H, T, w, b, out);
}

__global__ void k_fill_i32(int* p, int n, int v) {
  const int i = threadIdx.x + blockIdx.x * blockDim.x;
  if (i < n) p[i] = v;
}

void launch_fill_i32(int* p, int n, int v, hipStream_t st) {
  if (n <= 0) return;
  hipLaunchKernelGGL(k_fill_i32, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
}

__global__ void k_widen(const void* src, int bf16, float* dst, long long n) {
  for (long long i = threadIdx.x + (long long)blockIdx.x * blockDim.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    dst[i] = bf16 ? bf16_to_f32(((const uint16_t*)src)[i]) : ((const float*)src)[i];
}

void launch_widen(const void* src, bool bf16, float* dst, long long n, hipStream_t st) {
  if (n <= 0) return;
  long long g = (n + 255) / 256;
  if (g > 4096) g = 4096;
  hipLaunchKernelGGL(k_widen, dim3((unsigned)g), dim3(256), 0, st, src, (int)bf16, dst, n);
}

}  // namespace ember
