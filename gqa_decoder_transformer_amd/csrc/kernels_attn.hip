// Attention kernels.
//
// softmax(q.k * scale + mask) v per query head; query head h reads kv head h / (NH/NKV)
// (ember internals page, "grouped-query attention"); key s is admissible for a query at
// position t iff s <= t when causal ("LowLlamaBasic reference.py", self_attn), every key
// of the row otherwise ("PII-Tracer serving/reference_forward.py"). The softmax is the
// max-subtracted one, evaluated online (running max m, running sum l, rescaled
// accumulator). A key or tile with no admissible entry contributes nothing: no
// exp(-inf - (-inf)) is ever formed (ember internals page, "edge cases": fully masked
// rows). Every query the C ABI can issue admits at least one key.
#include "common.h"
#include "kernels.h"

namespace ember {

namespace {

EMBER_DEV float load_kv(const void* base, size_t idx, bool bf16) {
  return bf16 ? bf16_to_f32(((const uint16_t*)base)[idx]) : ((const float*)base)[idx];
}

// ------------------------------------------------------------------ flash prefill (VALU)
// Block: 64 queries x 4 lanes (each lane owns HD/4 dims), one query head. K/V tiles of
// 64 keys are staged in LDS as f32.
constexpr int kFlashQ = 64;
constexpr int kFlashK = 64;

template <int HD>
__global__ void __launch_bounds__(256) k_flash_prefill(FlashArgs a) {
  constexpr int DP = HD / 4;
  __shared__ float Ks[kFlashK * HD];
  __shared__ float Vs[kFlashK * HD];
  const int qt = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int b = a.b0 + r;
  const int kvh = h / (a.NH / a.NKV);
  const int qi = qt * kFlashQ + threadIdx.x / 4;
  const int part = threadIdx.x % 4;
  const bool qvalid = qi < a.tokens_per_row;
  const int m = r * a.tokens_per_row + (qvalid ? qi : a.tokens_per_row - 1);
  const int qpos = a.start_pos + (qvalid ? qi : a.tokens_per_row - 1);

  float q[DP], acc[DP];
  const float* qp = a.q + (size_t)m * a.NH * HD + (size_t)h * HD + part * DP;
#pragma unroll
  for (int d = 0; d < DP; ++d) { q[d] = qp[d]; acc[d] = 0.f; }
  float mrun = -INFINITY, l = 0.f;

  // keys of this block: causal -> up to the last query's position; else the whole row
  const int q_last = min(a.tokens_per_row, (qt + 1) * kFlashQ) - 1;
  const int key_end = a.causal ? a.start_pos + q_last + 1 : a.start_pos + a.tokens_per_row;
  const size_t kv_base = ((size_t)b * a.NKV + kvh) * a.max_seq * HD;

  for (int k0 = 0; k0 < key_end; k0 += kFlashK) {
    const int nk = min(kFlashK, key_end - k0);
    __syncthreads();
    for (int e = threadIdx.x; e < nk * HD; e += blockDim.x) {
      Ks[e] = load_kv(a.k_cache, kv_base + (size_t)k0 * HD + e, a.kv_bf16);
      Vs[e] = load_kv(a.v_cache, kv_base + (size_t)k0 * HD + e, a.kv_bf16);
    }
    __syncthreads();
    for (int j = 0; j < nk; ++j) {
      const float* kr = Ks + j * HD + part * DP;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < DP; ++d) s = fmaf(q[d], kr[d], s);
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s *= a.scale;
      const int kpos = k0 + j;
      if (a.causal && kpos > qpos) continue;          // inadmissible key: no contribution
      const float mnew = fmaxf(mrun, s);
      const float alpha = expf(mrun - mnew);          // mrun = -inf -> 0
      const float p = expf(s - mnew);
      l = l * alpha + p;
      const float* vr = Vs + j * HD + part * DP;
#pragma unroll
      for (int d = 0; d < DP; ++d) acc[d] = fmaf(p, vr[d], acc[d] * alpha);
      mrun = mnew;
    }
  }
  if (!qvalid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const size_t o = (size_t)m * a.NH * HD + (size_t)h * HD + part * DP;
#pragma unroll
  for (int d = 0; d < DP; ++d) {
    const float v = acc[d] * inv;
    if (a.out_f32) a.out_f32[o + d] = v;
    if (a.out_hi) {
      uint32_t hi, lo;
      split_bf16(v, hi, lo);
      a.out_hi[o + d] = (uint16_t)hi;
      if (a.out_lo) a.out_lo[o + d] = (uint16_t)lo;
    }
  }
}

// ------------------------------------------------------------------ split-K decode
// Block (split, kv head, row): the G query heads of the group share every K/V read.
// A group of LPK lanes reads one key (16 bytes per lane); per head the partial dot
// products are summed with lane shuffles, then each lane group keeps an online softmax
// state; groups are merged through LDS in a fixed order. Output per (row, head, split):
// (m, l, acc[HD]) with acc unnormalised.
constexpr int kMaxG = 8;

EMBER_DEV void split_range(int S, int nsplit, int chunk_min, int split, int& s0, int& s1) {
  int chunk = (S + nsplit - 1) / nsplit;
  if (chunk < chunk_min) chunk = chunk_min;
  s0 = split * chunk;
  s1 = min(S, s0 + chunk);
}

template <int HD, bool KV_BF16, int G>
__global__ void __launch_bounds__(256) k_decode_attn(DecodeAttnArgs a) {
  constexpr int ES = KV_BF16 ? 2 : 4;
  constexpr int DPL = 16 / ES;                 // dims per lane
  constexpr int LPK = HD / DPL;                // lanes per key
  static_assert(LPK >= 1 && LPK <= 64, "head_dim");
  constexpr int KPW = kWave / LPK;             // keys per wave pass
  constexpr int NGRP = 4 * KPW;                // lane groups per block
  __shared__ float qs[G * HD];
  __shared__ float sm[NGRP], sl[NGRP];
  __shared__ float sacc[NGRP * HD];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int S = *a.d_pos + 1;
  int s0, s1;
  split_range(S, a.nsplit, a.chunk_min, split, s0, s1);
  if (s0 >= S) return;                         // beyond the valid splits: never read

  const int h0 = kvh * G;
  for (int e = threadIdx.x; e < G * HD; e += blockDim.x)
    qs[e] = a.q[(size_t)b * a.NH * HD + (size_t)h0 * HD + e];
  __syncthreads();

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int grp = wave * KPW + lane / LPK;     // 0..NGRP-1
  const int sub = lane % LPK;
  float qv[G][DPL];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int d = 0; d < DPL; ++d) qv[g][d] = qs[g * HD + sub * DPL + d];

  float mrun[G], l[G], acc[G][DPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    mrun[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[g][d] = 0.f;
  }
  const size_t base = ((size_t)b * a.NKV + kvh) * a.max_seq * HD;
  for (int key = s0 + grp; key < s1; key += NGRP) {
    const size_t off = base + (size_t)key * HD + sub * DPL;
    u32x4_t kraw, vraw;
    if (KV_BF16) {
      kraw = *(const u32x4_t*)((const uint16_t*)a.k_cache + off);
      vraw = *(const u32x4_t*)((const uint16_t*)a.v_cache + off);
    } else {
      kraw = *(const u32x4_t*)((const float*)a.k_cache + off);
      vraw = *(const u32x4_t*)((const float*)a.v_cache + off);
    }
    float kf[DPL], vf[DPL];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (KV_BF16) {
        kf[2 * i] = bf16_lo(kraw[i]); kf[2 * i + 1] = bf16_hi(kraw[i]);
        vf[2 * i] = bf16_lo(vraw[i]); vf[2 * i + 1] = bf16_hi(vraw[i]);
      } else {
        kf[i] = __uint_as_float(kraw[i]);
        vf[i] = __uint_as_float(vraw[i]);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < DPL; ++d) s = fmaf(qv[g][d], kf[d], s);
      s = group_sum(s, LPK) * a.scale;
      const float mnew = fmaxf(mrun[g], s);
      const float alpha = expf(mrun[g] - mnew);
      const float p = expf(s - mnew);
      l[g] = l[g] * alpha + p;
#pragma unroll
      for (int d = 0; d < DPL; ++d) acc[g][d] = fmaf(p, vf[d], acc[g][d] * alpha);
      mrun[g] = mnew;
    }
  }
  // merge lane groups through LDS (fixed order), one head at a time
  const int h_base = b * a.NH + h0;
  for (int g = 0; g < G; ++g) {
    if (sub == 0) {
      sm[grp] = mrun[g];
      sl[grp] = l[g];
    }
#pragma unroll
    for (int d = 0; d < DPL; ++d) sacc[grp * HD + sub * DPL + d] = acc[g][d];
    __syncthreads();
    for (int d = threadIdx.x; d < HD; d += blockDim.x) {
      float M = -INFINITY;
      for (int i = 0; i < NGRP; ++i) M = fmaxf(M, sm[i]);
      float L = 0.f, A = 0.f;
      if (M != -INFINITY) {
        for (int i = 0; i < NGRP; ++i) {
          const float w = (sm[i] == -INFINITY) ? 0.f : expf(sm[i] - M);
          L += sl[i] * w;
          A += sacc[i * HD + d] * w;
        }
      }
      float* out = a.part + (((size_t)(h_base + g)) * a.nsplit + split) * (HD + 2);
      if (d == 0) { out[0] = M; out[1] = L; }
      out[2 + d] = A;
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(128) k_attn_combine(const float* part, int NH, int HD,
                                                      int nsplit, const int* d_pos, int chunk_min,
                                                      float* out_f32, uint16_t* out_hi,
                                                      uint16_t* out_lo) {
  const int bh = blockIdx.x;                   // b * NH + h
  const int S = *d_pos + 1;
  int chunk = (S + nsplit - 1) / nsplit;
  if (chunk < chunk_min) chunk = chunk_min;
  const int nvalid = (S + chunk - 1) / chunk;
  const int stride = HD + 2;
  const float* ph = part + (size_t)bh * nsplit * stride;
  for (int d = threadIdx.x; d < HD; d += blockDim.x) {
    float M = -INFINITY;
    for (int j = 0; j < nvalid; ++j) M = fmaxf(M, ph[(size_t)j * stride]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
      for (int j = 0; j < nvalid; ++j) {
        const float mj = ph[(size_t)j * stride];
        const float w = (mj == -INFINITY) ? 0.f : expf(mj - M);
        L += ph[(size_t)j * stride + 1] * w;
        A += ph[(size_t)j * stride + 2 + d] * w;
      }
    }
    const float v = L > 0.f ? A / L : 0.f;
    const size_t o = (size_t)bh * HD + d;
    if (out_f32) out_f32[o] = v;
    if (out_hi) {
      uint32_t hi, lo;
      split_bf16(v, hi, lo);
      out_hi[o] = (uint16_t)hi;
      if (out_lo) out_lo[o] = (uint16_t)lo;
    }
  }
}

template <int HD, bool BF>
void launch_decode_hd(const DecodeAttnArgs& a, hipStream_t st) {
  const int G = a.NH / a.NKV;
  dim3 grid(a.nsplit, a.NKV, a.B);
#define EMBER_G(GV) \
  case GV: hipLaunchKernelGGL((k_decode_attn<HD, BF, GV>), grid, dim3(256), 0, st, a); break;
  switch (G) {
    EMBER_G(1) EMBER_G(2) EMBER_G(3) EMBER_G(4) EMBER_G(5) EMBER_G(6) EMBER_G(7) EMBER_G(8)
    default: break;
  }
#undef EMBER_G
}

}  // namespace

void launch_flash_prefill(const FlashArgs& a, hipStream_t st) {
  dim3 grid((a.tokens_per_row + kFlashQ - 1) / kFlashQ, a.NH, a.rows);
  switch (a.HD) {
    case 8: hipLaunchKernelGGL(k_flash_prefill<8>, grid, dim3(256), 0, st, a); break;
    case 16: hipLaunchKernelGGL(k_flash_prefill<16>, grid, dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL(k_flash_prefill<32>, grid, dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL(k_flash_prefill<64>, grid, dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL(k_flash_prefill<128>, grid, dim3(256), 0, st, a); break;
    default: break;
  }
}

void launch_decode_attn(const DecodeAttnArgs& a, hipStream_t st) {
  switch (a.HD) {
#define EMBER_HD(HDV)                                               \
  case HDV:                                                         \
    if (a.kv_bf16) launch_decode_hd<HDV, true>(a, st);              \
    else launch_decode_hd<HDV, false>(a, st);                       \
    break;
    EMBER_HD(8) EMBER_HD(16) EMBER_HD(32) EMBER_HD(64) EMBER_HD(128)
#undef EMBER_HD
    default: break;
  }
}

void launch_attn_combine(const float* part, int B, int NH, int HD, int nsplit, const int* d_pos,
                         int chunk_min, float* out_f32, uint16_t* out_hi, uint16_t* out_lo,
                         hipStream_t st) {
  if (B <= 0) return;
  hipLaunchKernelGGL(k_attn_combine, dim3(B * NH), dim3(128), 0, st, part, NH, HD, nsplit, d_pos,
                     chunk_min, out_f32, out_hi, out_lo);
}

void decode_split_plan(int B, int NKV, int max_seq, int* nsplit, int* chunk_min) {
  const int cmin = 64;
  int target = (2048 + NKV * B - 1) / (NKV * B);
  int maxs = (max_seq + cmin - 1) / cmin;
  int ns = target < maxs ? target : maxs;
  if (ns < 1) ns = 1;
  *nsplit = ns;
  *chunk_min = cmin;
}

}  // namespace ember
