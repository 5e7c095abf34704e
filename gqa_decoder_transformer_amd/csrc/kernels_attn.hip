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
// Block (split, head block, row): G query heads of one kv group, either the whole group
// (every K/V read shared by G heads: bandwidth-bound grids) or one head (short
// per-wave instruction streams when the grid is small; the group's other heads re-read
// the same keys through L2). The block first issues its K/V loads, then builds the
// current token's roped q (G heads) and -- in the split that holds position pos -- the
// roped k and v, which the group's first head block also stores into the cache at pos
// (qkv epilogue fused: q/k
// RMSNorm when configured, rotate-half RoPE from the tables, K/V store at the explicit
// position). A group of LPK lanes reads one key (16 bytes per lane); per head the
// partial dot products are summed with lane shuffles and each lane group keeps an online
// softmax state; key batches are double-buffered in registers. Groups are merged through
// LDS in a fixed order. Output per (row, head, split): (m, l, acc[HD]), acc unnormalised.
EMBER_DEV void split_range(int S, int nsplit, int chunk_min, int split, int& s0, int& s1) {
  int chunk = (S + nsplit - 1) / nsplit;
  if (chunk < chunk_min) chunk = chunk_min;
  s0 = split * chunk;
  s1 = min(S, s0 + chunk);
}

template <int HD, bool KV_BF16, int G>
__global__ void __launch_bounds__(256) k_decode_attn(DecodeAttnArgs a) {
  constexpr int NT = 256;
  constexpr int ES = KV_BF16 ? 2 : 4;
  constexpr int DPL = 16 / ES;                 // dims per lane
  constexpr int LPK = HD / DPL;                // lanes per key
  static_assert(LPK >= 1 && LPK <= 64, "head_dim");
  constexpr int KPW = kWave / LPK;             // keys per wave pass
  constexpr int NGRP = (NT / kWave) * KPW;     // lane groups per block
  // keys per group per batch (fewer for wide bf16 groups: 256 VGPRs per lane)
  constexpr int KI = (KV_BF16 && G > 4) ? 2 : 4;
  constexpr int HALF = HD / 2;
  constexpr bool ONE_PASS = NGRP * G * (HD + 2) * 4 <= 48 * 1024;
  constexpr int MG = ONE_PASS ? G : 1;
  __shared__ float qs[G * HD];
  __shared__ float kc[HD], vc[HD];
  __shared__ float cs[HALF], sn[HALF];
  __shared__ float sm[NGRP * MG], sl[NGRP * MG], smax[MG];
  __shared__ float sacc[NGRP * MG * HD];

  const int split = blockIdx.x, b = blockIdx.z;
  const int group = a.NH / a.NKV;
  const int h0 = blockIdx.y * G;               // first query head of this block
  const int kvh = h0 / group;
  const bool kv_writer = h0 % group == 0;
  // The key range of a split does not depend on the position (chunk_min is at least
  // ceil(max_seq / nsplit)), so the first K/V batch is issued before the position is
  // known; keys at or past the position are masked afterwards.
  const int s0 = split * a.chunk_min;
  const int s_hi = min(a.max_seq, s0 + a.chunk_min);

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int grp = wave * KPW + lane / LPK;     // 0..NGRP-1
  const int sub = lane % LPK;
  const size_t base = ((size_t)b * a.NKV + kvh) * a.max_seq * HD;
  auto batches = [&](int end) {
    const int nkeys = end - s0 - grp > 0 ? (end - s0 - grp + NGRP - 1) / NGRP : 0;
    return (nkeys + KI - 1) / KI;
  };

  // K/V loads are unconditional, keys clamped into [0, s_hi) (always inside the cache;
  // entries past the valid range are zeroed before use): guarded loads made the compiler
  // wait for every outstanding load before issuing the next batch
  u32x4_t kb0[KI], vb0[KI], kb1[KI], vb1[KI];
  auto load = [&](int batch, u32x4_t* kb, u32x4_t* vb) {
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int key = max(0, min(s0 + grp + NGRP * (batch * KI + i), s_hi - 1));
      const size_t off = base + (size_t)key * HD + sub * DPL;
      if (KV_BF16) {
        kb[i] = ld_stream((const uint16_t*)a.k_cache + off);
        vb[i] = ld_stream((const uint16_t*)a.v_cache + off);
      } else {
        kb[i] = ld_stream((const float*)a.k_cache + off);
        vb[i] = ld_stream((const float*)a.v_cache + off);
      }
    }
  };
  load(0, kb0, vb0);

  // current token: raw q (G heads), this step's RoPE row and, in the split that holds
  // the position, raw k/v of head kvh
  const int qkv_n = (a.NH + 2 * a.NKV) * HD;
  // projection column c of this row: stored by the QKV GEMM, or the sum of its deferred
  // split-K planes in plane order plus the bias (what the split-K reduce would have stored)
  // (every plane's load issued before the first add; past the last plane the loads repeat
  // it, unused: 1.4 us per layer faster than branching around them)
  auto proj = [&](int c) -> float {
    if (a.qkv_splits <= 0) return a.qkv[(size_t)b * qkv_n + c];
    const float* pp = a.qkv_part + (size_t)b * qkv_n + c;
    const size_t plane = (size_t)a.B * qkv_n;
    float pv[kMaxDeferredPlanes];
#pragma unroll
    for (int s = 0; s < kMaxDeferredPlanes; ++s) pv[s] = pp[min(s, a.qkv_splits - 1) * plane];
    float acc = pv[0];
#pragma unroll
    for (int s = 1; s < kMaxDeferredPlanes; ++s)
      if (s < a.qkv_splits) acc += pv[s];
    return acc + (a.qkv_bias ? a.qkv_bias[c] : 0.f);
  };
  for (int e = threadIdx.x; e < G * HD; e += blockDim.x) qs[e] = proj(h0 * HD + e);
  for (int e = threadIdx.x; e < HALF; e += blockDim.x) {
    cs[e] = a.rope_cur[(size_t)b * HD + e];
    sn[e] = a.rope_cur[(size_t)b * HD + HALF + e];
  }
  const int pos = a.d_pos[b];
  const int S = pos + 1;
  if (s0 >= S) return;                         // beyond the valid splits: never read
  const int s1 = min(S, s_hi);
  const bool has_cur = s1 == S;
  const int nb = batches(s1);
  if (has_cur)
    for (int e = threadIdx.x; e < HD; e += blockDim.x) {
      kc[e] = proj((a.NH + kvh) * HD + e);
      vc[e] = proj((a.NH + a.NKV + kvh) * HD + e);
    }
  __syncthreads();
  // RoPE (and q/k norm) in place: pair e (thread e + 256 j) is pair e % HALF of head
  // e / HALF, head G being the current key
  const int npairs = (G + (has_cur ? 1 : 0)) * HALF;
  constexpr int PJ = ((G + 1) * HALF + NT - 1) / NT;
  float y0[PJ], y1[PJ];
#pragma unroll
  for (int j = 0; j < PJ; ++j) {
    const int e = threadIdx.x + NT * j;
    if (e >= npairs) continue;
    const int hh = e / HALF, i = e % HALF;
    const float* src = hh < G ? qs + hh * HD : kc;
    const float* nw = hh < G ? a.q_norm : a.k_norm;
    float x0 = src[i], x1 = src[i + HALF];
    if (nw) {
      float ss = 0.f;
      for (int d = 0; d < HD; ++d) ss += src[d] * src[d];
      const float rms = sqrtf(ss / (float)HD + a.eps);
      x0 = x0 / rms * nw[i];
      x1 = x1 / rms * nw[i + HALF];
    }
    y0[j] = x0 * cs[i] - x1 * sn[i];
    y1[j] = x1 * cs[i] + x0 * sn[i];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PJ; ++j) {
    const int e = threadIdx.x + NT * j;
    if (e >= npairs) continue;
    const int hh = e / HALF, i = e % HALF;
    float* dst = hh < G ? qs + hh * HD : kc;
    float v0 = y0[j], v1 = y1[j];
    if (hh == G && KV_BF16) {                  // the cache holds bf16: use the stored values
      v0 = bf16_to_f32(f32_to_bf16_rne(v0));
      v1 = bf16_to_f32(f32_to_bf16_rne(v1));
    }
    dst[i] = v0;
    dst[i + HALF] = v1;
  }
  if (has_cur && KV_BF16)
    for (int e = threadIdx.x; e < HD; e += blockDim.x) vc[e] = bf16_to_f32(f32_to_bf16_rne(vc[e]));
  __syncthreads();
  if (has_cur && kv_writer) {                  // store this token's K/V at position pos
    const size_t off = base + (size_t)pos * HD;
    for (int e = threadIdx.x; e < HD; e += blockDim.x) {
      if (KV_BF16) {
        ((uint16_t*)a.k_cache)[off + e] = (uint16_t)f32_to_bf16_rne(kc[e]);
        ((uint16_t*)a.v_cache)[off + e] = (uint16_t)f32_to_bf16_rne(vc[e]);
      } else {
        ((float*)a.k_cache)[off + e] = kc[e];
        ((float*)a.v_cache)[off + e] = vc[e];
      }
    }
  }

  // q pre-multiplied by scale * log2(e): scores and the running maxima are base-2
  // logits (hardware exp2 per probability); the partial's maximum goes out in natural
  // units
  const float c2 = a.scale * 1.4426950408889634f;
  float qv[G][DPL];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int d = 0; d < DPL; ++d) qv[g][d] = qs[g * HD + sub * DPL + d] * c2;

  float mrun[G], l[G], acc[G][DPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    mrun[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[g][d] = 0.f;
  }
  // one batch of KI keys: scores first, then one running-max update per head, then the
  // value accumulation; each key's K and V are widened just before use (only one key's
  // worth of f32 values is live at a time)
  auto widen = [&](const u32x4_t& raw, const float* cur, int key, bool valid, float* f) {
    if (key == pos) {
#pragma unroll
      for (int d = 0; d < DPL; ++d) f[d] = cur[sub * DPL + d];
    } else if (!valid) {                       // never-written or stale entries: zeros
#pragma unroll
      for (int d = 0; d < DPL; ++d) f[d] = 0.f;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (KV_BF16) {
          f[2 * j] = bf16_lo(raw[j]);
          f[2 * j + 1] = bf16_hi(raw[j]);
        } else {
          f[j] = __uint_as_float(raw[j]);
        }
      }
    }
  };
  auto compute = [&](int batch, const u32x4_t* kb, const u32x4_t* vb) {
    float sc[G][KI];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int key = s0 + grp + NGRP * (batch * KI + i);
      const bool valid = key < s1;
      float kf[DPL];
      widen(kb[i], kc, key, valid, kf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < DPL; ++d) s = fmaf(qv[g][d], kf[d], s);
        s = group_sum<LPK>(s);
        sc[g][i] = valid ? s : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mb = -INFINITY;
#pragma unroll
      for (int i = 0; i < KI; ++i) mb = fmaxf(mb, sc[g][i]);
      const float mnew = fmaxf(mrun[g], mb);
      const bool none = mnew == -INFINITY;     // no admissible key yet: nothing changes
      const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(mrun[g] - mnew);  // -inf -> 0
      l[g] *= alpha;
#pragma unroll
      for (int d = 0; d < DPL; ++d) acc[g][d] *= alpha;
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const float p = none ? 0.f : __builtin_amdgcn_exp2f(sc[g][i] - mnew);  // -inf -> 0
        sc[g][i] = p;
        l[g] += p;
      }
      mrun[g] = mnew;
    }
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int key = s0 + grp + NGRP * (batch * KI + i);
      float vf[DPL];
      widen(vb[i], vc, key, key < s1, vf);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int d = 0; d < DPL; ++d) acc[g][d] = fmaf(sc[g][i], vf[d], acc[g][d]);
    }
  };
  for (int bt = 0; bt < nb; bt += 2) {
    load(bt + 1, kb1, vb1);                    // past the last batch: clamped reloads
    compute(bt, kb0, vb0);
    if (bt + 1 >= nb) break;
    load(bt + 2, kb0, vb0);
    compute(bt + 1, kb1, vb1);
  }

  // merge lane groups through LDS (fixed order): per head the group weights
  // w_i = 2^{m_i - M} once (base-2 maxima), then every output dimension sums acc_i w_i
  // over the groups
  const int h_base = b * a.NH + h0;
  for (int g0 = 0; g0 < G; g0 += MG) {
#pragma unroll
    for (int gg = 0; gg < MG; ++gg) {
      const int g = g0 + gg;
      if (sub == 0) {
        sm[grp * MG + gg] = mrun[g];
        sl[grp * MG + gg] = l[g];
      }
#pragma unroll
      for (int d = 0; d < DPL; ++d) sacc[(grp * MG + gg) * HD + sub * DPL + d] = acc[g][d];
    }
    __syncthreads();
    if (threadIdx.x < MG) {
      const int gg = threadIdx.x;
      float M = -INFINITY;
      for (int i = 0; i < NGRP; ++i) M = fmaxf(M, sm[i * MG + gg]);
      smax[gg] = M;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < NGRP * MG; e += blockDim.x) {
      const float M = smax[e % MG];
      sm[e] = (M == -INFINITY || sm[e] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sm[e] - M);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < MG * HD; e += blockDim.x) {
      const int gg = e / HD, d = e % HD;
      float L = 0.f, A = 0.f;
      for (int i = 0; i < NGRP; ++i) {
        const float w = sm[i * MG + gg];
        L = fmaf(sl[i * MG + gg], w, L);
        A = fmaf(sacc[(i * MG + gg) * HD + d], w, A);
      }
      if (a.nsplit == 1) {                     // the only split: final, normalised
        const float v = L > 0.f ? A / L : 0.f;
        const size_t o = (size_t)(h_base + g0 + gg) * HD + d;
        if (a.out_f32) a.out_f32[o] = v;
        if (a.out_hi) {
          uint32_t hi, lo;
          split_bf16(v, hi, lo);
          a.out_hi[o] = (uint16_t)hi;
          if (a.out_lo) a.out_lo[o] = (uint16_t)lo;
        }
      } else {
        float* out = a.part + (((size_t)(h_base + g0 + gg)) * a.nsplit + split) * (HD + 2);
        if (d == 0) { out[0] = smax[gg] * 0.6931471805599453f; out[1] = L; }   // natural units
        out[2 + d] = A;
      }
    }
    __syncthreads();
  }

}

// Combine of the split partials of one (row, head):
// att = sum_j acc_j w_j / L, w_j = e^{m_j - M}, M = max_j m_j, L = sum_j l_j w_j.
// Every split's partial is staged in LDS before the position is read (the loads do not
// wait for it); only the splits that hold a key up to the position are summed.
constexpr int kCombineMaxElems = 64 * (128 + 2);
__global__ void __launch_bounds__(128) k_attn_combine(const float* part, int NH, int HD,
                                                      int nsplit, const int* d_pos, int chunk_min,
                                                      float* out_f32, uint16_t* out_hi,
                                                      uint16_t* out_lo) {
  __shared__ float sp[kCombineMaxElems];
  __shared__ float w[64];
  __shared__ float inv_l;
  const int bh = blockIdx.x;                   // b * NH + h
  const int stride = HD + 2;
  const float* ph = part + (size_t)bh * nsplit * stride;
  for (int e = threadIdx.x; e < nsplit * stride; e += blockDim.x) sp[e] = ph[e];
  const int S = d_pos[bh / NH] + 1;
  int chunk = (S + nsplit - 1) / nsplit;
  if (chunk < chunk_min) chunk = chunk_min;
  const int nv = (S + chunk - 1) / chunk;
  __syncthreads();
  if (threadIdx.x < kWave) {                   // split j on lane j (nsplit <= 64)
    const int j = threadIdx.x;
    const float mj = j < nv ? sp[j * stride] : -INFINITY;
    const float M = wave_max(mj);
    const float wj = (mj == -INFINITY) ? 0.f : expf(mj - M);
    const float L = wave_sum(j < nv ? sp[j * stride + 1] * wj : 0.f);
    w[j] = wj;
    if (j == 0) inv_l = L > 0.f ? 1.f / L : 0.f;
  }
  __syncthreads();
  for (int d = threadIdx.x; d < HD; d += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < nv; ++j) acc = fmaf(sp[j * stride + 2 + d], w[j], acc);
    const float v = acc * inv_l;
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
  const int G = a.heads_per_block;
  dim3 grid(a.nsplit, a.NH / G, a.B);
#define EMBER_G(GV) \
  case GV: hipLaunchKernelGGL((k_decode_attn<HD, BF, GV>), grid, dim3(256), 0, st, a); break;
  switch (G) {
    EMBER_G(1) EMBER_G(2) EMBER_G(3) EMBER_G(4) EMBER_G(5) EMBER_G(6) EMBER_G(7) EMBER_G(8)
    default: report_unlaunched("decode attention: more than 8 heads per block"); break;
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
    default: report_unlaunched("prefill attention: head_dim"); break;
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
    default: report_unlaunched("decode attention: head_dim"); break;
  }
}

void launch_attn_combine(const float* part, int B, int NH, int HD, int nsplit, const int* d_pos,
                         int chunk_min, float* out_f32, uint16_t* out_hi, uint16_t* out_lo,
                         hipStream_t st) {
  if (B <= 0) return;
  hipLaunchKernelGGL(k_attn_combine, dim3(B * NH), dim3(128), 0, st, part, NH, HD, nsplit, d_pos,
                     chunk_min, out_f32, out_hi, out_lo);
}

DecodePlan decode_split_plan(int B, int NH, int NKV, int max_seq, int max_splits) {
  // Keys are split so that the grid covers the CUs: chunks of >= 64 keys, at most 64
  // splits (the combine keeps per-split weights in LDS). Few (row, head) pairs: one
  // query head per block, about 512 blocks; otherwise a whole kv group per block
  // (every K/V byte read once), about 256 blocks for one row and 2048 for batches (none
  // split once the batch alone makes 512 blocks).
  DecodePlan p{1, max_seq, NH / NKV};
  const int maxs = (max_seq + 63) / 64;
  int ns;
  if (B * NH <= 64) {
    p.heads_per_block = 1;
    ns = (512 + B * NH - 1) / (B * NH);
  } else {
    // batches whose (row, kv group) blocks already fill the GPU twice over take no key
    // split (no combine launch: the 64 x 8192 long-context decode 4.77 -> 4.70 ms/step)
    const int target_blocks = B == 1 ? 256 : (B * NKV >= 512 ? 512 : 2048);
    ns = (target_blocks + NKV * B - 1) / (NKV * B);
  }
  if (ns > maxs) ns = maxs;
  if (ns > 64) ns = 64;
  if (ns > max_splits) ns = max_splits;
  if (ns >= 2) {
    p.nsplit = ns;
    p.chunk_min = (max_seq + ns - 1) / ns;     // fixed ranges: split j holds [j c, j c + c)
  }
  return p;
}

}  // namespace ember
