// Prefill attention on MFMA (head_dim 64 or 128): flash-style, one (row, query head,
// 64-query tile) per block, 4 waves x 16 queries, K/V tiles staged in LDS.
//
// Math (per query head h, kv head h / (NH/NKV)): o = softmax(q.k * scale + mask) v with
// the causal mask key <= query position ("LowLlamaBasic reference.py", self_attn) or no
// mask ("PII-Tracer serving/reference_forward.py"); max-subtracted online softmax.
//
// Everything is computed transposed so the two products chain without lane shuffles:
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16 with A = K tile (keys x head dims) and
//                 B = Q^T; lane l ends up holding query l%16 and keys 4*(l/16)+i of each
//                 16-key block;
//   O^T = V^T P^T A = V^T (head dims x keys), B = P^T. The B operand of lane l must hold
//                 8 keys of query l%16: exactly the 8 probabilities the lane holds for two
//                 consecutive 16-key blocks. The MFMA's k slots are therefore the key
//                 permutation slot 8g+j -> 4g+j (j<4), 16+4g+(j-4) (j>=4), and V^T is read
//                 from LDS with the same permutation (two 8-byte reads).
// Scores, the running max/sum and the rescaling are per lane (query l%16): the row
// statistics only need the lanes l, l^16, l^32, l^48.
//
// Precision: EXACT splits q, k, v and p into bf16 hi + lo and forms hi*hi + hi*lo + lo*hi
// (3 MFMAs per product, ~2^-17 relative); FAST uses bf16 hi only.
#include "common.h"
#include "kernels.h"

namespace ember {

namespace {

constexpr int kQ = 64;                 // queries per block (4 waves x 16)

template <int HD> struct FlashCfg {
  static constexpr int BK = HD == 64 ? 64 : 32;        // keys per LDS tile
  static constexpr int KS = HD + 8;                    // K tile row stride (bf16)
  static constexpr int VS = BK + 8;                    // V^T row stride (bf16)
};

EMBER_DEV bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

EMBER_DEV uint32_t pack2(uint32_t lo, uint32_t hi) { return (lo & 0xFFFFu) | (hi << 16); }

template <int HD, bool SPLIT>
__global__ void __launch_bounds__(256) k_flash_mfma(FlashArgs a) {
  using C = FlashCfg<HD>;
  constexpr int BK = C::BK, KS = C::KS, VS = C::VS;
  constexpr int NKB = BK / 16;         // 16-key score blocks per tile
  constexpr int NST = BK / 32;         // 32-key MFMA steps per tile (P V)
  constexpr int NKS = HD / 32;         // 32-dim MFMA steps (Q K)
  constexpr int NDB = HD / 16;         // 16-dim output blocks
  __shared__ __align__(16) uint16_t Kh[BK * KS];
  __shared__ __align__(16) uint16_t Kl[SPLIT ? BK * KS : 8];
  __shared__ __align__(16) uint16_t Vh[HD * VS];
  __shared__ __align__(16) uint16_t Vl[SPLIT ? HD * VS : 8];

  const int qt = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int b = a.b0 + r;
  const int kvh = h / (a.NH / a.NKV);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int ql = lane % 16, g = lane / 16;
  const int qi = qt * kQ + wave * 16 + ql;               // query index within the row
  const bool qvalid = qi < a.tokens_per_row;
  const int qc = qvalid ? qi : a.tokens_per_row - 1;
  const int qpos = a.start_pos + qc;
  const size_t mrow = (size_t)r * a.tokens_per_row + qc;

  // Q^T operand: lane holds q[query ql][ks*32 + 8g .. +7], split into hi/lo
  bf16x8_t qh[NKS], qlo[NKS];
  {
    const float* qp = a.q + mrow * a.NH * HD + (size_t)h * HD;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4_t hv, lv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t h0, l0, h1, l1;
        split_bf16(qp[ks * 32 + 8 * g + 2 * j], h0, l0);
        split_bf16(qp[ks * 32 + 8 * g + 2 * j + 1], h1, l1);
        hv[j] = pack2(h0, h1);
        lv[j] = pack2(l0, l1);
      }
      qh[ks] = as_bf16x8(hv);
      qlo[ks] = as_bf16x8(lv);
    }
  }

  const int q_last = min(a.tokens_per_row, (qt + 1) * kQ) - 1;
  const int key_end = a.causal ? a.start_pos + q_last + 1 : a.start_pos + a.tokens_per_row;
  const size_t kv_base = ((size_t)b * a.NKV + kvh) * a.max_seq * HD;

  f32x4_t o[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) o[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;

  // staging: BK keys x HD values of K and V; thread t handles 4-value chunks
  constexpr int CH = BK * HD / 4 / 256;                  // chunks per thread per tensor
  float kreg[CH][4], vreg[CH][4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int id = threadIdx.x + 256 * c;
      const int key = id / (HD / 4), d4 = (id % (HD / 4)) * 4;
      const int kk = min(k0 + key, key_end - 1);         // clamp: masked keys never count
      const size_t off = kv_base + (size_t)kk * HD + d4;
      if (a.kv_bf16) {
        const uint2 kr = *(const uint2*)((const uint16_t*)a.k_cache + off);
        const uint2 vr = *(const uint2*)((const uint16_t*)a.v_cache + off);
        kreg[c][0] = bf16_lo(kr.x); kreg[c][1] = bf16_hi(kr.x);
        kreg[c][2] = bf16_lo(kr.y); kreg[c][3] = bf16_hi(kr.y);
        vreg[c][0] = bf16_lo(vr.x); vreg[c][1] = bf16_hi(vr.x);
        vreg[c][2] = bf16_lo(vr.y); vreg[c][3] = bf16_hi(vr.y);
      } else {
        const float4 kr = *(const float4*)((const float*)a.k_cache + off);
        const float4 vr = *(const float4*)((const float*)a.v_cache + off);
        kreg[c][0] = kr.x; kreg[c][1] = kr.y; kreg[c][2] = kr.z; kreg[c][3] = kr.w;
        vreg[c][0] = vr.x; vreg[c][1] = vr.y; vreg[c][2] = vr.z; vreg[c][3] = vr.w;
      }
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int id = threadIdx.x + 256 * c;
      const int key = id / (HD / 4), d4 = (id % (HD / 4)) * 4;
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) split_bf16(kreg[c][j], hi[j], lo[j]);
      *(uint2*)(Kh + key * KS + d4) = make_uint2(pack2(hi[0], hi[1]), pack2(hi[2], hi[3]));
      if (SPLIT) *(uint2*)(Kl + key * KS + d4) = make_uint2(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t vh, vl;
        split_bf16(vreg[c][j], vh, vl);
        Vh[(d4 + j) * VS + key] = (uint16_t)vh;
        if (SPLIT) Vl[(d4 + j) * VS + key] = (uint16_t)vl;
      }
    }
  };

  gload(0);
  for (int k0 = 0; k0 < key_end; k0 += BK) {
    __syncthreads();                                     // previous tile fully consumed
    lstore();
    __syncthreads();
    if (k0 + BK < key_end) gload(k0 + BK);               // prefetch the next tile

    // ---- S^T = K Q^T for this tile
    f32x4_t s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int ro = (kb * 16 + ql) * KS + ks * 32 + 8 * g;
        const bf16x8_t kh = as_bf16x8(*(const u32x4_t*)(Kh + ro));
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qh[ks], s[kb], 0, 0, 0);
        if (SPLIT) {
          const bf16x8_t kl = as_bf16x8(*(const u32x4_t*)(Kl + ro));
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qlo[ks], s[kb], 0, 0, 0);
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qh[ks], s[kb], 0, 0, 0);
        }
      }
    }
    // ---- mask, scale, online softmax (lane = query ql, keys k0 + 16kb + 4g + i)
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = k0 + kb * 16 + 4 * g + i;
        float v = s[kb][i] * a.scale;
        if (key >= key_end || (a.causal && key > qpos)) v = -INFINITY;
        s[kb][i] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mnew = fmaxf(mrun, mt);
    const float alpha = mnew == -INFINITY ? 1.f : expf(mrun - mnew);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = s[kb][i] == -INFINITY ? 0.f : expf(s[kb][i] - mnew);
        s[kb][i] = p;
        psum += p;
      }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    lrun = lrun * alpha + psum;
    mrun = mnew;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[d][i] *= alpha;

    // ---- O^T += V^T P^T: 32-key steps; P^T operand = this lane's 8 probabilities
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      u32x4_t ph, pl;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
        split_bf16(s[2 * st + j][0], h0, l0);
        split_bf16(s[2 * st + j][1], h1, l1);
        split_bf16(s[2 * st + j][2], h2, l2);
        split_bf16(s[2 * st + j][3], h3, l3);
        ph[2 * j] = pack2(h0, h1);
        ph[2 * j + 1] = pack2(h2, h3);
        pl[2 * j] = pack2(l0, l1);
        pl[2 * j + 1] = pack2(l2, l3);
      }
      const bf16x8_t pbh = as_bf16x8(ph), pbl = as_bf16x8(pl);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int vo = (db * 16 + ql) * VS + st * 32 + 4 * g;
        u32x4_t vh;
        const uint2 v0 = *(const uint2*)(Vh + vo);
        const uint2 v1 = *(const uint2*)(Vh + vo + 16);
        vh[0] = v0.x; vh[1] = v0.y; vh[2] = v1.x; vh[3] = v1.y;
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vh), pbh, o[db], 0, 0, 0);
        if (SPLIT) {
          u32x4_t vl;
          const uint2 w0 = *(const uint2*)(Vl + vo);
          const uint2 w1 = *(const uint2*)(Vl + vo + 16);
          vl[0] = w0.x; vl[1] = w0.y; vl[2] = w1.x; vl[3] = w1.y;
          o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vh), pbl, o[db], 0, 0, 0);
          o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vl), pbh, o[db], 0, 0, 0);
        }
      }
    }
  }

  if (!qvalid) return;
  const float inv = lrun > 0.f ? 1.f / lrun : 0.f;
  const size_t ob = mrow * a.NH * HD + (size_t)h * HD;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = db * 16 + 4 * g + i;
      const float v = o[db][i] * inv;
      if (a.out_f32) a.out_f32[ob + d] = v;
      if (a.out_hi) {
        uint32_t hi, lo;
        split_bf16(v, hi, lo);
        a.out_hi[ob + d] = (uint16_t)hi;
        if (a.out_lo) a.out_lo[ob + d] = (uint16_t)lo;
      }
    }
}

}  // namespace

bool flash_mfma_supported(int HD) { return HD == 64 || HD == 128; }

void launch_flash_mfma(const FlashArgs& a, bool split, hipStream_t st) {
  dim3 grid((a.tokens_per_row + kQ - 1) / kQ, a.NH, a.rows);
  if (a.HD == 64) {
    if (split) hipLaunchKernelGGL((k_flash_mfma<64, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_flash_mfma<64, false>), grid, dim3(256), 0, st, a);
  } else if (a.HD == 128) {
    if (split) hipLaunchKernelGGL((k_flash_mfma<128, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((k_flash_mfma<128, false>), grid, dim3(256), 0, st, a);
  }
}

}  // namespace ember
