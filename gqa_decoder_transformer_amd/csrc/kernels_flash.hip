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
// Precision: EXACT splits q and k into three bf16 planes and forms the six products
// q_i k_j with i + j <= 2 (the scores are exponentiated, so their absolute error must stay
// at the f32 level of q.k whatever their size); v and p into two planes hi + lo with
// hi*hi + hi*lo + lo*hi (~2^-17 relative, 3 MFMAs). FAST uses one bf16 plane of each.
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

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two f32 -> packed bf16 (round to nearest even) with gfx950's v_cvt_pk_bf16_f32.
EMBER_DEV uint32_t cvt_pk_bf16(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

template <int HD, bool SPLIT>
__global__ void __launch_bounds__(256) k_flash_mfma(FlashArgs a) {
  using C = FlashCfg<HD>;
  constexpr int BK = C::BK, KS = C::KS, VS = C::VS;
  constexpr int NKB = BK / 16;         // 16-key score blocks per tile
  constexpr int NST = BK / 32;         // 32-key MFMA steps per tile (P V)
  constexpr int NKS = HD / 32;         // 32-dim MFMA steps (Q K)
  constexpr int NDB = HD / 16;         // 16-dim output blocks
  __shared__ __align__(16) uint16_t Kh[BK * KS];
  __shared__ __align__(16) uint16_t Km[SPLIT ? BK * KS : 8];
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

  // Q^T operand: lane holds q[query ql][ks*32 + 8g .. +7], split into three planes
  bf16x8_t qh[NKS], qm[NKS], qlo[NKS];
  {
    const float* qp = a.q + mrow * a.NH * HD + (size_t)h * HD;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4_t hv, mv, lv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t a0, a1, a2, b0, b1, b2;
        split3_bf16(qp[ks * 32 + 8 * g + 2 * j], a0, a1, a2);
        split3_bf16(qp[ks * 32 + 8 * g + 2 * j + 1], b0, b1, b2);
        hv[j] = pack2(a0, b0);
        mv[j] = pack2(a1, b1);
        lv[j] = pack2(a2, b2);
      }
      qh[ks] = as_bf16x8(hv);
      qm[ks] = as_bf16x8(mv);
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
      uint32_t hi[4], mi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) split3_bf16(kreg[c][j], hi[j], mi[j], lo[j]);
      *(uint2*)(Kh + key * KS + d4) = make_uint2(pack2(hi[0], hi[1]), pack2(hi[2], hi[3]));
      if (SPLIT) {
        *(uint2*)(Km + key * KS + d4) = make_uint2(pack2(mi[0], mi[1]), pack2(mi[2], mi[3]));
        *(uint2*)(Kl + key * KS + d4) = make_uint2(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]));
      }
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
        if (SPLIT) {
          const bf16x8_t km = as_bf16x8(*(const u32x4_t*)(Km + ro));
          const bf16x8_t kl = as_bf16x8(*(const u32x4_t*)(Kl + ro));
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qh[ks], s[kb], 0, 0, 0);
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qlo[ks], s[kb], 0, 0, 0);
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(km, qm[ks], s[kb], 0, 0, 0);
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(km, qh[ks], s[kb], 0, 0, 0);
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qm[ks], s[kb], 0, 0, 0);
        }
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qh[ks], s[kb], 0, 0, 0);
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


// ------------------------------------------------------------------ packed K / V^T planes
// One block per (64-key tile, kv head, pass row): K is copied row-major (bf16 planes), V
// is transposed through LDS so that every V^T row is written with 16-byte stores. Keys
// from key_end up to the tile boundary are zero.
template <int HD>
__global__ void __launch_bounds__(256) k_kv_pack(KvPackArgs a) {
  __shared__ float vs[64 * (HD + 1)];
  const int kt = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int k0 = kt * 64;
  const size_t cbase = ((size_t)(a.b0 + r) * a.NKV + g) * a.max_seq * HD;
  const size_t kplane = (size_t)a.rows * a.NKV * a.LK * HD;      // elements per plane
  const size_t kb = ((size_t)r * a.NKV + g) * a.LK * HD;
  for (int it = threadIdx.x; it < 64 * HD / 8; it += 256) {
    const int key = it / (HD / 8), d8 = (it % (HD / 8)) * 8;
    const int pos = k0 + key;
    float kv[8], vv[8];
    if (pos < a.key_end) {
      const size_t off = cbase + (size_t)pos * HD + d8;
      if (a.kv_bf16) {
        const u32x4_t kr = ld_stream((const uint16_t*)a.k_cache + off);   // read once
        const u32x4_t vr = ld_stream((const uint16_t*)a.v_cache + off);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kv[2 * j] = bf16_lo(kr[j]); kv[2 * j + 1] = bf16_hi(kr[j]);
          vv[2 * j] = bf16_lo(vr[j]); vv[2 * j + 1] = bf16_hi(vr[j]);
        }
      } else {
        const float* kf = (const float*)a.k_cache + off;
        const float* vf = (const float*)a.v_cache + off;
        const float4 k0v = ld_stream_f4(kf), k1v = ld_stream_f4(kf + 4);   // read once
        const float4 v0v = ld_stream_f4(vf), v1v = ld_stream_f4(vf + 4);
        kv[0] = k0v.x; kv[1] = k0v.y; kv[2] = k0v.z; kv[3] = k0v.w;
        kv[4] = k1v.x; kv[5] = k1v.y; kv[6] = k1v.z; kv[7] = k1v.w;
        vv[0] = v0v.x; vv[1] = v0v.y; vv[2] = v0v.z; vv[3] = v0v.w;
        vv[4] = v1v.x; vv[5] = v1v.y; vv[6] = v1v.z; vv[7] = v1v.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) { kv[j] = 0.f; vv[j] = 0.f; }
    }
    u32x4_t k0p, k1p, k2p;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t a0, a1, a2, b0, b1, b2;
      split3_bf16(kv[2 * j], a0, a1, a2);
      split3_bf16(kv[2 * j + 1], b0, b1, b2);
      k0p[j] = pack2(a0, b0);
      k1p[j] = pack2(a1, b1);
      k2p[j] = pack2(a2, b2);
    }
    const size_t ko = kb + (size_t)pos * HD + d8;
    *(u32x4_t*)(a.kp + ko) = k0p;
    if (a.split) {
      *(u32x4_t*)(a.kp + kplane + ko) = k1p;
      *(u32x4_t*)(a.kp + 2 * kplane + ko) = k2p;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) vs[key * (HD + 1) + d8 + j] = vv[j];
  }
  __syncthreads();
  const size_t vb = ((size_t)r * a.NKV + g) * HD * a.LK;
  // V^T keys are stored in the order the attention kernel's MFMA operand wants them:
  // within every 16 keys the middle two runs of 4 swap places, so a lane's 8 keys
  // (0-3 and 8-11, or 4-7 and 12-15) are 16 contiguous bytes
  for (int it = threadIdx.x; it < HD * 8; it += 256) {
    const int d = it / 8, key8 = (it % 8) * 8;
    const int src0 = (key8 & ~15) + ((key8 & 8) ? 4 : 0);   // source keys src0 + {0..3, 8..11}
    u32x4_t hi, lo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ka = src0 + (2 * j < 4 ? 2 * j : 2 * j + 4);
      uint32_t h0, l0, h1, l1;
      split_bf16(vs[ka * (HD + 1) + d], h0, l0);
      split_bf16(vs[(ka + 1) * (HD + 1) + d], h1, l1);
      hi[j] = pack2(h0, h1);
      lo[j] = pack2(l0, l1);
    }
    const size_t vo = vb + (size_t)d * a.LK + k0 + key8;
    *(u32x4_t*)(a.vt + vo) = hi;
    if (a.split) *(u32x4_t*)(a.vt + kplane + vo) = lo;
  }
}

// ------------------------------------------------------------------ tiled MFMA attention
// Block: 128 queries of one (pass row, query head), 4 waves x 32 queries (EXACT head_dim
// 64: 8 waves, 256 queries); K tiles of 64
// keys. v_mfma_f32_32x32x16_bf16 throughout, everything transposed so the two products
// chain without lane shuffles:
//   S^T = K Q^T: A = K rows (keys) x 16 head dims, B = Q^T; lane l holds query l % 32 and
//                keys 8 (e / 4) + 4 (l / 32) + e % 4 (e < 16) of each 32-key block.
//   O^T = V^T P^T: B = P^T must hold 8 keys of query l % 32 per lane: the lane's own 8
//                probabilities of a 16-key half block, so MFMA slot 8 (l / 32) + i stands
//                for key 16 t + (i < 4 ? 4 (l / 32) + i : 8 + 4 (l / 32) + i - 4), and V^T
//                is packed in that order (k_kv_pack swaps the middle two runs of 4 keys of every
//                16), so each V^T fragment is one 16-byte LDS read.
// Both tiles are double-buffered in LDS, loaded one tile ahead through registers from the
// packed planes (16-byte loads, rows padded by 16 bytes). The softmax is the online one
// in base 2 (scores pre-multiplied by scale * log2 e) with lazy rescaling (the running
// maximum moves only when exceeded by more than 2^8); masks are applied only on tiles
// that cross the causal diagonal or the end of the keys (scale * log2 e is folded into Q
// before its bf16 rounding; P is rounded with the hardware pack-convert); under the causal mask a wave
// skips the tiles wholly past its last query; blocks are ordered so that each half of the
// grid pairs long and short causal rows. Output rows go through LDS and leave as 16-byte stores.
constexpr int kTK = 64;

// EXACT keeps three K planes and two V planes per stage (k_kv_pack). At head_dim 64 two
// such stages take 92 KB, one block per CU: the block has 8 waves (256 queries) so every
// SIMD still runs two, except on grids too small to give every CU a block (short
// prompts), which take 4 waves (an 8-wave block over 128 tokens ran half its waves on
// no queries, 9.2 -> 12.6 us). At head_dim 128 two stages exceed the LDS, so that form
// runs one stage (tile j + 1 waits in registers while tile j is consumed, then one more
// barrier per tile) with 4 waves.
template <int HD, bool SPLIT, int W = 4>
struct TiledCfg {
  static constexpr int NW = W;                                  // waves of 32 queries
  static constexpr int NT = NW * kWave, TQ = NW * 32;
  static constexpr int NPK = SPLIT ? 3 : 1, NPV = SPLIT ? 2 : 1;
  static constexpr int KS = HD + 8, VS = kTK + 8;
  static constexpr int KTILE = kTK * KS, VTILE = HD * VS;
  static constexpr int STAGE = NPK * KTILE + NPV * VTILE;      // bf16 elements
  static constexpr int NST = (SPLIT && HD == 128) ? 1 : 2;     // LDS stages
  static constexpr size_t LDS = (size_t)NST * STAGE * 2;       // bytes
  static_assert(LDS <= 160 * 1024, "LDS of one CU");
  static_assert((size_t)NW * 32 * (HD + 1) * 4 <= LDS, "output staging fits");
  static_assert(kTK * HD / 8 % NT == 0, "tile chunks per thread");
};

template <int HD, bool SPLIT, int W>
__global__ void __launch_bounds__((TiledCfg<HD, SPLIT, W>::NT)) k_flash_tiled(FlashArgs a,
                                                                            const uint16_t* kp,
                                                                            const uint16_t* vt, int LK,
                                                                            int longest_first) {
  using C = TiledCfg<HD, SPLIT, W>;
  constexpr int NPK = C::NPK, NPV = C::NPV, KS = C::KS, VS = C::VS, NT = C::NT, TQ = C::TQ;
  constexpr int NKS = HD / 16, NDB = HD / 32;
  constexpr int CK = kTK * HD / 8 / NT;                          // 16-byte chunks per thread
  extern __shared__ __align__(16) uint16_t sm[];

  // Dispatch order L (x fastest, then heads, then rows) -> tile. A grid larger than the
  // CUs hold at once is dispatched as blocks finish: there the tiles go in decreasing
  // query position (long causal rows first, the short ones fill in at the end).
  // Otherwise the first half of the grid takes the tiles in decreasing position and the
  // second half in increasing position, so blocks half a grid apart (dispatched into the
  // same slots) carry complementary amounts of work.
  const int nq = gridDim.x, HR = gridDim.y * gridDim.z, total = nq * HR;
  int L = blockIdx.x + nq * (blockIdx.y + gridDim.y * blockIdx.z);
  {
    // blocks are dealt round-robin to the 8 XCDs: within each run of 8 G dispatched
    // blocks, XCD x takes G consecutive work items, the G query heads of one kv group at
    // one query tile, so their K/V tiles are fetched into one L2 at about one time
    const int G = a.NH / a.NKV, chunk = 8 * G;
    if (total % chunk == 0) L = L / chunk * chunk + G * (L % 8) + L % chunk / 8;
  }
  const int half = (total + 1) / 2;
  const int tix = longest_first ? L : L < half ? L : total - 1 - (L - half);
  const int qt = nq - 1 - tix / HR;
  const int h = (tix % HR) % gridDim.y, r = (tix % HR) / gridDim.y;
  const int g = h / (a.NH / a.NKV);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int lq = lane % 32, hl = lane / 32;
  const int T = a.tokens_per_row;
  const int q0 = qt * TQ + wave * 32;
  const int qc = min(q0 + lq, T - 1);
  const int qpos = a.start_pos + qc;
  const size_t mrow = (size_t)r * T + qc;
  const int key_end = a.start_pos + T;
  const int kend_blk = a.causal ? a.start_pos + min(T, (qt + 1) * TQ) : key_end;
  const int ntiles = (kend_blk + kTK - 1) / kTK;
  const int wq_first = a.start_pos + min(T - 1, q0);
  const int wq_last = a.start_pos + min(T - 1, q0 + 31);

  // Q^T operand: query lq, head dims 16 ks + 8 hl .. + 8, pre-multiplied by
  // scale * log2(e) so that the products are base-2 logits directly; EXACT: three planes
  // q0 + q1 + q2 (as K), and the score is the sum of the six products q_i k_j with
  // i + j <= 2 (the three left out are below 2^-24 of |q| |k|)
  const float c2 = a.scale * 1.4426950408889634f;
  bf16x8_t qh[NKS], qm[SPLIT ? NKS : 1], qlo[SPLIT ? NKS : 1];
  {
    const float* qp = a.q + mrow * a.NH * HD + (size_t)h * HD + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const float4 x0 = *(const float4*)(qp + 16 * ks), x1 = *(const float4*)(qp + 16 * ks + 4);
      const float xv[8] = {x0.x * c2, x0.y * c2, x0.z * c2, x0.w * c2,
                           x1.x * c2, x1.y * c2, x1.z * c2, x1.w * c2};
      u32x4_t hv, mv, lv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t a0, a1, a2, b0, b1, b2;
        split3_bf16(xv[2 * j], a0, a1, a2);
        split3_bf16(xv[2 * j + 1], b0, b1, b2);
        hv[j] = pack2(a0, b0);
        mv[j] = pack2(a1, b1);
        lv[j] = pack2(a2, b2);
      }
      qh[ks] = as_bf16x8(hv);
      if (SPLIT) {
        qm[ks] = as_bf16x8(mv);
        qlo[ks] = as_bf16x8(lv);
      }
    }
  }

  // tile staging: thread chunk c covers K key id / (HD / 8), dims (id % (HD / 8)) * 8 and
  // V^T head dim id / 8, keys (id % 8) * 8 (id = tid + NT c)
  const size_t plane = (size_t)a.rows * a.NKV * LK * HD;
  const uint16_t* kg = kp + ((size_t)r * a.NKV + g) * LK * HD;
  const uint16_t* vg = vt + ((size_t)r * a.NKV + g) * HD * LK;
  u32x4_t rk[NPK][CK], rv[NPV][CK];
  auto gload = [&](int j) {
    const int k0 = j * kTK;
#pragma unroll
    for (int c = 0; c < CK; ++c) {
      const int id = threadIdx.x + NT * c;
      const size_t ko = (size_t)(k0 + id / (HD / 8)) * HD + (id % (HD / 8)) * 8;
      const size_t vo = (size_t)(id / 8) * LK + k0 + (id % 8) * 8;
#pragma unroll
      for (int p = 0; p < NPK; ++p) rk[p][c] = *(const u32x4_t*)(kg + p * plane + ko);
#pragma unroll
      for (int p = 0; p < NPV; ++p) rv[p][c] = *(const u32x4_t*)(vg + p * plane + vo);
    }
  };
  auto sstore = [&](int s) {
    uint16_t* st = sm + s * C::STAGE;
#pragma unroll
    for (int c = 0; c < CK; ++c) {
      const int id = threadIdx.x + NT * c;
      const int ko = (id / (HD / 8)) * KS + (id % (HD / 8)) * 8;
      const int vo = (id / 8) * VS + (id % 8) * 8;
#pragma unroll
      for (int p = 0; p < NPK; ++p) *(u32x4_t*)(st + p * C::KTILE + ko) = rk[p][c];
#pragma unroll
      for (int p = 0; p < NPV; ++p) *(u32x4_t*)(st + NPK * C::KTILE + p * C::VTILE + vo) = rv[p][c];
    }
  };

  f32x16_t o[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[d][e] = 0.f;
  float mrun = -INFINITY;
  // FAST: the softmax denominators come from the matrix core: an all-ones A operand
  // against P^T gives every row of `lsum` the per-query sum of exactly the bf16
  // probabilities the P V product uses. EXACT: each lane sums its f32 probabilities
  // (lpart; the query's other half is in lane ^ 32), which the hi + lo planes of P carry
  // to 2^-17, so no MFMA is spent on it
  f32x16_t lsum;
  float lpart = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) lsum[e] = 0.f;
  const u32x4_t ones_u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const bf16x8_t ones = as_bf16x8(ones_u);

  gload(0);
  sstore(0);
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    const int s = C::NST == 2 ? (j & 1) : 0;
    if (j + 1 < ntiles) gload(j + 1);
    const int k0 = j * kTK;
    if (!a.causal || k0 <= wq_last) {                          // wave-uniform
      const uint16_t* st = sm + s * C::STAGE;
      f32x16_t sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[kb][e] = 0.f;
      if (!SPLIT) {
        // every K fragment of the tile is read first; the two 32-key blocks' MFMA chains
        // then alternate, so consecutive MFMAs are independent
        bf16x8_t kfh[2][NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            kfh[kb][ks] = as_bf16x8(*(const u32x4_t*)(st + (kb * 32 + lq) * KS + 16 * ks + 8 * hl));
        if (HD == 64) __builtin_amdgcn_sched_barrier(0); // reads ahead of the MFMAs (HD 128:
                                                         // too many registers for all of them)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfh[kb][ks], qh[ks], sc[kb], 0, 0, 0);
      } else {
        // one 16-dim step at a time (three K planes of both 32-key blocks), the smaller
        // products first; the two blocks' chains alternate
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          bf16x8_t k0f[2], k1f[2], k2f[2];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const int ro = (kb * 32 + lq) * KS + 16 * ks + 8 * hl;
            k0f[kb] = as_bf16x8(*(const u32x4_t*)(st + ro));
            k1f[kb] = as_bf16x8(*(const u32x4_t*)(st + C::KTILE + ro));
            k2f[kb] = as_bf16x8(*(const u32x4_t*)(st + 2 * C::KTILE + ro));
          }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k2f[kb], qh[ks], sc[kb], 0, 0, 0);
            sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0f[kb], qlo[ks], sc[kb], 0, 0, 0);
          }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1f[kb], qm[ks], sc[kb], 0, 0, 0);
            sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1f[kb], qh[ks], sc[kb], 0, 0, 0);
          }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0f[kb], qm[ks], sc[kb], 0, 0, 0);
            sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0f[kb], qh[ks], sc[kb], 0, 0, 0);
          }
        }
      }
      // keys past `klim` are masked with one compare and select per score, only on tiles
      // that cross the causal diagonal or the end of the keys (a wave-uniform branch)
      const bool need_mask = (a.causal && k0 + kTK - 1 > wq_first) || k0 + kTK > key_end;
      if (__builtin_expect(__builtin_amdgcn_readfirstlane((int)need_mask), 0)) {
        const int klim = (a.causal ? min(key_end - 1, qpos) : key_end - 1) - k0 - 4 * hl;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int kofs = kb * 32 + 8 * (e / 4) + (e % 4);    // key - k0 - 4 hl
            sc[kb][e] = kofs > klim ? -INFINITY : sc[kb][e];
          }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sc[kb][e]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      // Lazy rescaling: the reference maximum mrun moves (and O and l are rescaled) only
      // when a score exceeds it by more than 2^8 in any row of the wave; otherwise the
      // probabilities are taken against the stale maximum, at most 2^8. The first tile
      // always moves it (mrun = -inf; key 0 is in tile 0, so it becomes finite).
      if (__ballot(mt > mrun + 8.f) != 0) {
        const float mnew = fmaxf(mrun, mt);
        const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);   // mrun = -inf -> 0
#pragma unroll
        for (int e = 0; e < 16; ++e) lsum[e] *= alpha;
        lpart *= alpha;
#pragma unroll
        for (int d = 0; d < NDB; ++d)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
        mrun = mnew;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          sc[kb][e] = __builtin_amdgcn_exp2f(sc[kb][e] - mrun);   // masked (-inf) -> 0
      if (SPLIT) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) lpart += sc[kb][e];
      }
#pragma unroll
      for (int t = 0; t < kTK / 16; ++t) {
        const int kb = t / 2, e0 = 8 * (t % 2);
        u32x4_t ph, pl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p0 = sc[kb][e0 + 2 * i], p1 = sc[kb][e0 + 2 * i + 1];
          ph[i] = cvt_pk_bf16(p0, p1);
          if (SPLIT) pl[i] = cvt_pk_bf16(p0 - bf16_lo(ph[i]), p1 - bf16_hi(ph[i]));
        }
        const bf16x8_t pbh = as_bf16x8(ph), pbl = as_bf16x8(pl);
        if (!SPLIT) lsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pbh, lsum, 0, 0, 0);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int vo = (db * 32 + lq) * VS + 16 * t + 8 * hl;   // keys stored permuted
          const uint16_t* vb = st + NPK * C::KTILE;
          const u32x4_t vh = *(const u32x4_t*)(vb + vo);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vh), pbh, o[db], 0, 0, 0);
          if (SPLIT) {
            const u32x4_t vl = *(const u32x4_t*)(vb + C::VTILE + vo);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vh), pbl, o[db], 0, 0, 0);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vl), pbh, o[db], 0, 0, 0);
          }
        }
      }
    }
    if (C::NST == 2) {
      if (j + 1 < ntiles) sstore(s ^ 1);
      __syncthreads();
    } else {
      __syncthreads();                                         // tile j consumed
      if (j + 1 < ntiles) {
        sstore(0);
        __syncthreads();
      }
    }
  }

  // normalise and stage the wave's 32 output rows (f32, padded) through LDS
  float* ow = (float*)sm + wave * 32 * (HD + 1);
  const float lrun = SPLIT ? lpart + __shfl_xor(lpart, 32) : lsum[0];
  const float inv = lrun > 0.f ? 1.f / lrun : 0.f;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      ow[lq * (HD + 1) + db * 32 + 8 * (e / 4) + 4 * hl + (e % 4)] = o[db][e] * inv;
  __syncthreads();
  for (int it = lane; it < 32 * (HD / 8); it += kWave) {
    const int row = it / (HD / 8), c8 = (it % (HD / 8)) * 8;
    if (q0 + row >= T) continue;
    const float* src = ow + row * (HD + 1) + c8;
    const size_t ob = ((size_t)r * T + q0 + row) * a.NH * HD + (size_t)h * HD + c8;
    if (a.out_f32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) a.out_f32[ob + i] = src[i];
    }
    if (a.out_hi) {
      u32x4_t hv, lv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t h0, l0, h1, l1;
        split_bf16(src[2 * i], h0, l0);
        split_bf16(src[2 * i + 1], h1, l1);
        hv[i] = pack2(h0, h1);
        lv[i] = pack2(l0, l1);
      }
      *(u32x4_t*)(a.out_hi + ob) = hv;
      if (a.out_lo) *(u32x4_t*)(a.out_lo + ob) = lv;
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
  } else {
    report_unlaunched("MFMA attention: head_dim");
  }
}

}  // namespace ember

namespace ember {

void launch_kv_pack(const KvPackArgs& a, hipStream_t st) {
  if (a.rows <= 0 || a.key_end <= 0) return;
  dim3 grid(a.LK / 64, a.NKV, a.rows);
  if (a.HD == 64) hipLaunchKernelGGL(k_kv_pack<64>, grid, dim3(256), 0, st, a);
  else if (a.HD == 128) hipLaunchKernelGGL(k_kv_pack<128>, grid, dim3(256), 0, st, a);
  else report_unlaunched("K/V packing: head_dim");
}

namespace {
// blocks of each tiled-attention form that the device holds at once (CUs x blocks per
// CU), and its CU count, per device: [device][HD 128][split][8 waves]
constexpr int kMaxDevices = 64;
int g_tiled_resident[kMaxDevices][2][2][2];
int g_cus[kMaxDevices];

template <int HD, bool SPLIT, int W>
void tiled_init(int dev, int cus) {
  using TC = TiledCfg<HD, SPLIT, W>;
  (void)hipFuncSetAttribute((const void*)k_flash_tiled<HD, SPLIT, W>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)TC::LDS);
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k_flash_tiled<HD, SPLIT, W>,
                                                   TC::NT, TC::LDS) != hipSuccess)
    per_cu = 0;
  g_tiled_resident[dev][HD == 128][SPLIT][W == 8] = per_cu * cus;
}
}  // namespace

void flash_init() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
  g_cus[dev] = cus;
  tiled_init<64, false, 4>(dev, cus);
  tiled_init<64, true, 4>(dev, cus);
  tiled_init<64, true, 8>(dev, cus);
  tiled_init<128, false, 4>(dev, cus);
  tiled_init<128, true, 4>(dev, cus);
}

void launch_flash_tiled(const FlashArgs& a, const uint16_t* kp, const uint16_t* vt, int LK,
                        bool split, hipStream_t st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
#define EMBER_TILED(HDV, SP, WV)                                                       \
  {                                                                                    \
    using TC = TiledCfg<HDV, SP, WV>;                                                  \
    const dim3 grid((a.tokens_per_row + TC::TQ - 1) / TC::TQ, a.NH, a.rows);            \
    const long long blocks = (long long)grid.x * grid.y * grid.z;                      \
    const int resident = g_tiled_resident[dev][HDV == 128][SP][WV == 8];               \
    const int lf = resident > 0 && blocks > resident;                                  \
    hipLaunchKernelGGL((k_flash_tiled<HDV, SP, WV>), grid, dim3(TC::NT), TC::LDS, st, a, kp, vt, LK, lf); \
  }
  if (a.HD == 64) {
    // EXACT: 8-wave blocks unless that grid leaves CUs without a block
    const long long b8 = (long long)((a.tokens_per_row + 255) / 256) * a.NH * a.rows;
    if (!split) EMBER_TILED(64, false, 4)
    else if (b8 >= g_cus[dev]) EMBER_TILED(64, true, 8)
    else EMBER_TILED(64, true, 4)
  } else if (a.HD == 128) {
    if (split) EMBER_TILED(128, true, 4) else EMBER_TILED(128, false, 4)
  } else {
    report_unlaunched("tiled attention: head_dim");
  }
#undef EMBER_TILED
}

}  // namespace ember
