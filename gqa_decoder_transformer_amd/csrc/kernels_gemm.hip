// Prefill GEMM: C[M, N] = A[M, K] . W[N, K]^T with bf16 weights on gfx950 MFMA
// (v_mfma_f32_32x32x16_bf16), f32 accumulation.
//
// A (activations) arrives as bf16 planes written by the producing kernel: in EXACT mode
// x = hi + lo (hi = bf16(x), lo = bf16(x - hi)) and every weight fragment is multiplied
// by both planes, which makes each product f32-accurate to ~2^-17 relative (the weights
// are exactly bf16, and bf16 x bf16 products are exact in f32); in FAST mode only hi.
//
// Two main loops share the tiling and the epilogues. k_gemm: global loads of 16 bytes per
// lane, 8 lanes per 128-byte row segment, PF stages ahead in registers, then stored to an
// LDS of two stages (rows padded by 16 bytes, so the 32 rows a fragment read touches fall
// on distinct banks); it serves every K. k_gemm_dl (K a multiple of 64): the tiles go
// straight from global memory into LDS (below). Block tile BM x BN, K stage 64; each wave
// computes a WM x WN share of it with 32x32x16 MFMAs and reads the fragments of k-step
// t + 1 while the MFMAs of step t run (scheduling groups pin that interleave). Blocks are
// remapped so that the tiles one XCD runs at a time share A rows and weight columns in
// its L2.
//
// Epilogues: store (+bias), residual add (x += C), SiLU*up over the gate/up rows that
// the weight repack interleaves in blocks of 32 (the lane holding gate column j of
// fragment 2q holds the matching up column in fragment 2q + 1), the QKV post-processing
// of a prefill pass for head_dim 64 (bias, q/k RMSNorm, rotate-half RoPE with the pair
// (d, d + 32) in one lane, q out, K/V into the cache), or raw f32 partial tiles for
// split-K. A second weight plane (w_lo: weights that bf16 cannot hold, as a bf16 pair)
// runs as a second pass.
#include "common.h"
#include "kernels.h"

namespace ember {

namespace {

constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;   // bf16 elements per LDS row (128 + 16 bytes)

typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int BM, int BN, bool SPLIT>
constexpr size_t gemm_lds_bytes() {
  return (size_t)2 * ((SPLIT ? 2 : 1) * BM + BN) * LDS_STRIDE * 2;
}

// Epilogue of one wave's TM x TN fragments: element e of fragment (i, j) is C[row][col]
// with row = m0 + wm0 + 32 i + 4 (lane / 32) + 8 (e / 4) + e % 4,
// col = n0 + wn0 + 32 j + lane % 32.
template <int TM, int TN, int EPI>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& a, f32x16_t (&acc)[TM][TN],
                                              const float (&biasv)[TN], int m0, int n0,
                                              int wm0, int wn0, int lane) {
  const int fr = lane % 32;
  // One 64-bit base per fragment, 32-bit row offsets after it (fewer live registers
  // across the whole kernel than a 64-bit product per element).
  const int rb0 = m0 + wm0 + 4 * (lane / 32);
  if (a.partial) {                         // split-K: raw f32 tile into this slice's plane
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = n0 + wn0 + j * 32 + fr;
        const int row0 = rb0 + i * 32;
        float* pb = a.partial + ((size_t)blockIdx.y * a.M + row0) * a.N + col;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int dr = 8 * (e / 4) + e % 4;
          if (col < a.N && row0 + dr < a.M) pb[dr * a.N] = acc[i][j][e];
        }
      }
    return;
  }
  if constexpr (EPI == GEMM_QKV) {
    // head_dim 64: the wave's columns start on a head, so fragment j (even) holds dims
    // 0..31 of head (n0 + wn0 + 32 j) / 64 in this lane's column and fragment j + 1 dims
    // 32..63: the rotate-half pair (d, d + 32) of a row sits in one lane, and the 32 lanes
    // of a half-wave hold one row's 64 dims (the per-head norm is a 5-step lane sum).
    // Heads run q, then k, then v ("ember scripts/reference_forward.py", rope; q/k norm
    // before RoPE: "PII-Tracer serving/reference_forward.py", forward); K and V land at the
    // token's explicit position (ember internals page, "cursor semantics").
    const QkvPostArgs& qp = a.post;
    const int start = qp.d_pos ? *qp.d_pos : qp.start_pos;
#pragma unroll
    for (int j = 0; j < TN; j += 2) {
      const int hcol = n0 + wn0 + 32 * j;
      if (hcol >= a.N) continue;                            // wave-uniform
      const int h = hcol / 64;
      const bool is_q = h < qp.NH, is_v = h >= qp.NH + qp.NKV;
      const float* nw = is_q ? qp.q_norm : qp.k_norm;
      const bool norm = nw != nullptr && !is_v;             // wave-uniform
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row0 = rb0 + i * 32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = row0 + 8 * (e / 4) + e % 4;
          float x0 = acc[i][j][e] + biasv[j], x1 = acc[i][j + 1][e] + biasv[j + 1];
          if (norm) {
            float ss = x0 * x0 + x1 * x1;
#pragma unroll
            for (int o = 1; o < 32; o <<= 1) ss += __shfl_xor(ss, o);
            const float rms = sqrtf(ss / 64.f + qp.eps);
            x0 = x0 / rms * nw[fr];
            x1 = x1 / rms * nw[fr + 32];
          }
          if (row >= a.M) continue;
          const int p = start + row % qp.tokens_per_row;
          float y0 = x0, y1 = x1;
          if (!is_v) {
            const float cs = qp.cos_t[(size_t)p * 32 + fr], sn = qp.sin_t[(size_t)p * 32 + fr];
            y0 = x0 * cs - x1 * sn;
            y1 = x1 * cs + x0 * sn;
          }
          if (is_q) {
            float* dst = qp.q_out + (size_t)row * qp.NH * 64 + h * 64 + fr;
            dst[0] = y0;
            dst[32] = y1;
          } else {
            const int b = qp.b0 + row / qp.tokens_per_row;
            const int kvh = is_v ? h - qp.NH - qp.NKV : h - qp.NH;
            const size_t off = (((size_t)b * qp.NKV + kvh) * qp.max_seq + p) * 64 + fr;
            void* cache = is_v ? qp.v_cache : qp.k_cache;
            if (qp.kv_bf16) {
              ((uint16_t*)cache)[off] = (uint16_t)f32_to_bf16_rne(y0);
              ((uint16_t*)cache)[off + 32] = (uint16_t)f32_to_bf16_rne(y1);
            } else {
              ((float*)cache)[off] = y0;
              ((float*)cache)[off + 32] = y1;
            }
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn0 + j * 32 + fr;
      const int row0 = rb0 + i * 32;
      if (EPI == GEMM_SILU) {
        // fragment j (even) holds gate outputs, fragment j + 1 the matching up outputs
        if (j % 2) continue;
        const int ocol = (col / (2 * kGuBlock)) * kGuBlock + col % kGuBlock;
        const size_t ob = (size_t)row0 * a.ldo + ocol;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int dr = 8 * (e / 4) + e % 4;
          if (row0 + dr >= a.M || col >= a.N) continue;
          const float v = silu(acc[i][j][e]) * acc[i][j + 1][e];
          const size_t o = ob + dr * a.ldo;
          if (a.o_f32) a.o_f32[o] = v;
          if (a.o_hi) {
            uint32_t h, l;
            split_bf16(v, h, l);
            a.o_hi[o] = (uint16_t)h;
            if (a.o_lo) a.o_lo[o] = (uint16_t)l;
          }
        }
      } else {
        float* cb = a.c + (size_t)row0 * a.ldc + col;
        const int ld = (int)a.ldc;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int dr = 8 * (e / 4) + e % 4;
          if (col >= a.N || row0 + dr >= a.M) continue;
          if (EPI == GEMM_RESID) cb[dr * ld] += acc[i][j][e];
          else cb[dr * ld] = acc[i][j][e] + biasv[j];
        }
      }
    }
  }
}

// KG > 1: KG groups of WM x WN waves compute the same tile over consecutive parts of
// its K range, each with its own two LDS stages; the groups' accumulators are summed
// through LDS in group order before the epilogue (occupancy without partial planes).
template <int BM, int BN, int WM, int WN, int PF, bool SPLIT, int EPI, bool TAIL, bool DB = true,
          int KG = 1>
__global__ void __launch_bounds__(WM * WN * KG * kWave) k_gemm(GemmArgs a) {
  constexpr int NT = WM * WN * kWave;                     // threads of one K group
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;    // 32x32 fragments per wave
  constexpr int RS = NT / 8;                              // rows per load round
  constexpr int CA = BM / RS, CB = BN / RS;               // 16-byte loads per plane
  constexpr int NP = SPLIT ? 2 : 1;
  constexpr int PLANE = BM * LDS_STRIDE;                  // A plane size in a stage
  constexpr int STAGE = NP * PLANE + BN * LDS_STRIDE;
  static_assert(CA * RS == BM && CB * RS == BN, "tile rows");
  static_assert(EPI != GEMM_SILU || TN % 2 == 0, "SiLU pairs gate/up fragments");
  static_assert((size_t)(KG - 1) * WM * WN * TM * TN * 16 * kWave * 4 <= (size_t)KG * 2 * STAGE * 2,
                "group reduction fits in the stages");
  extern __shared__ __align__(16) uint16_t smem[];

  // XCD-aware tile order: blocks are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous run of logical tiles. Within the run, tiles go in bands of kBandM M-tiles:
  // a band's M-tiles fastest, then the next N-tile, so the tiles an XCD runs at one time
  // form a band-high window that shares both its A rows and its weight columns in the
  // XCD's L2 (with M-tiles fastest over all of M, as at M = 8192, every N-tile re-read
  // all of A: 33x the operand bytes fetched from the memory side).
  const int mt = (a.M + BM - 1) / BM, nt = (a.N + BN - 1) / BN;
  const int nblk = mt * nt;
  int lin = blockIdx.x;
  if (nblk % 8 == 0) lin = (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
  constexpr int kBandM = 8;
  const int band = lin / (kBandM * nt), m_first = band * kBandM;
  const int band_m = min(mt - m_first, kBandM);
  const int in_band = lin - band * kBandM * nt;
  const int tm = m_first + in_band % band_m, tn = in_band / band_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kg = threadIdx.x / NT, tg = threadIdx.x % NT;  // K group, thread in group
  const int wave = tg / kWave, lane = tg % kWave;
  const int wm0 = (wave / WN) * (BM / WM), wn0 = (wave % WN) * (BN / WN);
  const int fr = lane % 32, fk = (lane / 32) * 8;

  // K range of this block (split-K over gridDim.y slices of k_chunk columns), then of
  // this K group (the host gives every group the same number of stages)
  const int kbb = blockIdx.y * a.k_chunk;
  const int kend = min(a.K, kbb + a.k_chunk);
  const int nk = (kend - kbb + BK - 1) / BK / KG;
  const int kb0 = kbb + kg * nk * BK;

  // this thread's load rows (clamped: rows past M/N are loaded but never stored) and
  // its 8-element k chunk within a stage
  const int r0 = tg / 8, kc = (tg % 8) * 8;
  const uint16_t* pa_hi = a.a_hi + (size_t)min(m0 + r0, a.M - 1) * a.lda + kc;
  const uint16_t* pa_lo = SPLIT ? a.a_lo + (size_t)min(m0 + r0, a.M - 1) * a.lda + kc : nullptr;
  const uint16_t* pw = a.w + (size_t)min(n0 + r0, a.N - 1) * a.K + kc;
  int oa[CA], ob[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) oa[i] = (min(m0 + r0 + RS * i, a.M - 1) - min(m0 + r0, a.M - 1)) * a.lda;
#pragma unroll
  for (int i = 0; i < CB; ++i) ob[i] = (min(n0 + r0 + RS * i, a.N - 1) - min(n0 + r0, a.N - 1)) * a.K;
  const int lofs = r0 * LDS_STRIDE + kc;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  // the bias of this lane's output columns, read before the main loop (a load in the
  // epilogue raised the register pressure of the whole kernel)
  float biasv[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j)
    biasv[j] = ((EPI == GEMM_STORE || EPI == GEMM_QKV) && a.bias && !a.partial)
                   ? a.bias[min(n0 + wn0 + j * 32 + fr, a.N - 1)] : 0.f;

  u32x4_t rh[PF][CA], rl[PF][SPLIT ? CA : 1], rw[PF][CB];
  bool okb[PF];
  // stage t of this block: k0 = kb0 + 64 t. With TAIL (K range not a multiple of 64) a
  // chunk wholly past the range is zeroed when it is stored to LDS (K is a multiple of
  // 8, so a chunk is either inside or past it); without it no select touches the data.
  auto gload = [&](int b, int t) {
    const int k0 = kb0 + t * BK;
    const bool ok = !TAIL || k0 + kc < kend;
    const int kk = ok ? k0 : kb0;
    okb[b] = ok;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      rh[b][i] = *(const u32x4_t*)(pa_hi + oa[i] + kk);
      if (SPLIT) rl[b][i] = *(const u32x4_t*)(pa_lo + oa[i] + kk);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) rw[b][i] = *(const u32x4_t*)(pw + ob[i] + kk);
  };
  uint16_t* const sg = smem + kg * 2 * STAGE;             // this group's two stages
  auto sstore = [&](int b, int s) {
    uint16_t* base = sg + s * STAGE + lofs;
    const u32x4_t z = {0, 0, 0, 0};
    const bool ok = okb[b];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      *(u32x4_t*)(base + RS * i * LDS_STRIDE) = !TAIL || ok ? rh[b][i] : z;
      if (SPLIT) *(u32x4_t*)(base + PLANE + RS * i * LDS_STRIDE) = !TAIL || ok ? rl[b][i] : z;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i)
      *(u32x4_t*)(base + NP * PLANE + RS * i * LDS_STRIDE) = !TAIL || ok ? rw[b][i] : z;
  };
  constexpr int NF = DB ? 2 : 1;                          // fragment buffers
  bf16x8_t fh[NF][TM], fl[NF][SPLIT ? TM : 1], fw[NF][TN];
  auto rdfrag = [&](int f, int s, int ks) {
    const uint16_t* st = sg + s * STAGE;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int o = (wm0 + i * 32 + fr) * LDS_STRIDE + ks + fk;
      fh[f][i] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(st + o));
      if (SPLIT) fl[f][i] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(st + PLANE + o));
    }
#pragma unroll
    for (int j = 0; j < TN; ++j)
      fw[f][j] = __builtin_bit_cast(bf16x8_t,
                                    *(const u32x4_t*)(st + NP * PLANE + (wn0 + j * 32 + fr) * LDS_STRIDE + ks + fk));
  };
  auto mfmas = [&](int f) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fh[f][i], fw[f][j], acc[i][j], 0, 0, 0);
        if (SPLIT)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fl[f][i], fw[f][j], acc[i][j], 0, 0, 0);
      }
  };
  constexpr int NMF = NP * TM * TN, NRD = NP * TM + TN, NLD = NP * CA + CB;

  // prologue: stages 0 .. PF-1 in flight (past the end: the last stage again), stage 0
  // stored
#pragma unroll
  for (int b = 0; b < PF; ++b) gload(b, min(b, nk - 1));
  sstore(0, 0);
  __syncthreads();
  for (int k0 = 0; k0 < nk; k0 += PF) {
#pragma unroll
    for (int ph = 0; ph < PF; ++ph) {
      const int k = k0 + ph;                   // stage computed now, from LDS k & 1
      const int s = k & 1;
      gload(ph, min(k + PF, nk - 1));          // the registers of stage k are free
      rdfrag(0, s, 0);
#pragma unroll
      for (int t = 0; t < BK / 16; ++t) {
        if (DB) {
          if (t + 1 < BK / 16) rdfrag((t + 1) & 1, s, (t + 1) * 16);
          mfmas(t & 1);
        } else {
          // one fragment buffer: the next step's reads overwrite it behind these MFMAs
          mfmas(0);
          if (t + 1 < BK / 16) rdfrag(0, s, (t + 1) * 16);
        }
      }
      sstore((ph + 1) % PF, s ^ 1);            // stage k + 1 (past the end: unused)
      __builtin_amdgcn_sched_group_barrier(0x020, NLD, 0);        // global loads
      __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);        // step-0 fragments
#pragma unroll
      for (int t = 0; t < BK / 16 - 1; ++t)
#pragma unroll
        for (int r = 0; r < NRD; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, NMF / NRD > 0 ? NMF / NRD : 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
      for (int r = 0; r < NLD; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, NMF / NLD > 0 ? NMF / NLD : 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      }
      __syncthreads();
      if (k + 1 >= nk) break;
    }
  }

  if constexpr (KG > 1) {
    // groups 1.. hand their accumulators to group 0 through LDS (the stages are free)
    float* red = (float*)smem;                  // [group - 1][wave][i][j][e][lane]
    __syncthreads();
    if (kg > 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            red[(((((size_t)(kg - 1) * WM * WN + wave) * TM + i) * TN + j) * 16 + e) * kWave + lane] =
                acc[i][j][e];
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int g = 1; g < KG; ++g)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            acc[i][j][e] += red[(((((size_t)(g - 1) * WM * WN + wave) * TM + i) * TN + j) * 16 + e) * kWave + lane];
  }

  gemm_epilogue<TM, TN, EPI>(a, acc, biasv, m0, n0, wm0, wn0, lane);
}

// ------------------------------------------------------------------ direct-to-LDS main loop
// The operand tiles go from global memory straight into LDS with global_load_lds_dwordx4
// (each lane's 16 bytes land at the wave's LDS address + 16 x lane), NS stages deep: no
// register staging, no LDS store instructions, and the loads of NS - 1 stages in flight
// behind the MFMAs. One wave-wide load moves RPI whole rows of a BK-column stage. Rows are
// unpadded (a wave-wide load is 1 KB of consecutive LDS), so the 16-byte chunks of a row
// are stored XOR-swizzled: chunk c of stage row r sits in slot c ^ swz(r). A 16-byte LDS
// read is served in four passes of 16 lanes over 64 four-byte banks (256 bytes), and a
// fragment read has 16 consecutive rows in a pass at one logical chunk: with 128-byte
// rows, rows r and r + 1 differ in the bank half and swz(r) = (r / 2) mod 8 gives the
// eight row pairs distinct slots (r mod 8 put rows r and r + 8 on the same banks: 4.0
// conflict cycles per LDS instruction, measured). One barrier per stage: a stage's slot is
// refilled only after every wave has passed the barrier that follows its use.
template <int BK>
EMBER_DEV int dl_swz(int r) { return BK == 64 ? ((r >> 1) & 7) : ((r >> 2) & 3); }

// s_waitcnt immediate: vector-memory count <= n, the other counters unconstrained
constexpr int vmcnt_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4) | (15 << 8); }

// wait until at most min(younger, Y) stages of NI loads each are in flight (immediate
// operands: one s_waitcnt per possible count); LGKM: also every LDS read done
template <int NI, int Y, bool LGKM>
EMBER_DEV void wait_stages(int younger) {
  constexpr int lg = LGKM ? ~(15 << 8) : ~0;
  if constexpr (Y <= 0) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & lg);
  } else {
    if (younger >= Y) __builtin_amdgcn_s_waitcnt(vmcnt_imm(Y * NI) & lg);
    else wait_stages<NI, Y - 1, LGKM>(younger);
  }
}

template <int BM, int BN, int WM, int WN, int BK, int NS, int NP, int EPI>
__global__ void __launch_bounds__(WM * WN * kWave) k_gemm_dl(GemmArgs a) {
  // NP activation planes: hi (1), + lo (2), + x2 (3: a_x2, the EXACT QKV input)
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;     // 32x32 fragments per wave
  constexpr int CPR = BK / 8, RPI = kWave / CPR;          // chunks per row, rows per load
  constexpr int ROWS = NP * BM + BN;                      // stage rows: A planes, then W
  constexpr int IA = BM / (RPI * NW), NI = ROWS / (RPI * NW);
  constexpr int STAGE = ROWS * BK;                        // bf16 elements
  static_assert(BK == 32 || BK == 64, "stage width");
  static_assert(BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "a load stays in one operand");
  static_assert(NS >= 2 && (NS - 1) * NI <= 63, "stages in flight within the vmcnt range");
  static_assert(EPI != GEMM_SILU || TN % 2 == 0, "SiLU pairs gate/up fragments");
  extern __shared__ __align__(16) uint16_t smem[];

  // XCD-aware band order of the tiles (as in k_gemm)
  const int mt = (a.M + BM - 1) / BM, nt = (a.N + BN - 1) / BN;
  const int nblk = mt * nt;
  int lin = blockIdx.x;
  if (nblk % 8 == 0) lin = (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
  constexpr int kBandM = 8;
  const int band = lin / (kBandM * nt), m_first = band * kBandM;
  const int band_m = min(mt - m_first, kBandM);
  const int in_band = lin - band * kBandM * nt;
  const int tm = m_first + in_band % band_m, tn = in_band / band_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int wm0 = (wave / WN) * (BM / WM), wn0 = (wave % WN) * (BN / WN);
  const int fr = lane % 32;

  // K range of this block (split-K slices of k_chunk columns; whole stages)
  const int kb0 = blockIdx.y * a.k_chunk;
  const int nk = (min(a.K, kb0 + a.k_chunk) - kb0) / BK;

  // load i of a stage covers stage rows (i NW + wave) RPI .. + RPI; this lane takes row
  // lr of them and stores its chunk in slot ls, so it loads chunk ls ^ swz(row)
  const int lr = lane / CPR, ls = lane % CPR;
  uint32_t off[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int srow = (i * NW + wave) * RPI + lr;
    const int c = ls ^ dl_swz<BK>(srow);
    if (i < NP * IA) {
      const int r = srow - (i / IA) * BM;
      off[i] = (uint32_t)min(m0 + r, a.M - 1) * (uint32_t)a.lda + c * 8;
    } else {
      const int r = srow - NP * BM;
      off[i] = (uint32_t)min(n0 + r, a.N - 1) * (uint32_t)a.K + c * 8;
    }
  }
  auto issue = [&](int slot, int t) {
    const int k0 = kb0 + t * BK;
    uint16_t* st = smem + slot * STAGE;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint16_t* base = i < IA ? a.a_hi : (NP > 1 && i < 2 * IA) ? a.a_lo
                                             : (NP > 2 && i < 3 * IA) ? a.a_x2 : a.w;
      auto* dst = (__attribute__((address_space(3))) void*)(st + (i * NW + wave) * RPI * BK);
      // the 64 x 64 form serves GEMMs of at most 128 rows, whose weights are read once:
      // their loads carry the non-temporal hint
      if (BM == 64 && i >= NP * IA)
        __builtin_amdgcn_global_load_lds((const void*)(base + off[i] + k0), dst, 16, 0, 2);
      else
        __builtin_amdgcn_global_load_lds((const void*)(base + off[i] + k0), dst, 16, 0, 0);
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  float biasv[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j)
    biasv[j] = ((EPI == GEMM_STORE || EPI == GEMM_QKV) && a.bias && !a.partial)
                   ? a.bias[min(n0 + wn0 + j * 32 + fr, a.N - 1)] : 0.f;

  // fragment reads: A fragment i is stage row wm0 + 32 i + fr, W fragment j stage row
  // NP BM + wn0 + 32 j + fr; k-step kk reads logical chunk 2 kk + lane / 32 (these rows
  // start on multiples of 32, so their swizzle depends on fr alone)
  const int sw = dl_swz<BK>(fr);
  int cofs[BK / 16];
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) cofs[kk] = ((2 * kk + lane / 32) ^ sw) * 8;
  const int arow = (wm0 + fr) * BK, wrow = (NP * BM + wn0 + fr) * BK;
  bf16x8_t fh[2][TM], fl[2][NP > 1 ? TM : 1], fx[2][NP > 2 ? TM : 1], fw[2][TN];
  auto rdfrag = [&](int f, const uint16_t* st, int kk) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      fh[f][i] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(st + arow + i * 32 * BK + cofs[kk]));
      if (NP > 1)
        fl[f][i] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(st + BM * BK + arow + i * 32 * BK + cofs[kk]));
      if (NP > 2)
        fx[f][i] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(st + 2 * BM * BK + arow + i * 32 * BK + cofs[kk]));
    }
#pragma unroll
    for (int j = 0; j < TN; ++j)
      fw[f][j] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(st + wrow + j * 32 * BK + cofs[kk]));
  };
  auto mfmas = [&](int f) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fh[f][i], fw[f][j], acc[i][j], 0, 0, 0);
        if (NP > 1)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fl[f][i], fw[f][j], acc[i][j], 0, 0, 0);
        if (NP > 2)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fx[f][i], fw[f][j], acc[i][j], 0, 0, 0);
      }
  };

  // Stage t sits in slot t % NS. The barrier between stages t and t + 1 comes after every
  // wave has read all of stage t (lgkmcnt 0) and seen stage t + 1 land (vmcnt); behind it
  // the wave refills slot t % NS with stage t + NS, reads stage t + 1's first fragments
  // and only then issues stage t's last MFMAs, so no wave restarts with an empty pipe.
  constexpr int KS = BK / 16;
  constexpr int NMF = NP * TM * TN, NRD = NP * TM + TN;   // MFMAs, fragment reads per k-step
  static_assert(KS % 2 == 0, "stage t + 1 starts in fragment buffer 0");
#pragma unroll
  for (int p = 0; p < NS; ++p)
    if (p < nk) issue(p, p);
  int slot = 0;
  if (nk > 0) {
    // stage 0 has landed once at most min(NS, nk) - 1 younger stages are in flight
    wait_stages<NI, NS - 1, false>(min(NS, nk) - 1);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    rdfrag(0, smem, 0);
  }
  for (int t = 0; t < nk; ++t) {
    const uint16_t* st = smem + slot * STAGE;
#pragma unroll
    for (int kk = 0; kk + 1 < KS; ++kk) {
      rdfrag((kk + 1) & 1, st, kk + 1);
      mfmas(kk & 1);
    }
    // one fragment read of the next k-step after every NMF / NRD MFMAs of this one
#pragma unroll
    for (int kk = 0; kk + 1 < KS; ++kk)
#pragma unroll
      for (int r = 0; r < NRD; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, NMF / NRD > 0 ? NMF / NRD : 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    const int nslot = slot + 1 == NS ? 0 : slot + 1;
    {
      // stages t + 2 .. min(t + NS - 1, nk - 1) may stay in flight (after the last stage
      // nothing is in flight; its barrier and reads are harmless: the reads fetch a slot's
      // stale data and are never used)
      wait_stages<NI, NS - 2, true>(min(NS - 2, nk - 2 - t));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      // the last k-step's fragments pass through an empty asm statement behind the
      // barrier: its MFMAs cannot be scheduled above it
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        asm volatile("" : "+v"(fh[(KS - 1) & 1][i]));
        if (NP > 1) asm volatile("" : "+v"(fl[(KS - 1) & 1][i]));
        if (NP > 2) asm volatile("" : "+v"(fx[(KS - 1) & 1][i]));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) asm volatile("" : "+v"(fw[(KS - 1) & 1][j]));
      if (t + NS < nk) issue(slot, t + NS);
      rdfrag(0, smem + nslot * STAGE, 0);
    }
    mfmas((KS - 1) & 1);
#pragma unroll
    for (int r = 0; r < NRD; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, NMF / NRD > 0 ? NMF / NRD : 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    slot = nslot;
  }
  gemm_epilogue<TM, TN, EPI>(a, acc, biasv, m0, n0, wm0, wn0, lane);
}

template <int BM, int BN, int BK, int NS, int NP>
constexpr size_t gemm_dl_lds_bytes() {
  return (size_t)NS * (NP * BM + BN) * BK * 2;
}

// Tile configurations: block BM x BN, WM x WN waves, register prefetch depth PF, KG
// groups of waves over the K range.
enum GemmCfg { CFG_128x256 = 1, CFG_128x128 = 2, CFG_64x128 = 3, CFG_256x256 = 4, CFG_64x64 = 5,
               CFG_128x128_K2 = 6, CFG_128x256_W8 = 7,
               // direct-to-LDS main loop (k_gemm_dl), BK 64, two stages
               CFG_DL_256x256 = 8,        // one plane: 8 waves of 128 x 64
               CFG_DL_S128x256 = 9,       // two planes: 8 waves of 64 x 64
               CFG_DL_64x64 = 10,         // 2 waves of 32 x 64, three stages (two: three planes)
               CFG_DL_64x256 = 11,        // two planes, M <= 64: 4 waves of 64 x 64, three stages
               CFG_DL_128x128 = 12 };     // two planes: 4 waves of 64 x 64, three stages

template <int BM, int BN, int WM, int WN, int PF, bool SPLIT, int EPI, int KG = 1>
void set_attr() {
  (void)hipFuncSetAttribute((const void*)k_gemm<BM, BN, WM, WN, PF, SPLIT, EPI, false, true, KG>,
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(KG * gemm_lds_bytes<BM, BN, SPLIT>()));
  (void)hipFuncSetAttribute((const void*)k_gemm<BM, BN, WM, WN, PF, SPLIT, EPI, true, true, KG>,
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(KG * gemm_lds_bytes<BM, BN, SPLIT>()));
}

template <int BM, int BN, int WM, int WN, int PF, bool SPLIT, int EPI, int KG = 1>
void launch_cfg(const GemmArgs& a, int splits, hipStream_t st) {
  const int blocks = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const size_t lds = KG * gemm_lds_bytes<BM, BN, SPLIT>();
  // every K slice a whole number of 64-column stages: no tail handling
  const bool tail = a.K % BK != 0 || a.k_chunk % BK != 0;
  if (tail)
    hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, PF, SPLIT, EPI, true, true, KG>), dim3(blocks, splits),
                       dim3(WM * WN * KG * kWave), lds, st, a);
  else
    hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, PF, SPLIT, EPI, false, true, KG>), dim3(blocks, splits),
                       dim3(WM * WN * KG * kWave), lds, st, a);
}

template <int BM, int BN, int WM, int WN, int BK, int NS, int NP, int EPI>
void set_attr_dl() {
  static_assert(gemm_dl_lds_bytes<BM, BN, BK, NS, NP>() <= 160 * 1024, "LDS of one CU");
  (void)hipFuncSetAttribute((const void*)k_gemm_dl<BM, BN, WM, WN, BK, NS, NP, EPI>,
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)gemm_dl_lds_bytes<BM, BN, BK, NS, NP>());
}

template <int BM, int BN, int WM, int WN, int BK, int NS, int NP, int EPI>
void launch_dl(const GemmArgs& a, int splits, hipStream_t st) {
  const int blocks = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  constexpr size_t lds = gemm_dl_lds_bytes<BM, BN, BK, NS, NP>();
  hipLaunchKernelGGL((k_gemm_dl<BM, BN, WM, WN, BK, NS, NP, EPI>), dim3(blocks, splits),
                     dim3(WM * WN * kWave), lds, st, a);
}

int tiles_of(const GemmArgs& a, int bm, int bn) {
  return ((a.M + bm - 1) / bm) * ((a.N + bn - 1) / bn);
}

// A 32x32x16 MFMA of a wave tile of TM x TN fragments reads (TM + TN) / (TM TN) fragments
// of 1 KB from LDS, so small wave tiles are bound by LDS bandwidth: one-plane input takes
// 256 x 256 tiles over 8 waves (128 x 64 each, two waves per SIMD) when they make at
// least one tile per CU (measured faster there at every K), else 128 x 128; the
// two-plane (EXACT) input (a third LDS plane) takes 128 x 256 when that leaves ~0.7
// tiles per CU. M <= 128 (batched decode, short prompts) takes 64 x 64 tiles over 2
// waves: at M = 128 they fill the GPU without the split-K planes and reduce that
// 128 x 128 tiles need (0.5B prefill GEMMs 10-20 % faster).
int pick_cfg(const GemmArgs& a) {
  // K in whole 64-column stages: the tile forms load straight from global memory into
  // LDS (k_gemm_dl; 4-10 % faster than register staging on the 1B-shape GEMMs)
  const bool dl = a.K % BK == 0;
  // a wide two-plane GEMM of at most 64 rows (the EXACT LM head of a decode batch): a
  // 64 x 64 tile reads its two activation planes from L2 at twice its weight bytes, a
  // 64 x 256 tile at half (64-row LM head 155 -> 138 us; with one plane, or with 64 x 128
  // tiles on the 16384-column gate/up, no faster)
  if (a.M <= 64 && dl && a.a_lo && !a.a_x2 && tiles_of(a, 64, 64) >= 1024) return CFG_DL_64x256;
  // the 64 x 64 direct-to-LDS form when its blocks fit the CUs (more tiles, as in the
  // one-plane LM head or a 128-row gate/up, run faster register staged); three stages
  // (72 KB of LDS, 48 KB with one plane) run as fast as six or eight and leave room for
  // a second block per CU (64-row EXACT decode layer 91.2 -> 87.8 us, FAST 80.0 -> 76.8)
  if (a.M <= 128) return dl && tiles_of(a, 64, 64) <= 256 ? CFG_DL_64x64 : CFG_64x64;
  // two-plane input: 128 x 256 tiles over 8 waves of 64 x 64 (two waves per SIMD; over 4
  // waves of 64 x 128 the accumulators and fragments held a wave to one per SIMD); with
  // fewer such tiles, 128 x 128 straight into LDS over three stages (the 1B shape's output
  // and down projections at M = 2048: 53.5 -> 51 us and 152-160 -> 142 us against register
  // staging; with one plane the same form was slower, the QKV projection 50 -> 69 us)
  if (a.a_lo) {
    if (tiles_of(a, 128, 256) >= 180) return dl ? CFG_DL_S128x256 : CFG_128x256_W8;
    return dl ? CFG_DL_128x128 : CFG_128x128;
  }
  if (tiles_of(a, 256, 256) >= 256) return dl ? CFG_DL_256x256 : CFG_256x256;
  // long K against N (the down projection at M = 2048): 256 x 256 tiles over four K
  // slices, whose partial planes cost less than the halved operand traffic saves there
  // (measured slower for K <= N)
  if (a.partial && a.K >= 4 * a.N && a.K >= 4096 && tiles_of(a, 256, 256) >= 64 &&
      (size_t)4 * a.M * a.N <= a.partial_elems)
    return dl ? CFG_DL_256x256 : CFG_256x256;
  // about one 128 x 128 tile per CU: two K groups per tile (two waves per SIMD) when the
  // stages split evenly
  const int t128 = tiles_of(a, 128, 128);
  if (t128 >= 192 && t128 <= 256 && a.K % (2 * BK) == 0) return CFG_128x128_K2;
  return CFG_128x128;
}

void cfg_dims(int cfg, int& bm, int& bn) {
  switch (cfg) {
    case CFG_256x256: bm = 256; bn = 256; break;
    case CFG_128x256: case CFG_128x256_W8: case CFG_DL_S128x256: bm = 128; bn = 256; break;
    case CFG_DL_256x256: bm = 256; bn = 256; break;
    case CFG_128x128: case CFG_128x128_K2: bm = 128; bn = 128; break;
    case CFG_64x64: case CFG_DL_64x64: bm = 64; bn = 64; break;
    case CFG_DL_64x256: bm = 64; bn = 256; break;
    case CFG_DL_128x128: bm = 128; bn = 128; break;
    default: bm = 64; bn = 128; break;
  }
}

template <bool SPLIT, int EPI>
void launch_split(const GemmArgs& a, int cfg, int splits, hipStream_t st) {
  switch (cfg) {
    case CFG_256x256:
      if constexpr (!SPLIT) launch_cfg<256, 256, 2, 4, 1, false, EPI>(a, splits, st);
      else report_unlaunched("GEMM: one-plane tile form with two planes");
      break;
    case CFG_128x256: launch_cfg<128, 256, 2, 2, 2, SPLIT, EPI>(a, splits, st); break;
    case CFG_128x256_W8: launch_cfg<128, 256, 2, 4, 2, SPLIT, EPI>(a, splits, st); break;
    case CFG_128x128: launch_cfg<128, 128, 2, 2, 2, SPLIT, EPI>(a, splits, st); break;
    case CFG_128x128_K2:
      if constexpr (!SPLIT) launch_cfg<128, 128, 2, 2, 2, false, EPI, 2>(a, splits, st);
      else report_unlaunched("GEMM: one-plane tile form with two planes");
      break;
    case CFG_64x64: launch_cfg<64, 64, 2, 1, 4, SPLIT, EPI>(a, splits, st); break;
    case CFG_DL_256x256:
      if constexpr (!SPLIT) launch_dl<256, 256, 2, 4, 64, 2, 1, EPI>(a, splits, st);
      else report_unlaunched("GEMM: one-plane tile form with two planes");
      break;
    case CFG_DL_S128x256:
      if constexpr (SPLIT) launch_dl<128, 256, 2, 4, 64, 2, 2, EPI>(a, splits, st);
      else report_unlaunched("GEMM: two-plane tile form with one plane");
      break;
    case CFG_DL_64x64:
      if constexpr (SPLIT) launch_dl<64, 64, 2, 1, 64, 3, 2, EPI>(a, splits, st);
      else launch_dl<64, 64, 2, 1, 64, 3, 1, EPI>(a, splits, st);
      break;
    case CFG_DL_64x256:
      if constexpr (SPLIT) launch_dl<64, 256, 1, 4, 64, 3, 2, EPI>(a, splits, st);
      else report_unlaunched("GEMM: two-plane tile form with one plane");
      break;
    case CFG_DL_128x128:
      if constexpr (SPLIT) launch_dl<128, 128, 2, 2, 64, 3, 2, EPI>(a, splits, st);
      else report_unlaunched("GEMM: two-plane tile form with one plane");
      break;
    default: launch_cfg<64, 128, 2, 2, 2, SPLIT, EPI>(a, splits, st); break;
  }
}

// three activation planes (EXACT QKV input): the direct-to-LDS forms only, with the store
// or the QKV post-processing epilogue
template <int EPI>
void launch_three(const GemmArgs& a, int cfg, int splits, hipStream_t st) {
  if constexpr (EPI == GEMM_STORE || EPI == GEMM_QKV) {
    if (cfg == CFG_DL_S128x256) {
      launch_dl<128, 256, 2, 4, 64, 2, 3, EPI>(a, splits, st);
      return;
    }
    if (cfg == CFG_DL_64x64) {
      launch_dl<64, 64, 2, 1, 64, 2, 3, EPI>(a, splits, st);
      return;
    }
  }
  report_unlaunched("GEMM: three activation planes in this tile form or epilogue");
}

template <int EPI>
void launch_epi(const GemmArgs& a, int cfg, int splits, hipStream_t st) {
  if (a.a_x2) launch_three<EPI>(a, cfg, splits, st);
  else if (a.a_lo) launch_split<true, EPI>(a, cfg, splits, st);
  else launch_split<false, EPI>(a, cfg, splits, st);
}

template <bool SPLIT, int EPI>
void set_attrs_split() {
  if constexpr (!SPLIT) {
    set_attr<256, 256, 2, 4, 1, false, EPI>();
    set_attr<128, 128, 2, 2, 2, false, EPI, 2>();
  }
  set_attr<128, 256, 2, 2, 2, SPLIT, EPI>();
  set_attr<128, 256, 2, 4, 2, SPLIT, EPI>();
  set_attr<128, 128, 2, 2, 2, SPLIT, EPI>();
  set_attr<64, 128, 2, 2, 2, SPLIT, EPI>();
  set_attr<64, 64, 2, 1, 4, SPLIT, EPI>();
  if constexpr (!SPLIT) {
    set_attr_dl<256, 256, 2, 4, 64, 2, 1, EPI>();
    set_attr_dl<64, 64, 2, 1, 64, 3, 1, EPI>();
  } else {
    set_attr_dl<128, 256, 2, 4, 64, 2, 2, EPI>();
    set_attr_dl<64, 64, 2, 1, 64, 3, 2, EPI>();
    set_attr_dl<64, 256, 1, 4, 64, 3, 2, EPI>();
    set_attr_dl<128, 128, 2, 2, 64, 3, 2, EPI>();
  }
}

template <int EPI>
void set_attrs_epi() {
  set_attrs_split<false, EPI>();
  set_attrs_split<true, EPI>();
}

// Fixed-order sum of the split-K partial planes, then the epilogue.
template <int EPI>
__global__ void __launch_bounds__(256) k_splitk_reduce(GemmArgs a, int splits) {
  const int nout = EPI == GEMM_SILU ? a.N / 2 : a.N;
  const size_t total = (size_t)a.M * nout;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const int row = (int)(e / nout), col = (int)(e % nout);
    if (EPI == GEMM_SILU) {
      const int gcol = gu_row(col, 0), ucol = gu_row(col, 1);
      float g = 0.f, u = 0.f;
      for (int s = 0; s < splits; ++s) {
        const float* pp = a.partial + (size_t)s * a.M * a.N + (size_t)row * a.N;
        g += pp[gcol];
        u += pp[ucol];
      }
      const float v = silu(g) * u;
      const size_t o = (size_t)row * a.ldo + col;
      if (a.o_f32) a.o_f32[o] = v;
      if (a.o_hi) {
        uint32_t h, l;
        split_bf16(v, h, l);
        a.o_hi[o] = (uint16_t)h;
        if (a.o_lo) a.o_lo[o] = (uint16_t)l;
      }
    } else {
      float acc = 0.f;
      for (int s = 0; s < splits; ++s) acc += a.partial[(size_t)s * a.M * a.N + (size_t)row * a.N + col];
      float* cp = a.c + (size_t)row * a.ldc + col;
      if (EPI == GEMM_RESID) *cp += acc;
      else *cp = acc + (a.bias ? a.bias[col] : 0.f);
    }
  }
}

// The same sum four columns per thread (16-byte partial loads and output stores) when
// every row length and output pointer allows it; same split order.
template <int EPI>
__global__ void __launch_bounds__(256) k_splitk_reduce4(GemmArgs a, int splits) {
  const int nout = EPI == GEMM_SILU ? a.N / 2 : a.N;
  const int nq = nout / 4;
  const size_t total = (size_t)a.M * nq;
  const size_t plane = (size_t)a.M * a.N;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const int row = (int)(e / nq), col = (int)(e % nq) * 4;
    if (EPI == GEMM_SILU) {
      // four outputs of one block of 32 read four consecutive gate and up columns
      const float* pg = a.partial + (size_t)row * a.N + gu_row(col, 0);
      const float* pu = a.partial + (size_t)row * a.N + gu_row(col, 1);
      float4 g = ld_stream_f4(pg), u = ld_stream_f4(pu);   // partial planes: read once
      for (int s = 1; s < splits; ++s) {
        const float4 gs = ld_stream_f4(pg + s * plane), us = ld_stream_f4(pu + s * plane);
        g.x += gs.x; g.y += gs.y; g.z += gs.z; g.w += gs.w;
        u.x += us.x; u.y += us.y; u.z += us.z; u.w += us.w;
      }
      const float v[4] = {silu(g.x) * u.x, silu(g.y) * u.y, silu(g.z) * u.z, silu(g.w) * u.w};
      const size_t o = (size_t)row * a.ldo + col;
      if (a.o_f32) *(float4*)(a.o_f32 + o) = make_float4(v[0], v[1], v[2], v[3]);
      if (a.o_hi) {
        uint32_t h[4], l[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) split_bf16(v[i], h[i], l[i]);
        *(uint2*)(a.o_hi + o) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        if (a.o_lo) *(uint2*)(a.o_lo + o) = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
      }
    } else {
      const float* pp = a.partial + (size_t)row * a.N + col;
      float4 acc = ld_stream_f4(pp);                     // partial planes: read once
      for (int s = 1; s < splits; ++s) {
        const float4 ps = ld_stream_f4(pp + s * plane);
        acc.x += ps.x; acc.y += ps.y; acc.z += ps.z; acc.w += ps.w;
      }
      float4* cp = (float4*)(a.c + (size_t)row * a.ldc + col);
      if (EPI == GEMM_RESID) {
        const float4 c0 = *cp;
        *cp = make_float4(c0.x + acc.x, c0.y + acc.y, c0.z + acc.z, c0.w + acc.w);
      } else {
        const float4 bv = a.bias ? *(const float4*)(a.bias + col) : make_float4(0.f, 0.f, 0.f, 0.f);
        *cp = make_float4(acc.x + bv.x, acc.y + bv.y, acc.z + bv.z, acc.w + bv.w);
      }
    }
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Split K when the tiles cannot fill the GPU: slices of >= 256 columns, about 512 blocks
// (256 for the 64 x 64 tiles of small M, whose blocks each stream their weights, and for 256 x 256
// tiles, whose slices keep >= 1024 columns: every split adds an f32 partial plane to write
// and reduce).
int pick_splits(const GemmArgs& a, int cfg) {
  if (!a.partial) return 1;
  int bm, bn;
  cfg_dims(cfg, bm, bn);
  const int tiles = tiles_of(a, bm, bn);
  if (tiles >= 192) return 1;
  const bool big = bm == 256 && bn == 256;
  const int target = (bm == 64 && bn == 64) || big ? 256 : 512;
  int s = (target + tiles - 1) / tiles;
  const int max_s = a.K / (big ? 1024 : 256);
  if (s > max_s) s = max_s;
  if ((size_t)s * a.M * a.N > a.partial_elems) s = (int)(a.partial_elems / ((size_t)a.M * a.N));
  return s < 2 ? 1 : s;
}

// ------------------------------------------------------------------ f32-weight VALU GEMM
// For models stored in f32 (the tiny configuration): one thread per output (pair), f32 FMA.
template <int EPI>
__global__ void __launch_bounds__(256) k_gemm_f32w(GemmF32Args a) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  const int m = blockIdx.y;
  const int nout = (EPI == GEMM_SILU) ? a.N / 2 : a.N;
  if (n >= nout || m >= a.M) return;
  const float* x = a.a + (size_t)m * a.lda;
  if (EPI == GEMM_SILU) {
    const int rg = gu_row(n, 0), ru = gu_row(n, 1);
    float g = 0.f, u = 0.f;
    for (int k = 0; k < a.K; ++k) {
      g = fmaf(a.w[(size_t)rg * a.K + k], x[k], g);
      u = fmaf(a.w[(size_t)ru * a.K + k], x[k], u);
    }
    a.o_f32[(size_t)m * a.ldo + n] = silu(g) * u;
    return;
  }
  float acc = 0.f;
  for (int k = 0; k < a.K; ++k) acc = fmaf(a.w[(size_t)n * a.K + k], x[k], acc);
  float* cp = a.c + (size_t)m * a.ldc + n;
  if (EPI == GEMM_RESID) *cp += acc;
  else *cp = acc + (a.bias ? a.bias[n] : 0.f);
}

// Fixed-order sum of `used` partial planes with the epilogue.
void launch_reduce(const GemmArgs& a, int epi, int used, hipStream_t st) {
  const int nout = epi == GEMM_SILU ? a.N / 2 : a.N;
  const bool vec = a.N % 4 == 0 && nout % 4 == 0 && aligned16(a.partial) &&
                   (epi == GEMM_SILU ? (a.ldo % 4 == 0 && aligned16(a.o_f32) && aligned16(a.o_hi) &&
                                        aligned16(a.o_lo))
                                     : (a.ldc % 4 == 0 && aligned16(a.c) && aligned16(a.bias)));
  if (vec) {
    long long blocks = ((long long)a.M * (nout / 4) + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    switch (epi) {
      case GEMM_STORE: hipLaunchKernelGGL(k_splitk_reduce4<GEMM_STORE>, dim3((unsigned)blocks), dim3(256), 0, st, a, used); break;
      case GEMM_RESID: hipLaunchKernelGGL(k_splitk_reduce4<GEMM_RESID>, dim3((unsigned)blocks), dim3(256), 0, st, a, used); break;
      case GEMM_SILU: hipLaunchKernelGGL(k_splitk_reduce4<GEMM_SILU>, dim3((unsigned)blocks), dim3(256), 0, st, a, used); break;
      default: report_unlaunched("split-K reduce: epilogue"); break;
    }
    return;
  }
  long long blocks = ((long long)a.M * nout + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  switch (epi) {
    case GEMM_STORE: hipLaunchKernelGGL(k_splitk_reduce<GEMM_STORE>, dim3((unsigned)blocks), dim3(256), 0, st, a, used); break;
    case GEMM_RESID: hipLaunchKernelGGL(k_splitk_reduce<GEMM_RESID>, dim3((unsigned)blocks), dim3(256), 0, st, a, used); break;
    case GEMM_SILU: hipLaunchKernelGGL(k_splitk_reduce<GEMM_SILU>, dim3((unsigned)blocks), dim3(256), 0, st, a, used); break;
    default: report_unlaunched("split-K reduce: epilogue"); break;
  }
}

}  // namespace

bool gemm_three_planes(const GemmArgs& a) {
  // a second weight plane (dequantised q8_0) adds its pass with the residual epilogue,
  // which has no three-plane form: such weights keep the separate third-plane pass
  if (!a.a_lo || !a.a_x2 || a.w_lo) return false;
  const int cfg = pick_cfg(a);
  return cfg == CFG_DL_S128x256 || cfg == CFG_DL_64x64;
}

void gemm_init() {
  set_attr_dl<128, 256, 2, 4, 64, 2, 3, GEMM_STORE>();
  set_attr_dl<64, 64, 2, 1, 64, 2, 3, GEMM_STORE>();
  set_attr_dl<128, 256, 2, 4, 64, 2, 3, GEMM_QKV>();
  set_attr_dl<64, 64, 2, 1, 64, 2, 3, GEMM_QKV>();
  set_attrs_epi<GEMM_STORE>();
  set_attrs_epi<GEMM_RESID>();
  set_attrs_epi<GEMM_SILU>();
  set_attrs_epi<GEMM_QKV>();
}

int launch_gemm(const GemmArgs& a0, int epi, hipStream_t st, bool defer) {
  if (a0.M <= 0 || a0.N <= 0) return 0;
  if (epi == GEMM_QKV) {
    GemmArgs a = a0;
    const int cfg = pick_cfg(a);
    const int splits = pick_splits(a, cfg);
    if (!a0.w_lo && splits > 1) {
      // split K: the post-processing kernel sums the partial planes itself (no reduce)
      a.k_chunk = ((a.K + splits - 1) / splits + 63) / 64 * 64;
      const int used = (a.K + a.k_chunk - 1) / a.k_chunk;
      launch_epi<GEMM_STORE>(a, cfg, used, st);    // partial planes (epilogue skipped)
      QkvPostArgs pa = a0.post;
      pa.partial = a.partial;
      pa.splits = used;
      pa.bias = a0.bias;
      launch_qkv_post(pa, st);
      return 0;
    }
    if (a0.post.HD != 64 || a0.w_lo) {
      QkvPostArgs pa = a0.post;
      pa.qkv = a0.c;
      launch_gemm(a, GEMM_STORE, st);                // raw projections into c, then
      launch_qkv_post(pa, st);                       // the separate post-processing
      return 0;
    }
    a.partial = nullptr;
    a.k_chunk = a.K;
    launch_epi<GEMM_QKV>(a, cfg, 1, st);
    return 0;
  }
  GemmArgs a = a0;
  a.w_lo = nullptr;
  const bool two = a0.w_lo != nullptr;
  // two weight planes: each takes half of the partial planes
  if (two) a.partial_elems /= 2;
  const int cfg = pick_cfg(a);
  int splits = pick_splits(a, cfg);
  if (two && !a.partial && epi == GEMM_SILU) {          // needs the split-K planes
    report_unlaunched("two-plane SiLU GEMM without split-K planes");
    return 0;
  }
  if (two && (splits <= 1 || !a.partial) && epi != GEMM_SILU) {
    // tiles that fill the GPU: the second plane's pass adds into the output
    a.partial = nullptr;
    a.k_chunk = a.K;
    if (epi == GEMM_STORE) launch_epi<GEMM_STORE>(a, cfg, 1, st);
    else launch_epi<GEMM_RESID>(a, cfg, 1, st);
    GemmArgs b = a;
    b.w = a0.w_lo;
    b.bias = nullptr;
    launch_epi<GEMM_RESID>(b, cfg, 1, st);
    return 0;
  }
  if (!two && splits <= 1) {
    a.partial = nullptr;
    a.k_chunk = a.K;
    switch (epi) {
      case GEMM_STORE: launch_epi<GEMM_STORE>(a, cfg, 1, st); break;
      case GEMM_RESID: launch_epi<GEMM_RESID>(a, cfg, 1, st); break;
      case GEMM_SILU: launch_epi<GEMM_SILU>(a, cfg, 1, st); break;
      default: report_unlaunched("GEMM: epilogue"); break;
    }
    return 0;
  }
  if (splits < 1) splits = 1;
  // K slices are whole 64-column stages
  a.k_chunk = ((a.K + splits - 1) / splits + 63) / 64 * 64;
  const int used = (a.K + a.k_chunk - 1) / a.k_chunk;
  launch_epi<GEMM_STORE>(a, cfg, used, st);      // partial planes (epilogue skipped)
  if (two) {                                     // the second plane's slices follow
    GemmArgs b = a;
    b.w = a0.w_lo;
    b.partial = a.partial + (size_t)used * a.M * a.N;
    launch_epi<GEMM_STORE>(b, cfg, used, st);
  }
  // deferred: the caller's next kernel sums the partial planes itself (the same fixed
  // order as the reduce: planes 0, 1, ... then the residual or the bias)
  if (defer && !two && (epi == GEMM_STORE || epi == GEMM_RESID) && used <= kMaxDeferredPlanes)
    return used;
  launch_reduce(a, epi, two ? 2 * used : used, st);
  return 0;
}

void launch_gemm_f32w(const GemmF32Args& a, int epi, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return;
  const int nout = (epi == GEMM_SILU) ? a.N / 2 : a.N;
  dim3 grid((nout + 255) / 256, a.M);
  switch (epi) {
    case GEMM_STORE: hipLaunchKernelGGL(k_gemm_f32w<GEMM_STORE>, grid, dim3(256), 0, st, a); break;
    case GEMM_RESID: hipLaunchKernelGGL(k_gemm_f32w<GEMM_RESID>, grid, dim3(256), 0, st, a); break;
    case GEMM_SILU: hipLaunchKernelGGL(k_gemm_f32w<GEMM_SILU>, grid, dim3(256), 0, st, a); break;
    default: report_unlaunched("f32-weight GEMM: epilogue"); break;
  }
}

}  // namespace ember
