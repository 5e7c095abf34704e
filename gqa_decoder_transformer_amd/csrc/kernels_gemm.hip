// Prefill GEMM: C[M, N] = A[M, K] . W[N, K]^T with bf16 weights on gfx950 MFMA
// (v_mfma_f32_16x16x32_bf16), f32 accumulation.
//
// A (activations) arrives as bf16 planes written by the producing kernel: in EXACT mode
// x = hi + lo (hi = bf16(x), lo = bf16(x - hi)) and every weight fragment is multiplied
// by both planes, which makes each product f32-accurate to ~2^-17 relative (the weights
// are exactly bf16, and bf16 x bf16 products are exact in f32); in FAST mode only hi.
//
// Tiling: 256 threads (4 waves, WM x WN), block tile BM x BN, K-stage 64. Global ->
// registers (16-byte loads, next stage prefetched during the MFMAs of the current
// one) -> LDS (rows padded by 16 bytes: the 16 rows a fragment read touches fall on
// distinct banks) -> MFMA fragments. Blocks are remapped so that consecutive tiles of
// one weight column block run on the same XCD (its L2 serves the repeated weight reads).
//
// Epilogues: store (+bias), residual add (x += C), SiLU*up over the gate/up rows that
// the weight repack interleaves in blocks of 16 (the lane holding gate column j holds
// the matching up column in the next 16-column fragment).
#include "common.h"
#include "kernels.h"

namespace ember {

namespace {

constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;   // bf16 elements per LDS row (128 + 16 bytes)

template <int ROWS>
struct TileLoader {
  // ROWS x BK bf16 tile = ROWS * 8 chunks of 16 bytes; 256 threads.
  static constexpr int CHUNKS = ROWS * (BK / 8) / 256;
  u32x4_t r[CHUNKS];
  EMBER_DEV void load(const uint16_t* base, int ld, int row0, int nrows, int k0, int K) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int id = threadIdx.x + 256 * i;
      int row = row0 + id / (BK / 8);
      row = row < nrows ? row : nrows - 1;          // clamp: rows beyond M/N never stored
      const int col = k0 + (id % (BK / 8)) * 8;
      // K is a multiple of 8: a chunk is either inside K or wholly past it (zeros)
      r[i] = col < K ? *(const u32x4_t*)(base + (size_t)row * ld + col) : u32x4_t{0, 0, 0, 0};
    }
  }
  EMBER_DEV void store(uint16_t* lds) const {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int id = threadIdx.x + 256 * i;
      const int row = id / (BK / 8);
      const int col = (id % (BK / 8)) * 8;
      *(u32x4_t*)(lds + row * LDS_STRIDE + col) = r[i];
    }
  }
};

EMBER_DEV bf16x8_t lds_frag(const uint16_t* lds, int row, int k) {
  const u32x4_t v = *(const u32x4_t*)(lds + row * LDS_STRIDE + k);
  return __builtin_bit_cast(bf16x8_t, v);
}

template <int BM, int BN, int WM, int WN, bool SPLIT, int EPI>
__global__ void __launch_bounds__(256) k_gemm(GemmArgs a) {
  constexpr int TM = BM / WM / 16;
  constexpr int TN = BN / WN / 16;
  static_assert(WM * WN == 4, "4 waves");
  static_assert(EPI != GEMM_SILU || TN % 2 == 0, "SiLU pairs 16-column fragments");
  __shared__ __align__(16) uint16_t As_hi[BM * LDS_STRIDE];
  __shared__ __align__(16) uint16_t As_lo[SPLIT ? BM * LDS_STRIDE : 8];
  __shared__ __align__(16) uint16_t Bs[BN * LDS_STRIDE];

  // XCD-aware tile order: blocks are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous run of logical tiles, M-tiles fastest, so a weight column block stays
  // within one XCD's L2.
  const int mt = (a.M + BM - 1) / BM, nt = (a.N + BN - 1) / BN;
  const int nblk = mt * nt;
  int lin = blockIdx.x;
  if (nblk % 8 == 0) lin = (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
  const int tm = lin % mt, tn = lin / mt;
  const int m0 = tm * BM, n0 = tn * BN;

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int wm0 = wm * (BM / WM), wn0 = wn * (BN / WN);
  const int fr = lane % 16, fk = (lane / 16) * 8;

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  TileLoader<BM> la_hi, la_lo;
  TileLoader<BN> lb;
  // K range of this block (split-K over gridDim.y slices of k_chunk columns)
  const int kb0 = blockIdx.y * a.k_chunk;
  const int kend = min(a.K, kb0 + a.k_chunk);
  const int nk = (kend - kb0 + BK - 1) / BK;
  la_hi.load(a.a_hi, a.lda, m0, a.M, kb0, kend);
  if (SPLIT) la_lo.load(a.a_lo, a.lda, m0, a.M, kb0, kend);
  lb.load(a.w, a.K, n0, a.N, kb0, kend);
  la_hi.store(As_hi);
  if (SPLIT) la_lo.store(As_lo);
  lb.store(Bs);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) {
      la_hi.load(a.a_hi, a.lda, m0, a.M, kb0 + (kt + 1) * BK, kend);
      if (SPLIT) la_lo.load(a.a_lo, a.lda, m0, a.M, kb0 + (kt + 1) * BK, kend);
      lb.load(a.w, a.K, n0, a.N, kb0 + (kt + 1) * BK, kend);
    }
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      bf16x8_t bf[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) bf[j] = lds_frag(Bs, wn0 + j * 16 + fr, ks + fk);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const bf16x8_t ah = lds_frag(As_hi, wm0 + i * 16 + fr, ks + fk);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bf[j], acc[i][j], 0, 0, 0);
        if (SPLIT) {
          const bf16x8_t al = lds_frag(As_lo, wm0 + i * 16 + fr, ks + fk);
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bf[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    __syncthreads();
    if (kt + 1 < nk) {
      la_hi.store(As_hi);
      if (SPLIT) la_lo.store(As_lo);
      lb.store(Bs);
      __syncthreads();
    }
  }

  // epilogue: lane holds C[row0 + e][col] for e < 4 of each 16x16 fragment
  const int rbase = m0 + wm0 + (lane / 16) * 4;
  if (a.partial) {                         // split-K: raw f32 tile into this slice's plane
    float* pp = a.partial + (size_t)blockIdx.y * a.M * a.N;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = n0 + wn0 + j * 16 + fr;
        if (col >= a.N) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = rbase + i * 16 + e;
          if (row < a.M) pp[(size_t)row * a.N + col] = acc[i][j][e];
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn0 + j * 16 + fr;
      if (EPI == GEMM_SILU) {
        if (j % 2) continue;
        const int ocol = (col / 32) * 16 + (col % 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = rbase + i * 16 + e;
          if (row >= a.M || col >= a.N) continue;
          const float v = silu(acc[i][j][e]) * acc[i][j + 1][e];
          const size_t o = (size_t)row * a.ldo + ocol;
          if (a.o_f32) a.o_f32[o] = v;
          if (a.o_hi) {
            uint32_t h, l;
            split_bf16(v, h, l);
            a.o_hi[o] = (uint16_t)h;
            if (a.o_lo) a.o_lo[o] = (uint16_t)l;
          }
        }
      } else {
        if (col >= a.N) continue;
        const float bias = (EPI == GEMM_STORE && a.bias) ? a.bias[col] : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = rbase + i * 16 + e;
          if (row >= a.M) continue;
          float* cp = a.c + (size_t)row * a.ldc + col;
          if (EPI == GEMM_RESID) *cp += acc[i][j][e];
          else *cp = acc[i][j][e] + bias;
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int EPI>
void launch_cfg(const GemmArgs& a, int splits, hipStream_t st) {
  const int blocks = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  if (a.a_lo)
    hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, true, EPI>), dim3(blocks, splits), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, false, EPI>), dim3(blocks, splits), dim3(256), 0, st, a);
}

template <int EPI>
void launch_epi(const GemmArgs& a, int splits, hipStream_t st) {
  // small M (decode batches, short prompts): 64-row tiles
  if (a.M <= 64) launch_cfg<64, 128, 2, 2, EPI>(a, splits, st);
  else launch_cfg<128, 128, 2, 2, EPI>(a, splits, st);
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
      const int gcol = (col / 16) * 32 + (col % 16), ucol = gcol + 16;
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

// Split K when the tiles cannot fill the GPU: slices of >= 256 columns, about 512 blocks.
int pick_splits(const GemmArgs& a) {
  if (!a.partial) return 1;
  const int BM = a.M <= 64 ? 64 : 128;
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + 127) / 128);
  if (tiles >= 192) return 1;
  int s = (512 + tiles - 1) / tiles;
  const int max_s = a.K / 256;
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
    const int rg = (n >> 4) * 32 + (n & 15), ru = rg + 16;
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

}  // namespace

void launch_gemm(const GemmArgs& a0, int epi, hipStream_t st) {
  if (a0.M <= 0 || a0.N <= 0) return;
  GemmArgs a = a0;
  const int splits = pick_splits(a);
  if (splits <= 1) {
    a.partial = nullptr;
    a.k_chunk = a.K;
    switch (epi) {
      case GEMM_STORE: launch_epi<GEMM_STORE>(a, 1, st); break;
      case GEMM_RESID: launch_epi<GEMM_RESID>(a, 1, st); break;
      case GEMM_SILU: launch_epi<GEMM_SILU>(a, 1, st); break;
      default: break;
    }
    return;
  }
  // K slices are whole 64-column stages
  a.k_chunk = ((a.K + splits - 1) / splits + 63) / 64 * 64;
  const int used = (a.K + a.k_chunk - 1) / a.k_chunk;
  launch_epi<GEMM_STORE>(a, used, st);            // partial planes (epilogue skipped)
  const int nout = epi == GEMM_SILU ? a.N / 2 : a.N;
  long long blocks = ((long long)a.M * nout + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  switch (epi) {
    case GEMM_STORE: hipLaunchKernelGGL(k_splitk_reduce<GEMM_STORE>, dim3((unsigned)blocks), dim3(256), 0, st, a, used); break;
    case GEMM_RESID: hipLaunchKernelGGL(k_splitk_reduce<GEMM_RESID>, dim3((unsigned)blocks), dim3(256), 0, st, a, used); break;
    case GEMM_SILU: hipLaunchKernelGGL(k_splitk_reduce<GEMM_SILU>, dim3((unsigned)blocks), dim3(256), 0, st, a, used); break;
    default: break;
  }
}

void launch_gemm_f32w(const GemmF32Args& a, int epi, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return;
  const int nout = (epi == GEMM_SILU) ? a.N / 2 : a.N;
  dim3 grid((nout + 255) / 256, a.M);
  switch (epi) {
    case GEMM_STORE: hipLaunchKernelGGL(k_gemm_f32w<GEMM_STORE>, grid, dim3(256), 0, st, a); break;
    case GEMM_RESID: hipLaunchKernelGGL(k_gemm_f32w<GEMM_RESID>, grid, dim3(256), 0, st, a); break;
    case GEMM_SILU: hipLaunchKernelGGL(k_gemm_f32w<GEMM_SILU>, grid, dim3(256), 0, st, a); break;
    default: break;
  }
}

}  // namespace ember
