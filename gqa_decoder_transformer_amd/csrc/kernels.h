// Host-side launch wrappers of the gfx950 kernels (one translation unit per kernel
// family). Pointers are device pointers; every launch is asynchronous on `st`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define EMBER_INLINE_HD __host__ __device__ inline

namespace ember {

// Flags raised by kernels and reported by ember_sync.
enum DeviceFlag { kFlagBadToken = 0, kFlagNaN = 1, kNumFlags = 4 };

// A launch wrapper that has no kernel for its arguments (a shape the host validation
// should have refused) launches nothing and records `what` here; the C ABI call that
// enqueued it then fails with EMBER_E_DEVICE instead of leaving stale outputs.
void report_unlaunched(const char* what);

// ------------------------------------------------------------------ misc (kernels_misc.hip)

// x[m, :] = widen(E[ids[m], :]) for m < M; ids outside [0, V) read row 0 and raise
// flags[kFlagBadToken] (host-validated prefill ids never do).
// Storage of the weight matrices. q8_0 ("ember internals", section "GGUF format and
// quantization", subsection "q8_0 block quantization": 32 int8 values and one f16 scale per
// block along the row) is repacked at load into two planes: [N][K] bytes holding q + 128
// (so a byte converts to f32 in one instruction), then [N][K / 32] f16 scale bits.
enum WeightKind { WK_F32 = 0, WK_BF16 = 1, WK_Q8 = 2 };
constexpr int kQ8Block = 32;
constexpr int kQ8BlockBytes = 34;

// x[m] = row ids[m] of the embedding E (bf16 / f32 [V, H], or q8 planes with scales
// e_scale); an id outside [0, V) takes row 0 and raises kFlagBadToken.
void launch_embed(const int32_t* ids, const void* E, int e_wk, const uint16_t* e_scale, float* x,
                  int M, int H, int V, int* flags, hipStream_t st);

// q8_0 blocks of src ([N][K / 32] blocks of 34 bytes: f16 scale little-endian, 32 int8)
// into the two planes. Destination row of source row n: dst_row0 + n (gu < 0), or
// gu_row(n, gu) (gate: gu = 0, up: gu = 1; the interleaved gate/up matrix).
void launch_q8_unpack(const uint8_t* src, int N, int K, uint8_t* dst_q, uint16_t* dst_s,
                      int dst_row0, int gu, hipStream_t st);
// The dequantised matrix w = q * d, [N, K] row-major: Q8_TO_F32 (exact), Q8_TO_BF16
// (round to nearest even), or Q8_TO_BF16_PAIR: bf16(w) at dst and the bf16 rounding of
// w - bf16(w) at dst + N K (their sum is w within 2^-17 relative).
enum Q8DequantMode { Q8_TO_F32 = 0, Q8_TO_BF16 = 1, Q8_TO_BF16_PAIR = 2 };
void launch_q8_dequant(const uint8_t* q, const uint16_t* s, int N, int K, void* dst, int mode,
                       hipStream_t st);

// Row-wise RMSNorm of rows src_row(r) = r * row_step + row_off, r < R, of x [*, H]:
// y = x / sqrt(mean(x^2) + eps) * w. Writes any of: out_f32 [R, H], planes hi/lo
// [R, ld_plane] bf16 (lo may be null: single plane); with x2 (needs lo) the three planes
// y = hi + lo + x2 of split3_bf16 instead of the pair. With nsplit > 0 (row_step 1,
// row_off 0, and rmsnorm_adds_partials(H, ld_plane)) it first completes a deferred
// split-K residual GEMM: x += the sum of the partial planes part [nsplit][R][H], in plane
// order, written back to x.
void launch_rmsnorm(const float* x, const float* w, float eps, int R, int H, int row_step,
                    int row_off, float* out_f32, uint16_t* hi, uint16_t* lo, int ld_plane,
                    hipStream_t st, uint16_t* x2 = nullptr, const float* part = nullptr,
                    int nsplit = 0);
bool rmsnorm_adds_partials(int H, int ld_plane);

struct QkvPostArgs {
  const float* qkv;        // [M, (NH + 2 NKV) HD] raw projections (bias included)
  int M, NH, NKV, HD;
  int tokens_per_row;      // token m belongs to row b0 + m / tpr at position start + m % tpr
  int b0, start_pos;
  const int* d_pos;        // if non-null, start_pos is read from *d_pos
  const float* cos_t;      // [max_seq, HD/2]
  const float* sin_t;
  const float* q_norm;     // [HD] or null (per-head RMSNorm before RoPE)
  const float* k_norm;
  float eps;
  float* q_out;            // [M, NH*HD] f32 (roped, normed)
  void* k_cache;           // layer base: [B_cache][NKV][max_seq][HD]
  void* v_cache;
  bool kv_bf16;
  int max_seq;
  // or (splits > 0) the projections as `splits` split-K partial planes [splits][M][N]
  // (N = (NH + 2 NKV) HD) summed in plane order, plus `bias` [N] (or null); qkv unused
  const float* partial;
  int splits;
  const float* bias;
};
// Per-head q/k RMSNorm (optional), rotate-half RoPE from the tables, K/V store at the
// tokens' explicit positions.
void launch_qkv_post(const QkvPostArgs& a, hipStream_t st);

// next[r] = argmax over the partial keys part[r, 0..nparts); NaN flag handled upstream.
void launch_argmax_reduce(const unsigned long long* part, int nparts, int R, int32_t* next,
                          hipStream_t st);
// next[r] = argmax(logits[r, 0..n)) (lowest index on ties); raises kFlagNaN on NaN.
void launch_argmax_rows(const float* logits, int R, int n, long long ld, int32_t* next,
                        int* flags, hipStream_t st);

// Token classification head: out[m, c] = dot(h[m], W[c]) + b[c] (h already normalised),
// next[m] = argmax_c out[m, c].
void launch_cls_head(const float* h, const void* W, bool w_bf16, const float* b, int M, int H,
                     int C, float* out, int32_t* next, hipStream_t st);

// Copy R rows of n logits (row stride ld) to f32 or bf16 (round to nearest even).
void launch_convert_logits(const float* src, int R, int n, long long ld, void* dst,
                           bool to_bf16, hipStream_t st);

// Begin a decode step. Row r's position p_r: pos for every row, or (ragged) the value
// already in row_pos[r]; then row_pos[r] = p_r, rope_cur[r] = (cos, sin) row of p_r, row r
// of x the embedding of ids[r] (out-of-range ids -> 0 + flag), *d_pos = p_0.
struct StepBeginArgs {
  const int32_t* ids;
  int R, V, pos;
  bool ragged;
  int* row_pos;            // [R]
  int* d_pos;
  int* flags;
  const float* cos_t;
  const float* sin_t;
  int half;
  float* rope_cur;         // [R][HD]: cos[HD/2], sin[HD/2] per row
  const void* E;
  int e_wk;                // WeightKind of E
  const uint16_t* e_scale; // q8: scale plane of E
  float* x;
  int H;
};
void launch_step_begin(const StepBeginArgs& a, hipStream_t st);
// ---------------------------------------------------------------- sampling (kernels_sample.hip)

constexpr int kSampleMaxTiles = 4096;                 // 256-token tiles per row
constexpr int kSampleMaxVocab = kSampleMaxTiles * 256;
constexpr int kSampleBins = 2048;                     // radix digit of 11 bits
constexpr int kSampleChunk = 2048;                    // tokens per block of a row

// Per-row state the phases of one draw hand to each other through global memory. All
// zero between draws (the last phase clears what the others leave behind).
struct SampleState {
  uint32_t hist_k[3][kSampleBins];                    // top-k counts per digit
  unsigned long long hist_p[3][kSampleBins];          // top-p fixed-point weights per digit
  unsigned long long ptotal;                          // top-p weight of all survivors
  unsigned long long above;                           // weight above the current prefix
  uint32_t maxkey;                                    // ordered key of the largest z
  uint32_t count;                                     // blocks done in the current phase
  uint32_t prefix, pmask;                             // radix search so far
  float thr;                                          // survivors: z >= thr
  int live_k, live_p;                                 // the searches found their keys
  int pad;
};

// Tile sums per row: [R][sample_tiles_ld(V)] floats.
EMBER_INLINE_HD int sample_blocks(int V) { return (V + kSampleChunk - 1) / kSampleChunk; }
EMBER_INLINE_HD int sample_tiles_ld(int V) { return sample_blocks(V) * (kSampleChunk / 256); }

// next[r] = a token drawn from row r of the logits through temperature, top-k, top-p,
// softmax and an inverse-CDF draw with u = uniform[row * u_ld + col0 + r], where row is
// d_pos[r] (each row's position) when d_pos is non-null, else pos (clamped to u_rows - 1).
// temperature > 0.
// Raises kFlagNaN when a row holds a NaN. state / tiles: R rows of the buffers above.
struct SampleArgs {
  const float* logits;
  long long ld;
  int R, V;
  float temperature;
  int top_k;
  float top_p;
  const float* uniform;    // null: on-device draws (Philox4x32-10 keyed by seed, see
                           // kernels_sample.hip)
  int u_rows;
  long long u_ld;
  unsigned long long seed;
  int col0;
  int pos;
  const int* d_pos;
  int32_t* next;
  int* flags;
  SampleState* state;
  float* tiles;
};
void launch_sample(const SampleArgs& a, hipStream_t st);

void launch_fill_i32(int* p, int n, int v, hipStream_t st);
// dst[r * dst_stride + i] = src[(r * row_step + row_off) * H + i], r < R, i < H.
void launch_copy_rows(const float* src, int R, int row_step, int row_off, int H, float* dst,
                      long long dst_stride, hipStream_t st);
// Mean-pooled sequence score: acc[r][d] (= if first, else +=) sum over the row's tpr tokens
// of h[r * tpr + t][d]; then out[r] = sum_d (acc[r][d] / T) w[d] + b[0].
void launch_pool_accum(const float* h, int R, int tpr, int H, float* acc, bool first,
                       hipStream_t st);
void launch_pool_head(const float* acc, int R, int H, int T, const float* w, const float* b,
                      float* out, hipStream_t st);
// dst[i] = widen(src[i]) for i < n (bf16 or f32 source).
void launch_widen(const void* src, bool bf16, float* dst, long long n, hipStream_t st);

// ------------------------------------------------------------------ GEMV (kernels_gemv.hip)

// The gate and up projections are stored as one matrix of 2*FF rows, interleaved in
// blocks of kGuBlock rows: [g 0..31][u 0..31][g 32..63][u 32..63]... (one 32-column MFMA
// fragment of gate outputs is followed by the fragment of the matching up outputs).
constexpr int kGuBlock = 32;
EMBER_INLINE_HD int gu_row(int n, int up) {
  return (n / kGuBlock) * 2 * kGuBlock + (up ? kGuBlock : 0) + n % kGuBlock;
}

enum GemvEpi { GEMV_STORE = 0, GEMV_RESID = 1, GEMV_SILU = 2, GEMV_LOGITS = 3 };

struct GemvArgs {
  const void* W;           // [N_rows, K] row-major, bf16 or f32, or the q8 byte plane
  bool w_bf16;
  const uint16_t* w_scale; // q8 weights when non-null: [N_rows][K / 32] f16 scale bits
  int N;                   // outputs per token (SILU: FF outputs from 2*FF packed rows)
  int K;
  int M;                   // tokens: must be 1
  // input: x [K] f32; when norm_w != null the kernel applies RMSNorm to x first
  const float* x;
  const float* norm_w;
  // or (x == null) the input rebuilt from decode-attention split partials of one row:
  // xpart [K / xp_hd heads][xp_nsplit][xp_hd + 2] = (m, l, acc[xp_hd]);
  // x[h xp_hd + d] = sum_j acc_j[d] w_j / sum_j l_j w_j, w_j = e^(m_j - max m), over the
  // splits that hold a key up to the position (the k_attn_combine arithmetic); residual
  // epilogue only, 1 <= xp_nsplit <= gemv_parts_max(N, K, wk)
  const float* xpart;
  int xp_nsplit, xp_hd, xp_chunk_min;
  const int* xp_pos;
  float eps;
  // outputs
  const float* bias;       // [N] or null (STORE)
  float* y;                // STORE/SILU/LOGITS: [N]; RESID: x_res [N] (+=)
  int ldy;
  unsigned long long* argmax_part;   // LOGITS: [gridDim.x]
  int* flags;
};
void launch_gemv(const GemvArgs& a, int epi, hipStream_t st);
// The most decode-attention splits the residual GEMV of this shape can take as its input
// (xpart): 4 in the row-per-wave layout (K <= 1024), 8 in the row-per-block layout with one
// chunk per thread (bf16 / f32), 0 otherwise.
int gemv_parts_max(int N, int K, int wk);
int gemv_num_blocks(int N, int epi, int K, int wk);

// ------------------------------------------------------------------ GEMM (kernels_gemm.hip)

// GEMM_QKV: the QKV projection of a prefill pass with its post-processing fused when
// head_dim is 64 and K is not split (bias, optional q/k RMSNorm, rotate-half RoPE, q to
// post.q_out, K/V into the cache at their positions; `c` is not written); otherwise a
// plain store into `c` followed by launch_qkv_post(post).
enum GemmEpi { GEMM_STORE = 0, GEMM_RESID = 1, GEMM_SILU = 2, GEMM_QKV = 3 };

struct GemmArgs {
  // A: activations as bf16 planes [M, lda] (hi, and lo in EXACT mode; lo == null: one pass)
  const uint16_t* a_hi;
  const uint16_t* a_lo;
  // optional third plane x2 = bf16(x - hi - lo) in the same layout (EXACT QKV input); only
  // where gemm_three_planes() holds, and with GEMM_STORE
  const uint16_t* a_x2;
  int lda;
  // B: weights bf16 [N, K] row-major (K contiguous). With w_lo (same layout) the weights
  // are w + w_lo (a value that bf16 cannot hold, such as a dequantised q8_0 weight, as a
  // bf16 part and the bf16 rounding of its remainder), one pass per plane: the second
  // adds into the output, or, when K is split or the epilogue is SiLU, both passes write
  // split-K planes; `partial` must then hold 2 M N floats.
  const uint16_t* w;
  const uint16_t* w_lo;
  int M, N, K;
  const float* bias;       // STORE: [N] or null
  float* c;                // STORE: [M, ldc] f32; RESID: [M, ldc] +=
  long long ldc;
  uint16_t* o_hi;          // SILU: planes [M, ldo] of silu(g)*u (o_lo may be null)
  uint16_t* o_lo;
  float* o_f32;            // SILU: optional f32 [M, ldo]
  int ldo;
  // split-K scratch (optional): when the tiles cannot fill the GPU, K is cut into slices
  // whose f32 partial tiles land here ([slices][M][N]) and a fixed-order sum applies the
  // epilogue. null: never split.
  float* partial;
  size_t partial_elems;
  int k_chunk;             // set by launch_gemm
  QkvPostArgs post;        // GEMM_QKV only (post.qkv = c)
};
// Returns 0 when the output is complete. With `defer`, a store or residual GEMM that
// splits K into at most kMaxDeferredPlanes slices leaves its f32 partial planes
// ([n][M][N] at a.partial) for the caller's next kernel to sum (planes 0..n-1 in order,
// then + bias or into the residual) and returns n.
constexpr int kMaxDeferredPlanes = 8;
int launch_gemm(const GemmArgs& a, int epi, hipStream_t st, bool defer = false);
// true when launch_gemm takes a_x2 as a third activation plane in the same pass (tile forms
// that load straight into LDS); otherwise the caller adds that plane's product separately
bool gemm_three_planes(const GemmArgs& a);
// Sets the dynamic LDS limit of every GEMM kernel (call once before the first launch).
void gemm_init();

// f32-weight path (VALU), same epilogues; A is f32 [M, lda].
struct GemmF32Args {
  const float* a;
  int lda;
  const float* w;          // [N, K]
  int M, N, K;
  const float* bias;
  float* c;
  long long ldc;
  float* o_f32;            // SILU output [M, ldo] f32
  int ldo;
};
void launch_gemm_f32w(const GemmF32Args& a, int epi, hipStream_t st);

// ------------------------------------------------------------------ attention (kernels_attn.hip)

struct FlashArgs {
  const float* q;          // [M, NH*HD] f32, roped
  const void* k_cache;     // layer base [B_cache][NKV][max_seq][HD]
  const void* v_cache;
  bool kv_bf16;
  int NH, NKV, HD, max_seq;
  int tokens_per_row, rows, b0, start_pos;   // queries: rows x tokens_per_row
  bool causal;             // causal: keys 0..pos; else keys 0..start+tpr-1
  float scale;
  float* out_f32;          // [M, NH*HD] or null
  uint16_t* out_hi;        // planes [M, NH*HD] or null
  uint16_t* out_lo;
};
void launch_flash_prefill(const FlashArgs& a, hipStream_t st);
// MFMA flash attention (kernels_flash.hip) for head_dim 64 / 128; `split`: EXACT hi+lo.
bool flash_mfma_supported(int HD);
void launch_flash_mfma(const FlashArgs& a, bool split, hipStream_t st);

// Packed K and V^T bf16 planes of one prefill pass (keys 0 .. key_end-1 of each pass row,
// zero up to LK = key_end rounded up to 64), read by the tiled attention:
//   K   plane p: kp[(((p * rows + r) * NKV + g) * LK + key) * HD + d]
//   V^T plane p: vt[(((p * rows + r) * NKV + g) * HD + d) * LK + key]
// FAST: one plane each, bf16(x). EXACT (split): K in three planes x0 = bf16(x),
// x1 = bf16(x - x0), x2 = bf16(x - x0 - x1) (their sum is x within ~2^-25 relative: the
// scores q.k feed exp, so their absolute error must stay at f32 level however large they
// are); V in two planes x0, x1 (within 2^-17: the P V product is a weighted mean).
struct KvPackArgs {
  const void* k_cache;     // layer base [B_cache][NKV][max_seq][HD]
  const void* v_cache;
  bool kv_bf16;
  int NKV, HD, max_seq;
  int rows, b0, key_end, LK;
  bool split;
  uint16_t* kp;
  uint16_t* vt;
};
inline int kv_pack_lk(int key_end) { return (key_end + 63) / 64 * 64; }
inline int kv_pack_kplanes(bool split) { return split ? 3 : 1; }
inline int kv_pack_vplanes(bool split) { return split ? 2 : 1; }
inline size_t kv_pack_elems(int rows, int NKV, int HD, int key_end, bool split) {
  return (size_t)(kv_pack_kplanes(split) + kv_pack_vplanes(split)) * rows * NKV *
         kv_pack_lk(key_end) * HD;
}
void launch_kv_pack(const KvPackArgs& a, hipStream_t st);

// Tiled MFMA prefill attention (head_dim 64 / 128) over the packed planes; queries from
// `a.q`, output to a.out_hi / a.out_lo (planes) or a.out_f32. Sets its LDS limit on the
// first call.
void launch_flash_tiled(const FlashArgs& a, const uint16_t* kp, const uint16_t* vt, int LK,
                        bool split, hipStream_t st);
void flash_init();

// Measurement kernels (kernels_peak.hip): a streaming copy of `bytes` from src to dst, and
// an MFMA-only loop over kPeakMfmaBlocks blocks of 256 threads that writes one float per
// thread to `out` and returns the flops of one launch.
constexpr int kPeakMfmaBlocks = 1024;
constexpr int kPeakReadBlocks = 256 * 8;
void launch_peak_copy(const void* src, void* dst, size_t bytes, hipStream_t st);
// A streaming read of `bytes` at src; one word per thread of kPeakReadBlocks x 256 to out.
void launch_peak_read(const void* src, size_t bytes, uint32_t* out, hipStream_t st);
double launch_peak_mfma(float* out, hipStream_t st);

struct DecodeAttnArgs {
  const float* qkv;        // [B, (NH + 2 NKV) HD] raw projections of the current token
  const float* rope_cur;   // [B][HD]: cos[HD/2], sin[HD/2] of each row's position
  const float* q_norm;     // [HD] or null
  const float* k_norm;
  float eps;
  void* k_cache;           // layer base [B_cache][NKV][max_seq][HD]; K/V at d_pos[b] written
  void* v_cache;
  bool kv_bf16;
  int B, NH, NKV, HD, max_seq;
  const int* d_pos;        // [B] each row's current position; row b's keys 0..d_pos[b]
  int nsplit, chunk_min;   // nsplit == 1 or chunk_min >= ceil(max_seq / nsplit)
  float scale;
  float* part;             // [B][NH][nsplit][HD + 2] split partials (m, l, acc)
  // qkv_splits > 0: qkv is not written; the current token's projections are the sum of
  // the deferred split-K planes qkv_part [qkv_splits][B][(NH + 2 NKV) HD] (in plane
  // order) plus qkv_bias (may be null)
  const float* qkv_part;
  int qkv_splits;
  const float* qkv_bias;
  float* out_f32;          // nsplit == 1: the normalised output [B, NH*HD] (f32 and/or
  uint16_t* out_hi;        // bf16 planes) is written directly and no combine follows
  uint16_t* out_lo;
  int heads_per_block;     // 1 or NH / NKV (a whole kv group per block)
};
// Split-K decode attention with the QKV epilogue (q/k norm, RoPE, K/V store at the
// current position) fused in.
void launch_decode_attn(const DecodeAttnArgs& a, hipStream_t st);
// att = combine(part) for B rows (nsplit <= 64), written as f32 [B, NH*HD] and/or planes;
// d_pos[b] is row b's position (the splits holding keys 0..d_pos[b] are combined).
void launch_attn_combine(const float* part, int B, int NH, int HD, int nsplit, const int* d_pos,
                         int chunk_min, float* out_f32, uint16_t* out_hi, uint16_t* out_lo,
                         hipStream_t st);

// Launch plan of decode attention: number of splits (1: no combine), minimum chunk of
// keys per split, threads per block.
struct DecodePlan { int nsplit, chunk_min, heads_per_block; };
DecodePlan decode_split_plan(int B, int NH, int NKV, int max_seq, int max_splits = 64);

}  // namespace ember
