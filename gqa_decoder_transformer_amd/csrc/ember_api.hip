// C ABI of the GQA decoder forward pass: host validation, the workspace plan, weight
// repacking, the prefill and decode schedules, HIP-graph replay of decode steps.
//
// The interface follows the "ember internals" page (ForwardModel: create_cache,
// forward_with_cache(token_ids, cache, start_pos); explicit write positions from
// "cursor semantics") and the checks of "Falcon-H1-0.5B-Rust src/lib.rs"
// (Config::validate, validate_weights, Model::logits). No device memory is allocated
// here: everything lives in the caller's workspace and KV buffer.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "../../include/ember.h"
#include "kernels.h"

using namespace ember;

namespace {

thread_local std::string g_last_error;

ember_status fail(ember_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

// The first launch wrapper of this thread's current call that found no kernel for its
// arguments (see report_unlaunched), or null.
thread_local const char* g_unlaunched = nullptr;

}  // namespace

void ember::report_unlaunched(const char* what) {
  if (!g_unlaunched) g_unlaunched = what;
}

namespace {

// EMBER_E_DEVICE if a launch of the current call launched nothing; clears the record.
ember_status check_launched() {
  const char* w = g_unlaunched;
  g_unlaunched = nullptr;
  if (w) return fail(EMBER_E_DEVICE, "internal error: no kernel for these arguments (%s)", w);
  return EMBER_OK;
}

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) return fail(EMBER_E_DEVICE, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

size_t dtype_size(int dt) { return dt == EMBER_BF16 ? 2 : 4; }

int weight_kind(int dt) { return dt == EMBER_Q8_0 ? WK_Q8 : (dt == EMBER_BF16 ? WK_BF16 : WK_F32); }

// The GEMMs of multi-token passes run on bf16 MFMA for bf16 and q8 weights (q8 from a
// dequantised copy: bf16 in FAST precision, in EXACT a bf16 pair whose sum is the weight
// within 2^-17, one GEMM pass per plane); f32 weights take the f32 path.
bool uses_mfma(const ember_config& c) {
  return c.weight_dtype == EMBER_BF16 || c.weight_dtype == EMBER_Q8_0;
}
bool q8_pair(const ember_config& c) {
  return c.weight_dtype == EMBER_Q8_0 && c.precision == EMBER_EXACT;
}

struct LayerOff {
  size_t ln1, wqkv, bqkv, wo, qn, kn, ln2, wgu, wd;
  size_t wqkv_s, wo_s, wgu_s, wd_s;   // q8: scale planes
};

struct Plan {
  // weights
  size_t embed, fnorm, cls_w, cls_b, cos_t, sin_t;
  std::vector<LayerOff> layer;
  // activations
  size_t ids, pos, row_pos, rope_cur, next, flags, x, xb, pa_hi, pa_lo, pa_x2, pb_hi, pb_lo, qkv, q, att, act, part,
      logits, argpart, splitk, kvpack, samp_state, samp_tiles, embed_s, q8_scratch, sens_w,
      sens_b, sens_acc, sens_out;
  size_t splitk_elems, kvpack_elems;
  size_t total;
  int Mx, qkv_n, ka, nsplit_max, argparts;
};

// Config validation (cf. Falcon-H1 Rust reference, Config::validate: zero dimensions,
// heads % kv_heads, odd head_dim), plus what the kernels assume.
ember_status validate_config(const ember_config* c) {
  if (!c) return fail(EMBER_E_ARG, "config is NULL");
  if (c->vocab <= 0 || c->hidden <= 0 || c->layers <= 0 || c->heads <= 0 || c->kv_heads <= 0 ||
      c->head_dim <= 0 || c->ffn <= 0)
    return fail(EMBER_E_CONFIG, "zero dimension");
  if (c->heads % c->kv_heads != 0 || c->head_dim % 2 != 0)
    return fail(EMBER_E_CONFIG, "invalid GQA/RoPE shape");
  if (c->heads / c->kv_heads > 8) return fail(EMBER_E_CONFIG, "GQA group above 8 is not supported");
  const int hd = c->head_dim;
  if (hd != 8 && hd != 16 && hd != 32 && hd != 64 && hd != 128)
    return fail(EMBER_E_CONFIG, "head_dim must be one of 8, 16, 32, 64, 128");
  if (c->weight_dtype != EMBER_F32 && c->weight_dtype != EMBER_BF16 && c->weight_dtype != EMBER_Q8_0)
    return fail(EMBER_E_DTYPE, "unsupported weight dtype %d", c->weight_dtype);
  if (c->weight_dtype == EMBER_Q8_0 && c->head_kind != EMBER_HEAD_TIED_LM)
    return fail(EMBER_E_CONFIG, "q8_0 weights need the tied LM head");
  if (c->kv_dtype != EMBER_F32 && c->kv_dtype != EMBER_BF16)
    return fail(EMBER_E_DTYPE, "unsupported KV dtype %d", c->kv_dtype);
  if (c->precision != EMBER_EXACT && c->precision != EMBER_FAST)
    return fail(EMBER_E_CONFIG, "unknown precision mode");
  if (c->precision == EMBER_EXACT && c->kv_dtype != EMBER_F32)
    return fail(EMBER_E_CONFIG, "EXACT precision needs an f32 KV cache");
  if (c->head_kind != EMBER_HEAD_TIED_LM && c->head_kind != EMBER_HEAD_CLS)
    return fail(EMBER_E_CONFIG, "unknown head kind");
  if (c->head_kind == EMBER_HEAD_CLS && (c->n_classes <= 0 || c->n_classes > 64))
    return fail(EMBER_E_CONFIG, "n_classes must be in 1..64");
  if (c->head_kind == EMBER_HEAD_TIED_LM && !c->causal)
    return fail(EMBER_E_CONFIG, "a tied LM head needs a causal model");
  if (c->sens_head != 0 && (c->sens_head != 1 || c->head_kind != EMBER_HEAD_CLS))
    return fail(EMBER_E_CONFIG, "the sequence-score head is a 0/1 flag of classification models");
  if (c->ffn % kGuBlock != 0) return fail(EMBER_E_CONFIG, "ffn must be a multiple of %d", kGuBlock);
  const int K8 = c->weight_dtype == EMBER_Q8_0 ? kQ8Block : (c->weight_dtype == EMBER_BF16 ? 8 : 4);
  if (c->hidden % K8 || c->ffn % K8 || (c->heads * hd) % K8)
    return fail(EMBER_E_CONFIG, "hidden, ffn and heads*head_dim must be multiples of %d", K8);
  if (c->hidden > 8192 || c->ffn > 32768 || c->heads * hd > 8192)
    return fail(EMBER_E_CONFIG, "dimension above the supported maximum");
  if (c->max_batch <= 0 || c->max_seq <= 0 || c->max_tokens <= 0)
    return fail(EMBER_E_CONFIG, "max_batch, max_seq and max_tokens must be positive");
  if (c->max_seq > 65536) return fail(EMBER_E_CONFIG, "max_seq above 65536");
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.0))
    return fail(EMBER_E_CONFIG, "rms_eps must be >= 0 and rope_theta > 0");
  if (c->rope_llama3 && (!(c->llama3_factor > 0) ||
                         !(c->llama3_high_freq_factor > c->llama3_low_freq_factor) ||
                         !(c->llama3_original_max_pos > 0)))
    return fail(EMBER_E_CONFIG, "invalid llama3 RoPE scaling parameters");
  return EMBER_OK;
}

Plan make_plan(const ember_config& c) {
  Plan p{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  const bool q8 = c.weight_dtype == EMBER_Q8_0;
  const size_t ws = q8 ? 1 : dtype_size(c.weight_dtype);
  const int H = c.hidden, HD = c.head_dim, NH = c.heads, NKV = c.kv_heads, FF = c.ffn;
  // a matrix [N, K]: its values (q8: the byte plane), then for q8 the scale plane
  auto mat = [&](size_t N, size_t K, size_t& scales) {
    const size_t o = take(N * K * ws);
    scales = q8 ? take(N * (K / kQ8Block) * 2) : 0;
    return o;
  };
  p.qkv_n = (NH + 2 * NKV) * HD;
  p.embed = mat(c.vocab, H, p.embed_s);
  p.layer.resize(c.layers);
  for (int l = 0; l < c.layers; ++l) {
    LayerOff& L = p.layer[l];
    L.ln1 = take((size_t)H * 4);
    L.wqkv = mat(p.qkv_n, H, L.wqkv_s);
    L.bqkv = c.qkv_bias ? take((size_t)p.qkv_n * 4) : 0;
    L.wo = mat(H, (size_t)NH * HD, L.wo_s);
    L.qn = c.qk_norm ? take((size_t)HD * 4) : 0;
    L.kn = c.qk_norm ? take((size_t)HD * 4) : 0;
    L.ln2 = take((size_t)H * 4);
    L.wgu = mat((size_t)2 * FF, H, L.wgu_s);
    L.wd = mat(H, FF, L.wd_s);
  }
  p.fnorm = take((size_t)H * 4);
  p.cls_w = c.head_kind == EMBER_HEAD_CLS ? take((size_t)c.n_classes * H * ws) : 0;
  p.cls_b = c.head_kind == EMBER_HEAD_CLS ? take((size_t)c.n_classes * 4) : 0;
  p.sens_w = c.sens_head ? take((size_t)H * 4) : 0;
  p.sens_b = c.sens_head ? take(4) : 0;
  p.sens_acc = c.sens_head ? take((size_t)c.max_batch * H * 4) : 0;
  p.sens_out = c.sens_head ? take((size_t)c.max_batch * 4) : 0;
  p.cos_t = take((size_t)c.max_seq * (HD / 2) * 4);
  p.sin_t = take((size_t)c.max_seq * (HD / 2) * 4);

  const int Mx = c.max_tokens > c.max_batch ? c.max_tokens : c.max_batch;
  p.Mx = Mx;
  p.ka = H > NH * HD ? H : NH * HD;
  const int out_dim = c.head_kind == EMBER_HEAD_CLS ? c.n_classes : c.vocab;
  p.nsplit_max = (c.max_seq + 63) / 64;
  p.argparts = gemv_num_blocks(c.vocab, GEMV_LOGITS, H, weight_kind(c.weight_dtype));
  p.ids = take((size_t)Mx * 4);
  p.pos = take(4);
  p.row_pos = take((size_t)c.max_batch * 4);
  p.rope_cur = take((size_t)c.max_batch * c.head_dim * 4);
  p.next = take((size_t)Mx * 4);
  p.flags = take(kNumFlags * 4);
  p.x = take((size_t)Mx * H * 4);
  p.xb = take((size_t)Mx * H * 4);
  p.pa_hi = take((size_t)Mx * p.ka * 2);
  p.pa_lo = take((size_t)Mx * p.ka * 2);
  // EXACT multi-token passes: the third plane of the QKV projection's input (q and k
  // feed the attention scores, whose absolute error the softmax amplifies)
  p.pa_x2 = uses_mfma(c) && c.precision == EMBER_EXACT ? take((size_t)Mx * p.ka * 2) : 0;
  p.pb_hi = take((size_t)Mx * FF * 2);
  p.pb_lo = take((size_t)Mx * FF * 2);
  p.qkv = take((size_t)Mx * p.qkv_n * 4);
  p.q = take((size_t)Mx * NH * HD * 4);
  p.att = take((size_t)Mx * NH * HD * 4);
  p.act = take((size_t)Mx * FF * 4);
  p.part = take((size_t)c.max_batch * NH * p.nsplit_max * (HD + 2) * 4);
  p.logits = take((size_t)c.max_batch * out_dim * 4);
  p.argpart = take((size_t)p.argparts * 8);
  // sampler state and tile sums, one per batch row (tied LM head only)
  const bool can_sample = c.head_kind == EMBER_HEAD_TIED_LM && c.vocab <= kSampleMaxVocab;
  p.samp_state = can_sample ? take((size_t)c.max_batch * sizeof(SampleState)) : 0;
  p.samp_tiles = can_sample ? take((size_t)c.max_batch * sample_tiles_ld(c.vocab) * 4) : 0;
  {
    // split-K partial planes for GEMMs whose tiles cannot fill the GPU (M <= 128)
    int maxn = 2 * FF > p.qkv_n ? 2 * FF : p.qkv_n;
    if (H > maxn) maxn = H;
    const int mrows = Mx < 128 ? Mx : 128;
    p.splitk_elems = uses_mfma(c) ? (size_t)16 * mrows * maxn : 0;
    // two weight planes: both passes of a SiLU GEMM land in partial planes
    if (q8_pair(c) && p.splitk_elems < (size_t)2 * Mx * maxn) p.splitk_elems = (size_t)2 * Mx * maxn;
    p.splitk = p.splitk_elems ? take(p.splitk_elems * 4) : 0;
  }
  {
    // packed K / V^T planes for the tiled prefill attention: one pass holds at most Mx
    // tokens, or one row of up to max_seq keys, each row rounded up to a 64-key tile
    const bool tiled = uses_mfma(c) && (HD == 64 || HD == 128);
    const int cap_keys = (Mx > c.max_seq ? Mx : c.max_seq) + 64 * c.max_batch;
    const bool ex = c.precision == EMBER_EXACT;
    p.kvpack_elems = tiled ? (size_t)(kv_pack_kplanes(ex) + kv_pack_vplanes(ex)) * NKV * cap_keys * HD : 0;
    p.kvpack = p.kvpack_elems ? take(p.kvpack_elems * 2) : 0;
  }
  if (q8) {
    // the dequantised copy of one matrix for the GEMMs of multi-token passes (bf16, or
    // the bf16 pair in EXACT precision): the largest of a layer's matrices and the
    // embedding
    size_t elems = (size_t)c.vocab * H;
    const size_t cand[4] = {(size_t)p.qkv_n * H, (size_t)H * NH * HD, (size_t)2 * FF * H,
                            (size_t)H * FF};
    for (size_t e : cand) elems = e > elems ? e : elems;
    p.q8_scratch = take(elems * (q8_pair(c) ? 4 : 2));
  }
  p.total = off;
  return p;
}

// RoPE frequencies: freq_i = theta^(-2i/HD) ("ember scripts/reference_forward.py",
// inv_freq), llama3-scaled by lerp(1/factor, 1, clip(z, 0, 1)) with
// z = (orig * freq / (2 pi) - low) / (high - low) ("LowLlamaBasic reference.py",
// rotary_cos_sin). Angles pos * freq and their cos/sin in f64, rounded once to f32.
void rope_host(const ember_config& c, int n_pos, float* cs, float* sn) {
  const int half = c.head_dim / 2;
  std::vector<double> freq(half);
  for (int i = 0; i < half; ++i) {
    double f = 1.0 / std::pow(c.rope_theta, 2.0 * (double)i / (double)c.head_dim);
    if (c.rope_llama3) {
      const double lo = c.llama3_low_freq_factor, hi = c.llama3_high_freq_factor;
      double z = (c.llama3_original_max_pos * f / (2.0 * M_PI) - lo) / (hi - lo);
      z = z < 0.0 ? 0.0 : (z > 1.0 ? 1.0 : z);
      const double start = 1.0 / c.llama3_factor;
      f *= start + z * (1.0 - start);
    }
    freq[i] = f;
  }
  for (int p = 0; p < n_pos; ++p)
    for (int i = 0; i < half; ++i) {
      const double ang = (double)p * freq[i];
      cs[(size_t)p * half + i] = (float)std::cos(ang);
      sn[(size_t)p * half + i] = (float)std::sin(ang);
    }
}

}  // namespace

struct ember_model {
  ember_config cfg;
  Plan plan;
  char* ws;
  int wk;                   // WeightKind of the matrices
  bool mfma;                // multi-token passes on bf16 MFMA (see uses_mfma)
  int has_logits_rows;      // rows in the logits buffer, 0 before any forward
  int sens_rows = 0;        // rows of sequence scores of the last prefill
  int last_decode_batch = 0;
  struct { int M, rows, tpr, b0, start; } last_pass = {0, 0, 0, 0, 0};
  // decode graph cache
  hipGraphExec_t graph = nullptr;
  const ember_cache* graph_cache = nullptr;
  int graph_batch = -1;
  hipStream_t graph_stream = nullptr;
  int32_t* graph_next = nullptr;
  // sampler of the next-token outputs (greedy argmax when `sampling` is false)
  ember_sampler samp{};
  bool sampling = false;
  template <typename T> T* at(size_t off) const { return (T*)(ws + off); }
  float* splitk() const { return plan.splitk_elems ? (float*)(ws + plan.splitk) : nullptr; }
};

struct ember_cache {
  ember_model* model;
  char* kv;
  size_t layer_bytes;
  std::vector<int> filled;  // per batch row: positions 0..filled[r]-1 hold K/V
};

namespace {

struct Ctx {
  ember_model* m;
  ember_cache* c;
  hipStream_t st;
  int only = -1;     // >= 0: launch only the kernel of this ember_kernel kind (timing)
};

bool want(const Ctx& cx, int kind) { return cx.only < 0 || cx.only == kind; }
bool want_aux(const Ctx& cx) { return cx.only < 0; }

// GEMV weight arguments of one matrix (values at `off`, q8 scales at `soff`).
void gemv_weights(const ember_model* md, GemvArgs& g, size_t off, size_t soff) {
  g.W = md->ws + off;
  g.w_bf16 = md->wk == WK_BF16;
  g.w_scale = md->wk == WK_Q8 ? (const uint16_t*)(md->ws + soff) : nullptr;
}

// Weights of one matrix [N, K] for the GEMM of a multi-token pass: in place for bf16 and
// f32; q8 matrices are first dequantised into the scratch copy, stream-ordered before the
// GEMM that reads it: bf16, or in EXACT precision the bf16 pair (the second plane in *lo).
const void* gemm_weights(const Ctx& cx, size_t off, size_t soff, int N, int K,
                         const uint16_t** lo = nullptr) {
  ember_model* md = cx.m;
  if (lo) *lo = nullptr;
  if (md->wk != WK_Q8) return md->ws + off;
  void* dst = md->ws + md->plan.q8_scratch;
  const bool pair = q8_pair(md->cfg);
  if (want_aux(cx))
    launch_q8_dequant((const uint8_t*)(md->ws + off), (const uint16_t*)(md->ws + soff), N, K, dst,
                      pair ? Q8_TO_BF16_PAIR : Q8_TO_BF16, cx.st);
  if (pair && lo) *lo = (const uint16_t*)dst + (size_t)N * K;
  return dst;
}

// Next ids of R rows of logits [R, ld] drawn with the model's sampler: draw row u_pos
// (the device position of a decode step when u_pos < 0), columns u_col0 + r.
void launch_draw(const Ctx& cx, const float* logits, int R, long long ld, int32_t* next,
                 int u_col0, int u_pos) {
  ember_model* md = cx.m;
  SampleArgs a{};
  a.logits = logits; a.ld = ld; a.R = R; a.V = md->cfg.vocab;
  a.temperature = md->samp.temperature; a.top_k = md->samp.top_k; a.top_p = md->samp.top_p;
  a.uniform = md->samp.d_uniform; a.u_rows = md->samp.n_pos; a.u_ld = md->samp.ld;
  a.seed = md->samp.seed;
  a.col0 = u_col0; a.pos = u_pos < 0 ? 0 : u_pos;
  a.d_pos = u_pos < 0 ? md->at<int>(md->plan.row_pos) : nullptr;
  a.next = next; a.flags = md->at<int>(md->plan.flags);
  a.state = md->at<SampleState>(md->plan.samp_state);
  a.tiles = md->at<float>(md->plan.samp_tiles);
  launch_sample(a, cx.st);
}

// Whether a call drawing `rows` rows from draw row `u_pos` fits the sampler's draws.
ember_status check_draws(const ember_model* md, int rows, long long u_pos) {
  if (!md->sampling || !md->samp.d_uniform) return EMBER_OK;   // on-device draws: no array
  if (u_pos >= md->samp.n_pos)
    return fail(EMBER_E_CAPACITY, "draw row %lld beyond the sampler's %d rows", u_pos,
                md->samp.n_pos);
  if (rows > md->samp.ld)
    return fail(EMBER_E_CAPACITY, "batch %d beyond the sampler's row stride %d", rows,
                md->samp.ld);
  return EMBER_OK;
}

void* k_layer(const ember_cache* c, int l) { return c->kv + (size_t)l * c->layer_bytes; }
void* v_layer(const ember_cache* c, int l) {
  return c->kv + (size_t)(c->model->cfg.layers + l) * c->layer_bytes;
}

enum Path { PATH_GEMV, PATH_MFMA, PATH_F32W };
enum Attn { ATTN_FLASH, ATTN_DECODE };

struct Pass {
  int M;             // tokens in the pass = rows * tpr
  int rows, tpr, b0, start;
  const int* d_pos;  // decode: each row's position, from device [rows]
  Path path;
  Attn attn;
};

// One decoder block over the pass's tokens: x += attn(norm(x)); x += mlp(norm(x)).
// One layer of a pass. `pending` > 0: the previous layer's down projection left that many
// split-K partial planes for this layer's first norm to add into x. With `defer_down` (the
// caller runs the next layer right after this one, with no reader of x in between) this
// layer's down projection may do the same; returns its plane count (0: x is complete).
int run_layer(const Ctx& cx, int li, const Pass& ps, int pending = 0, bool defer_down = false) {
  ember_model* md = cx.m;
  const ember_config& c = md->cfg;
  const Plan& p = md->plan;
  const LayerOff& L = p.layer[li];
  hipStream_t st = cx.st;
  const int H = c.hidden, NH = c.heads, NKV = c.kv_heads, HD = c.head_dim, FF = c.ffn;
  const bool exact = c.precision == EMBER_EXACT;
  float* x = md->at<float>(p.x);
  float* xb = md->at<float>(p.xb);
  float* qkv = md->at<float>(p.qkv);
  float* q = md->at<float>(p.q);
  float* att = md->at<float>(p.att);
  float* act = md->at<float>(p.act);
  float* part = md->at<float>(p.part);
  uint16_t* pa_hi = md->at<uint16_t>(p.pa_hi);
  uint16_t* pa_lo = exact ? md->at<uint16_t>(p.pa_lo) : nullptr;
  uint16_t* pb_hi = md->at<uint16_t>(p.pb_hi);
  uint16_t* pb_lo = exact ? md->at<uint16_t>(p.pb_lo) : nullptr;
  const float* ln1 = md->at<float>(L.ln1);
  const float* ln2 = md->at<float>(L.ln2);
  const float* bqkv = c.qkv_bias ? md->at<float>(L.bqkv) : nullptr;
  const float scale = (float)(1.0 / std::sqrt((double)HD));
  // one-row decode: the output-projection GEMV can rebuild its input from up to
  // `fold_max` attention split partials (no combine launch); its row-per-block layout
  // takes up to 8, so the plan is capped there
  const int fold_max = ps.attn == ATTN_DECODE && ps.path == PATH_GEMV
                           ? gemv_parts_max(H, NH * HD, md->wk) : 0;
  DecodePlan dp{1, c.max_seq, NH / NKV};
  if (ps.attn == ATTN_DECODE)
    dp = decode_split_plan(ps.M, NH, NKV, c.max_seq, fold_max > 4 ? fold_max : 64);
  const bool fuse_combine = fold_max > 0 && dp.nsplit > 1 && dp.nsplit <= fold_max;

  // q/k norm, RoPE and the K/V store of a prefill pass (QKV post-processing)
  QkvPostArgs qa{};
  qa.qkv = qkv; qa.M = ps.M; qa.NH = NH; qa.NKV = NKV; qa.HD = HD;
  qa.tokens_per_row = ps.tpr; qa.b0 = ps.b0; qa.start_pos = ps.start; qa.d_pos = ps.d_pos;
  qa.cos_t = md->at<float>(p.cos_t); qa.sin_t = md->at<float>(p.sin_t);
  qa.q_norm = c.qk_norm ? md->at<float>(L.qn) : nullptr;
  qa.k_norm = c.qk_norm ? md->at<float>(L.kn) : nullptr;
  qa.eps = c.rms_eps; qa.q_out = q;
  qa.k_cache = k_layer(cx.c, li); qa.v_cache = v_layer(cx.c, li);
  qa.kv_bf16 = c.kv_dtype == EMBER_BF16; qa.max_seq = c.max_seq;

  // ---- attention block
  int qkv_deferred = 0;
  if (ps.path == PATH_GEMV) {
    GemvArgs g{};
    gemv_weights(md, g, L.wqkv, L.wqkv_s);
    g.N = p.qkv_n; g.K = H; g.M = ps.M;
    g.x = x; g.norm_w = ln1; g.eps = c.rms_eps; g.bias = bqkv; g.y = qkv; g.ldy = p.qkv_n;
    if (want(cx, EMBER_K_QKV)) launch_gemv(g, GEMV_STORE, st);
  } else if (ps.path == PATH_MFMA) {
    uint16_t* pa_x2 = exact ? md->at<uint16_t>(p.pa_x2) : nullptr;
    // one-token decode: a split-K QKV GEMM leaves its partial planes to the attention
    // kernel, which sums the few projections it reads (no reduce launch)
    const bool defer_qkv = want_aux(cx) && ps.attn == ATTN_DECODE;
    if (want_aux(cx))
      launch_rmsnorm(x, ln1, c.rms_eps, ps.M, H, 1, 0, nullptr, pa_hi, pa_lo, p.ka, st, pa_x2,
                     md->splitk(), pending);
    GemmArgs g{};
    g.partial = md->splitk(); g.partial_elems = p.splitk_elems;
    g.a_hi = pa_hi; g.a_lo = pa_lo; g.lda = p.ka;
    g.w = (const uint16_t*)gemm_weights(cx, L.wqkv, L.wqkv_s, p.qkv_n, H, &g.w_lo);
    g.M = ps.M; g.N = p.qkv_n; g.K = H; g.bias = bqkv; g.c = qkv; g.ldc = p.qkv_n;
    if (exact) {
      // EXACT: the input as three bf16 planes (within ~2^-25), so q and k are f32-level:
      // planes hi + lo store the projections (+bias), the third plane adds into them
      // (v as well: with peaked attention the output is one value row, and two planes
      // leave it ~2^-17 sqrt(K) off, 1e-4 in the logits); the post-processing (prefill)
      // or the decode attention then reads them. Where one pass takes all three planes,
      // a prefill with head_dim 64 does the post-processing in that GEMM's epilogue
      // (the f32 projections never reach memory)
      GemmArgs g3 = g;
      g3.a_x2 = pa_x2;
      const bool three = gemm_three_planes(g3);
      const bool fused = three && ps.attn == ATTN_FLASH && HD == 64;
      if (want(cx, EMBER_K_QKV)) {
        if (fused) {
          g3.post = qa;
          launch_gemm(g3, GEMM_QKV, st);
        } else if (three) {
          qkv_deferred = launch_gemm(g3, GEMM_STORE, st, defer_qkv);   // all three planes, one pass
        } else {
          launch_gemm(g, GEMM_STORE, st);
          g3.a_hi = pa_x2; g3.a_lo = nullptr; g3.a_x2 = nullptr; g3.bias = nullptr;
          launch_gemm(g3, GEMM_RESID, st);
        }
      }
      if (want_aux(cx) && ps.attn == ATTN_FLASH && !fused) launch_qkv_post(qa, st);
    } else if (ps.attn == ATTN_FLASH) {
      g.post = qa;
      if (want(cx, EMBER_K_QKV)) launch_gemm(g, GEMM_QKV, st);
    } else if (want(cx, EMBER_K_QKV)) {
      qkv_deferred = launch_gemm(g, GEMM_STORE, st, defer_qkv);
    }
  } else {
    if (want_aux(cx)) launch_rmsnorm(x, ln1, c.rms_eps, ps.M, H, 1, 0, xb, nullptr, nullptr, 0, st);
    GemmF32Args g{};
    g.a = xb; g.lda = H; g.w = (const float*)gemm_weights(cx, L.wqkv, L.wqkv_s, p.qkv_n, H);
    g.M = ps.M; g.N = p.qkv_n; g.K = H;
    g.bias = bqkv; g.c = qkv; g.ldc = p.qkv_n;
    if (want(cx, EMBER_K_QKV)) launch_gemm_f32w(g, GEMM_STORE, st);
  }

  // prefill on MFMA: the QKV GEMM applies the post-processing itself (GEMM_QKV)
  if (want_aux(cx) && ps.attn == ATTN_FLASH && ps.path != PATH_MFMA) launch_qkv_post(qa, st);

  const bool planes_out = ps.path == PATH_MFMA;
  if (ps.attn == ATTN_FLASH) {
    FlashArgs fa{};
    fa.q = q; fa.k_cache = qa.k_cache; fa.v_cache = qa.v_cache; fa.kv_bf16 = qa.kv_bf16;
    fa.NH = NH; fa.NKV = NKV; fa.HD = HD; fa.max_seq = c.max_seq;
    fa.tokens_per_row = ps.tpr; fa.rows = ps.rows; fa.b0 = ps.b0; fa.start_pos = ps.start;
    fa.causal = c.causal != 0; fa.scale = scale;
    fa.out_f32 = planes_out ? nullptr : att;
    fa.out_hi = planes_out ? pa_hi : nullptr;
    fa.out_lo = planes_out ? pa_lo : nullptr;
    if (want(cx, EMBER_K_ATTN)) {
      const int key_end = ps.start + ps.tpr;
      const size_t need = kv_pack_elems(ps.rows, NKV, HD, key_end, exact);
      if (planes_out && flash_mfma_supported(HD) && need <= p.kvpack_elems) {
        // pack this pass's keys into bf16 K and V^T planes, then the tiled MFMA kernel
        KvPackArgs ka{};
        ka.k_cache = qa.k_cache; ka.v_cache = qa.v_cache; ka.kv_bf16 = qa.kv_bf16;
        ka.NKV = NKV; ka.HD = HD; ka.max_seq = c.max_seq;
        ka.rows = ps.rows; ka.b0 = ps.b0; ka.key_end = key_end; ka.LK = kv_pack_lk(key_end);
        ka.split = exact;
        ka.kp = md->at<uint16_t>(p.kvpack);
        ka.vt = ka.kp + (size_t)kv_pack_kplanes(exact) * ps.rows * NKV * ka.LK * HD;
        launch_kv_pack(ka, st);
        launch_flash_tiled(fa, ka.kp, ka.vt, ka.LK, exact, st);
      } else if (planes_out && flash_mfma_supported(HD)) {
        launch_flash_mfma(fa, exact, st);
      } else {
        launch_flash_prefill(fa, st);
      }
    }
  } else {
    DecodeAttnArgs da{};
    da.qkv = qkv; da.rope_cur = md->at<float>(p.rope_cur); da.q_norm = qa.q_norm;
    da.k_norm = qa.k_norm; da.eps = c.rms_eps;
    da.k_cache = qa.k_cache; da.v_cache = qa.v_cache; da.kv_bf16 = qa.kv_bf16;
    da.B = ps.M; da.NH = NH; da.NKV = NKV; da.HD = HD; da.max_seq = c.max_seq;
    da.d_pos = ps.d_pos; da.nsplit = dp.nsplit; da.chunk_min = dp.chunk_min; da.scale = scale;
    da.part = part; da.heads_per_block = dp.heads_per_block;
    da.qkv_part = md->splitk(); da.qkv_splits = qkv_deferred; da.qkv_bias = bqkv;
    da.out_f32 = planes_out ? nullptr : att;
    da.out_hi = planes_out ? pa_hi : nullptr;
    da.out_lo = planes_out ? pa_lo : nullptr;
    if (want(cx, EMBER_K_ATTN)) launch_decode_attn(da, st);
    if (want_aux(cx) && dp.nsplit > 1 && !fuse_combine)
      launch_attn_combine(part, ps.M, NH, HD, dp.nsplit, ps.d_pos, dp.chunk_min,
                          da.out_f32, da.out_hi, da.out_lo, st);
  }

  int o_deferred = 0;
  if (ps.path == PATH_GEMV) {
    GemvArgs g{};
    gemv_weights(md, g, L.wo, L.wo_s);
    g.N = H; g.K = NH * HD; g.M = ps.M;
    g.x = att; g.y = x; g.ldy = H;
    if (fuse_combine) {
      g.x = nullptr;
      g.xpart = part; g.xp_nsplit = dp.nsplit; g.xp_hd = HD; g.xp_chunk_min = dp.chunk_min;
      g.xp_pos = ps.d_pos;
    }
    if (want(cx, EMBER_K_O)) launch_gemv(g, GEMV_RESID, st);
  } else if (ps.path == PATH_MFMA) {
    GemmArgs g{};
    g.partial = md->splitk(); g.partial_elems = p.splitk_elems;
    g.a_hi = pa_hi; g.a_lo = pa_lo; g.lda = p.ka;
    g.w = (const uint16_t*)gemm_weights(cx, L.wo, L.wo_s, H, NH * HD, &g.w_lo);
    g.M = ps.M; g.N = H; g.K = NH * HD; g.c = x; g.ldc = H;
    // a split-K residual add is left to the norm that follows (it reads x anyway)
    if (want(cx, EMBER_K_O))
      o_deferred = launch_gemm(g, GEMM_RESID, st, want_aux(cx) && rmsnorm_adds_partials(H, p.ka));
  } else {
    GemmF32Args g{};
    g.a = att; g.lda = NH * HD; g.w = (const float*)gemm_weights(cx, L.wo, L.wo_s, H, NH * HD);
    g.M = ps.M; g.N = H; g.K = NH * HD;
    g.c = x; g.ldc = H;
    if (want(cx, EMBER_K_O)) launch_gemm_f32w(g, GEMM_RESID, st);
  }

  // ---- MLP block
  int down_deferred = 0;
  if (ps.path == PATH_GEMV) {
    GemvArgs g{};
    gemv_weights(md, g, L.wgu, L.wgu_s);
    g.N = FF; g.K = H; g.M = ps.M;
    g.x = x; g.norm_w = ln2; g.eps = c.rms_eps; g.y = act; g.ldy = FF;
    if (want(cx, EMBER_K_GATE_UP)) launch_gemv(g, GEMV_SILU, st);
    GemvArgs d{};
    gemv_weights(md, d, L.wd, L.wd_s);
    d.N = H; d.K = FF; d.M = ps.M; d.x = act; d.y = x; d.ldy = H;
    if (want(cx, EMBER_K_DOWN)) launch_gemv(d, GEMV_RESID, st);
  } else if (ps.path == PATH_MFMA) {
    if (want_aux(cx))
      launch_rmsnorm(x, ln2, c.rms_eps, ps.M, H, 1, 0, nullptr, pa_hi, pa_lo, p.ka, st, nullptr,
                     md->splitk(), o_deferred);
    GemmArgs g{};
    g.partial = md->splitk(); g.partial_elems = p.splitk_elems;
    g.a_hi = pa_hi; g.a_lo = pa_lo; g.lda = p.ka;
    g.w = (const uint16_t*)gemm_weights(cx, L.wgu, L.wgu_s, 2 * FF, H, &g.w_lo);
    g.M = ps.M; g.N = 2 * FF; g.K = H; g.o_hi = pb_hi; g.o_lo = pb_lo; g.ldo = FF;
    GemmArgs d{};
    d.partial = md->splitk(); d.partial_elems = p.splitk_elems;
    d.a_hi = pb_hi; d.a_lo = pb_lo; d.lda = FF;
    d.M = ps.M; d.N = H; d.K = FF; d.c = x; d.ldc = H;
    if (want(cx, EMBER_K_GATE_UP)) launch_gemm(g, GEMM_SILU, st);
    d.w = (const uint16_t*)gemm_weights(cx, L.wd, L.wd_s, H, FF, &d.w_lo);   // after the gate/up GEMM
    if (want(cx, EMBER_K_DOWN))
      down_deferred = launch_gemm(d, GEMM_RESID, st,
                                  defer_down && want_aux(cx) && rmsnorm_adds_partials(H, p.ka));
  } else {
    if (want_aux(cx)) launch_rmsnorm(x, ln2, c.rms_eps, ps.M, H, 1, 0, xb, nullptr, nullptr, 0, st);
    GemmF32Args g{};
    g.a = xb; g.lda = H; g.w = (const float*)gemm_weights(cx, L.wgu, L.wgu_s, 2 * FF, H);
    g.M = ps.M; g.N = 2 * FF; g.K = H;
    g.o_f32 = act; g.ldo = FF;
    if (want(cx, EMBER_K_GATE_UP)) launch_gemm_f32w(g, GEMM_SILU, st);
    GemmF32Args d{};
    d.a = act; d.lda = FF; d.w = (const float*)gemm_weights(cx, L.wd, L.wd_s, H, FF);
    d.M = ps.M; d.N = H; d.K = FF;
    d.c = x; d.ldc = H;
    if (want(cx, EMBER_K_DOWN)) launch_gemm_f32w(d, GEMM_RESID, st);
  }
  return down_deferred;
}

// Tied LM head over R rows of x (row r = x[r * row_step + row_off]): final RMSNorm, then
// logits = E . h ("ember scripts/reference_forward.py", end of forward), then the greedy
// argmax, or the sampler's draw (draw row u_pos, or the device position when u_pos < 0;
// columns u_col0 + r). Writes logits [R, ld] at `out` and next ids when `next` is
// non-null.
void run_lm_head(const Ctx& cx, int R, int row_step, int row_off, float* out, long long ld,
                 int32_t* next, int u_col0 = 0, int u_pos = -1) {
  const bool draw = next && cx.m->sampling && (want_aux(cx) || cx.only == EMBER_K_SAMPLE);
  ember_model* md = cx.m;
  const ember_config& c = md->cfg;
  const Plan& p = md->plan;
  hipStream_t st = cx.st;
  const int H = c.hidden, V = c.vocab;
  const float* fn = md->at<float>(p.fnorm);
  if (R == 1 && ld == V) {
    // the final RMSNorm is fused into the GEMV
    GemvArgs g{};
    gemv_weights(md, g, p.embed, p.embed_s);
    g.N = V; g.K = H; g.M = 1;
    g.x = md->at<float>(p.x) + (size_t)row_off * H; g.norm_w = fn; g.eps = c.rms_eps;
    g.y = out; g.ldy = V;
    g.argmax_part = md->at<unsigned long long>(p.argpart);
    g.flags = md->at<int>(p.flags);
    if (want(cx, EMBER_K_LM_HEAD)) launch_gemv(g, GEMV_LOGITS, st);
    if (draw)
      launch_draw(cx, out, 1, ld, next, u_col0, u_pos);
    else if (next && want_aux(cx))
      launch_argmax_reduce(g.argmax_part, gemv_num_blocks(V, GEMV_LOGITS, H, md->wk), 1, next, st);
    return;
  }
  // R rows (at most the pass capacity Mx at a time: the plane / xb buffers hold Mx rows)
  const int G = p.Mx;
  float* xb = md->at<float>(p.xb);
  const uint16_t* Ew_lo = nullptr;
  const void* Ew = gemm_weights(cx, p.embed, p.embed_s, V, H, &Ew_lo);
  for (int r0 = 0; r0 < R; r0 += G) {
    const int rn = R - r0 < G ? R - r0 : G;
    const int off = row_off + r0 * row_step;
    if (md->mfma) {
      uint16_t* hi = md->at<uint16_t>(p.pa_hi);
      uint16_t* lo = c.precision == EMBER_EXACT ? md->at<uint16_t>(p.pa_lo) : nullptr;
      if (want_aux(cx))
        launch_rmsnorm(md->at<float>(p.x), fn, c.rms_eps, rn, H, row_step, off, nullptr, hi, lo,
                       p.ka, st);
      GemmArgs g{};
      g.partial = md->splitk(); g.partial_elems = p.splitk_elems;
      g.a_hi = hi; g.a_lo = lo; g.lda = p.ka; g.w = (const uint16_t*)Ew; g.w_lo = Ew_lo;
      g.M = rn; g.N = V; g.K = H; g.c = out + (size_t)r0 * ld; g.ldc = ld;
      if (want(cx, EMBER_K_LM_HEAD)) launch_gemm(g, GEMM_STORE, st);
    } else {
      if (want_aux(cx))
        launch_rmsnorm(md->at<float>(p.x), fn, c.rms_eps, rn, H, row_step, off, xb, nullptr,
                       nullptr, 0, st);
      GemmF32Args g{};
      g.a = xb; g.lda = H; g.w = (const float*)Ew; g.M = rn; g.N = V; g.K = H;
      g.c = out + (size_t)r0 * ld; g.ldc = ld;
      if (want(cx, EMBER_K_LM_HEAD)) launch_gemm_f32w(g, GEMM_STORE, st);
    }
    if (draw)
      launch_draw(cx, out + (size_t)r0 * ld, rn, ld, next + r0, u_col0 + r0, u_pos);
    else if (next && want_aux(cx))
      launch_argmax_rows(out + (size_t)r0 * ld, rn, V, ld, next + r0, md->at<int>(p.flags), st);
  }
}

// Classification head over R rows of x: out[r] = Wc . rmsnorm(x_r) + bc, next[r] = argmax.
void run_cls_head(const Ctx& cx, int R, int row_step, int row_off, float* out, int32_t* next) {
  ember_model* md = cx.m;
  const ember_config& c = md->cfg;
  const Plan& p = md->plan;
  const int H = c.hidden;
  float* xb = md->at<float>(p.xb);
  const int G = p.Mx;
  for (int r0 = 0; r0 < R; r0 += G) {
    const int rn = R - r0 < G ? R - r0 : G;
    launch_rmsnorm(md->at<float>(p.x), md->at<float>(p.fnorm), c.rms_eps, rn, H, row_step,
                   row_off + r0 * row_step, xb, nullptr, nullptr, 0, cx.st);
    launch_cls_head(xb, md->ws + p.cls_w, md->wk == WK_BF16, md->at<float>(p.cls_b), rn, H, c.n_classes,
                    out ? out + (size_t)r0 * c.n_classes : nullptr, next ? next + r0 : nullptr,
                    cx.st);
  }
}

// One decode step's device work for B rows, ids in plan.ids, position in plan.pos.
// The layers and the LM head of one decode step (the step's embedding and staging run
// before it); the next ids (greedy or drawn) go to `next`.
void decode_body(const Ctx& cx, int B, int32_t* next, int only_layer = -1) {
  ember_model* md = cx.m;
  const ember_config& c = md->cfg;
  const Plan& p = md->plan;
  Pass ps{};
  ps.M = B; ps.rows = B; ps.tpr = 1; ps.b0 = 0; ps.start = 0; ps.d_pos = md->at<int>(p.row_pos);
  ps.path = B == 1 ? PATH_GEMV : (md->mfma ? PATH_MFMA : PATH_F32W);
  ps.attn = ATTN_DECODE;
  // layer l's down projection may leave its split-K planes to layer l + 1's first norm
  int pending = 0;
  for (int l = 0; l < c.layers; ++l)
    if (only_layer < 0 || l == only_layer)
      pending = run_layer(cx, l, ps, pending, only_layer < 0 && l + 1 < c.layers);
  if ((want(cx, EMBER_K_LM_HEAD) || cx.only == EMBER_K_SAMPLE) && (cx.only >= 0 || only_layer < 0))
    run_lm_head(cx, B, 1, 0, md->at<float>(p.logits), c.vocab, next);
}

bool graphs_enabled() {
  const char* e = getenv("EMBER_NO_GRAPH");
  return !(e && e[0] && e[0] != '0');
}

}  // namespace

// =================================================================== C ABI

extern "C" {

const char* ember_last_error(void) { return g_last_error.c_str(); }

size_t ember_workspace_bytes(const ember_config* cfg) {
  if (validate_config(cfg) != EMBER_OK) return 0;
  return make_plan(*cfg).total;
}

size_t ember_kv_cache_bytes(const ember_config* cfg) {
  if (validate_config(cfg) != EMBER_OK) return 0;
  return (size_t)2 * cfg->layers * cfg->max_batch * cfg->kv_heads * cfg->max_seq *
         cfg->head_dim * dtype_size(cfg->kv_dtype);
}

ember_status ember_rope_table(const ember_config* cfg, int32_t n_pos, float* h_cos,
                              float* h_sin) {
  ember_status s = validate_config(cfg);
  if (s != EMBER_OK) return s;
  if (n_pos <= 0 || !h_cos || !h_sin) return fail(EMBER_E_ARG, "bad RoPE table arguments");
  rope_host(*cfg, n_pos, h_cos, h_sin);
  return EMBER_OK;
}

ember_status ember_load_weights(const ember_config* cfg, const ember_tensor* tensors,
                                int32_t n_tensors, void* d_workspace, size_t workspace_bytes,
                                void* stream, ember_model** out) {
  g_last_error.clear();
  if (!out) return fail(EMBER_E_ARG, "out is NULL");
  *out = nullptr;
  ember_status s = validate_config(cfg);
  if (s != EMBER_OK) return s;
  if (!d_workspace || (n_tensors > 0 && !tensors)) return fail(EMBER_E_ARG, "NULL pointer");
  const ember_config& c = *cfg;
  Plan plan = make_plan(c);
  gemm_init();
  flash_init();
  if (workspace_bytes < plan.total)
    return fail(EMBER_E_ARG, "workspace too small: %zu < %zu bytes", workspace_bytes, plan.total);

  // name -> tensor, with shape checks (cf. Falcon-H1 Rust reference, validate_weights)
  std::map<std::string, const ember_tensor*> byname;
  for (int i = 0; i < n_tensors; ++i) {
    if (!tensors[i].name || !tensors[i].data) return fail(EMBER_E_ARG, "tensor %d has NULL name/data", i);
    byname[tensors[i].name] = &tensors[i];
  }
  const bool q8 = c.weight_dtype == EMBER_Q8_0;
  auto need = [&](const std::string& n, std::vector<int64_t> shape,
                  const ember_tensor** t) -> ember_status {
    auto it = byname.find(n);
    if (it == byname.end()) return fail(EMBER_E_TENSOR_MISSING, "missing tensor %s", n.c_str());
    const ember_tensor* e = it->second;
    if (e->dtype != EMBER_F32 && e->dtype != EMBER_BF16 && e->dtype != EMBER_Q8_0)
      return fail(EMBER_E_DTYPE, "unsupported dtype %d for %s", e->dtype, n.c_str());
    // q8_0 configs: matrices in q8_0, vectors (norms, biases) in f32
    const int want_dt = q8 ? (shape.size() == 2 ? EMBER_Q8_0 : EMBER_F32) : c.weight_dtype;
    if (e->dtype != want_dt)
      return fail(EMBER_E_DTYPE, "tensor %s dtype %d differs from the config's (%d expected)",
                  n.c_str(), e->dtype, want_dt);
    bool ok = e->ndim == (int)shape.size();
    for (size_t d = 0; ok && d < shape.size(); ++d) ok = e->shape[d] == shape[d];
    if (!ok) return fail(EMBER_E_TENSOR_SHAPE, "bad shape for %s", n.c_str());
    *t = e;
    return EMBER_OK;
  };
  const int H = c.hidden, V = c.vocab, NH = c.heads, NKV = c.kv_heads, HD = c.head_dim, FF = c.ffn;
  struct LT { const ember_tensor *ln1, *q, *k, *v, *qb, *kb, *vb, *o, *qn, *kn, *ln2, *g, *u, *d; };
  std::vector<LT> lt(c.layers);
  const ember_tensor *emb = nullptr, *fn = nullptr, *clsw = nullptr, *clsb = nullptr,
                    *sensw = nullptr, *sensb = nullptr;
#define NEED(n, shape, dst) do { ember_status s_ = need(n, shape, dst); if (s_ != EMBER_OK) return s_; } while (0)
  NEED("model.embed_tokens.weight", (std::vector<int64_t>{V, H}), &emb);
  for (int l = 0; l < c.layers; ++l) {
    const std::string pf = "model.layers." + std::to_string(l) + ".";
    LT& t = lt[l];
    NEED(pf + "input_layernorm.weight", (std::vector<int64_t>{H}), &t.ln1);
    NEED(pf + "self_attn.q_proj.weight", (std::vector<int64_t>{NH * HD, H}), &t.q);
    NEED(pf + "self_attn.k_proj.weight", (std::vector<int64_t>{NKV * HD, H}), &t.k);
    NEED(pf + "self_attn.v_proj.weight", (std::vector<int64_t>{NKV * HD, H}), &t.v);
    if (c.qkv_bias) {
      NEED(pf + "self_attn.q_proj.bias", (std::vector<int64_t>{NH * HD}), &t.qb);
      NEED(pf + "self_attn.k_proj.bias", (std::vector<int64_t>{NKV * HD}), &t.kb);
      NEED(pf + "self_attn.v_proj.bias", (std::vector<int64_t>{NKV * HD}), &t.vb);
    }
    NEED(pf + "self_attn.o_proj.weight", (std::vector<int64_t>{H, NH * HD}), &t.o);
    if (c.qk_norm) {
      NEED(pf + "self_attn.q_norm.weight", (std::vector<int64_t>{HD}), &t.qn);
      NEED(pf + "self_attn.k_norm.weight", (std::vector<int64_t>{HD}), &t.kn);
    }
    NEED(pf + "post_attention_layernorm.weight", (std::vector<int64_t>{H}), &t.ln2);
    NEED(pf + "mlp.gate_proj.weight", (std::vector<int64_t>{FF, H}), &t.g);
    NEED(pf + "mlp.up_proj.weight", (std::vector<int64_t>{FF, H}), &t.u);
    NEED(pf + "mlp.down_proj.weight", (std::vector<int64_t>{H, FF}), &t.d);
  }
  NEED("model.norm.weight", (std::vector<int64_t>{H}), &fn);
  if (c.head_kind == EMBER_HEAD_CLS) {
    NEED("token_cls_head.weight", (std::vector<int64_t>{c.n_classes, H}), &clsw);
    NEED("token_cls_head.bias", (std::vector<int64_t>{c.n_classes}), &clsb);
  }
  if (c.sens_head) {
    NEED("sensitivity_head.weight", (std::vector<int64_t>{1, H}), &sensw);
    NEED("sensitivity_head.bias", (std::vector<int64_t>{1}), &sensb);
  }
#undef NEED

  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)d_workspace;
  const size_t es = dtype_size(c.weight_dtype);
  const bool bf = c.weight_dtype == EMBER_BF16;
  auto copy = [&](size_t dst, const ember_tensor* t, size_t bytes) -> hipError_t {
    return hipMemcpyAsync(ws + dst, t->data, bytes, hipMemcpyDeviceToDevice, st);
  };
  // q8_0 blocks into the byte and scale planes (rows placed as the copies below place them)
  auto unpack = [&](const ember_tensor* t, int N, int K, size_t off, size_t soff, int row0, int gu) {
    launch_q8_unpack((const uint8_t*)t->data, N, K, (uint8_t*)(ws + off), (uint16_t*)(ws + soff),
                     row0, gu, st);
  };
  if (q8) unpack(emb, V, H, plan.embed, plan.embed_s, 0, -1);
  else HIP_TRY(copy(plan.embed, emb, (size_t)V * H * es));
  for (int l = 0; l < c.layers; ++l) {
    const LayerOff& L = plan.layer[l];
    const LT& t = lt[l];
    launch_widen(t.ln1->data, bf, (float*)(ws + L.ln1), H, st);
    launch_widen(t.ln2->data, bf, (float*)(ws + L.ln2), H, st);
    // fused QKV rows: q, then k, then v
    if (q8) {
      unpack(t.q, NH * HD, H, L.wqkv, L.wqkv_s, 0, -1);
      unpack(t.k, NKV * HD, H, L.wqkv, L.wqkv_s, NH * HD, -1);
      unpack(t.v, NKV * HD, H, L.wqkv, L.wqkv_s, (NH + NKV) * HD, -1);
    } else {
      HIP_TRY(copy(L.wqkv, t.q, (size_t)NH * HD * H * es));
      HIP_TRY(copy(L.wqkv + (size_t)NH * HD * H * es, t.k, (size_t)NKV * HD * H * es));
      HIP_TRY(copy(L.wqkv + (size_t)(NH + NKV) * HD * H * es, t.v, (size_t)NKV * HD * H * es));
    }
    if (c.qkv_bias) {
      launch_widen(t.qb->data, bf, (float*)(ws + L.bqkv), NH * HD, st);
      launch_widen(t.kb->data, bf, (float*)(ws + L.bqkv) + NH * HD, NKV * HD, st);
      launch_widen(t.vb->data, bf, (float*)(ws + L.bqkv) + (NH + NKV) * HD, NKV * HD, st);
    }
    if (q8) unpack(t.o, H, NH * HD, L.wo, L.wo_s, 0, -1);
    else HIP_TRY(copy(L.wo, t.o, (size_t)H * NH * HD * es));
    if (c.qk_norm) {
      launch_widen(t.qn->data, bf, (float*)(ws + L.qn), HD, st);
      launch_widen(t.kn->data, bf, (float*)(ws + L.kn), HD, st);
    }
    // gate/up rows interleaved in blocks of kGuBlock (see gu_row)
    if (q8) {
      unpack(t.g, FF, H, L.wgu, L.wgu_s, 0, 0);
      unpack(t.u, FF, H, L.wgu, L.wgu_s, 0, 1);
      unpack(t.d, H, FF, L.wd, L.wd_s, 0, -1);
    } else {
      const size_t blk = (size_t)kGuBlock * H * es;
      HIP_TRY(hipMemcpy2DAsync(ws + L.wgu, 2 * blk, t.g->data, blk, blk, FF / kGuBlock,
                               hipMemcpyDeviceToDevice, st));
      HIP_TRY(hipMemcpy2DAsync(ws + L.wgu + blk, 2 * blk, t.u->data, blk, blk, FF / kGuBlock,
                               hipMemcpyDeviceToDevice, st));
      HIP_TRY(copy(L.wd, t.d, (size_t)H * FF * es));
    }
  }
  launch_widen(fn->data, bf, (float*)(ws + plan.fnorm), H, st);
  if (clsw) {
    HIP_TRY(copy(plan.cls_w, clsw, (size_t)c.n_classes * H * es));
    launch_widen(clsb->data, bf, (float*)(ws + plan.cls_b), c.n_classes, st);
  }
  if (sensw) {
    launch_widen(sensw->data, bf, (float*)(ws + plan.sens_w), H, st);
    launch_widen(sensb->data, bf, (float*)(ws + plan.sens_b), 1, st);
  }
  {
    std::vector<float> cs((size_t)c.max_seq * (HD / 2)), sn(cs.size());
    rope_host(c, c.max_seq, cs.data(), sn.data());
    HIP_TRY(hipMemcpyAsync(ws + plan.cos_t, cs.data(), cs.size() * 4, hipMemcpyHostToDevice, st));
    HIP_TRY(hipMemcpyAsync(ws + plan.sin_t, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, st));
    HIP_TRY(hipStreamSynchronize(st));
  }
  launch_fill_i32((int*)(ws + plan.flags), kNumFlags, 0, st);
  if (plan.samp_state)
    launch_fill_i32((int*)(ws + plan.samp_state),
                    (int)((size_t)c.max_batch * sizeof(SampleState) / 4), 0, st);
  HIP_TRY(hipGetLastError());
  HIP_TRY(hipStreamSynchronize(st));

  ember_model* m = new ember_model();
  m->cfg = c;
  m->plan = plan;
  m->ws = ws;
  m->wk = weight_kind(c.weight_dtype);
  m->mfma = uses_mfma(c);
  m->has_logits_rows = 0;
  *out = m;
  return EMBER_OK;
}

ember_status ember_cache_bind(ember_model* model, void* d_kv, size_t kv_bytes, ember_cache** out) {
  g_last_error.clear();
  if (!model || !d_kv || !out) return fail(EMBER_E_ARG, "NULL argument");
  *out = nullptr;
  const size_t need = ember_kv_cache_bytes(&model->cfg);
  if (kv_bytes < need) return fail(EMBER_E_CAPACITY, "KV buffer too small: %zu < %zu", kv_bytes, need);
  ember_cache* c = new ember_cache();
  c->model = model;
  c->kv = (char*)d_kv;
  c->layer_bytes = need / (2 * (size_t)model->cfg.layers);
  c->filled.assign((size_t)model->cfg.max_batch, 0);
  *out = c;
  return EMBER_OK;
}

namespace {

// The prefill of ember_prefill, optionally keeping each block's output at every row's
// last position in d_acts [batch][layers][hidden].
ember_status prefill_impl(ember_model* md, ember_cache* cache, const int32_t* h_ids,
                          int32_t batch, int32_t n_tokens, int32_t start_pos,
                          float* d_all_logits, int32_t* d_next, float* d_acts, void* stream,
                          int row0 = 0) {
  if (!md || !cache || !h_ids) return fail(EMBER_E_ARG, "NULL argument");
  if (cache->model != md) return fail(EMBER_E_ARG, "cache bound to another model");
  const ember_config& c = md->cfg;
  if (n_tokens <= 0) return fail(EMBER_E_ARG, "input_ids must not be empty");
  if (batch <= 0 || row0 < 0 || row0 + batch > c.max_batch)
    return fail(EMBER_E_CAPACITY, "batch %d outside 1..%d", batch, c.max_batch);
  if (start_pos < 0 || (long long)start_pos + n_tokens > c.max_seq)
    return fail(EMBER_E_CAPACITY, "positions [%d, %d) exceed max_seq %d", start_pos,
                start_pos + n_tokens, c.max_seq);
  for (int r = row0; r < row0 + batch; ++r)
    if (start_pos > cache->filled[r])
      return fail(EMBER_E_STATE, "start_pos %d leaves a gap after %d cached positions of row %d",
                  start_pos, cache->filled[r], r);
  if (!c.causal && start_pos != 0)
    return fail(EMBER_E_ARG, "a bidirectional model takes whole sequences (start_pos 0)");
  if (!c.causal && n_tokens > (c.max_tokens > c.max_batch ? c.max_tokens : c.max_batch))
    return fail(EMBER_E_CAPACITY, "a bidirectional row of %d tokens must fit one pass of %d",
                n_tokens, c.max_tokens > c.max_batch ? c.max_tokens : c.max_batch);
  for (long long i = 0; i < (long long)batch * n_tokens; ++i)
    if (h_ids[i] < 0 || h_ids[i] >= c.vocab)
      return fail(EMBER_E_TOKEN, "token %d outside vocabulary", h_ids[i]);
  if (d_next && c.head_kind == EMBER_HEAD_TIED_LM) {
    const ember_status s = check_draws(md, batch, (long long)start_pos + n_tokens - 1);
    if (s != EMBER_OK) return s;
  }

  hipStream_t st = (hipStream_t)stream;
  const Plan& p = md->plan;
  Ctx cx{md, cache, st};
  const int out_dim = c.head_kind == EMBER_HEAD_CLS ? c.n_classes : c.vocab;
  g_unlaunched = nullptr;
  // passes: whole rows when a row fits max_tokens, else position chunks of one row
  const int T = n_tokens;
  const int rows_per_pass = T <= p.Mx ? (p.Mx / T < batch ? p.Mx / T : batch) : 1;
  const int tok_chunk = T <= p.Mx ? T : p.Mx;
  for (int bi = 0; bi < batch; bi += rows_per_pass) {
    const int rows = batch - bi < rows_per_pass ? batch - bi : rows_per_pass;
    const int b0 = row0 + bi;               // cache / state row of the pass's first row
    for (int t0 = 0; t0 < T; t0 += tok_chunk) {
      const int tpr = T - t0 < tok_chunk ? T - t0 : tok_chunk;
      const int M = rows * tpr;
      // stage ids of this pass (rows x tpr)
      std::vector<int32_t> ids((size_t)M);
      for (int r = 0; r < rows; ++r)
        memcpy(&ids[(size_t)r * tpr], h_ids + (size_t)(bi + r) * T + t0, (size_t)tpr * 4);
      HIP_TRY(hipMemcpyAsync(md->at<int32_t>(p.ids), ids.data(), (size_t)M * 4,
                             hipMemcpyHostToDevice, st));
      launch_embed(md->at<int32_t>(p.ids), md->ws + p.embed, md->wk,
                   md->wk == WK_Q8 ? md->at<uint16_t>(p.embed_s) : nullptr, md->at<float>(p.x), M,
                   c.hidden, c.vocab, md->at<int>(p.flags), st);
      Pass ps{};
      ps.M = M; ps.rows = rows; ps.tpr = tpr; ps.b0 = b0; ps.start = start_pos + t0;
      ps.d_pos = nullptr;
      ps.path = M == 1 ? PATH_GEMV : (md->mfma ? PATH_MFMA : PATH_F32W);
      ps.attn = ATTN_FLASH;
      const bool last_chunk = t0 + tpr == T;
      const bool taps = d_acts && last_chunk;      // x is read after every layer
      int pending = 0;
      for (int l = 0; l < c.layers; ++l) {
        pending = run_layer(cx, l, ps, pending, !taps && l + 1 < c.layers);
        if (taps)
          launch_copy_rows(md->at<float>(p.x), rows, tpr, tpr - 1, c.hidden,
                           d_acts + ((size_t)bi * c.layers + l) * c.hidden,
                           (long long)c.layers * c.hidden, st);
      }
      md->last_pass = {M, rows, tpr, b0, start_pos + t0};
      if (c.sens_head) {
        // the sequence score: every token's final-normed state summed per row (across the
        // passes of a row), then mean and head at the row's last chunk
        float* hn = md->at<float>(p.xb);
        launch_rmsnorm(md->at<float>(p.x), md->at<float>(p.fnorm), c.rms_eps, M, c.hidden, 1, 0,
                       hn, nullptr, nullptr, 0, st);
        float* acc = md->at<float>(p.sens_acc) + (size_t)b0 * c.hidden;
        launch_pool_accum(hn, rows, tpr, c.hidden, acc, t0 == 0, st);
        if (last_chunk)
          launch_pool_head(acc, rows, c.hidden, T, md->at<float>(p.sens_w), md->at<float>(p.sens_b),
                           md->at<float>(p.sens_out) + b0, st);
      }
      if (c.head_kind == EMBER_HEAD_TIED_LM) {
        if (d_all_logits) {
          for (int r = 0; r < rows; ++r)
            run_lm_head(cx, tpr, 1, r * tpr,
                        d_all_logits + ((size_t)(bi + r) * T + t0) * out_dim, out_dim, nullptr);
        }
        if (last_chunk)
          run_lm_head(cx, rows, tpr, tpr - 1, md->at<float>(p.logits) + (size_t)b0 * out_dim,
                      out_dim, d_next ? d_next + bi : nullptr, b0, start_pos + T - 1);
      } else {
        for (int r = 0; r < rows; ++r)
          if (d_all_logits || d_next)
            run_cls_head(cx, tpr, 1, r * tpr,
                         d_all_logits ? d_all_logits + ((size_t)(bi + r) * T + t0) * out_dim : nullptr,
                         d_next ? d_next + (size_t)(bi + r) * T + t0 : nullptr);
        if (last_chunk)
          run_cls_head(cx, rows, tpr, tpr - 1, md->at<float>(p.logits) + (size_t)b0 * out_dim,
                       nullptr);
      }
      HIP_TRY(hipGetLastError());
      const ember_status ls = check_launched();
      if (ls != EMBER_OK) return ls;
    }
  }
  for (int r = row0; r < row0 + batch; ++r)
    if (start_pos + T > cache->filled[r]) cache->filled[r] = start_pos + T;
  md->has_logits_rows = row0 + batch;
  md->sens_rows = c.sens_head ? row0 + batch : 0;
  return EMBER_OK;
}

}  // namespace

ember_status ember_prefill(ember_model* md, ember_cache* cache, const int32_t* h_ids,
                           int32_t batch, int32_t n_tokens, int32_t start_pos,
                           float* d_all_logits, int32_t* d_next, void* stream) {
  g_last_error.clear();
  return prefill_impl(md, cache, h_ids, batch, n_tokens, start_pos, d_all_logits, d_next,
                      nullptr, stream);
}

ember_status ember_forward_with_activations(ember_model* md, ember_cache* cache,
                                            const int32_t* h_ids, int32_t batch,
                                            int32_t n_tokens, int32_t start_pos, float* d_acts,
                                            int32_t* d_next, void* stream) {
  g_last_error.clear();
  if (!d_acts) return fail(EMBER_E_ARG, "NULL activations buffer");
  return prefill_impl(md, cache, h_ids, batch, n_tokens, start_pos, nullptr, d_next, d_acts,
                      stream);
}

ember_status ember_prefill_rows(ember_model* md, ember_cache* cache, const int32_t* h_ids,
                                const int32_t* h_lengths, const int32_t* h_start,
                                int32_t batch, int32_t* d_next, void* stream) {
  g_last_error.clear();
  if (!md || !cache || !h_ids || !h_lengths || !h_start) return fail(EMBER_E_ARG, "NULL argument");
  if (cache->model != md) return fail(EMBER_E_ARG, "cache bound to another model");
  const ember_config& c = md->cfg;
  if (batch <= 0 || batch > c.max_batch)
    return fail(EMBER_E_CAPACITY, "batch %d outside 1..%d", batch, c.max_batch);
  // every row is checked before anything is enqueued
  long long off = 0;
  for (int r = 0; r < batch; ++r) {
    const int n = h_lengths[r], s0 = h_start[r];
    if (n <= 0) return fail(EMBER_E_ARG, "row %d: input_ids must not be empty", r);
    if (s0 < 0 || (long long)s0 + n > c.max_seq)
      return fail(EMBER_E_CAPACITY, "row %d: positions [%d, %d) exceed max_seq %d", r, s0, s0 + n,
                  c.max_seq);
    if (s0 > cache->filled[r])
      return fail(EMBER_E_STATE, "row %d: start_pos %d leaves a gap after %d cached positions", r,
                  s0, cache->filled[r]);
    if (!c.causal && s0 != 0)
      return fail(EMBER_E_ARG, "a bidirectional model takes whole sequences (start_pos 0)");
    if (!c.causal && n > (c.max_tokens > c.max_batch ? c.max_tokens : c.max_batch))
      return fail(EMBER_E_CAPACITY, "row %d: a bidirectional row must fit one pass", r);
    for (int i = 0; i < n; ++i)
      if (h_ids[off + i] < 0 || h_ids[off + i] >= c.vocab)
        return fail(EMBER_E_TOKEN, "token %d outside vocabulary", h_ids[off + i]);
    if (d_next && c.head_kind == EMBER_HEAD_TIED_LM) {
      const ember_status s = check_draws(md, r + 1, (long long)s0 + n - 1);
      if (s != EMBER_OK) return s;
    }
    off += n;
  }
  const int per_row = c.head_kind == EMBER_HEAD_CLS ? 0 : 1;   // next ids per row (LM head)
  off = 0;
  for (int r = 0; r < batch; ++r) {
    int32_t* nx = nullptr;
    if (d_next) nx = per_row ? d_next + r : d_next + off;      // cls: one id per token
    const ember_status s = prefill_impl(md, cache, h_ids + off, 1, h_lengths[r], h_start[r],
                                        nullptr, nx, nullptr, stream, r);
    if (s != EMBER_OK) return s;
    off += h_lengths[r];
  }
  return EMBER_OK;
}

ember_status ember_sensitivity(ember_model* md, float* d_out, void* stream) {
  g_last_error.clear();
  if (!md || !d_out) return fail(EMBER_E_ARG, "NULL argument");
  if (!md->cfg.sens_head) return fail(EMBER_E_STATE, "the model has no sequence-score head");
  if (md->sens_rows <= 0) return fail(EMBER_E_STATE, "no prefill has run yet");
  HIP_TRY(hipMemcpyAsync(d_out, md->at<float>(md->plan.sens_out), (size_t)md->sens_rows * 4,
                         hipMemcpyDeviceToDevice, (hipStream_t)stream));
  return EMBER_OK;
}

namespace {

// One cached step for `batch` rows: at position `pos` for every row, or (h_pos non-null)
// at row r's own position h_pos[r].
ember_status decode_impl(ember_model* md, ember_cache* cache, const int32_t* d_ids, int32_t batch,
                         int32_t pos, const int32_t* h_pos, int32_t* d_next, void* stream) {
  if (!md || !cache || !d_ids || !d_next) return fail(EMBER_E_ARG, "NULL argument");
  if (cache->model != md) return fail(EMBER_E_ARG, "cache bound to another model");
  const ember_config& c = md->cfg;
  if (!c.causal) return fail(EMBER_E_STATE, "decode steps need a causal model");
  if (batch <= 0 || batch > c.max_batch)
    return fail(EMBER_E_CAPACITY, "batch %d outside 1..%d", batch, c.max_batch);
  int max_pos = 0;
  for (int r = 0; r < batch; ++r) {
    const int pr = h_pos ? h_pos[r] : pos;
    if (pr < 0 || pr >= c.max_seq)
      return fail(EMBER_E_CAPACITY, "row %d: position %d outside [0, max_seq %d)", r, pr, c.max_seq);
    if (cache->filled[r] == 0) return fail(EMBER_E_STATE, "row %d: decode step before any prefill", r);
    if (pr > cache->filled[r])
      return fail(EMBER_E_STATE, "row %d: position %d leaves a gap after %d cached positions", r,
                  pr, cache->filled[r]);
    max_pos = pr > max_pos ? pr : max_pos;
  }
  {
    const ember_status s = check_draws(md, batch, max_pos);
    if (s != EMBER_OK) return s;
  }
  hipStream_t st = (hipStream_t)stream;
  const Plan& p = md->plan;
  Ctx cx{md, cache, st};
  g_unlaunched = nullptr;
  if (h_pos)
    HIP_TRY(hipMemcpyAsync(md->at<int>(p.row_pos), h_pos, (size_t)batch * 4, hipMemcpyHostToDevice, st));
  StepBeginArgs sb{};
  sb.ids = d_ids; sb.R = batch; sb.V = c.vocab; sb.pos = pos;
  sb.ragged = h_pos != nullptr; sb.row_pos = md->at<int>(p.row_pos);
  sb.d_pos = md->at<int>(p.pos); sb.flags = md->at<int>(p.flags);
  sb.cos_t = md->at<float>(p.cos_t); sb.sin_t = md->at<float>(p.sin_t); sb.half = c.head_dim / 2;
  sb.rope_cur = md->at<float>(p.rope_cur);
  sb.E = md->ws + p.embed; sb.e_wk = md->wk;
  sb.e_scale = md->wk == WK_Q8 ? md->at<uint16_t>(p.embed_s) : nullptr;
  sb.x = md->at<float>(p.x); sb.H = c.hidden;
  launch_step_begin(sb, st);
  const bool use_graph = st != nullptr && graphs_enabled();
  if (use_graph) {
    if (!md->graph || md->graph_cache != cache || md->graph_batch != batch || md->graph_stream != st ||
        md->graph_next != d_next) {
      if (md->graph) {
        (void)hipGraphExecDestroy(md->graph);
        md->graph = nullptr;
      }
      HIP_TRY(hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal));
      decode_body(cx, batch, d_next);
      hipGraph_t g = nullptr;
      HIP_TRY(hipStreamEndCapture(st, &g));
      hipError_t e = hipGraphInstantiate(&md->graph, g, nullptr, nullptr, 0);
      (void)hipGraphDestroy(g);
      if (e != hipSuccess) return fail(EMBER_E_DEVICE, "graph instantiate: %s", hipGetErrorString(e));
      const ember_status ls = check_launched();
      if (ls != EMBER_OK) {                 // never replay a step that misses a kernel
        (void)hipGraphExecDestroy(md->graph);
        md->graph = nullptr;
        return ls;
      }
      md->graph_cache = cache;
      md->graph_batch = batch;
      md->graph_stream = st;
      md->graph_next = d_next;
    }
    HIP_TRY(hipGraphLaunch(md->graph, st));
  } else {
    decode_body(cx, batch, d_next);
  }
  HIP_TRY(hipGetLastError());
  {
    const ember_status ls = check_launched();
    if (ls != EMBER_OK) return ls;
  }
  for (int r = 0; r < batch; ++r) {
    const int pr = h_pos ? h_pos[r] : pos;
    if (pr + 1 > cache->filled[r]) cache->filled[r] = pr + 1;
  }
  md->has_logits_rows = batch;
  md->last_decode_batch = batch;
  return EMBER_OK;
}

}  // namespace

ember_status ember_decode_step(ember_model* md, ember_cache* cache, const int32_t* d_ids,
                               int32_t batch, int32_t pos, int32_t* d_next, void* stream) {
  g_last_error.clear();
  return decode_impl(md, cache, d_ids, batch, pos, nullptr, d_next, stream);
}

ember_status ember_decode_step_rows(ember_model* md, ember_cache* cache, const int32_t* d_ids,
                                    int32_t batch, const int32_t* h_pos, int32_t* d_next,
                                    void* stream) {
  g_last_error.clear();
  if (!h_pos) return fail(EMBER_E_ARG, "NULL positions");
  return decode_impl(md, cache, d_ids, batch, 0, h_pos, d_next, stream);
}

ember_status ember_time_kernel(ember_model* md, ember_cache* cache, int32_t kernel, int32_t phase,
                               int32_t iters, void* stream, float* avg_us) {
  g_last_error.clear();
  if (!md || !cache || !avg_us || iters <= 0) return fail(EMBER_E_ARG, "bad arguments");
  if (kernel < EMBER_K_LM_HEAD || kernel > EMBER_K_SAMPLE) return fail(EMBER_E_ARG, "unknown kernel");
  if (kernel == EMBER_K_SAMPLE && (phase != 0 || !md->sampling))
    return fail(EMBER_E_ARG, "the sampler is timed on decode steps with a sampler set");
  hipStream_t st = (hipStream_t)stream;
  Ctx cx{md, cache, st, kernel == EMBER_K_LAYER ? -1 : kernel};
  const ember_config& c = md->cfg;
  const Plan& p = md->plan;
  // the launches are captured into a graph (non-null stream) so that back-to-back
  // execution, not the host launch rate, sets the measured time
  auto enqueue = [&](int n) -> ember_status {
    if (phase == 0) {
      if (md->last_decode_batch <= 0) return fail(EMBER_E_STATE, "no decode step has run");
      for (int i = 0; i < n; ++i)
        decode_body(cx, md->last_decode_batch, md->at<int32_t>(p.next), i % c.layers);
    } else {
      if (md->last_pass.M <= 0) return fail(EMBER_E_STATE, "no prefill has run");
      Pass ps{};
      ps.M = md->last_pass.M; ps.rows = md->last_pass.rows; ps.tpr = md->last_pass.tpr;
      ps.b0 = md->last_pass.b0; ps.start = md->last_pass.start; ps.d_pos = nullptr;
      ps.path = ps.M == 1 ? PATH_GEMV : (md->mfma ? PATH_MFMA : PATH_F32W);
      ps.attn = ATTN_FLASH;
      for (int i = 0; i < n; ++i) {
        if (kernel == EMBER_K_LM_HEAD)
          run_lm_head(cx, ps.rows, ps.tpr, ps.tpr - 1, md->at<float>(p.logits), c.vocab, nullptr);
        else
          run_layer(cx, i % c.layers, ps);
      }
    }
    return EMBER_OK;
  };
  hipGraphExec_t ge = nullptr;
  g_unlaunched = nullptr;
  if (st != nullptr && graphs_enabled()) {
    HIP_TRY(hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal));
    ember_status s0 = enqueue(iters);
    hipGraph_t g = nullptr;
    HIP_TRY(hipStreamEndCapture(st, &g));
    if (s0 != EMBER_OK) { (void)hipGraphDestroy(g); return s0; }
    hipError_t e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (e != hipSuccess) return fail(EMBER_E_DEVICE, "graph instantiate: %s", hipGetErrorString(e));
    HIP_TRY(hipGraphLaunch(ge, st));     // warm-up replay
    HIP_TRY(hipStreamSynchronize(st));
  }
  // The timed replays are queued behind a running warm-up replay, so the start event and
  // the first timed kernel follow it back to back: host submission time never lands
  // inside the measured span.
  const int reps = ge ? 2 : 1;
  hipEvent_t e0, e1;
  HIP_TRY(hipEventCreate(&e0));
  HIP_TRY(hipEventCreate(&e1));
  if (ge) HIP_TRY(hipGraphLaunch(ge, st));
  HIP_TRY(hipEventRecord(e0, st));
  for (int rep = 0; rep < reps; ++rep) {
    if (ge) {
      HIP_TRY(hipGraphLaunch(ge, st));
    } else {
      ember_status s1 = enqueue(iters);
      if (s1 != EMBER_OK) return s1;
    }
  }
  HIP_TRY(hipEventRecord(e1, st));
  HIP_TRY(hipEventSynchronize(e1));
  float ms = 0.f;
  HIP_TRY(hipEventElapsedTime(&ms, e0, e1));
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (ge) (void)hipGraphExecDestroy(ge);
  HIP_TRY(hipGetLastError());
  *avg_us = ms * 1000.f / (float)(iters * reps);
  return check_launched();
}

ember_status ember_measure_peak(int32_t kind, void* d_buf, size_t bytes, int32_t iters,
                                void* stream, float* out) {
  g_last_error.clear();
  if (!d_buf || !out || iters <= 0) return fail(EMBER_E_ARG, "bad arguments");
  hipStream_t st = (hipStream_t)stream;
  const size_t half = bytes / 2 / 4096 * 4096;
  const size_t read_out = (size_t)kPeakReadBlocks * 256 * 4;
  if (kind == EMBER_PEAK_COPY) {
    if (half == 0) return fail(EMBER_E_ARG, "buffer too small for the copy");
  } else if (kind == EMBER_PEAK_READ) {
    if (bytes < 2 * read_out) return fail(EMBER_E_ARG, "buffer too small for the read");
  } else if (kind == EMBER_PEAK_MFMA) {
    if (bytes < (size_t)kPeakMfmaBlocks * 256 * 4)
      return fail(EMBER_E_ARG, "the MFMA loop needs %zu bytes", (size_t)kPeakMfmaBlocks * 256 * 4);
  } else {
    return fail(EMBER_E_ARG, "unknown peak kind %d", kind);
  }
  double work = 0.0;
  auto launch = [&]() {
    if (kind == EMBER_PEAK_COPY) {
      launch_peak_copy(d_buf, (char*)d_buf + half, half, st);
      work = 2.0 * (double)half;
    } else if (kind == EMBER_PEAK_READ) {
      const size_t n = (bytes - read_out) / 65536 * 65536;      // whole 64 KB segments
      launch_peak_read((const char*)d_buf + read_out, n, (uint32_t*)d_buf, st);
      work = (double)n;
    } else {
      work = launch_peak_mfma((float*)d_buf, st);
    }
  };
  launch();                                  // warm-up
  hipEvent_t e0, e1;
  HIP_TRY(hipEventCreate(&e0));
  HIP_TRY(hipEventCreate(&e1));
  HIP_TRY(hipEventRecord(e0, st));
  for (int i = 0; i < iters; ++i) launch();
  HIP_TRY(hipEventRecord(e1, st));
  HIP_TRY(hipEventSynchronize(e1));
  float ms = 0.f;
  HIP_TRY(hipEventElapsedTime(&ms, e0, e1));
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  HIP_TRY(hipGetLastError());
  const double per_s = work * iters / (ms * 1e-3);
  *out = (float)(kind == EMBER_PEAK_MFMA ? per_s / 1e12 : per_s / 1e9);
  return EMBER_OK;
}

ember_status ember_set_sampler(ember_model* md, const ember_sampler* s) {
  g_last_error.clear();
  if (!md) return fail(EMBER_E_ARG, "NULL model");
  if (s && !(s->temperature >= 0.f && std::isfinite(s->temperature)))
    return fail(EMBER_E_ARG, "temperature must be finite and >= 0");
  const bool on = s && s->temperature > 0.f;
  if (on) {
    if (!std::isfinite(s->top_p) || s->top_p < 0.f) return fail(EMBER_E_ARG, "top_p must be finite and >= 0");
    if (s->top_k < 0) return fail(EMBER_E_ARG, "top_k must be >= 0");
    if (s->d_uniform && (s->n_pos < 1 || s->ld < 1))
      return fail(EMBER_E_ARG, "draws d_uniform need n_pos >= 1 and ld >= 1");
    if (md->cfg.head_kind != EMBER_HEAD_TIED_LM)
      return fail(EMBER_E_STATE, "sampling needs the tied LM head");
    if (md->cfg.vocab > kSampleMaxVocab)
      return fail(EMBER_E_CAPACITY, "vocabulary %d beyond the sampler's %d", md->cfg.vocab,
                  kSampleMaxVocab);
  }
  if (md->graph) {
    (void)hipGraphExecDestroy(md->graph);
    md->graph = nullptr;
    md->graph_cache = nullptr;
  }
  md->sampling = on;
  md->samp = on ? *s : ember_sampler{};
  return EMBER_OK;
}

ember_status ember_sample(ember_model* md, const float* d_logits, int32_t rows,
                          int64_t ld_logits, int32_t pos, int32_t* d_next, void* stream) {
  g_last_error.clear();
  if (!md || !d_logits || !d_next) return fail(EMBER_E_ARG, "NULL argument");
  if (md->cfg.head_kind != EMBER_HEAD_TIED_LM) return fail(EMBER_E_STATE, "sampling needs the tied LM head");
  if (rows < 1) return fail(EMBER_E_ARG, "rows must be >= 1");
  if (rows > md->cfg.max_batch)
    return fail(EMBER_E_CAPACITY, "%d rows beyond max_batch %d", rows, md->cfg.max_batch);
  if (ld_logits < md->cfg.vocab) return fail(EMBER_E_ARG, "row stride below the vocabulary");
  if (pos < 0) return fail(EMBER_E_ARG, "negative draw row");
  const ember_status s = check_draws(md, rows, pos);
  if (s != EMBER_OK) return s;
  Ctx cx{md, nullptr, (hipStream_t)stream};
  g_unlaunched = nullptr;
  if (md->sampling)
    launch_draw(cx, d_logits, rows, ld_logits, d_next, 0, pos);
  else
    launch_argmax_rows(d_logits, rows, md->cfg.vocab, ld_logits, d_next, md->at<int>(md->plan.flags),
                       cx.st);
  HIP_TRY(hipGetLastError());
  return check_launched();
}

// ------------------------------------------------------------------ no-allocation draw
// ember_sample_noalloc keeps the sampler's per-row state and tile sums in this file-scope
// device array instead of the model's workspace. Each GPU holds its own copy; host code
// uses only the address hipGetSymbolAddress returns for the current device (the array's
// name is a host-side stand-in, not a device address).
namespace {

constexpr size_t kNoAllocRowBytes =
    (sizeof(SampleState) + (size_t)kSampleMaxTiles * 4 + 255) / 256 * 256;
constexpr size_t kNoAllocBytes = (size_t)EMBER_NOALLOC_MAX_ROWS * kNoAllocRowBytes;

static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device.
ember_status scratch_for_device(char** out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(EMBER_E_DEVICE, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(EMBER_E_DEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = (char*)g_scratch_ptr[dev];
  return EMBER_OK;
}

}  // namespace

ember_status ember_sample_noalloc(ember_model* md, const float* d_logits, int32_t rows,
                                  int64_t ld_logits, int32_t pos, int32_t* d_next, void* stream) {
  g_last_error.clear();
  if (!md || !d_logits || !d_next) return fail(EMBER_E_ARG, "NULL argument");
  if (md->cfg.head_kind != EMBER_HEAD_TIED_LM) return fail(EMBER_E_STATE, "sampling needs the tied LM head");
  if (rows < 1) return fail(EMBER_E_ARG, "rows must be >= 1");
  if (rows > EMBER_NOALLOC_MAX_ROWS)
    return fail(EMBER_E_CAPACITY, "%d rows beyond the no-allocation draw's maximum of %d", rows,
                EMBER_NOALLOC_MAX_ROWS);
  if (md->cfg.vocab > kSampleMaxVocab)
    return fail(EMBER_E_CAPACITY, "vocabulary %d beyond the sampler's %d", md->cfg.vocab, kSampleMaxVocab);
  if (ld_logits < md->cfg.vocab) return fail(EMBER_E_ARG, "row stride below the vocabulary");
  if (pos < 0) return fail(EMBER_E_ARG, "negative draw row");
  {
    const ember_status s = check_draws(md, rows, pos);
    if (s != EMBER_OK) return s;
  }
  hipStream_t st = (hipStream_t)stream;
  g_unlaunched = nullptr;
  if (!md->sampling) {
    // greedy: one block per row, no scratch
    launch_argmax_rows(d_logits, rows, md->cfg.vocab, ld_logits, d_next, md->at<int>(md->plan.flags), st);
    HIP_TRY(hipGetLastError());
    return check_launched();
  }
  char* base = nullptr;
  {
    const ember_status s = scratch_for_device(&base);
    if (s != EMBER_OK) return s;
  }
  // the phases expect zeroed per-row state: clear it (a fill kernel, capture-safe) rather
  // than trusting what the previous call on this GPU left
  SampleState* state = (SampleState*)base;
  float* tiles = (float*)(base + (size_t)EMBER_NOALLOC_MAX_ROWS * sizeof(SampleState));
  launch_fill_i32((int*)state, (int)((size_t)rows * sizeof(SampleState) / 4), 0, st);
  SampleArgs a{};
  a.logits = d_logits; a.ld = ld_logits; a.R = rows; a.V = md->cfg.vocab;
  a.temperature = md->samp.temperature; a.top_k = md->samp.top_k; a.top_p = md->samp.top_p;
  a.uniform = md->samp.d_uniform; a.u_rows = md->samp.n_pos; a.u_ld = md->samp.ld;
  a.seed = md->samp.seed;
  a.col0 = 0; a.pos = pos; a.d_pos = nullptr;
  a.next = d_next; a.flags = md->at<int>(md->plan.flags);
  a.state = state;
  a.tiles = tiles;
  launch_sample(a, st);
  HIP_TRY(hipGetLastError());
  return check_launched();
}

ember_status ember_logits(ember_model* md, void* d_out, int32_t dtype, void* stream) {
  g_last_error.clear();
  if (!md || !d_out) return fail(EMBER_E_ARG, "NULL argument");
  if (dtype != EMBER_F32 && dtype != EMBER_BF16) return fail(EMBER_E_DTYPE, "unsupported dtype %d", dtype);
  if (md->has_logits_rows <= 0) return fail(EMBER_E_STATE, "no forward has run yet");
  const int out_dim = md->cfg.head_kind == EMBER_HEAD_CLS ? md->cfg.n_classes : md->cfg.vocab;
  launch_convert_logits(md->at<float>(md->plan.logits), md->has_logits_rows, out_dim, out_dim,
                        d_out, dtype == EMBER_BF16, (hipStream_t)stream);
  HIP_TRY(hipGetLastError());
  return EMBER_OK;
}

ember_status ember_sync(ember_model* md, void* stream) {
  g_last_error.clear();
  if (!md) return fail(EMBER_E_ARG, "NULL model");
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipStreamSynchronize(st));
  int flags[kNumFlags];
  HIP_TRY(hipMemcpy(flags, md->at<int>(md->plan.flags), sizeof flags, hipMemcpyDeviceToHost));
  launch_fill_i32(md->at<int>(md->plan.flags), kNumFlags, 0, st);
  HIP_TRY(hipStreamSynchronize(st));
  if (flags[kFlagNaN]) return fail(EMBER_E_NONFINITE, "NaN in logits");
  if (flags[kFlagBadToken]) return fail(EMBER_E_TOKEN, "decode id outside vocabulary");
  return EMBER_OK;
}

void ember_cache_free(ember_cache* cache) {
  if (!cache) return;
  ember_model* m = cache->model;
  if (m && m->graph_cache == cache && m->graph) {
    (void)hipGraphExecDestroy(m->graph);
    m->graph = nullptr;
    m->graph_cache = nullptr;
  }
  delete cache;
}

void ember_free(ember_model* model) {
  if (!model) return;
  if (model->graph) (void)hipGraphExecDestroy(model->graph);
  delete model;
}

}  // extern "C"
