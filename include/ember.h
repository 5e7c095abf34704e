/*
 * ember.h -- C ABI of the MI355X (gfx950) GQA decoder forward pass.
 *
 * The forward pass is the one the pages define: bf16 (or f32) weights widened to f32,
 * RMSNorm, rotate-half RoPE with optional llama3 frequency scaling, grouped-query
 * attention over a causal KV cache (prefill once, then one cached step per new token)
 * or bidirectional attention, SwiGLU MLP, tied LM head (or a token classification head)
 * and greedy argmax. Interface shape: "ember internals" page, section "ForwardModel
 * trait" (create_cache, forward_with_cache(token_ids, cache, start_pos)), with the
 * explicit write position of section "cursor semantics", and the validation and error
 * cases of "Falcon-H1-0.5B-Rust src/lib.rs" (Config::validate, validate_weights,
 * Model::logits).
 *
 * Conventions
 *  - Every call returns ember_status (0 = EMBER_OK). When the host detects an error
 *    nothing is enqueued; ember_last_error() returns a message (thread-local).
 *  - Device memory is owned by the caller. The library allocates no device memory: the
 *    weights, activations and scratch live in a caller-provided workspace, the KV cache
 *    in a caller-provided buffer. Handles (ember_model, ember_cache) are host objects
 *    owned by the library and released with ember_free / ember_cache_free.
 *  - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued
 *    asynchronously; calls on one model must be ordered on one stream. A model handle is
 *    not thread-safe.
 *  - All tensors are row-major and contiguous. Batch rows share positions.
 */
#ifndef EMBER_H
#define EMBER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ember_status {
  EMBER_OK = 0,
  EMBER_E_ARG = 1,             /* bad argument: NULL pointer, size 0, workspace too small */
  EMBER_E_CONFIG = 2,          /* zero dimension, heads % kv_heads != 0, odd head_dim, ... */
  EMBER_E_TENSOR_MISSING = 3,  /* a required named tensor is absent */
  EMBER_E_TENSOR_SHAPE = 4,    /* a tensor's shape differs from the config */
  EMBER_E_DTYPE = 5,           /* unsupported dtype, or a tensor dtype != weight_dtype */
  EMBER_E_TOKEN = 6,           /* token id outside [0, vocab) */
  EMBER_E_CAPACITY = 7,        /* positions or rows beyond the cache / config capacity */
  EMBER_E_STATE = 8,           /* call out of order (e.g. decode before any prefill) */
  EMBER_E_DEVICE = 9,          /* a HIP runtime error */
  EMBER_E_NONFINITE = 10       /* the device saw a NaN logit */
} ember_status;

/* EMBER_Q8_0: a weight matrix [N, K] (K a multiple of 32) stored as q8_0 blocks ("ember
 * internals" page, section "GGUF format and quantization", subsection "q8_0 block
 * quantization"): N x K/32 blocks of 34 bytes, row by row, each a little-endian f16 scale d
 * followed by 32 signed int8 values q; the weights are q * d. The blocks run along K.
 * Weights only (never a KV cache or an output dtype). */
typedef enum ember_dtype { EMBER_F32 = 0, EMBER_BF16 = 1, EMBER_Q8_0 = 2 } ember_dtype;

/* EXACT: f32 arithmetic on the bf16 weights (f32 logits, 1e-4 tier). Decode: f32 FMA on
 *        weights widened in registers. Multi-token passes on bf16 MFMA: every GEMM
 *        activation is split into two bf16 planes hi + lo (their sum within 2^-17 of the
 *        f32 value; weights are exact in bf16, products exact in f32); the attention
 *        scores q.k are formed from three planes of q and of k (six products, absolute
 *        error at the f32 level of q.k however large the scores: they are exponentiated),
 *        P and V from two planes each. KV cache must be F32. The softmax amplifies a
 *        score error by its size, so with scores of magnitude ~100 and more (far beyond
 *        initialised or typical trained models) f32 implementations themselves, this one
 *        and a plain f32 reference, differ from the exact result by more than 1e-4.
 * FAST:  single-pass bf16 activations into the MFMA GEMMs and attention, f32
 *        accumulation, norms, softmax and residual (bf16 logits, 2e-2 tier). */
typedef enum ember_precision { EMBER_EXACT = 0, EMBER_FAST = 1 } ember_precision;

typedef enum ember_head_kind {
  EMBER_HEAD_TIED_LM = 0,      /* logits = E . rmsnorm(h), E = model.embed_tokens.weight */
  EMBER_HEAD_CLS = 1           /* logits = Wc . rmsnorm(h) + bc at every token */
} ember_head_kind;

typedef struct ember_config {
  double rope_theta;           /* RoPE base theta */
  double llama3_factor;        /* llama3 frequency scaling (used when rope_llama3 != 0) */
  double llama3_low_freq_factor;
  double llama3_high_freq_factor;
  double llama3_original_max_pos;
  float rms_eps;               /* RMSNorm epsilon (also for per-head q/k norm) */
  /* head_dim in {8, 16, 32, 64, 128}; heads a multiple of kv_heads with at most 8 query
   * heads per kv head; ffn a multiple of 32; hidden, ffn and heads * head_dim multiples
   * of 8 (bf16 weights) or 4 (f32); hidden <= 8192, ffn <= 32768, heads * head_dim <=
   * 8192, max_seq <= 65536. Other shapes fail with EMBER_E_CONFIG. */
  int32_t vocab, hidden, layers, heads, kv_heads, head_dim, ffn;
  int32_t rope_llama3;         /* 0/1 */
  int32_t qkv_bias;            /* 0/1: q/k/v projections carry a bias (Qwen2 family) */
  int32_t qk_norm;             /* 0/1: per-head RMSNorm of q and k before RoPE (Qwen3) */
  int32_t causal;              /* 1 = causal decoder, 0 = bidirectional encoder */
  int32_t head_kind;           /* ember_head_kind */
  int32_t n_classes;           /* classes of the EMBER_HEAD_CLS head */
  int32_t weight_dtype;        /* ember_dtype of every stored tensor; EMBER_Q8_0: every
                                * matrix in q8_0 and every vector (norm weights, biases) in
                                * F32, tied LM head only, hidden, ffn and heads * head_dim
                                * multiples of 32. A one-token pass (batch-1 decode) reads
                                * the blocks directly; multi-token passes dequantise each
                                * matrix into a workspace copy first: bf16 for FAST; for
                                * EXACT a bf16 pair hi + lo (within 2^-17 of q * d), one
                                * MFMA pass per plane */
  int32_t kv_dtype;            /* ember_dtype of the KV cache */
  int32_t precision;           /* ember_precision */
  int32_t max_batch;           /* rows per call */
  int32_t max_seq;             /* positions per row: capacity of the cache and RoPE table */
  int32_t max_tokens;          /* tokens processed per prefill pass (>= max_batch) */
  int32_t sens_head;           /* 0/1, classification-head models only: the mean-pooled
                                * sequence score ("PII-Tracer serving/reference_forward.py",
                                * forward: tensors sensitivity_head.weight [1, hidden] and
                                * .bias [1]); read with ember_sensitivity after a prefill */
} ember_config;

/* A named weight tensor, HuggingFace naming ("model.embed_tokens.weight",
 * "model.layers.{i}.self_attn.q_proj.weight", ".bias", "...k_norm.weight",
 * "model.norm.weight", "token_cls_head.weight", ...). `data` is a device pointer,
 * borrowed for the duration of ember_load_weights only. */
typedef struct ember_tensor {
  const char* name;
  const void* data;
  int64_t shape[4];
  int32_t ndim;
  int32_t dtype;               /* ember_dtype */
} ember_tensor;

typedef struct ember_model ember_model;
typedef struct ember_cache ember_cache;

/* Bytes of workspace ember_load_weights needs for `cfg` (repacked weights, RoPE tables,
 * activations for max_tokens tokens, split-K partials, logits [max_batch, out_dim] f32).
 * Sized once for the capacities in `cfg` so that no step allocates: the "ember internals"
 * page, section "qk_scratch", keeps one score buffer reserved for max_seq_len and resized
 * in place, so the hot path never calls the allocator; here every such buffer (scores,
 * split partials, activations) is a fixed region of this workspace.
 * Returns 0 if the config is invalid (no error code; ember_last_error() explains). */
size_t ember_workspace_bytes(const ember_config* cfg);

/* Bytes of a KV cache for `cfg`: K and V, [layers][max_batch][kv_heads][max_seq][head_dim]
 * of kv_dtype. Layout of the "ember internals" page, section "kv cache" / "layout": one
 * contiguous block per layer holding every (kv) head and position, addressed by fixed
 * strides; only kv_heads heads are stored (section "grouped-query attention (GQA)": the
 * cache shrinks by heads / kv_heads). Returns 0 if the config is invalid. */
size_t ember_kv_cache_bytes(const ember_config* cfg);

/* Model::new of "Falcon-H1-0.5B-Rust src/lib.rs": validate the config as its
 * Config::validate does (zero dimensions -> EMBER_E_CONFIG, heads % kv_heads or odd
 * head_dim -> EMBER_E_CONFIG; here also dtypes and capacities) and every tensor as its
 * validate_weights does (a missing name -> EMBER_E_TENSOR_MISSING, a shape other than the
 * config's -> EMBER_E_TENSOR_SHAPE; here also the dtype -> EMBER_E_DTYPE), then repack the
 * weights into
 * `d_workspace` (QKV rows fused, gate/up rows interleaved, norm vectors and biases as
 * f32) and upload the RoPE cos/sin tables (angles in f64, rounded once to f32).
 * `d_workspace` must stay allocated and untouched while the model lives. Synchronises
 * `stream` before returning. */
ember_status ember_load_weights(const ember_config* cfg, const ember_tensor* tensors,
                                int32_t n_tensors, void* d_workspace, size_t workspace_bytes,
                                void* stream, ember_model** out);

/* Bind a caller-owned KV buffer of at least ember_kv_cache_bytes(cfg) bytes
 * ("ForwardModel::create_cache"). The buffer holds no valid positions until a prefill. */
ember_status ember_cache_bind(ember_model* model, void* d_kv, size_t kv_bytes,
                              ember_cache** out);

/* Forward `n_tokens` tokens of each of `batch` rows at positions
 * [start_pos, start_pos + n_tokens) ("forward_with_cache(token_ids, cache, start_pos)"),
 * writing their K/V at those explicit positions. `h_ids` is host memory [batch, n_tokens]
 * int32, validated (EMBER_E_TOKEN). start_pos must not leave a gap after the positions
 * already held by the cache (EMBER_E_STATE); start_pos + n_tokens <= max_seq
 * (EMBER_E_CAPACITY). The head output at each row's last position is kept for
 * ember_logits. Optional outputs (NULL to skip), device memory:
 *   d_all_logits  f32 [batch, n_tokens, out_dim]: head output at every position;
 *   d_next        int32 [batch] (decoder: argmax of the last position, lowest index on
 *                 ties) or [batch, n_tokens] (classification head: argmax per token).
 * For a bidirectional config, start_pos must be 0, every token attends to every token of
 * its row, and a row must fit one pass (n_tokens <= max_tokens, else EMBER_E_CAPACITY). */
ember_status ember_prefill(ember_model* model, ember_cache* cache, const int32_t* h_ids,
                           int32_t batch, int32_t n_tokens, int32_t start_pos,
                           float* d_all_logits, int32_t* d_next, void* stream);

/* Ragged prefill: row r (r < batch) forwards h_lengths[r] tokens at positions
 * [h_start[r], h_start[r] + h_lengths[r]) ("ember internals" page, section "ForwardModel
 * trait": forward_with_cache(token_ids, cache, start_pos) per sequence). h_ids (host) holds
 * the rows' tokens one after the other; h_lengths and h_start are host [batch]. Each row is
 * checked as in ember_prefill (against its own cached length) before anything is
 * enqueued. d_next (optional): [batch] next ids of the LM head (each row's last
 * position), or one id per token (classification head, packed like h_ids). The rows run
 * one pass each (a row's tokens are not batched with another row's). */
ember_status ember_prefill_rows(ember_model* model, ember_cache* cache, const int32_t* h_ids,
                                const int32_t* h_lengths, const int32_t* h_start,
                                int32_t batch, int32_t* d_next, void* stream);

/* ember_prefill that also writes the hidden state after every block at each row's last
 * position ("ember internals" page, section "ForwardModel trait",
 * forward_with_activations; section "probing pipeline": activations[layer][d]) into
 * d_acts, device f32 [batch][layers][hidden]: the residual stream before the final norm.
 * The head output at the last position is kept for ember_logits as after ember_prefill;
 * d_next as there (NULL to skip). Same errors as ember_prefill, and EMBER_E_ARG for a
 * NULL d_acts. */
ember_status ember_forward_with_activations(ember_model* model, ember_cache* cache,
                                            const int32_t* h_ids, int32_t batch,
                                            int32_t n_tokens, int32_t start_pos, float* d_acts,
                                            int32_t* d_next, void* stream);

/* The mean-pooled sequence scores of the most recent prefill, [batch] f32 into d_out
 * (device): the final-normed hidden states averaged over each row's n_tokens tokens, then
 * . sensitivity_head.weight + sensitivity_head.bias. EMBER_E_STATE without the head or
 * before any prefill. */
ember_status ember_sensitivity(ember_model* model, float* d_out, void* stream);

/* One cached greedy step for `batch` rows at position `pos` (causal configs only; every
 * row at the same position -- ember_decode_step_rows takes one per row). The "ember
 * internals" page, section "attention": after one prefill, one cached step per new token;
 * section "cursor semantics": the step's K/V are written at the explicit position `pos`
 * (never at an implicit cursor), read back by the same step's attention over 0..pos:
 * reads the ids d_ids [batch] int32 (device), writes their K/V at `pos`, attends over
 * positions 0..pos, and writes the argmax of the new logits to d_next [batch] int32
 * (device; may alias d_ids). Requires pos <= the cache's filled length (EMBER_E_STATE)
 * and pos < max_seq (EMBER_E_CAPACITY). The step is replayed from a HIP graph and does
 * not synchronise; the graph is captured again whenever the batch, the cache, the stream
 * or d_next differ from the previous step's (keep d_next fixed across steps). An id
 * outside [0, vocab) is replaced by 0 and flagged; ember_sync reports it as
 * EMBER_E_TOKEN. */
ember_status ember_decode_step(ember_model* model, ember_cache* cache, const int32_t* d_ids,
                               int32_t batch, int32_t pos, int32_t* d_next, void* stream);

/* ember_decode_step with a position per row: row r's token is at h_pos[r] (host [batch]),
 * each row checked against its own cached length. The positions are copied to the device
 * before the step's graph, which reads them there (the graph is shared with
 * ember_decode_step). */
ember_status ember_decode_step_rows(ember_model* model, ember_cache* cache,
                                    const int32_t* d_ids, int32_t batch, const int32_t* h_pos,
                                    int32_t* d_next, void* stream);

/* Copy the head output of the most recent prefill / decode step, [batch, out_dim], into
 * d_out (device, caller-owned) as EMBER_F32 or EMBER_BF16 (round to nearest even). For
 * the tied LM head these are the logits E . rmsnorm(h) at each row's last position
 * ("ember scripts/reference_forward.py", end of forward: the final norm, then the
 * embedding matrix as the output projection). EMBER_E_STATE before any forward,
 * EMBER_E_DTYPE for another dtype. Asynchronous on `stream`. */
ember_status ember_logits(ember_model* model, void* d_out, int32_t dtype, void* stream);

/* Synchronise `stream` and report device-side conditions raised since the last call:
 * an out-of-range decode id (EMBER_E_TOKEN) or a NaN logit (EMBER_E_NONFINITE); then
 * clear them. These are the errors Model::logits of "Falcon-H1-0.5B-Rust src/lib.rs"
 * returns as Result::Err(String) ("token ... outside vocabulary"; its test_cpu_logits
 * requires finite logits), found here on the device after the work was enqueued, hence
 * reported at the next sync. A HIP runtime error is EMBER_E_DEVICE. */
ember_status ember_sync(ember_model* model, void* stream);

/* Sampling ("ember internals" page, section "sampler"): the token of ember_prefill's and
 * ember_decode_step's d_next is drawn instead of taken greedily. The stages, in order:
 * z = logit / temperature; top-k (0 < top_k < vocab): z below the top_k-th largest z is
 * dropped, ties with it kept; top-p (0 < top_p < 1): tokens whose probability under the
 * softmax of the remaining z lies below the nucleus cutoff (the smallest probability of
 * the shortest decreasing-order prefix whose sum exceeds top_p) are dropped; softmax of
 * the rest (uniform when every z is -inf); the first index whose running probability sum
 * in index order exceeds the draw u, or the last index of the maximum when rounding
 * leaves none.
 * The draw u of batch row b for the token predicted from the logits at position q (a
 * decode step at `pos` draws for q = pos, a prefill of positions [start_pos, start_pos +
 * n) for q = start_pos + n - 1; the page draws it from a seeded generator it does not
 * name) comes from one of two sources:
 *  - d_uniform non-null: an input array, device f32 [n_pos, ld] with values in [0, 1),
 *    borrowed while the sampler is set; u = d_uniform[q * ld + b];
 *  - d_uniform null: generated on the device by the counter-based generator
 *    Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1,
 *    2, 3", SC'11): its first output word at counter (q, b, 0, 0) and key (seed mod 2^32,
 *    seed div 2^32), u = (word >> 8) * 2^-24. No position or batch capacity applies. */
typedef struct ember_sampler {
  float temperature;           /* > 0 draws; 0 = greedy argmax (the default) */
  int32_t top_k;               /* 0 or >= vocab: stage off */
  float top_p;                 /* outside (0, 1): stage off */
  const float* d_uniform;      /* device [n_pos, ld] f32, or null: draws from `seed` */
  int32_t n_pos;               /* rows of d_uniform */
  int32_t ld;                  /* row stride of d_uniform in floats */
  uint64_t seed;               /* key of the on-device draws (d_uniform null) */
} ember_sampler;

/* Set the sampler of `model` (copied), or with NULL or temperature 0 return to greedy
 * argmax. A negative or non-finite temperature or top_p, top_k < 0, or a d_uniform with
 * n_pos < 1 or ld < 1 fail with EMBER_E_ARG, a classification-head model with
 * EMBER_E_STATE, a vocabulary above 1048576 with EMBER_E_CAPACITY. Afterwards a prefill
 * or decode step whose draw row lies beyond n_pos - 1 or whose batch exceeds ld fails
 * with EMBER_E_CAPACITY. The next decode step captures its graph again. */
ember_status ember_set_sampler(ember_model* model, const ember_sampler* sampler);

/* Draw one token for each of `rows` rows of caller logits d_logits f32 [rows, vocab]
 * (row stride ld_logits >= vocab, device) with the model's sampler, u = d_uniform[pos *
 * ld + r], into d_next [rows] int32 (device); greedy argmax when no sampler is set. A
 * NaN logit raises the model's NaN flag (ember_sync). EMBER_E_CAPACITY when rows exceeds
 * max_batch (the sampler's per-row state lives in the workspace) or ld, or pos lies
 * beyond n_pos - 1. Draws share that state with the model's own, so calls on one model
 * stay ordered on one stream. */
ember_status ember_sample(ember_model* model, const float* d_logits, int32_t rows,
                          int64_t ld_logits, int32_t pos, int32_t* d_next, void* stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid device allocation): ember_sample with the same arguments and
 * results, whose draw keeps its per-row scratch (radix-search histograms, counters and
 * tile sums) in a fixed device array inside the library instead of the model's
 * workspace. It calls no allocator. The array holds EMBER_NOALLOC_MAX_ROWS rows (about
 * 90 KB each, ~1.4 MB per GPU, kept until the process ends); more rows fail with
 * EMBER_E_CAPACITY and enqueue nothing. Each GPU has one such array shared by every call
 * on it (every model): calls that overlap on one GPU (different streams, or threads)
 * race and must not be issued; calls ordered on one stream are safe (each clears the
 * state it uses first). With no sampler set it is the greedy argmax, which needs no
 * scratch. Other errors as ember_sample. */
#define EMBER_NOALLOC_MAX_ROWS 16
ember_status ember_sample_noalloc(ember_model* model, const float* d_logits, int32_t rows,
                                  int64_t ld_logits, int32_t pos, int32_t* d_next, void* stream);

/* Release the host handles of ember_cache_bind ("ForwardModel::create_cache" of the "ember
 * internals" page) and ember_load_weights (Model::new of "Falcon-H1-0.5B-Rust
 * src/lib.rs"). The caller's device buffers are not touched or freed; NULL is a no-op.
 * Free a cache before the model it is bound to. */
void ember_cache_free(ember_cache* cache);
void ember_free(ember_model* model);

/* Thread-local message describing the last error of this thread ("" if none): the
 * String of the Result::Err that Config::validate, validate_weights and Model::logits of
 * "Falcon-H1-0.5B-Rust src/lib.rs" return, here beside the ember_status code. The pointer
 * stays valid until the thread's next ember_* call. */
const char* ember_last_error(void);

/* Host-only: the RoPE tables the library uploads, cos/sin [n_pos, head_dim/2] f32
 * (angles pos * freq in f64, freq = theta^(-2i/head_dim), llama3-scaled when enabled,
 * rounded once to f32). No device call. */
ember_status ember_rope_table(const ember_config* cfg, int32_t n_pos, float* h_cos,
                              float* h_sin);

/* Measurement support (not part of the forward pass): the kernels of one step that
 * ember_time_kernel can time. The projection kinds time the GEMV of a one-row decode
 * step or the MFMA GEMM of a multi-row pass. */
typedef enum ember_kernel {
  EMBER_K_LM_HEAD = 0,         /* tied LM head over the vocabulary (+ argmax partials) */
  EMBER_K_QKV = 1,             /* fused QKV projection (+ bias; RMSNorm fused in the GEMV) */
  EMBER_K_ATTN = 2,            /* split-K decode attention, or flash prefill attention */
  EMBER_K_O = 3,               /* output projection + residual (GEMV: + split-K combine) */
  EMBER_K_GATE_UP = 4,         /* gate/up projection + SiLU*up */
  EMBER_K_DOWN = 5,            /* down projection + residual */
  EMBER_K_LAYER = 6,          /* every kernel of one layer, in step order */
  EMBER_K_SAMPLE = 7           /* the sampler of a decode step (phase 0, sampler set) */
} ember_kernel;

/* Launch kernel `kernel` of the most recent decode step (phase 0) or prefill pass
 * (phase 1) `iters` times back to back on `stream`, launch i on layer i mod layers (so
 * the weights stream from HBM as in a real step), with that step's launch arguments, and
 * return the mean duration per launch in microseconds. On a non-null stream the launches
 * form a graph replayed twice between two HIP events, queued behind a warm-up replay
 * so that host submission time stays outside the measured span. The launches work on the model's own buffers: afterwards the
 * activations, logits and the cache entries of the step's positions are unspecified, so
 * time only a finished sequence. EMBER_E_STATE if no such step has run. */
ember_status ember_time_kernel(ember_model* model, ember_cache* cache, int32_t kernel,
                               int32_t phase, int32_t iters, void* stream, float* avg_us);

/* Measurement support (not part of the forward pass): the achievable peaks that the
 * kernels' roofline fractions are also reported against, beside the published ones.
 *   EMBER_PEAK_COPY: a plain streaming copy from the first half of d_buf to the second
 *     (16-byte loads and stores); *out = GB/s, counting bytes read plus bytes written.
 *   EMBER_PEAK_READ: a streaming read of d_buf past its first 2 MiB (16-byte non-temporal loads,
 *     sixteen in flight per thread), which receive one word per thread; *out = GB/s read.
 *   EMBER_PEAK_MFMA: chains of v_mfma_f32_32x32x16_bf16 on register operands with no
 *     memory traffic, 2048 blocks of 256 threads; *out = TFLOP/s (dense bf16); d_buf (at
 *     least 2 MiB, device) receives one float per thread.
 * One warm-up launch, then `iters` launches between two HIP events on `stream`
 * (synchronised before returning). EMBER_E_ARG for a NULL pointer, iters < 1, an unknown
 * kind or a buffer too small. */
typedef enum ember_peak { EMBER_PEAK_COPY = 0, EMBER_PEAK_MFMA = 1, EMBER_PEAK_READ = 2 } ember_peak;
ember_status ember_measure_peak(int32_t kind, void* d_buf, size_t bytes, int32_t iters,
                                void* stream, float* out);

#ifdef __cplusplus
}
#endif

#endif /* EMBER_H */
