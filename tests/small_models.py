"""Small model shapes, one per family of the five workloads, for CPU pins and quick GPU
parity cases. Shapes only; the weights come from the seeded generator."""
from workloads import configs as C

TINY = C.TINY

QWEN_SMALL = C.shrink_model(C.QWEN05B, name="qwen-small", vocab=97, hidden=64, layers=2,
                            heads=4, kv_heads=2, head_dim=16, ffn=96)

LLAMA_SMALL = C.shrink_model(C.LLAMA1B, name="llama-small", vocab=101, hidden=64, layers=2,
                             heads=8, kv_heads=2, head_dim=8, ffn=128)

ENCODER_SMALL = C.shrink_model(C.ENCODER, name="encoder-small", vocab=89, hidden=64,
                               layers=2, heads=4, kv_heads=2, head_dim=32, ffn=96)

FAMILIES = [TINY, QWEN_SMALL, LLAMA_SMALL, ENCODER_SMALL]

# head_dim 64 / 128 shapes: exercise the MFMA attention kernels
LLAMA_HD64 = C.shrink_model(C.LLAMA1B, name="llama-hd64", vocab=131, hidden=128, layers=2,
                            heads=4, kv_heads=2, head_dim=64, ffn=192)

ENCODER_HD128 = C.shrink_model(C.ENCODER, name="encoder-hd128", vocab=83, hidden=128, layers=2,
                               heads=2, kv_heads=1, head_dim=128, ffn=160)

QWEN_HD64_G7 = C.shrink_model(C.QWEN05B, name="qwen-hd64-g7", vocab=97, hidden=448, layers=2,
                              heads=7, kv_heads=1, head_dim=64, ffn=320)

# plain multi-head attention (one kv head per query head)
LLAMA_MHA = C.shrink_model(C.LLAMA1B, name="llama-mha", vocab=131, hidden=128, layers=2,
                           heads=4, kv_heads=4, head_dim=64, ffn=192)

# at most 64 rows against >= 192 output tiles of 64 (vocabulary 16384, gate/up 12288
# rows): the 64 x 64 GEMM tiles without split-K
LLAMA_WIDE = C.shrink_model(C.LLAMA1B, name="llama-wide", vocab=16384, hidden=256, layers=2,
                            heads=4, kv_heads=2, head_dim=64, ffn=6144)

# head_dim 64 with 96 heads' worth of QKV columns (64 q + 2 x 16 kv): at 65-128 tokens per
# pass the QKV GEMM fills >= 192 tiles without split-K, so the post-processing (bias,
# q/k RMSNorm, RoPE, K/V store) runs in its epilogue
QWEN_QKV_WIDE = C.shrink_model(C.QWEN05B, name="qwen-qkv-wide", vocab=256, hidden=512, layers=2,
                               heads=64, kv_heads=16, head_dim=64, ffn=256, qk_norm=True)

# 32 heads of 64 (K = 2048 for the output projection: the row-per-block GEMV); one-row
# decode at 150+ positions of a 512-position cache runs many key splits and their combine
LLAMA_OFOLD = C.shrink_model(C.LLAMA1B, name="llama-ofold", vocab=256, hidden=256, layers=2,
                             heads=32, kv_heads=8, head_dim=64, ffn=512)

# long K against few output tiles: the projections take the split-K path
LLAMA_SPLITK = C.shrink_model(C.LLAMA1B, name="llama-splitk", vocab=131, hidden=256, layers=2,
                              heads=4, kv_heads=2, head_dim=64, ffn=1024)

# decode GEMV layouts past row-per-wave: the down projection's K takes the row-per-block
# layout with two chunks per thread (ffn 2304) and the K-looping kernel (ffn 8448 bf16 is
# more than 1024 chunks of 16 bytes)
QWEN_FF2K = C.shrink_model(C.QWEN05B, name="qwen-ff2k", vocab=97, hidden=64, layers=2,
                           heads=4, kv_heads=2, head_dim=16, ffn=2304)

LLAMA_FF8K = C.shrink_model(C.LLAMA1B, name="llama-ff8k", vocab=101, hidden=64, layers=2,
                            heads=8, kv_heads=2, head_dim=8, ffn=8448)

# q8_0 matrices (every K a multiple of 32). In the q8 GEMV a 16-byte chunk holds 16
# weights: ffn 2304 puts the down projection in the row-per-block layout, ffn 8448 in it
# with three chunks per thread, ffn 16896 past 1024 chunks (the K-looping kernel)
QWEN_SMALL_Q8 = C.shrink_model(QWEN_SMALL, name="qwen-small-q8", weight_dtype="q8_0")
LLAMA_SMALL_Q8 = C.shrink_model(LLAMA_SMALL, name="llama-small-q8", weight_dtype="q8_0")
LLAMA_HD64_Q8 = C.shrink_model(LLAMA_HD64, name="llama-hd64-q8", weight_dtype="q8_0")
QWEN_FF2K_Q8 = C.shrink_model(QWEN_FF2K, name="qwen-ff2k-q8", weight_dtype="q8_0")
LLAMA_FF8K_Q8 = C.shrink_model(LLAMA_FF8K, name="llama-ff8k-q8", weight_dtype="q8_0")
LLAMA_FF16K_Q8 = C.shrink_model(LLAMA_FF8K, name="llama-ff16k-q8", ffn=16896, weight_dtype="q8_0")
Q8_SMALL = [QWEN_SMALL_Q8, LLAMA_SMALL_Q8, LLAMA_HD64_Q8, QWEN_FF2K_Q8, LLAMA_FF8K_Q8,
            LLAMA_FF16K_Q8]
