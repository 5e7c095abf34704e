"""Model shapes and workloads of the decoder forward pass (shapes only, no arithmetic).

Five workloads are defined, each a model shape plus a batch/prompt/decode schedule:

* ``tiny``      -- the shape of the Falcon-H1 Rust reference's ``Config::demo`` (page
                   "Falcon-H1-0.5B-Rust src/lib.rs", ``Config::demo``): vocab 64, hidden 32,
                   2 layers, 4 q / 2 kv heads, head_dim 8, ff 64; f32 weights.
* ``qwen05b``   -- the Qwen2.5-0.5B shape that ember's NumPy reference runs (page
                   "ember scripts/reference_forward.py", module docstring and the config keys
                   read in ``main``): q/k/v biases, theta 1e6, eps 1e-6; bf16 weights.
* ``llama1b``   -- the Llama-3.2-1B shape of "LowLlamaBasic reference.py" (``predict`` and
                   ``rotary_cos_sin`` with llama3 frequency scaling); bf16 weights.
* ``encoder``   -- the Qwen3-style bidirectional encoder of "PII-Tracer-vLLM
                   serving/reference_forward.py" (``forward``: per-head q/k RMSNorm before
                   RoPE, no mask, token classification head); bf16 weights.
* ``longctx``   -- ``llama1b`` weights, 64 rows each holding an 8192-token cache, then
                   batched greedy decode.
* ``qwen05b-q8`` -- ``qwen05b`` with every matrix stored as q8_0 blocks (32 int8 values
                   and one f16 scale per 34 bytes), the weight format of the "ember
                   internals" page, section "GGUF format and quantization".

Hyper-parameters that the pages leave open are filled with the plainest reading: no
bias for ``tiny``, eps 1e-5 for the Llama shape, eps 1e-6 / vocab 151936 for the
Qwen3-style encoder, and a 2-way classification head with bias.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class ModelConfig:
    name: str
    vocab: int
    hidden: int
    layers: int
    heads: int
    kv_heads: int
    head_dim: int
    ffn: int
    rms_eps: float
    rope_theta: float
    # llama3 frequency scaling: (factor, low_freq_factor, high_freq_factor,
    # original_max_position_embeddings) or None.
    llama3: Optional[Tuple[float, float, float, float]] = None
    qkv_bias: bool = False
    qk_norm: bool = False
    causal: bool = True
    head: str = "tied_lm"          # "tied_lm" (logits = E . h) or "cls" (W h + b)
    n_classes: int = 0
    # the encoder's mean-pooled sequence score ("PII-Tracer serving/reference_forward.py",
    # ``forward``: sensitivity_head [1, hidden] + bias [1]); off unless asked for
    sens_head: bool = False
    weight_dtype: str = "bf16"     # "f32", "bf16" (every tensor) or "q8_0" (matrices; 1-D f32)

    @property
    def group(self) -> int:
        return self.heads // self.kv_heads

    @property
    def q_dim(self) -> int:
        return self.heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.kv_heads * self.head_dim

    @property
    def out_dim(self) -> int:
        return self.vocab if self.head == "tied_lm" else self.n_classes


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelConfig
    batch: int
    prompt_len: int
    decode_steps: int
    weight_seed: int
    ids_seed: int
    description: str = field(default="", compare=False)

    @property
    def max_pos(self) -> int:
        return self.prompt_len + self.decode_steps


TINY = ModelConfig(
    name="tiny", vocab=64, hidden=32, layers=2, heads=4, kv_heads=2, head_dim=8,
    ffn=64, rms_eps=1e-5, rope_theta=1e4, weight_dtype="f32")

QWEN05B = ModelConfig(
    name="qwen2.5-0.5b", vocab=151936, hidden=896, layers=24, heads=14, kv_heads=2,
    head_dim=64, ffn=4864, rms_eps=1e-6, rope_theta=1e6, qkv_bias=True)

LLAMA1B = ModelConfig(
    name="llama-3.2-1b", vocab=128256, hidden=2048, layers=16, heads=32, kv_heads=8,
    head_dim=64, ffn=8192, rms_eps=1e-5, rope_theta=5e5,
    llama3=(32.0, 1.0, 4.0, 8192.0))

ENCODER = ModelConfig(
    name="qwen3-encoder", vocab=151936, hidden=1024, layers=28, heads=16, kv_heads=8,
    head_dim=128, ffn=3072, rms_eps=1e-6, rope_theta=1e6, qk_norm=True, causal=False,
    head="cls", n_classes=2)

# the Qwen2.5-0.5B shape with q8_0 matrices ("ember internals", section
# "GGUF format and quantization", subsection "q8_0 block quantization"): the same seeded draws, quantised
QWEN05B_Q8 = ModelConfig(**{**QWEN05B.__dict__, "name": "qwen2.5-0.5b-q8_0",
                            "weight_dtype": "q8_0"})

WORKLOADS = {
    "tiny": Workload("tiny", TINY, batch=1, prompt_len=16, decode_steps=16,
                     weight_seed=1, ids_seed=101,
                     description="tiny GQA decoder, f32 weights, 1x16 prompt, 16 greedy steps"),
    "qwen05b": Workload("qwen05b", QWEN05B, batch=1, prompt_len=128, decode_steps=128,
                        weight_seed=2, ids_seed=102,
                        description="Qwen2.5-0.5B-shaped decoder, bf16, 1x128 prompt, 128 greedy steps"),
    "llama1b": Workload("llama1b", LLAMA1B, batch=1, prompt_len=2048, decode_steps=256,
                        weight_seed=3, ids_seed=103,
                        description="Llama-3.2-1B-shaped decoder, bf16, 1x2048 prompt, 256 greedy steps"),
    "encoder": Workload("encoder", ENCODER, batch=16, prompt_len=512, decode_steps=0,
                        weight_seed=4, ids_seed=104,
                        description="Qwen3-style bidirectional encoder, bf16, 16x512, 2-way token head"),
    "qwen05b-q8": Workload("qwen05b-q8", QWEN05B_Q8, batch=1, prompt_len=128, decode_steps=128, weight_seed=2,
                           ids_seed=102,
                           description="Qwen2.5-0.5B-shaped decoder, q8_0 matrices, 1x128 "
                                       "prompt, 128 greedy steps"),
    "longctx": Workload("longctx", LLAMA1B, batch=64, prompt_len=8192, decode_steps=128,
                        weight_seed=3, ids_seed=105,
                        description="Llama-3.2-1B-shaped decoder, bf16, 64 rows x 8192 cached, 128 greedy steps"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(w: Workload, **changes) -> Workload:
    """A copy of ``w`` with some fields replaced (used for reduced-size parity cases)."""
    d = dict(w.__dict__)
    d.update(changes)
    return Workload(**d)


def shrink_model(m: ModelConfig, **changes) -> ModelConfig:
    d = dict(m.__dict__)
    d.update(changes)
    return ModelConfig(**d)
