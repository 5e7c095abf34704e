"""Oracle for the GQA decoder forward pass -- TEST INFRASTRUCTURE, not part of the product.

A plain, slow, obviously correct CPU implementation (NumPy; scalar Python loops for the
brute-force form) of what the GPU path computes: bf16->f32 weight widening and q8_0
block dequantisation, RMSNorm,
rotate-half RoPE with optional llama3 frequency scaling, grouped-query attention with a
causal KV cache (or bidirectional), SwiGLU MLP, the tied LM head or a token
classification head, greedy argmax, and the sampler (temperature, top-k, top-p, softmax,
inverse-CDF draw; ``oracle.sampler``).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package. The HIP library and its Python binding never import, call or
link anything here, and nothing here imports them. The two sides share only the seeded
input generator (``workloads``), which holds none of the forward pass's arithmetic.

Precision: float32 storage and arithmetic by default, as the pages compute (bf16-valued
weights widened to f32, f32 caches and activations); ``dtype=np.float64`` gives the
shadow used to bound the f32 oracle's own rounding error.

Parity status: every function here is pinned by ``tests/test_oracle_*.py`` against
closed forms, invariants, library routines (torch, scipy, HuggingFace model classes) or
the brute-force loops; end-to-end values of the pages' trained checkpoints cannot be
pinned (the checkpoints are not available), so the model-level pins are invariants and
an independent library implementation of the same architectures.
"""
from .primitives import (apply_rope, attention, decode_tensor, dequant_q8_0,  # noqa: F401
                         f16_to_f32, greedy_argmax, rmsnorm, rope_inv_freq, rope_tables,
                         silu, softmax, swiglu, widen_bf16)
from .model import KVCache, OracleModel, generate, recompute_logits  # noqa: F401
from . import brute  # noqa: F401
from . import sampler  # noqa: F401
