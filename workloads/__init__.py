"""Seeded synthetic workloads shared by the oracle, the tests and the benchmark.

Holds model shapes and random-number draws only; none of the forward pass's arithmetic.
"""
from .configs import ModelConfig, Workload, WORKLOADS, get, scaled, shrink_model  # noqa: F401
from .synth import (f32_to_bf16_bits, make_ids, make_logits, make_uniforms,  # noqa: F401
                    make_weights, quantize_q8_0, tensor_shapes, weights_for)
