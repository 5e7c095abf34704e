"""The seeded input generator: determinism, shapes, bf16 rounding, norm weights."""
import numpy as np
import torch

import workloads as W
from tests.small_models import QWEN_SMALL


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 0.02,
                        # exact halfway cases between two bf16 values, both parities
                        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)])
    ours = W.f32_to_bf16_bits(a)
    lib = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)


def test_weights_are_deterministic_and_named_like_hf():
    a = W.make_weights(QWEN_SMALL, 5)
    b = W.make_weights(QWEN_SMALL, 5)
    c = W.make_weights(QWEN_SMALL, 6)
    assert list(a) == list(W.tensor_shapes(QWEN_SMALL))
    for n in a:
        assert a[n][0] == "bf16" and a[n][1].dtype == np.uint16
        assert a[n][1].shape == W.tensor_shapes(QWEN_SMALL)[n]
        assert np.array_equal(a[n][1], b[n][1])
    assert not np.array_equal(a["model.embed_tokens.weight"][1], c["model.embed_tokens.weight"][1])
    assert "model.layers.1.self_attn.k_proj.bias" in a


def test_norm_weights_are_one_and_draws_have_init_std():
    ck = W.make_weights(QWEN_SMALL, 5)
    one = W.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    for n, (_, arr) in ck.items():
        if n.endswith("norm.weight"):
            assert (arr == one).all()
    e = (ck["model.embed_tokens.weight"][1].astype(np.uint32) << 16).view(np.float32)
    assert abs(e.std() - 0.02) < 0.002 and abs(e.mean()) < 0.002


def test_ids_are_seeded_uniform_in_vocab():
    w = W.get("qwen05b")
    a, b = W.make_ids(w), W.make_ids(w)
    assert a.shape == (1, 128) and a.dtype == np.int32 and np.array_equal(a, b)
    assert a.min() >= 0 and a.max() < w.model.vocab
    big = W.make_ids(W.get("longctx"))
    assert big.shape == (64, 8192)


def test_workload_table():
    t = W.WORKLOADS
    assert (t["tiny"].model.vocab, t["tiny"].model.hidden, t["tiny"].model.layers) == (64, 32, 2)
    assert t["qwen05b"].model.qkv_bias and not t["llama1b"].model.qkv_bias
    assert t["llama1b"].model.llama3 == (32.0, 1.0, 4.0, 8192.0)
    assert not t["encoder"].model.causal and t["encoder"].model.qk_norm
    assert t["longctx"].model is t["llama1b"].model and t["longctx"].batch == 64
