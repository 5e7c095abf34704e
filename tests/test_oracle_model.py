"""Model-level pins of the oracle: invariants the pages fix, brute force on tiny shapes, and
independent library implementations of the same architectures (HuggingFace Qwen2 / Llama /
Qwen3 classes built offline from a config, random-init, loaded with our seeded weights)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from oracle import brute
from tests.small_models import ENCODER_SMALL, FAMILIES, LLAMA_SMALL, QWEN_SMALL, TINY

CAUSAL = [m for m in FAMILIES if m.causal]


def _sharpen(ck, factor=30.0):
    """Scale q/k projections so attention is peaked: at init std 0.02 on these tiny shapes
    the scores are ~0 and attention is near-uniform, which would hide RoPE errors."""
    out = {}
    for n, (t, a) in ck.items():
        if n.endswith(("q_proj.weight", "k_proj.weight")):
            a = W.f32_to_bf16_bits(O.widen_bf16(a) * np.float32(factor)) if t == "bf16" else a * factor
        out[n] = (t, a)
    return out


def _model(cfg, seed=7, dtype=np.float64, sharpen=True):
    ck = W.make_weights(cfg, seed)
    if sharpen:
        ck = _sharpen(ck)
    return O.OracleModel(cfg, ck, dtype), ck


def _ids(cfg, n, seed=3):
    return np.random.default_rng(seed).integers(0, cfg.vocab, n).astype(np.int32)


@pytest.mark.parametrize("cfg", FAMILIES, ids=lambda c: c.name)
def test_vectorised_forward_equals_scalar_loops(cfg):
    m, ck = _model(cfg)
    ids = _ids(cfg, 7)
    vec = m.forward_sequence(ids, all_positions=True)
    loops = brute.forward_all(cfg, ck, ids.tolist())
    assert np.allclose(vec, loops, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("cfg", CAUSAL, ids=lambda c: c.name)
def test_cached_decode_equals_full_prefix_recompute(cfg):
    # the ember internals page's KV-cache bug ("the model saw only the last token") would
    # make the cached logits differ from the recomputed ones after the first step
    m, _ = _model(cfg)
    prompt = _ids(cfg, 11)
    ids, cached = O.generate(m, prompt, 9)
    recomputed = O.recompute_logits(m, prompt, ids[:-1])
    assert np.allclose(cached, recomputed, rtol=1e-11, atol=1e-13)


def test_cached_decode_one_token_at_a_time_from_empty_cache():
    m, _ = _model(QWEN_SMALL)
    prompt = _ids(QWEN_SMALL, 6)
    cache = O.KVCache(QWEN_SMALL, 6, np.float64)
    for p, t in enumerate(prompt):
        out = m.forward_token(int(t), p, cache)
    assert np.allclose(out, m.forward_sequence(prompt), rtol=1e-11, atol=1e-13)


def test_prefill_in_two_chunks_equals_one():
    m, _ = _model(LLAMA_SMALL)
    prompt = _ids(LLAMA_SMALL, 13)
    c1 = O.KVCache(LLAMA_SMALL, 13, np.float64)
    m.forward_sequence(prompt[:5], 0, c1)
    two = m.forward_sequence(prompt[5:], 5, c1, all_positions=True)
    one = m.forward_sequence(prompt, all_positions=True)[5:]
    assert np.allclose(two, one, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("cfg", CAUSAL, ids=lambda c: c.name)
def test_causal_prefix_logits_unchanged_by_appended_tokens(cfg):
    m, _ = _model(cfg)
    ids = _ids(cfg, 12)
    short = m.forward_sequence(ids[:7], all_positions=True)
    long_ = m.forward_sequence(ids, all_positions=True)
    assert np.allclose(short, long_[:7], rtol=1e-12, atol=1e-14)


def test_bidirectional_encoder_sees_later_tokens():
    m, _ = _model(ENCODER_SMALL)
    ids = _ids(ENCODER_SMALL, 12)
    short = m.forward_sequence(ids[:7], all_positions=True)
    long_ = m.forward_sequence(ids, all_positions=True)
    assert not np.allclose(short, long_[:7], rtol=1e-6)


@pytest.mark.parametrize("cfg", [TINY, ENCODER_SMALL], ids=lambda c: c.name)
def test_every_layer_feeds_the_next(cfg):
    # a forgotten reassignment of a block's output (ember internals page) would leave the
    # output unchanged when that layer's weights change
    base, ck = _model(cfg)
    ids = _ids(cfg, 5)
    ref = base.forward_sequence(ids, all_positions=True)
    for li in range(cfg.layers):
        for part in ("self_attn.o_proj.weight", "mlp.down_proj.weight"):
            m = O.OracleModel(cfg, ck, np.float64)
            m.w[f"model.layers.{li}.{part}"] = m.w[f"model.layers.{li}.{part}"] * 1.5
            assert not np.allclose(m.forward_sequence(ids, all_positions=True), ref, rtol=1e-6)


def test_gqa_model_equals_mha_model_with_repeated_kv_weights():
    cfg = LLAMA_SMALL
    m, ck = _model(cfg)
    mha_cfg = W.shrink_model(cfg, kv_heads=cfg.heads)
    rep = cfg.group
    mk = {}
    for name, (tag, arr) in ck.items():
        if name.endswith(("k_proj.weight", "v_proj.weight")):
            arr = np.repeat(arr.reshape(cfg.kv_heads, cfg.head_dim, -1), rep, axis=0).reshape(-1, arr.shape[-1])
        mk[name] = (tag, arr)
    mha = O.OracleModel(mha_cfg, mk, np.float64)
    ids = _ids(cfg, 9)
    assert np.allclose(m.forward_sequence(ids, all_positions=True),
                       mha.forward_sequence(ids, all_positions=True), rtol=1e-12, atol=1e-14)


def test_f32_oracle_within_envelope_of_f64_shadow():
    w = W.get("tiny")
    ck = W.weights_for(w)
    ids = W.make_ids(w)[0]
    i32, l32 = O.generate(O.OracleModel(w.model, ck, np.float32), ids, w.decode_steps)
    i64, l64 = O.generate(O.OracleModel(w.model, ck, np.float64), ids, w.decode_steps)
    rel = np.abs(l32 - l64).max(-1) / np.abs(l64).max(-1)
    assert rel.max() < 1e-5
    assert np.array_equal(i32, i64)


def test_input_errors_of_the_rust_reference():
    m, _ = _model(TINY)
    with pytest.raises(ValueError):
        m.forward_sequence(np.array([], np.int32))
    with pytest.raises(ValueError):
        m.forward_sequence(np.array([1, TINY.vocab]))
    with pytest.raises(ValueError):
        m.forward_sequence(np.zeros(16385, np.int32))
    with pytest.raises(ValueError):
        O.KVCache(TINY, 4).write(0, np.array([4]), np.zeros((1, 2, 8)), np.zeros((1, 2, 8)))


def test_missing_tensor_is_an_error():
    ck = W.make_weights(TINY, 1)
    del ck["model.layers.1.mlp.up_proj.weight"]
    m = O.OracleModel(TINY, ck)
    with pytest.raises(KeyError):
        m.forward_sequence(np.array([1, 2]))


# ----------------------------------------------------------------------------- HuggingFace

def _rel(a, b):
    return np.abs(a - b).max() / np.abs(b).max()


# HuggingFace's rotary module computes its angles pos*freq in float32 while the oracle's
# tables are f64 angles rounded once; at position p that leaves HF ~p*2^-24 rad of angle
# error, which bounds how closely the two can agree.


def _hf_state(ck, dtype=torch.float64):
    return {n: torch.from_numpy(O.decode_tensor(t, a).astype(np.float64)).to(dtype) for n, (t, a) in ck.items()}


def _load(model, ck, skip=()):
    sd = {k: v for k, v in _hf_state(ck).items() if k not in skip}
    missing, unexpected = model.load_state_dict(sd, strict=False)
    assert not unexpected, unexpected
    assert all(k == "lm_head.weight" for k in missing), missing   # tied to the embedding
    return model.double().eval()


def test_matches_hf_qwen2_with_bias_and_tied_head():
    from transformers import Qwen2Config, Qwen2ForCausalLM
    c = QWEN_SMALL
    hc = Qwen2Config(vocab_size=c.vocab, hidden_size=c.hidden, intermediate_size=c.ffn,
                     num_hidden_layers=c.layers, num_attention_heads=c.heads,
                     num_key_value_heads=c.kv_heads, rms_norm_eps=c.rms_eps,
                     tie_word_embeddings=True, rope_theta=c.rope_theta,
                     max_position_embeddings=256, attn_implementation="eager")
    m, ck = _model(c)
    hf = _load(Qwen2ForCausalLM(hc).double(), ck)
    ids = _ids(c, 10)
    with torch.no_grad():
        ref = hf(torch.from_numpy(ids.astype(np.int64))[None]).logits[0].numpy()
    assert _rel(m.forward_sequence(ids, all_positions=True), ref) < 1e-6


def test_matches_hf_llama_with_llama3_rope_scaling_at_large_positions():
    from transformers import LlamaConfig, LlamaForCausalLM
    c = W.shrink_model(LLAMA_SMALL, head_dim=16, heads=4)
    hc = LlamaConfig(vocab_size=c.vocab, hidden_size=c.hidden, intermediate_size=c.ffn,
                     num_hidden_layers=c.layers, num_attention_heads=c.heads,
                     num_key_value_heads=c.kv_heads, head_dim=c.head_dim,
                     rms_norm_eps=c.rms_eps, tie_word_embeddings=True, rope_theta=c.rope_theta,
                     max_position_embeddings=16384, attn_implementation="eager",
                     rope_scaling={"rope_type": "llama3", "factor": 32.0, "low_freq_factor": 1.0,
                                   "high_freq_factor": 4.0, "original_max_position_embeddings": 8192})
    m, ck = _model(c)
    hf = _load(LlamaForCausalLM(hc).double(), ck)
    ids = _ids(c, 9)
    start = 6000
    with torch.no_grad():
        ref = hf(torch.from_numpy(ids.astype(np.int64))[None],
                 position_ids=torch.arange(start, start + 9)[None]).logits[0].numpy()
    ours = m.forward_sequence(ids, start, None, all_positions=True)
    assert _rel(ours, ref) < 5e-4
    # the bound discriminates: the same model without llama3 scaling is far outside it
    plain = O.OracleModel(W.shrink_model(c, llama3=None), ck, np.float64)
    assert _rel(plain.forward_sequence(ids, start, None, all_positions=True), ref) > 2e-3


def test_matches_hf_qwen3_qk_norm_bidirectional_with_token_head():
    from transformers import Qwen3Config, Qwen3Model
    c = ENCODER_SMALL
    hc = Qwen3Config(vocab_size=c.vocab, hidden_size=c.hidden, intermediate_size=c.ffn,
                     num_hidden_layers=c.layers, num_attention_heads=c.heads,
                     num_key_value_heads=c.kv_heads, head_dim=c.head_dim, rms_norm_eps=c.rms_eps,
                     rope_theta=c.rope_theta, attn_implementation="eager")
    m, ck = _model(c)
    sd = {k[len("model."):]: v for k, v in _hf_state(ck).items() if k.startswith("model.")}
    hf = Qwen3Model(hc).double().eval()
    missing, unexpected = hf.load_state_dict(sd, strict=True)
    ids = _ids(c, 11)
    T = len(ids)
    with torch.no_grad():   # an all-zero additive 4D mask: every key visible
        h = hf(torch.from_numpy(ids.astype(np.int64))[None],
               attention_mask=torch.zeros(1, 1, T, T, dtype=torch.float64)).last_hidden_state[0]
        st = _hf_state(ck)
        ref = (h @ st["token_cls_head.weight"].T + st["token_cls_head.bias"]).numpy()
    assert _rel(m.encode(ids[None])[0], ref) < 1e-6


def test_activations_match_hf_hidden_states():
    """forward_with_activations (ember internals, "ForwardModel trait"): the hidden state
    after every block at the last position. HuggingFace's hidden_states[l + 1] is block
    l's output for every block but the last, whose entry carries the final norm."""
    from transformers import Qwen2Config, Qwen2ForCausalLM
    c = W.shrink_model(QWEN_SMALL, layers=3)
    hc = Qwen2Config(vocab_size=c.vocab, hidden_size=c.hidden, intermediate_size=c.ffn,
                     num_hidden_layers=c.layers, num_attention_heads=c.heads,
                     num_key_value_heads=c.kv_heads, rms_norm_eps=c.rms_eps,
                     tie_word_embeddings=True, rope_theta=c.rope_theta,
                     max_position_embeddings=256, attn_implementation="eager")
    m, ck = _model(c)
    hf = _load(Qwen2ForCausalLM(hc).double(), ck)
    ids = _ids(c, 10)
    with torch.no_grad():
        out = hf(torch.from_numpy(ids.astype(np.int64))[None], output_hidden_states=True)
    hs = [h[0, -1].numpy() for h in out.hidden_states]
    acts, logits = m.forward_with_activations(ids)
    assert acts.shape == (c.layers, c.hidden)
    for li in range(c.layers - 1):
        assert _rel(acts[li], hs[li + 1]) < 1e-6
    assert _rel(O.rmsnorm(acts[-1], m.w["model.norm.weight"], c.rms_eps), hs[-1]) < 1e-6
    assert _rel(logits, out.logits[0, -1].numpy()) < 1e-6
    assert np.array_equal(logits, m.forward_sequence(ids))      # the same forward pass


def test_sensitivity_matches_mean_pooled_hf_hidden_state():
    """The encoder's mean-pooled sequence score ("PII-Tracer serving/reference_forward.py",
    ``forward``): the final-normed states averaged over tokens, then the head."""
    from transformers import Qwen3Config, Qwen3Model
    c = W.shrink_model(ENCODER_SMALL, sens_head=True)
    hc = Qwen3Config(vocab_size=c.vocab, hidden_size=c.hidden, intermediate_size=c.ffn,
                     num_hidden_layers=c.layers, num_attention_heads=c.heads,
                     num_key_value_heads=c.kv_heads, head_dim=c.head_dim, rms_norm_eps=c.rms_eps,
                     rope_theta=c.rope_theta, attn_implementation="eager")
    m, ck = _model(c)
    assert "sensitivity_head.weight" in ck and ck["sensitivity_head.weight"][1].shape == (1, c.hidden)
    sd = {k[len("model."):]: v for k, v in _hf_state(ck).items() if k.startswith("model.")}
    hf = Qwen3Model(hc).double().eval()
    hf.load_state_dict(sd, strict=True)
    ids = _ids(c, 13)
    T = len(ids)
    with torch.no_grad():
        h = hf(torch.from_numpy(ids.astype(np.int64))[None],
               attention_mask=torch.zeros(1, 1, T, T, dtype=torch.float64)).last_hidden_state[0]
        st = _hf_state(ck)
        ref = float((h.mean(0) @ st["sensitivity_head.weight"].T + st["sensitivity_head.bias"])[0])
    got = m.sensitivity(ids)
    assert abs(got - ref) <= 1e-9 * max(1.0, abs(ref))
    # pooling the states before the final norm gives a different number
    x = m.w["model.embed_tokens.weight"][ids].astype(np.float64)
    for li in range(c.layers):
        x = m.layer_sequence(li, x, np.arange(T), None)
    pre = float((x.mean(0) @ m.w["sensitivity_head.weight"].T + m.w["sensitivity_head.bias"])[0])
    assert abs(pre - ref) > 1e-6
