"""GPU parity of the probing taps through the C ABI against the oracle: the hidden state
after every block at each row's last position ("ember internals", "ForwardModel trait":
forward_with_activations) and the encoder's mean-pooled sequence score ("PII-Tracer
serving/reference_forward.py", forward: sensitivity head), in both precision tiers and
with prompts split over several passes."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.gpu_util import TOL_EXACT, TOL_FAST, check_greedy, rel_maxabs, say
from tests.small_models import ENCODER_SMALL, LLAMA_HD64, LLAMA_SMALL, QWEN_SMALL, QWEN_SMALL_Q8

pytestmark = pytest.mark.gpu


def _engine(model, ck, precision, max_batch, max_seq, max_tokens):
    from gqa_decoder_transformer_amd import binding as B
    cfg = B.make_config(model, precision=precision, max_batch=max_batch, max_seq=max_seq,
                        max_tokens=max_tokens)
    return B.Engine(cfg, ck, poison=True)


@pytest.mark.parametrize("model", [QWEN_SMALL, LLAMA_SMALL, LLAMA_HD64, QWEN_SMALL_Q8],
                         ids=lambda m: m.name)
@pytest.mark.parametrize("prec_name", ["exact", "fast"])
@pytest.mark.parametrize("max_tokens", [128, 16], ids=["one-pass", "chunked"])
def test_activations_after_every_block(model, prec_name, max_tokens):
    from gqa_decoder_transformer_amd import binding as B
    prec = B.EXACT if prec_name == "exact" else B.FAST
    tol = TOL_EXACT if prec == B.EXACT else TOL_FAST
    ck = W.make_weights(model, 19)
    Bn, T = 2, 37
    prompt = np.random.default_rng(21).integers(0, model.vocab, (Bn, T)).astype(np.int32)
    say(f"activations {model.name} {prec_name} max_tokens={max_tokens}")
    eng = _engine(model, ck, prec, Bn, 64, max(max_tokens, Bn))
    acts, nxt = eng.forward_with_activations(prompt)
    logits = eng.logits(Bn).cpu().numpy()
    acts = acts.cpu().numpy()
    nxt = nxt.cpu().numpy()
    eng.sync()
    om = O.OracleModel(model, ck)
    for b in range(Bn):
        o_acts, o_logits = om.forward_with_activations(prompt[b])
        err = rel_maxabs(acts[b], o_acts)                    # per layer
        say(f"row {b}: max rel err over layers {err.max():.3g}")
        assert err.max() < tol, err
        assert rel_maxabs(logits[b], o_logits) < tol
        if prec == B.EXACT:
            check_greedy(nxt[b:b + 1], np.array([np.argmax(o_logits)]), o_logits[None], tol)


def _scale(model, ck, ids):
    """Size of the score's terms (float64): sum_d |mean_d w_d| + |b|."""
    m64 = O.OracleModel(model, ck, np.float64)
    x = m64.w["model.embed_tokens.weight"][ids]
    for li in range(model.layers):
        x = m64.layer_sequence(li, x, np.arange(len(ids)), None)
    h = O.rmsnorm(x, m64.w["model.norm.weight"], model.rms_eps)
    return float(np.abs(h.mean(0) * m64.w["sensitivity_head.weight"][0]).sum()
                 + abs(m64.w["sensitivity_head.bias"][0]))


@pytest.mark.parametrize("prec_name", ["exact", "fast"])
@pytest.mark.parametrize("max_tokens", [128, 29], ids=["one-pass", "row-per-pass"])
def test_mean_pooled_sequence_score(prec_name, max_tokens):
    from gqa_decoder_transformer_amd import binding as B
    prec = B.EXACT if prec_name == "exact" else B.FAST
    tol = TOL_EXACT if prec == B.EXACT else TOL_FAST
    model = W.shrink_model(ENCODER_SMALL, sens_head=True)
    ck = W.make_weights(model, 22)
    Bn, T = 3, 29
    prompt = np.random.default_rng(23).integers(0, model.vocab, (Bn, T)).astype(np.int32)
    say(f"sequence score {prec_name} max_tokens={max_tokens}")
    eng = _engine(model, ck, prec, Bn, 32, max(max_tokens, Bn))
    eng.prefill(prompt)
    got = eng.sensitivity(Bn).cpu().numpy()
    eng.sync()
    om = O.OracleModel(model, ck)
    for b in range(Bn):
        want = om.sensitivity(prompt[b])
        scale = _scale(model, ck, prompt[b])
        say(f"row {b}: {got[b]:.6g} vs {want:.6g} (terms {scale:.3g})")
        assert abs(got[b] - want) <= tol * scale


def test_probe_errors():
    from gqa_decoder_transformer_amd import binding as B
    model = W.shrink_model(ENCODER_SMALL, sens_head=True)
    eng = _engine(model, W.make_weights(model, 22), B.EXACT, 1, 16, 16)
    with pytest.raises(B.EmberError) as e:
        eng.sensitivity(1)
    assert e.value.status == 8                           # before any prefill
    plain = _engine(ENCODER_SMALL, W.make_weights(ENCODER_SMALL, 22), B.EXACT, 1, 16, 16)
    plain.prefill(np.zeros((1, 4), np.int32))
    with pytest.raises(B.EmberError) as e:
        plain.sensitivity(1)
    assert e.value.status == 8                           # no sequence-score head
    with pytest.raises(B.EmberError) as e:
        B.ember_forward_with_activations(plain.model, plain.cache, np.zeros((1, 4), np.int32),
                                         0, 0, 0, plain.sp)
    assert e.value.status == 1                           # NULL activations buffer
    with pytest.raises(B.EmberError) as e:
        plain.prefill(np.zeros((1, 17), np.int32))
    assert e.value.status == 7                           # a bidirectional row over one pass
