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
from tests.small_models import (ENCODER_SMALL, LLAMA_HD64, LLAMA_SMALL, LLAMA_SPLITK, QWEN_SMALL,
                                 QWEN_SMALL_Q8)

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


@pytest.mark.parametrize("prec_name", ["exact", "fast"])
def test_taps_leave_the_logits_bitwise_unchanged(prec_name):
    """A split-K down projection leaves its partial planes to the next layer's first
    RMSNorm, which adds them into x; with activation taps x is read after every layer, so
    the separate fixed-order reduce runs instead. Both sum the planes in the same order:
    the last-token logits and ids of a tapped prefill equal a plain prefill's bit for bit,
    and so do the decode steps that follow. (llama-splitk: K = 1024 against 8 output
    tiles of 74 rows, so its down projection splits K into four slices.)"""
    from gqa_decoder_transformer_amd import binding as B
    prec = B.EXACT if prec_name == "exact" else B.FAST
    model = LLAMA_SPLITK
    ck = W.make_weights(model, 23)
    Bn, T = 2, 37
    prompt = np.random.default_rng(29).integers(0, model.vocab, (Bn, T)).astype(np.int32)
    say(f"taps vs plain prefill {model.name} {prec_name}")
    plain = _engine(model, ck, prec, Bn, 64, Bn * T)
    tapped = _engine(model, ck, prec, Bn, 64, Bn * T)
    ids_p = plain.prefill(prompt)[0].cpu().numpy()
    lg_p = plain.logits(Bn).cpu().numpy()
    _, ids_t = tapped.forward_with_activations(prompt)
    ids_t = ids_t.cpu().numpy()
    lg_t = tapped.logits(Bn).cpu().numpy()
    assert np.array_equal(lg_p.view(np.uint32), lg_t.view(np.uint32))
    assert np.array_equal(ids_p, ids_t)
    import torch
    cur_p = torch.tensor(ids_p, dtype=torch.int32, device="cuda:0")
    cur_t = torch.tensor(ids_t, dtype=torch.int32, device="cuda:0")
    for k in range(3):
        plain.decode_step(cur_p, T + k)
        tapped.decode_step(cur_t, T + k)
        a, b = plain.logits(Bn).cpu().numpy(), tapped.logits(Bn).cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), k
        assert np.array_equal(cur_p.cpu().numpy(), cur_t.cpu().numpy()), k
    plain.sync()
    tapped.sync()
