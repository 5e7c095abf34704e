"""The batch-1 LM head on the GPU (the fused final-norm GEMV that writes per-wave argmax
keys, then the key reduction) on crafted logits, and the bf16 -> f32 widening of every
bf16 bit pattern through that GEMV's weight loads.

Crafting: the final RMSNorm weight is `s e_0` with `s` the sign of the residual stream's
first component at the last position (read from the oracle), so h = rmsnorm(x) has one
nonzero component h_0 > 0 and every logit is E[j, 0] * h_0 exactly (the other products
are signed zeros). Column 0 of the tied embedding then sets each logit's value and sign:
equal entries give bitwise-equal logits (ties), +0 / -0 entries give zero logits, -inf
entries give -inf. The prompt uses tokens whose E[j, 0] is negative and keeps their rows
unchanged, so the crafted rows never feed the residual stream.

Greedy rule ("ember scripts/reference_forward.py", decode loop, np.argmax): the lowest
index of the maximum; -0.0 ties +0.0.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.gpu_util import say
from tests.small_models import LLAMA_SMALL

pytestmark = pytest.mark.gpu

CRAFT = W.shrink_model(LLAMA_SMALL, name="llama-craft", vocab=50021)


def _bits(a):
    return W.f32_to_bf16_bits(np.asarray(a, np.float32))


def _crafted(case, seed=71):
    """(checkpoint, prompt, expected id, crafted rows) for one crafted-logits case."""
    m = CRAFT
    ck = W.make_weights(m, seed)
    E = O.widen_bf16(ck["model.embed_tokens.weight"][1])
    rng = np.random.default_rng(seed)
    prompt = rng.choice(np.nonzero(E[:, 0] < 0)[0], 6, replace=False).astype(np.int32)
    acts, _ = O.OracleModel(m, ck).forward_with_activations(prompt)
    s = np.float32(1.0 if acts[-1, 0] > 0 else -1.0)
    fn = np.zeros(m.hidden, np.float32)
    fn[0] = s
    ck["model.norm.weight"] = ("bf16", _bits(fn))
    col = -np.abs(E[:, 0])                    # every logit negative ...
    col[prompt] = E[prompt, 0]                # ... the prompt's rows untouched (negative)
    free = np.setdiff1d(np.arange(m.vocab), prompt)
    V = m.vocab
    if case == "ties":
        rows = [r for r in (777, 20011, 33333, V - 2) if r in free]
        col[rows] = 8.0                       # equal maxima in different blocks
        want = rows[0]
    elif case == "zeros":
        rows = [r for r in (4099, 4100, 45000) if r in free]
        col[rows[0]] = -0.0                   # -0 first: it ties +0 and has the lower index
        col[rows[1]] = 0.0
        col[rows[2]] = 0.0
        col[[r for r in (0, 1, 4098, V - 1) if r in free]] = -np.inf
        want = rows[0]
    elif case == "last":
        rows = [V - 1]
        col[0] = -np.inf
        col[V - 1] = 8.0
        want = V - 1
    else:
        raise ValueError(case)
    Eb = ck["model.embed_tokens.weight"][1].copy()
    Eb[:, 0] = _bits(col)
    ck["model.embed_tokens.weight"] = ("bf16", Eb)
    return ck, prompt, want, rows


@pytest.mark.parametrize("case", ["ties", "zeros", "last"])
@pytest.mark.parametrize("prec_name", ["exact", "fast"])
def test_fused_lm_head_argmax_on_crafted_logits(case, prec_name):
    import torch
    from gqa_decoder_transformer_amd import binding as B
    m = CRAFT
    ck, prompt, want, rows = _crafted(case)
    om = O.OracleModel(m, ck)
    ref = om.forward_sequence(prompt)
    assert int(np.argmax(ref)) == want, "construction"
    # a decode token (from the prompt's rows) after which the crafted maximum still wins
    feed = None
    for t in prompt:
        ids, lg = O.generate(om, prompt, 1, pick=lambda k, x, t=t: int(t))
        if int(np.argmax(lg[1])) == want and lg[1][want] >= 0:
            feed, ref1 = int(t), lg[1]
            break
    assert feed is not None, "construction: no decode token keeps the crafted maximum"
    prec = B.EXACT if prec_name == "exact" else B.FAST
    cfg = B.make_config(m, precision=prec, max_batch=1, max_seq=16, max_tokens=16)
    eng = B.Engine(cfg, ck, poison=True)
    say(f"crafted LM head {case} {prec_name}: want {want}, rows {rows}")
    nxt, _ = eng.prefill(prompt[None])
    g0 = eng.logits(1).cpu().numpy()[0]
    cur = torch.tensor([feed], dtype=torch.int32, device=eng.device)
    out = torch.empty_like(cur)
    eng.decode_step(cur, len(prompt), out)
    g1 = eng.logits(1).cpu().numpy()[0]
    eng.sync()
    for step, (gid, g, o) in enumerate(((int(nxt.item()), g0, ref), (int(out.item()), g1, ref1))):
        assert gid == want, (step, gid, want)
        assert gid == int(np.argmax(g))                        # np.argmax of its own logits
        assert len(set(g[rows].tolist())) == 1 or case == "zeros"
        if case == "zeros":
            assert (g[rows] == 0).all()
        neg_inf = np.isneginf(o)
        assert np.array_equal(np.isneginf(g), neg_inf)
        fin = np.isfinite(o)
        tol = 1e-4 if prec == B.EXACT else 2e-2
        assert np.abs(g[fin] - o[fin]).max() <= tol * np.abs(o[fin]).max()
    eng.close()


WIDEN = W.shrink_model(LLAMA_SMALL, name="llama-widen", vocab=65536, layers=1, rms_eps=0.0)


@pytest.mark.parametrize("prec_name", ["exact", "fast"])
def test_bf16_widening_of_every_bit_pattern_through_the_lm_head(prec_name):
    """Column 0 of the tied embedding holds all 65 536 bf16 patterns (row j = pattern j,
    the other columns 0); the output and down projections are zero, so the residual
    stream is the embedding row of the input token 2.0 = 0x4000, i.e. [2, 0, ...]; with
    eps 0 its RMS is 1/4, and the final-norm weight 1/8 e_0 makes h = e_0 exactly. Each
    logit is then the widened weight times 1: the bits `pattern << 16` ("ember
    scripts/reference_forward.py", load_safetensors, BF16 branch), compared bitwise for
    every finite nonzero pattern and every infinity, as zero for +-0 (the sum starts at
    +0), and as NaN for the 254 NaN patterns (which raise the device NaN flag)."""
    import torch
    from gqa_decoder_transformer_amd import binding as B
    m = WIDEN
    ck = W.make_weights(m, 72)
    E = np.zeros((m.vocab, m.hidden), np.uint16)
    E[:, 0] = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ck["model.embed_tokens.weight"] = ("bf16", E)
    for n in list(ck):
        if n.endswith(("o_proj.weight", "down_proj.weight")):
            ck[n] = ("bf16", np.zeros_like(ck[n][1]))
    fn = np.zeros(m.hidden, np.float32)
    fn[0] = 0.125
    ck["model.norm.weight"] = ("bf16", _bits(fn))
    tok = 0x4000
    want = (np.arange(65536, dtype=np.uint32) << np.uint32(16)).view(np.float32)
    nan = np.isnan(want)
    zero = want == 0
    exact = ~nan & ~zero
    assert nan.sum() == 254
    with np.errstate(invalid="ignore"):
        ref = O.OracleModel(m, ck).forward_sequence(np.array([tok]))
    assert np.array_equal(ref[exact].view(np.uint32), want[exact].view(np.uint32))
    prec = B.EXACT if prec_name == "exact" else B.FAST
    cfg = B.make_config(m, precision=prec, max_batch=1, max_seq=4, max_tokens=4)
    eng = B.Engine(cfg, ck, poison=True)
    say(f"widening of all bf16 patterns {prec_name}")
    eng.prefill(np.array([[tok]], np.int32))
    g0 = eng.logits(1).cpu().numpy()[0]
    with pytest.raises(B.EmberError) as e:
        eng.sync()
    assert e.value.status == 10                      # NaN logits raise the device flag
    cur = torch.tensor([tok], dtype=torch.int32, device=eng.device)
    eng.decode_step(cur, 1, torch.empty_like(cur))
    g1 = eng.logits(1).cpu().numpy()[0]
    with pytest.raises(B.EmberError):
        eng.sync()
    eng.close()
    for g in (g0, g1):
        bad = np.nonzero(g[exact].view(np.uint32) != want[exact].view(np.uint32))[0]
        assert bad.size == 0, [hex(int(p)) for p in np.nonzero(exact)[0][bad][:8]]
        assert (g[zero] == 0).all()
        assert np.isnan(g[nan]).all()
