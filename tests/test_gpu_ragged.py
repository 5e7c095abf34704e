"""GPU parity of ragged batches through the C ABI: rows with their own prompt lengths,
start positions and decode positions ("ember internals", "ForwardModel trait":
forward_with_cache(token_ids, cache, start_pos) per sequence), against the oracle run
row by row."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from oracle import sampler as S
from tests.gpu_util import TOL_EXACT, TOL_FAST, check_greedy, rel_maxabs, say
from tests.small_models import LLAMA_HD64, LLAMA_SMALL, QWEN_HD64_G7, QWEN_SMALL_Q8

pytestmark = pytest.mark.gpu


def _engine(model, ck, precision, max_batch, max_seq, stream=None):
    from gqa_decoder_transformer_amd import binding as B
    cfg = B.make_config(model, precision=precision, max_batch=max_batch, max_seq=max_seq,
                        max_tokens=max_batch * max_seq)
    return B.Engine(cfg, ck, stream=stream, poison=True)


def _ragged_generate(eng, rows, n, starts=None, feed=None):
    """Ragged prefill, then n steps, row r at position len_r + start_r + k. Returns
    (ids [n + 1, B], logits [n + 1, B, V])."""
    import torch
    Bn = len(rows)
    starts = [0] * Bn if starts is None else starts
    nxt = eng.prefill_rows(rows, starts)
    ids, logs = [nxt.clone()], [eng.logits(Bn)]
    for k in range(n):
        pos = [starts[r] + len(rows[r]) + k for r in range(Bn)]
        cur = (torch.from_numpy(np.ascontiguousarray(feed[k], np.int32)).to(eng.device)
               if feed is not None else ids[-1].clone())
        out = torch.empty_like(cur)
        eng.decode_step_rows(cur, pos, out)
        ids.append(out)
        logs.append(eng.logits(Bn))
    eng.sync()
    return torch.stack(ids).cpu().numpy(), torch.stack(logs).float().cpu().numpy()


@pytest.mark.parametrize("model", [LLAMA_SMALL, LLAMA_HD64, QWEN_HD64_G7, QWEN_SMALL_Q8],
                         ids=lambda m: m.name)
@pytest.mark.parametrize("mode", ["graph", "direct"])
def test_ragged_prefill_and_decode_exact(model, mode):
    import torch
    from gqa_decoder_transformer_amd import binding as B
    ck = W.make_weights(model, 31)
    lens, N = [9, 20, 13], 8
    rng = np.random.default_rng(32)
    rows = [rng.integers(0, model.vocab, n).astype(np.int32) for n in lens]
    say(f"ragged {model.name} lens={lens} N={N} {mode}")
    # a side stream replays the step graph; the default stream launches directly
    stream = torch.cuda.Stream() if mode == "graph" else torch.cuda.current_stream()
    with torch.cuda.stream(stream):
        eng = _engine(model, ck, B.EXACT, len(rows), 48, stream=stream)
        g_ids, g_logits = _ragged_generate(eng, rows, N)
    torch.cuda.synchronize()
    om = O.OracleModel(model, ck)
    for r, row in enumerate(rows):
        or_ids, or_logits = O.generate(om, row, N)
        div = check_greedy(g_ids[:, r], or_ids, or_logits, TOL_EXACT)
        upto = N + 1 if div is None else div + 1
        err = rel_maxabs(g_logits[:upto, r], or_logits[:upto])
        say(f"row {r}: max rel err {err.max():.3g}")
        assert err.max() < TOL_EXACT, err


def test_ragged_fast_teacher_forced():
    from gqa_decoder_transformer_amd import binding as B
    model = LLAMA_HD64
    ck = W.make_weights(model, 33)
    lens, N = [5, 17, 11, 2], 6
    rng = np.random.default_rng(34)
    rows = [rng.integers(0, model.vocab, n).astype(np.int32) for n in lens]
    om = O.OracleModel(model, ck)
    orc = [O.generate(om, row, N) for row in rows]
    feed = np.stack([ids[:N] for ids, _ in orc], 1)
    eng = _engine(model, ck, B.FAST, len(rows), 32)
    _, g_logits = _ragged_generate(eng, rows, N, feed=feed)
    for r in range(len(rows)):
        err = rel_maxabs(g_logits[:, r], orc[r][1])
        say(f"row {r}: max rel err {err.max():.3g}")
        assert err.max() < TOL_FAST


def test_rows_continue_from_different_cached_lengths():
    """A uniform prefill, then a ragged continuation (each row from its own cached
    length), then ragged decode: equal to the oracle on the concatenated prompts."""
    import torch
    from gqa_decoder_transformer_amd import binding as B
    model = LLAMA_SMALL
    ck = W.make_weights(model, 35)
    rng = np.random.default_rng(36)
    head = rng.integers(0, model.vocab, (2, 10)).astype(np.int32)
    tails = [rng.integers(0, model.vocab, n).astype(np.int32) for n in (5, 12)]
    N = 6
    eng = _engine(model, ck, B.EXACT, 2, 40)
    eng.prefill(head)
    g_ids, g_logits = _ragged_generate(eng, tails, N, starts=[10, 10])
    om = O.OracleModel(model, ck)
    for r in range(2):
        full = np.concatenate([head[r], tails[r]])
        or_ids, or_logits = O.generate(om, full, N)
        div = check_greedy(g_ids[:, r], or_ids, or_logits, TOL_EXACT)
        upto = N + 1 if div is None else div + 1
        assert rel_maxabs(g_logits[:upto, r], or_logits[:upto]).max() < TOL_EXACT
    torch.cuda.synchronize()


def test_ragged_sampled_draws_use_each_rows_position():
    """With a sampler set, row r's draw at a step reads u[pos_r, r]: the GPU's tokens
    (teacher-forced with the oracle's draws) match the oracle's sampler on its own
    logits."""
    import torch
    from gqa_decoder_transformer_amd import binding as B
    from tests.test_gpu_sampler import candidates
    model = LLAMA_SMALL
    ck = W.make_weights(model, 37)
    t, k, p = 1.0, 0, 1.0
    e_t, e_a = ck["model.embed_tokens.weight"]
    ck["model.embed_tokens.weight"] = (e_t, W.f32_to_bf16_bits(O.widen_bf16(e_a) * np.float32(25.0)))
    lens, N = [7, 15, 3], 6
    rng = np.random.default_rng(38)
    rows = [rng.integers(0, model.vocab, n).astype(np.int32) for n in lens]
    U = W.make_uniforms(39, 40, len(rows))
    om = O.OracleModel(model, ck)
    orc = []
    for r, row in enumerate(rows):
        T = len(row)
        orc.append(O.generate(om, row, N,
                              pick=lambda s, lg, T=T, r=r: S.sample(lg, t, k, p, float(U[T - 1 + s, r]))))
    feed = np.stack([ids[:N] for ids, _ in orc], 1)
    eng = _engine(model, ck, B.EXACT, len(rows), 40)
    eng.set_sampler(t, k, p, torch.from_numpy(U).cuda())
    g_ids, _ = _ragged_generate(eng, rows, N, feed=feed)
    off = 0
    for r in range(len(rows)):
        or_ids, or_logits = orc[r]
        T = len(rows[r])
        for s in range(N + 1):
            if int(g_ids[s, r]) == int(or_ids[s]):
                continue
            off += 1
            d = 4.0 * TOL_EXACT * float(np.abs(or_logits[s]).max()) / t + 2e-5
            assert int(g_ids[s, r]) in candidates(or_logits[s], t, k, p, float(U[T - 1 + s, r]), d, d)
    say(f"{off} of {len(rows) * (N + 1)} draws differ within the candidates")
    assert off <= 2


def test_ragged_errors():
    import torch
    from gqa_decoder_transformer_amd import binding as B
    model = LLAMA_SMALL
    eng = _engine(model, W.make_weights(model, 40), B.EXACT, 2, 16)
    rows = [np.zeros(4, np.int32), np.zeros(6, np.int32)]
    with pytest.raises(B.EmberError) as e:
        eng.prefill_rows(rows, [0, 2])                       # row 1 would leave a gap
    assert e.value.status == 8
    with pytest.raises(B.EmberError) as e:
        eng.prefill_rows([np.zeros(4, np.int32), np.zeros(17, np.int32)])
    assert e.value.status == 7                               # past max_seq
    eng.prefill_rows(rows)
    ids = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(B.EmberError) as e:
        eng.decode_step_rows(ids, [4, 7])                    # row 1 has 6 positions
    assert e.value.status == 8
    with pytest.raises(B.EmberError) as e:
        eng.decode_step_rows(ids, [4, 16])
    assert e.value.status == 7
    eng.decode_step_rows(ids, [4, 6])
    eng.sync()
