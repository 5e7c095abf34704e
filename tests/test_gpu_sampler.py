"""GPU parity of the sampler ("ember internals" page, section "sampler") through the C ABI
against the oracle's sampler, on the same seeded logits and draws.

The drawn token depends on where u falls among the running sums; both sides compute those
sums in f32 in different orders (and, in the forward-pass cases, from logits that differ
within the EXACT tier). A token that differs from the oracle's is accepted only when its
interval of the float64 running sum lies within a small distance of u (the
"candidates"); peaked distributions leave a single candidate."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from oracle import rng as R
from oracle import sampler as S
from tests.gpu_util import TOL_EXACT, gpu_generate, say
from tests.small_models import LLAMA_SMALL, QWEN_SMALL
from workloads import configs as C

pytestmark = pytest.mark.gpu

# the Qwen2.5 vocabulary over a one-layer body: the sampler's passes at full width
BIGV = C.shrink_model(C.QWEN05B, name="qwen-vocab", vocab=151936, hidden=64, layers=1,
                      heads=4, kv_heads=2, head_dim=16, ffn=96)
ONE_BELOW_1 = float(np.nextafter(np.float32(1.0), np.float32(0.0)))


def _dist64(z, t, k, p):
    """The final distribution in float64 after the oracle's temperature and top-k (exact:
    no sums), with the temporary softmax, the nucleus cutoff and the final softmax taken
    in float64."""
    x = S.top_k_mask(S.apply_temperature(z, t), k).astype(np.float64)
    if np.isneginf(x).all():
        return np.full(x.size, 1.0 / x.size)
    e = np.exp(x - x.max())
    if 0.0 < p < 1.0:
        soft = e / e.sum()
        desc = np.sort(soft)[::-1]
        over = np.nonzero(np.cumsum(desc) > p)[0]
        cut = desc[over[0]] if over.size else desc[-1]
        e = np.where(soft < cut, 0.0, e)
    return e / e.sum()


def candidates(z, t, k, p, r, dr, dp):
    """Tokens whose interval of the float64 running sum contains a draw within dr of r,
    under the float64 distribution and the oracle's f32 one, for top-p in {p - dp, p,
    p + dp}; plus the oracle's own token. (The oracle's sequential f32 sums drift on flat
    rows: over ~10^5 nearly equal terms every add rounds the same way.)"""
    out = {S.sample(z, t, k, p, r)}
    ps = [p - dp, p, p + dp] if 0.0 < p < 1.0 else [p]
    for pp in ps:
        for dist in (_dist64(z, t, k, pp), S.final_distribution(z, t, k, pp).astype(np.float64)):
            dist = dist / dist.sum()
            hi = np.cumsum(dist)
            lo = hi - dist
            out.update(np.nonzero((dist > 0) & (hi >= r - dr) & (lo <= r + dr))[0].tolist())
    return out


def _engine(model, max_batch=1, max_seq=64, seed=21, stream=None, scale_embed=None):
    from gqa_decoder_transformer_amd import binding as B
    ck = W.make_weights(model, seed)
    if scale_embed is not None:
        t, a = ck["model.embed_tokens.weight"]
        a = W.f32_to_bf16_bits(O.widen_bf16(a) * np.float32(scale_embed)) if t == "bf16" else a * np.float32(scale_embed)
        ck["model.embed_tokens.weight"] = (t, a)
    cfg = B.make_config(model, precision=B.EXACT, max_batch=max_batch, max_seq=max_seq,
                        max_tokens=max_batch * max_seq)
    return B.Engine(cfg, ck, stream=stream, poison=True), ck


SETTINGS = [(1.0, 0, 1.0), (0.7, 50, 1.0), (1.0, 0, 0.9), (0.8, 50, 0.9), (1.3, 1000, 0.95),
            (1.0, 1, 1.0), (1.0, -1, 1.0), (1.0, -2, 0.5), (1.0, 0, 1e-6), (0.01, 0, 1.0),
            (1e4, 0, 1.0), (0.9, 20, 0.8)]


@pytest.fixture(scope="module")
def bigv():
    eng, _ = _engine(BIGV, max_batch=8, max_seq=16)
    return eng


@pytest.mark.parametrize("setting", SETTINGS, ids=lambda s: f"t{s[0]}-k{s[1]}-p{s[2]}")
def test_sample_full_vocabulary_matches_oracle(bigv, setting):
    import torch
    t, k, p = setting
    V = BIGV.vocab
    k = {-1: V - 1, -2: V}.get(k, k)                 # V - 1, and V (stage off)
    rows = 8
    ties = setting == SETTINGS[-1]
    logits = W.make_logits(100 + SETTINGS.index(setting), rows, V, ties=ties)
    U = W.make_uniforms(200 + SETTINGS.index(setting), 4, rows)
    U[3, 0], U[3, 1] = 0.0, ONE_BELOW_1               # extreme draws
    say(f"sampler V={V} rows={rows} t={t} k={k} p={p} ties={ties}")
    d_u = torch.from_numpy(U).cuda()
    bigv.set_sampler(t, k, p, d_u)
    d_l = torch.from_numpy(logits).cuda()
    got = []
    for pos in range(4):
        got.append(bigv.sample(d_l, pos).cpu().numpy())
    bigv.sync()
    bigv.set_sampler()
    off = 0
    for pos in range(4):
        want = S.sample_rows(logits, t, k, p, U[pos])
        for r in range(rows):
            if got[pos][r] != want[r]:
                off += 1
                cand = candidates(logits[r], t, k, p, float(U[pos, r]), 2e-5, 2e-5)
                assert got[pos][r] in cand, (pos, r, got[pos][r], want[r], sorted(cand)[:10])
    say(f"{off} of {4 * rows} draws differ from the f32 oracle, all within the candidates")


SEED = 0x9E3779B97F4A7C15              # both 32-bit key words nonzero


@pytest.mark.parametrize("setting", [(1.0, 0, 1.0), (0.8, 50, 0.9), (1e4, 0, 1.0)],
                         ids=["plain", "k50-p0.9", "flat"])
def test_sample_on_device_draws_match_oracle_generator(bigv, setting):
    """No draws passed: the sampler generates u on the device (Philox4x32-10 at counter
    (position, row), key = the seed). The oracle's generator, written independently from
    the published definition and pinned by its known-answer vectors, supplies the same
    u to the oracle's sampler. At t = 1e4 the distribution is nearly flat, so the token
    is a direct function of u (a wrong draw moves it)."""
    import torch
    t, k, p = setting
    V = BIGV.vocab
    rows = 8
    logits = W.make_logits(300 + int(t * 10) % 97, rows, V)
    d_l = torch.from_numpy(logits).cuda()
    bigv.set_sampler(t, k, p, seed=SEED)
    off = 0
    for pos in (0, 7, 4095, 70000):
        got = bigv.sample(d_l, pos).cpu().numpy()
        u = R.uniform(SEED, pos, np.arange(rows))
        want = S.sample_rows(logits, t, k, p, u)
        for r in range(rows):
            if got[r] != want[r]:
                off += 1
                cand = candidates(logits[r], t, k, p, float(u[r]), 2e-5, 2e-5)
                assert got[r] in cand, (pos, r, got[r], want[r])
    bigv.sync()
    bigv.set_sampler()
    say(f"on-device draws {setting}: {off} of {4 * rows} differ from the f32 oracle, within the candidates")


def test_sample_masked_and_uniform_rows(bigv):
    """A row of -inf only is drawn uniformly; a row with most tokens at -inf never draws
    one of them; temperature 0 is the greedy argmax (lowest index of the maximum)."""
    import torch
    V = BIGV.vocab
    rng = np.random.default_rng(7)
    logits = np.full((3, V), -np.inf, np.float32)
    live = rng.choice(V, 40, replace=False)
    logits[1, live] = rng.standard_normal(40).astype(np.float32)
    logits[2] = np.round(rng.standard_normal(V) * 2).astype(np.float32)   # many tied maxima
    U = np.array([[0.5, 0.3, 0.9], [0.0, ONE_BELOW_1, 0.123]], np.float32)
    d_u = torch.from_numpy(U).cuda()
    d_l = torch.from_numpy(logits).cuda()
    for t, k, p in [(1.0, 0, 1.0), (0.5, 10, 0.7), (2.0, 0, 0.3)]:
        bigv.set_sampler(t, k, p, d_u)
        for pos in range(2):
            got = bigv.sample(d_l, pos).cpu().numpy()
            want = S.sample_rows(logits, t, k, p, U[pos])
            say(f"masked rows t={t} k={k} p={p} pos={pos}: {got} vs {want}")
            assert got[1] in set(live.tolist())
            for r in range(3):
                if got[r] != want[r]:
                    assert got[r] in candidates(logits[r], t, k, p, float(U[pos, r]), 2e-5, 2e-5)
    bigv.set_sampler()
    got = bigv.sample(d_l, 0).cpu().numpy()
    assert got[2] == int(np.argmax(logits[2]))
    assert got[1] == int(live[np.argmax(logits[1, live])])
    bigv.sync()


def test_sampler_arguments_are_validated(bigv):
    import torch
    from gqa_decoder_transformer_amd import binding as B
    d_u = torch.rand((4, 2), device="cuda")
    for bad in [dict(temperature=-1.0), dict(temperature=float("nan")), dict(top_k=-3),
                dict(top_p=float("inf"))]:
        kw = dict(temperature=1.0, top_k=0, top_p=1.0)
        kw.update(bad)
        with pytest.raises(B.EmberError) as e:
            bigv.set_sampler(kw["temperature"], kw["top_k"], kw["top_p"], d_u)
        assert e.value.status == 1
    bigv.set_sampler(1.0, 0, 1.0, d_u)
    d_l = torch.zeros((3, BIGV.vocab), device="cuda")
    with pytest.raises(B.EmberError) as e:
        bigv.sample(d_l, 0)                          # 3 rows > ld 2
    assert e.value.status == 7
    with pytest.raises(B.EmberError) as e:
        bigv.sample(torch.zeros((9, BIGV.vocab), device="cuda"), 0)   # 9 rows > max_batch 8
    assert e.value.status == 7
    with pytest.raises(B.EmberError) as e:
        bigv.sample(d_l[:2], 4)                      # draw row 4 of 4
    assert e.value.status == 7
    bigv.set_sampler()


def _oracle_sampled(om, prompt_row, n, t, k, p, U, col):
    T = len(prompt_row)
    return O.generate(om, prompt_row, n,
                      pick=lambda s, lg: S.sample(lg, t, k, p, float(U[T - 1 + s, col])))


def _check_forward_draws(g_ids, or_ids, or_logits, t, k, p, U, T, col):
    """Step-by-step comparison of the GPU's draws (teacher-forced with the oracle's tokens)
    with the oracle's; a difference must lie within the candidates the logits' EXACT
    tolerance allows. Returns the number of differing steps."""
    off = 0
    for s in range(len(or_ids)):
        if int(g_ids[s]) == int(or_ids[s]):
            continue
        off += 1
        lg = or_logits[s]
        eps = TOL_EXACT * float(np.abs(lg).max())
        d = 4.0 * eps / t + 2e-5
        cand = candidates(lg, t, k, p, float(U[T - 1 + s, col]), d, d)
        if 0 < k < lg.size:                          # near-tie at the k-th largest
            zs = np.sort(lg.astype(np.float64))[::-1]
            if zs[k - 1] - zs[k] <= 2 * eps:
                for kk in (k - 1, k + 1):
                    cand |= candidates(lg, t, kk, p, float(U[T - 1 + s, col]), d, d)
        assert int(g_ids[s]) in cand, (s, int(g_ids[s]), int(or_ids[s]))
    return off


@pytest.mark.parametrize("model,batch,scale", [(QWEN_SMALL, 1, None), (QWEN_SMALL, 1, 25.0),
                                               (LLAMA_SMALL, 3, 25.0)],
                         ids=["qwen-b1-init", "qwen-b1-peaked", "llama-b3-peaked"])
@pytest.mark.parametrize("setting", [(1.0, 0, 1.0), (0.8, 20, 0.9)], ids=["plain", "k20-p0.9"])
@pytest.mark.parametrize("draws", ["array", "philox"])
def test_prefill_and_decode_draws_match_oracle(model, batch, scale, setting, draws):
    """The forward pass with a sampler set: the prefill's draw (row T - 1) and every decode
    step's draw (row pos), batch row b reading column b (or, with on-device draws, the
    generator at counter (pos, b)); decode steps on a side stream, so that they are
    replayed from the step graph."""
    import torch
    t, k, p = setting
    T, N = 13, 10
    prompt = np.random.default_rng(31).integers(0, model.vocab, (batch, T)).astype(np.int32)
    if draws == "array":
        U = W.make_uniforms(41, T + N, batch + 1)
    else:
        pos, col = np.meshgrid(np.arange(T + N), np.arange(batch + 1), indexing="ij")
        U = R.uniform(SEED, pos, col)
    say(f"forward draws {model.name} B={batch} scale={scale} t={t} k={k} p={p}")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        eng, ck = _engine(model, max_batch=batch, max_seq=32, seed=23, stream=s, scale_embed=scale)
        om = O.OracleModel(model, ck)
        orc = [_oracle_sampled(om, prompt[b], N, t, k, p, U, b) for b in range(batch)]
        feed = np.stack([ids[:N] for ids, _ in orc], 1)      # [N, batch]
        if draws == "array":
            eng.set_sampler(t, k, p, torch.from_numpy(U).cuda())
        else:
            eng.set_sampler(t, k, p, seed=SEED)
        g_ids, _ = gpu_generate(eng, prompt, N, feed=feed)
        eng.set_sampler()
    torch.cuda.synchronize()
    total = sum(_check_forward_draws(g_ids[:, b], orc[b][0], orc[b][1], t, k, p, U, T, b)
                for b in range(batch))
    say(f"{total} of {batch * (N + 1)} draws differ within the candidates")
    assert total <= max(1, batch * (N + 1) // 10)


def test_greedy_after_sampler_cleared_and_graph_recaptured():
    """Greedy, then a sampler, then greedy again on one engine and one side stream: the
    step graph is captured again at each change, and the greedy ids are the argmax of
    the logits the same steps write."""
    import torch
    model = QWEN_SMALL
    T, N = 9, 6
    prompt = np.random.default_rng(33).integers(0, model.vocab, (1, T)).astype(np.int32)
    U = W.make_uniforms(43, T + 3 * N, 1)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        eng, _ = _engine(model, max_seq=48, seed=24, stream=s, scale_embed=25.0)
        nxt, _ = eng.prefill(prompt)
        cur = nxt.clone()
        rec = []
        for phase in range(3):
            if phase == 1:
                eng.set_sampler(1.0, 0, 1.0, torch.from_numpy(U).cuda())
            elif phase == 2:
                eng.set_sampler()
            for j in range(N):
                pos = T + phase * N + j
                out = torch.empty_like(cur)
                eng.decode_step(cur, pos, out)
                rec.append((phase, out.clone(), eng.logits(1)))
                cur = out
        eng.sync()
    torch.cuda.synchronize()
    drawn_differs = 0
    for phase, ids, lg in rec:
        ids, lg = int(ids.cpu()[0]), lg.cpu().numpy()[0]
        if phase != 1:
            assert ids == int(np.argmax(lg))
        else:
            drawn_differs += ids != int(np.argmax(lg))
    say(f"{drawn_differs} of {N} drawn tokens differ from the argmax")
