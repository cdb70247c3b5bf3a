"""GPU parity of the sampler and of the generator frame ("One exact generator step")
against the oracle, through the C ABI.

Sampling decisions are integers decided in float64 from float32 logits; both sides take
them from the same float32 values, so a draw on the GPU's own logits must equal the
oracle sampler's draw exactly. The ring (temporal inputs, supplied-code placement,
output alignment) is integer bookkeeping and must match exactly; logits match the oracle
to the fp32 tolerance."""

import numpy as np
import pytest

from oracle import generator as OG
from oracle.sampling import sample_top_k
from personaplex_temporal_transformer_amd import pp, synth
from tests.helpers import max_abs_err, require_gpu, to_device

pytestmark = pytest.mark.gpu

FP32_TOL = 1e-4


def _gpu_sample(logits, temperature, top_k, u):
    import torch
    require_gpu()
    L = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
    U = torch.from_numpy(np.ascontiguousarray(u, np.float64)).cuda()
    out = torch.empty(L.shape[0], dtype=torch.int32, device="cuda")
    pp.sample_top_k(L, temperature, top_k, U, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check_rows(logits, temperature, top_k, u, label):
    got = _gpu_sample(logits, temperature, top_k, u)
    want = np.array([sample_top_k(logits[r], temperature, top_k, u[r]) for r in range(logits.shape[0])])
    bad = np.nonzero(got != want)[0]
    print("%s: %d rows, %d mismatches" % (label, logits.shape[0], len(bad)))
    assert len(bad) == 0, (label, bad[:5], got[bad[:5]], want[bad[:5]])


@pytest.mark.parametrize("n,k,t", [(2048, 250, 0.8), (32000, 25, 0.7), (1000, 250, 0.8), (5000, 40, 1.3),
                                   (2049, 1024, 0.5), (32768, 1024, 2.0), (2048, 1024, 1.0), (100, 250, 0.8),
                                   (1, 25, 0.7)])
def test_sampler_random_rows(n, k, t):
    g = np.random.default_rng(n + k)
    rows = 48
    logits = (3.0 * g.normal(size=(rows, n))).astype(np.float32)
    u = g.random(rows)
    u[0], u[1] = 0.0, np.nextafter(1.0, 0.0)
    _check_rows(logits, t, k, u, "random n=%d k=%d t=%g" % (n, k, t))


def test_sampler_ties_and_degenerate_rows():
    g = np.random.default_rng(9)
    n, rows = 2048, 40
    # heavy ties: values on a coarse grid, so the top-k cut falls inside a run of equals
    logits = (np.round(g.normal(size=(rows, n)) * 2) / 2).astype(np.float32)
    logits[0] = 0.0                                # all equal: candidates 0..k-1
    logits[1] = -0.0
    logits[2, ::2] = -0.0                          # -0 and +0 are one value
    logits[3, :] = -np.inf
    logits[3, 1500:1510] = 1.0                     # -inf outside the top k
    logits[4, 7] = 5.0                             # single clear maximum
    u = (np.arange(rows) + 0.5) / rows
    for k, t in ((250, 0.8), (25, 0.7), (1, 0.8), (250, 0.0), (2, 1.0)):
        _check_rows(logits, t, k, u, "ties k=%d t=%g" % (k, t))
    got = _gpu_sample(np.zeros((64, 300), np.float32), 1.0, 10, (np.arange(64) + 0.5) / 64)
    assert set(got.tolist()) == set(range(10))


def test_sampler_exact_boundaries():
    """Equal top weights put the threshold u * total exactly on a running sum at u = j / k;
    both sides take the first candidate whose running sum exceeds it strictly."""
    n = 300
    logits = np.full((6, n), -30.0, np.float32)
    logits[:, 10:14] = 0.0                          # four equal top logits, weights 1 each
    u = np.array([0.25, 0.5, 0.75, 0.25 - 2.0 ** -40, 0.0, 0.5 - 2.0 ** -40])
    _check_rows(logits, 1.0, 4, u, "exact boundaries k=4")
    got = _gpu_sample(logits, 1.0, 4, u)
    assert got.tolist() == [11, 12, 13, 10, 10, 11]


def _setup_generator(seed=0, **overrides):
    import torch
    require_gpu()
    ct, cd = synth.TINY_TEMPORAL, synth.TINY_DEPTH
    Wt = synth.temporal_weights(ct, seed, "fp32")
    Wd = synth.depth_weights(cd, seed + 1, "fp32")
    model = pp.TemporalModel(ct, to_device(Wt), "fp32")
    kv = model.kv_alloc()
    dep = pp.Depformer(cd, to_device(Wd), "fp32")
    gen = pp.Generator(model, kv, dep, **overrides)
    bufs = dict(inputs=torch.empty(17, dtype=torch.int32, device="cuda"),
                chosen=torch.empty(17, dtype=torch.int32, device="cuda"),
                text_logits=torch.empty(ct["text_vocab"] - 1, device="cuda"),
                depth_logits=torch.empty((cd["n_steps"], cd["n_out"]), device="cuda"),
                out=torch.empty(17, dtype=torch.int32, device="cuda"))
    return (Wt, ct, Wd, cd), (model, kv, dep, gen), bufs


def _user_codes(g, n, p_text=0.0):
    c = np.full((n, 17), -1, np.int64)
    c[:, 9:] = g.integers(0, 2048, (n, 8))
    sup = g.random(n) < p_text
    c[sup, 0] = g.integers(0, 32000, int(sup.sum()))
    return c


@pytest.mark.parametrize("text_prob", [0.0, 0.5])
def test_generator_tiny_fp32_matches_oracle(text_prob):
    import torch
    (Wt, ct, Wd, cd), (model, kv, dep, gen), b = _setup_generator()
    og = OG.Generator(Wt, ct, Wd, cd)
    g = np.random.default_rng(11)
    n = 9
    prov = _user_codes(g, n, text_prob)
    prov[3, 1:9] = g.integers(0, 2048, 8)          # one call also supplies agent codes
    U = g.random((n, 17))
    worst = 0.0
    for s in range(n):
        has = gen.step(prov[s], U[s], b["out"])
        want_out = og.step(prov[s], U[s])
        torch.cuda.synchronize()
        assert has == (want_out is not None), s
        if s == 0:
            continue
        gen.inspect(b["inputs"], b["chosen"], b["text_logits"], b["depth_logits"])
        torch.cuda.synchronize()
        inputs, chosen = b["inputs"].cpu().numpy(), b["chosen"].cpu().numpy()
        tl, dl = b["text_logits"].cpu().numpy(), b["depth_logits"].cpu().numpy()
        assert np.array_equal(inputs, og.last_inputs), s
        worst = max(worst, max_abs_err(tl, og.last_text_logits), max_abs_err(dl, og.last_depth_logits))
        # every selection: the supplied code, or the draw on the GPU's own logits
        tgt = s % 4
        for k in range(17):
            if og.prov[k, tgt]:
                continue
            want = (sample_top_k(tl, 0.7, 25, U[s][0]) if k == 0
                    else sample_top_k(dl[k - 1], 0.8, 250, U[s][k]))
            assert chosen[k] == want, (s, k)
        assert np.array_equal(chosen, og.last_chosen), s
        if want_out is not None:
            assert np.array_equal(b["out"].cpu().numpy(), want_out), s
    print("generator tiny fp32: %d calls, worst logit err %.3g" % (n, worst))
    assert worst <= FP32_TOL


def test_generator_greedy_and_defaults_validation():
    import torch
    (Wt, ct, Wd, cd), (model, kv, dep, gen), b = _setup_generator(seed=4, text_top_k=1, audio_top_k=1)
    og = OG.Generator(Wt, ct, Wd, cd, text_top_k=1, audio_top_k=1)
    g = np.random.default_rng(12)
    prov = _user_codes(g, 5)
    for s in range(5):
        gen.step(prov[s], g.random(17), b["out"])
        want = og.step(prov[s], None)
        torch.cuda.synchronize()
        if want is not None:
            assert np.array_equal(b["out"].cpu().numpy(), want), s
    with pytest.raises(pp.PPError):
        gen.step(np.full(17, 2048), None, b["out"])        # audio code outside [0, n_out)
    with pytest.raises(pp.PPError):
        gen.step(None, np.full(17, 1.0), b["out"])         # draw outside [0, 1)
    with pytest.raises(pp.PPError):
        pp.Generator(model, kv, dep, delays=(0,) * 16)     # wrong stream count


def test_generator_session_store_and_restore_resume_exactly():
    """A session stored after some calls (the model's ring with pp_kv_store and the
    delayed-code ring with pp_generator_store) and restored later resumes exactly: the same
    supplied codes and draws give the same selections, outputs and logits, bit for bit."""
    import torch
    (Wt, ct, Wd, cd), (model, kv, dep, gen), b = _setup_generator(seed=5)
    g = np.random.default_rng(21)
    n0, n1 = 5, 4
    prov = _user_codes(g, n0 + n1, 0.3)
    U = g.random((n0 + n1, 17))
    for s in range(n0):
        gen.step(prov[s], U[s], b["out"])
    cur, nbytes = gen.info()
    assert cur == n0
    ring = torch.empty(kv.info()[1] // 4, dtype=torch.float32, device="cuda")
    kv.store(ring)
    state = torch.empty((nbytes + 3) // 4, dtype=torch.int32, device="cuda")
    gen.store(state)
    pos = kv.info()[0]
    runs = []
    for rep in range(2):
        if rep == 1:
            kv.restore(ring, pos)
            gen.restore(state, cur)
            assert gen.info()[0] == cur
        got = []
        for s in range(n0, n0 + n1):
            has = gen.step(prov[s], U[s], b["out"])
            gen.inspect(b["inputs"], b["chosen"], b["text_logits"], b["depth_logits"])
            torch.cuda.synchronize()
            got.append((has, b["out"].cpu().numpy().copy() if has else None, b["chosen"].cpu().numpy().copy(),
                        b["text_logits"].cpu().numpy().copy(), b["depth_logits"].cpu().numpy().copy()))
        runs.append(got)
    for a, c in zip(runs[0], runs[1]):
        assert a[0] == c[0]
        for x, y in zip(a[1:], c[1:]):
            assert (x is None and y is None) or np.array_equal(x, y)
