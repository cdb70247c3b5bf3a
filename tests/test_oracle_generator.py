"""Pins of the oracle's generator frame (the delayed-code ring of the "One exact generator
step" passage): output alignment by stream delay, the temporal input each step reads,
supplied codes overriding selections, provided flags cleared after use, and the
greedy special case against the independently pinned temporal and depth oracles."""

import numpy as np
import pytest

from oracle import depformer as OD
from oracle import generator as OG
from oracle import temporal as OT
from oracle.sampling import sample_top_k
from personaplex_temporal_transformer_amd import synth

DELAY = np.array(OG.DELAYS)


_WEIGHTS = []


def make_weights():
    """The tiny temporal and depth weights the generator pins run on (built once)."""
    if not _WEIGHTS:
        ct = synth.TINY_TEMPORAL
        cd = synth.TINY_DEPTH
        _WEIGHTS.append((synth.temporal_weights(ct, 3, "fp32"), ct, synth.depth_weights(cd, 4, "fp32"), cd))
    return _WEIGHTS[0]


@pytest.fixture(scope="module")
def weights():
    return make_weights()


def _codes(g, n):
    c = np.empty((n, 17), np.int64)
    c[:, 0] = g.integers(0, 32000, n)
    c[:, 1:] = g.integers(0, 2048, (n, 16))
    return c


def test_first_model_step_reads_the_initial_tokens(weights):
    """Nothing supplied: the first call only primes the ring; the second (the first model
    step) feeds the temporal step the initial tokens -- text 32000, every audio stream
    2048 -- and a code supplied at the first call replaces its stream's initial token."""
    W_t, ct, W_d, cd = weights
    g = OG.Generator(W_t, ct, W_d, cd)
    assert g.step() is None
    g.step(uniforms=np.zeros(17))
    assert g.last_inputs.tolist() == [32000] + [2048] * 16
    g2 = OG.Generator(W_t, ct, W_d, cd)
    sup = np.full(17, -1)
    sup[9] = 77                       # user codebook 0, delay 0: slot 0 at the first call
    assert g2.step(provided=sup) is None
    g2.step(uniforms=np.zeros(17))
    assert g2.last_inputs.tolist() == [32000] + [2048] * 8 + [77] + [2048] * 7


def test_delay_table():
    assert OG.DELAYS[0] == 0 and OG.DELAYS[1] == 0 and OG.DELAYS[9] == 0
    assert all(OG.DELAYS[k] == 1 for k in list(range(2, 9)) + list(range(10, 17)))
    assert OG.MAX_DELAY == max(OG.DELAYS) == 1 and OG.RING == OG.MAX_DELAY + 3


def test_all_supplied_output_is_previous_call_and_inputs_are_delayed(weights):
    """Every stream supplied at every call: the aligned output of call s is exactly what
    was supplied at call s-1, whatever the stream's delay; the temporal input of call s holds, for delay-0 streams, the
    codes of call s-1 and, for delay-1 streams, those of call s-2 (initial tokens before
    the first call)."""
    W_t, ct, W_d, cd = weights
    gen = OG.Generator(W_t, ct, W_d, cd)
    g = np.random.default_rng(5)
    sup = _codes(g, 7)
    init = np.array([OG.TEXT_INITIAL] + [OG.AUDIO_INITIAL] * 16)
    u = g.random((7, 17))
    for s in range(7):
        out = gen.step(sup[s], u[s])
        if s == 0:
            assert out is None
            continue
        want_in = np.where(DELAY == 0, sup[s - 1], sup[s - 2] if s >= 2 else init)
        assert np.array_equal(gen.last_inputs, want_in), s
        # a delay-d code supplied at call s lands in the target slice of call s + d
        assert np.array_equal(gen.last_chosen, np.where(DELAY == 0, sup[s], sup[s - 1])), s
        if s == 1:
            assert out is None
        else:
            assert np.array_equal(out, sup[s - 1]), s
        assert not gen.prov[:, (s - 1) % 4].any()             # consumed flags cleared


def test_agent_streams_sampled_and_aligned(weights):
    """Only the user streams supplied: agent delay-0 outputs at call s are the selections
    of call s-1, agent delay-1 outputs those of call s; user outputs echo the supplied
    codes with the same alignment. Each selection is the sampler's draw on the logits
    its position produced, unless supplied."""
    W_t, ct, W_d, cd = weights
    gen = OG.Generator(W_t, ct, W_d, cd)
    g = np.random.default_rng(6)
    n = 6
    user = _codes(g, n)
    user[:, :9] = -1
    u = g.random((n, 17))
    chosen = {}
    for s in range(n):
        out = gen.step(user[s], u[s])
        if s == 0:
            continue
        chosen[s] = gen.last_chosen.copy()
        # user stream 9 (delay 0) is supplied into this call's target; 10..16 came last call
        assert chosen[s][9] == user[s][9]
        assert np.array_equal(chosen[s][10:], user[s - 1][10:])
        # the selections re-derived from the sampler on the same logits
        assert chosen[s][0] == sample_top_k(gen.last_text_logits, 0.7, 25, u[s][0])
        _, lg = OD.step_logits(gen.last_h, chosen[s][0], chosen[s][1:], W_d, cd)
        for q in range(16):
            k = q + 1
            if k >= 9:
                continue
            assert chosen[s][k] == sample_top_k(lg[q], 0.8, 250, u[s][k]), (s, k)
        if s >= 2:
            for k in range(17):
                src = chosen[s - 1][k] if DELAY[k] == 0 else chosen[s][k]
                assert out[k] == src, (s, k)


def test_greedy_generator_equals_temporal_then_depth(weights):
    """top_k = 1 for text and audio turns both samplers into argmax: the generator's
    selections must then equal an incremental temporal decode of its own inputs followed
    by the greedy depth loop -- two separately pinned oracles."""
    W_t, ct, W_d, cd = weights
    gen = OG.Generator(W_t, ct, W_d, cd, text_top_k=1, audio_top_k=1)
    g = np.random.default_rng(7)
    n = 4
    user = _codes(g, n)
    user[:, :9] = -1
    inputs, picks = [], []
    for s in range(n):
        gen.step(user[s], g.random(17))
        if s:
            inputs.append(gen.last_inputs.copy())
            picks.append(gen.last_chosen.copy())
    hs, lg = OT.decode_incremental(np.array(inputs), W_t, ct, with_logits=True)
    for t in range(n - 1):
        text = int(np.argmax(lg[t]))
        assert picks[t][0] == text
        forced = np.full(16, -1)
        forced[8] = picks[t][9]                              # supplied user codebook 0
        forced[9:] = picks[t][10:]                           # supplied user codebooks 1..7
        assert np.array_equal(picks[t][9:], np.concatenate([user[t + 1][9:10], user[t][10:]]))
        codes, _ = OD.step_logits(hs[t], text, forced, W_d, cd)
        assert np.array_equal(picks[t][1:], codes), t


def test_supplied_text_conditions_depth(weights):
    """A supplied agent-text code replaces the sampled text in the depth conditioning
    (greedy depth so the effect is checked exactly)."""
    W_t, ct, W_d, cd = weights
    gen = OG.Generator(W_t, ct, W_d, cd, audio_top_k=1)
    gen.step(None, None)
    sup = np.full(17, -1)
    sup[0] = 4242
    gen.step(sup, np.zeros(17))
    assert gen.last_chosen[0] == 4242
    codes, _ = OD.step_logits(gen.last_h, 4242, None, W_d, cd)
    assert np.array_equal(gen.last_chosen[1:], codes)
    # the initial tokens fill the first slot; the first model step reads them
    assert np.array_equal(gen.last_inputs, [OG.TEXT_INITIAL] + [OG.AUDIO_INITIAL] * 16)
