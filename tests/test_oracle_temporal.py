"""Pins of the temporal oracle against closed forms, brute force and invariants.

Each check is written independently of the oracle's own code (scalar loops with
math.*, hand-built weights whose effect is known), so a dropped term, a wrong sign or
index, or a transposed operand in the oracle fails at least one of them."""

import math

import numpy as np
import pytest

from oracle import temporal as O
from personaplex_temporal_transformer_amd import synth


def small_cfg(**kw):
    cfg = dict(n_layers=1, d_model=8, n_heads=2, d_head=4, d_ff=4, context=3000,
               text_vocab=5, audio_vocab=7, n_audio=2, rope_theta=10000.0, eps=1e-8)
    cfg.update(kw)
    return cfg


# --------------------------------------------------------------------------- embedding

def test_embed_minus_one_is_exact_zero():
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 0, "fp32", with_text_head=False, layers=[])
    x = O.embed([-1] * 17, W, cfg)
    assert np.all(x == 0.0)


def test_embed_single_id_is_that_row_and_sum_of_two():
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 0, "bf16", with_text_head=False, layers=[])
    ids = [-1] * 17
    ids[5] = 2048                                 # initial audio ID is a valid row
    row = W["emb.4.weight"][2048]
    x = O.embed(ids, W, cfg)
    widened = (row.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(x, widened)
    ids[0] = 32000                                # initial text ID
    x2 = O.embed(ids, W, cfg)
    t = (W["text_emb.weight"][32000].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(x2, t + widened)


def test_embed_f32_order_is_sequential_float32_sum():
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 3, "bf16", with_text_head=False, layers=[])
    ids = synth.stream_ids(cfg, 1, 9)[0]
    got = O.embed(ids, W, cfg, precision="f32")
    acc = np.zeros(cfg["d_model"], np.float32)
    for k in range(17):
        if ids[k] >= 0:
            tab = W["text_emb.weight"] if k == 0 else W["emb.%d.weight" % (k - 1)]
            acc = acc + synth.bf16_bits_to_f32(tab[ids[k]])
    assert np.array_equal(got, acc)
    assert np.max(np.abs(got - O.embed(ids, W, cfg))) < 1e-6


@pytest.mark.parametrize("bad", [(0, -2), (0, 32001), (3, 2049), (16, -5)])
def test_embed_rejects_invalid_ids(bad):
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 0, "fp32", with_text_head=False, layers=[])
    ids = [0] * 17
    ids[bad[0]] = bad[1]
    with pytest.raises(ValueError):
        O.embed(ids, W, cfg)


# --------------------------------------------------------------------------- pieces

def test_rmsnorm_closed_forms():
    D = 16
    alpha = np.linspace(0.5, 1.5, D)
    for c in (1e-4, 0.3, -2.0):
        got = O.rmsnorm(np.full(D, c), alpha, 1e-8)
        want = [a * c / math.sqrt(c * c + 1e-8) for a in alpha]
        assert np.allclose(got, want, rtol=1e-13, atol=0)
    z = O.rmsnorm(np.zeros(D), alpha, 1e-8)
    assert np.all(z == 0.0)
    v = np.arange(1.0, 5.0)            # mean square = 7.5
    got = O.rmsnorm(v, np.ones(4), 1e-8)
    assert np.allclose(got, v / math.sqrt(7.5 + 1e-8), rtol=1e-14)


def test_rope_inv_freq_closed_form():
    w = O.rope_inv_freq(128, 10000.0)
    assert len(w) == 64
    for j in (0, 1, 17, 63):
        assert abs(w[j] - math.exp(-math.log(10000.0) * 2 * j / 128)) < 1e-16
        assert abs(w[j] - 10000.0 ** (-2 * j / 128)) < 1e-15


def test_rope_adjacent_pairs_and_sign():
    d = 8
    for p in (0, 1, 7, 2999, 3100):
        e1 = np.zeros(d); e1[1] = 1.0            # second coordinate of pair j = 0 (omega = 1)
        out = O.rope(e1, p, 10000.0)
        want = np.zeros(d); want[0] = -math.sin(p); want[1] = math.cos(p)
        assert np.allclose(out, want, atol=1e-12)
        e2 = np.zeros(d); e2[2] = 1.0            # first coordinate of pair j = 1
        a = p * 10000.0 ** (-2 / d)
        out = O.rope(e2, p, 10000.0)
        want = np.zeros(d); want[2] = math.cos(a); want[3] = math.sin(a)
        assert np.allclose(out, want, atol=1e-12)


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(0)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for p in (0, 5, 2999):
        r = O.rope(q, p, 1e4)
        assert np.allclose(r[0::2] ** 2 + r[1::2] ** 2, q[0::2] ** 2 + q[1::2] ** 2)
    base = O.rope(q, 10, 1e4) @ O.rope(k, 3, 1e4)
    for s in (1, 100, 2990):
        assert abs(O.rope(q, 10 + s, 1e4) @ O.rope(k, 3 + s, 1e4) - base) < 1e-9


def _brute_attention(q, k, v, qp, kp, window):
    out = []
    for i in range(len(q)):
        keys = [j for j in range(len(k)) if 0 <= qp[i] - kp[j] < window]
        sc = [sum(q[i][d] * k[j][d] for d in range(len(q[i]))) / math.sqrt(len(q[i])) for j in keys]
        m = max(sc)
        e = [math.exp(s - m) for s in sc]
        tot = sum(e)
        out.append([sum(e[n] * v[j][d] for n, j in enumerate(keys)) / tot for d in range(len(v[0]))])
    return np.array(out)


def test_attention_brute_force():
    rng = np.random.default_rng(1)
    q, k, v = rng.standard_normal((6, 4)), rng.standard_normal((9, 4)), rng.standard_normal((9, 4))
    qp, kp = np.arange(3, 9), np.array([0, 1, 2, 3, 4, 5, 6, 7, 8])
    for window in (1, 3, 4, 3000):
        got = O.attention(q, k, v, qp, kp, window)
        assert np.allclose(got, _brute_attention(q, k, v, qp, kp, window), atol=1e-12)


def test_attention_single_key_returns_value_exactly():
    rng = np.random.default_rng(2)
    q, k, v = rng.standard_normal((1, 8)), rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    assert np.array_equal(O.attention(q, k, v, [5], [5], 3000), v)


def test_swiglu_hand_example():
    gz = np.array([0.0, 1.0, 5.0, 2.0])       # g = [0, 1], z = [5, 2]
    got = O.swiglu(gz, 2)
    assert got[0] == 0.0
    assert abs(got[1] - 1.0 / (1.0 + math.exp(-1.0)) * 2.0) < 1e-15


# --------------------------------------------------------------------------- block structure

def _perm(n, shift):
    P = np.zeros((n, n))
    for i in range(n):
        P[(i + shift) % n, (3 * i + 1) % n] = 1.0
    # a transposed operand must show: odd shifts give an involution (P = P^T) at n = 8
    assert not np.array_equal(P, P.T)
    return P


def test_block_with_hand_built_weights_single_frame():
    """One frame: attention sees one key, so A = V. With V = P_v u, W_O = P_o, W_in
    selecting g_i = 2 v_i and z_i = v_{i+4}, W_out placing silu(g_i) z_i at row
    (i + 1) mod 8, the block output has a closed form computed here with scalar math."""
    cfg = small_cfg()
    D, F = 8, 4
    rng = np.random.default_rng(3)
    Pv, Po = _perm(D, 2), _perm(D, 6)
    Wqkv = np.concatenate([rng.standard_normal((D, D)), rng.standard_normal((D, D)), Pv])
    Win = np.zeros((2 * F, D))
    for i in range(F):
        Win[i, i] = 2.0
        Win[F + i, i + 4] = 1.0
    Wout = np.zeros((D, F))
    for i in range(F):
        Wout[(i + 1) % D, i] = 1.0
    a1, a2 = np.linspace(0.5, 2, D), np.linspace(1.5, 0.7, D)
    W = {"transformer.layers.0.norm1.alpha": a1, "transformer.layers.0.norm2.alpha": a2,
         "transformer.layers.0.self_attn.in_proj_weight": Wqkv,
         "transformer.layers.0.self_attn.out_proj.weight": Po,
         "transformer.layers.0.gating.linear_in.weight": Win,
         "transformer.layers.0.gating.linear_out.weight": Wout}
    x = rng.standard_normal(D)
    got = O.block_full(x[None], np.array([7]), 0, W, cfg)[0]

    rms = math.sqrt(sum(t * t for t in x) / D + 1e-8)
    u = [a1[i] * x[i] / rms for i in range(D)]
    vv = [sum(Pv[i, j] * u[j] for j in range(D)) for i in range(D)]
    y = [x[i] + sum(Po[i, j] * vv[j] for j in range(D)) for i in range(D)]
    rms2 = math.sqrt(sum(t * t for t in y) / D + 1e-8)
    v2 = [a2[i] * y[i] / rms2 for i in range(D)]
    want = list(y)
    for i in range(F):
        g, z = 2.0 * v2[i], v2[i + 4]
        want[(i + 1) % D] += g / (1.0 + math.exp(-g)) * z
    assert np.allclose(got, want, atol=1e-13)


def test_block_window_by_uniform_attention():
    """Q = 0 makes every visible key equally weighted, so the attention output at t is
    the mean of the visible values. With V = u, W_O = I and a zero FFN, the block output
    is x_t + mean{u_j : 0 <= t - j < C}: a closed form that fixes the window (C keys,
    strictly causal) and that V is not rotated."""
    D, C, T = 8, 3, 7
    cfg = small_cfg(context=C)
    rng = np.random.default_rng(4)
    W = {"transformer.layers.0.norm1.alpha": np.ones(D), "transformer.layers.0.norm2.alpha": np.ones(D),
         "transformer.layers.0.self_attn.in_proj_weight":
             np.concatenate([np.zeros((D, D)), rng.standard_normal((D, D)), np.eye(D)]),
         "transformer.layers.0.self_attn.out_proj.weight": np.eye(D),
         "transformer.layers.0.gating.linear_in.weight": np.zeros((8, D)),
         "transformer.layers.0.gating.linear_out.weight": np.zeros((D, 4))}
    X = rng.standard_normal((T, D))
    got = O.block_full(X, np.arange(T) + 11, 0, W, cfg)
    U = [[X[t, i] / math.sqrt(sum(X[t] ** 2) / D + 1e-8) for i in range(D)] for t in range(T)]
    for t in range(T):
        vis = [j for j in range(T) if 0 <= t - j < C]
        want = [X[t, i] + sum(U[j][i] for j in vis) / len(vis) for i in range(D)]
        assert np.allclose(got[t], want, atol=1e-13), t


def test_text_head_orientation():
    cfg = small_cfg()
    D = 8
    Wt = np.zeros((3, D)); Wt[0, 5] = 1.0; Wt[1, 0] = -2.0; Wt[2, 7] = 0.5
    W = {"out_norm.alpha": np.ones(D), "text_linear.weight": Wt}
    x = np.arange(1.0, 9.0)
    h, logits = O.final(x, W, cfg, with_logits=True)
    assert np.allclose(logits, [h[5], -2 * h[0], 0.5 * h[7]], atol=1e-15)


def test_zero_blocks_leave_the_final_norm_of_the_embedding():
    """With every block matrix zero each block is the identity (q = k = v = 0, so the
    attention output is 0; SiLU(0) * 0 = 0), and h is the final RMSNorm of the embedding
    sum on both code paths: a text row holding 3 and 4 in a 256-wide model has
    mean(x^2) = 25 / 256, so h = (3, 4) * 16 / 5 = (9.6, 12.8) with unit scales."""
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 0, "fp32")
    for k in list(W):
        if k.startswith("transformer.layers.") and not k.endswith("alpha"):
            W[k] = np.zeros_like(W[k])
        if k == "text_emb.weight" or k.startswith("emb."):
            W[k] = np.zeros_like(W[k])
    W["text_emb.weight"][5, 0:2] = [3.0, 4.0]
    W["out_norm.alpha"] = np.ones(cfg["d_model"], np.float32)
    ids = np.full((2, 17), -1)
    ids[:, 0] = 5
    want = np.zeros(cfg["d_model"])
    want[0:2] = [9.6, 12.8]
    for h in (O.forward_full(ids, W, cfg), O.decode_incremental(ids, W, cfg)):
        assert np.allclose(h, want[None, :], rtol=1e-6, atol=1e-12)


# --------------------------------------------------------------------------- whole forward

def _tiny():
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 0, "fp32")
    ids = synth.stream_ids(cfg, 16, 1)
    return cfg, W, ids


def test_incremental_equals_full_sequence():
    cfg, W, ids = _tiny()
    full, lf = O.forward_full(ids, W, cfg, with_logits=True)
    inc, li = O.decode_incremental(ids, W, cfg, with_logits=True)
    assert np.max(np.abs(full - inc)) < 1e-12
    assert np.max(np.abs(lf - li)) < 1e-11


def test_incremental_equals_full_with_wrapping_window():
    cfg, W, ids = _tiny()
    cfg = synth.with_(cfg, context=4)
    full = O.forward_full(ids, W, cfg)
    inc = O.decode_incremental(ids, W, cfg)
    assert np.max(np.abs(full - inc)) < 1e-12
    # the window binds: a context of 3000 gives different late outputs
    assert np.max(np.abs(full[8:] - O.forward_full(ids, W, synth.TINY_TEMPORAL)[8:])) > 1e-3


def test_causality_future_frames_do_not_change_past_outputs():
    cfg, W, ids = _tiny()
    base = O.forward_full(ids, W, cfg)
    t0 = 9
    ids2 = ids.copy()
    ids2[t0 + 1:] = synth.stream_ids(cfg, 16 - t0 - 1, 77)
    pert = O.forward_full(ids2, W, cfg)
    assert np.array_equal(base[:t0 + 1], pert[:t0 + 1])
    assert np.max(np.abs(base[t0 + 1:] - pert[t0 + 1:])) > 1e-3


def test_shift_of_all_positions_leaves_outputs_unchanged():
    cfg, W, ids = _tiny()
    a = O.forward_full(ids[:6], W, cfg, p0=0)
    b = O.forward_full(ids[:6], W, cfg, p0=1234)
    assert np.max(np.abs(a - b)) < 1e-9


def _two_frame_qk_setup():
    """A 1-block stack of width 256 = 2 heads x 128 whose projections are built by hand
    (audit section 3, 'One of the 32 temporal blocks': one fused [Q, K, V] projection).

    Head h's query coordinate 0 is 4 u[2h] (Q section, rows h*128) and its key coordinate 0
    is 3 u[2h+1] (K section, rows 256 + h*128); every other query / key coordinate is 0, so
    RoPE rotates only pair 0, whose frequency is 1 for any theta. V = u (V section = I),
    W_O = I and the feed-forward is zero, so the block output is x + A."""
    D, H, dh = 256, 2, 128
    cfg = dict(n_layers=1, d_model=D, n_heads=H, d_head=dh, d_ff=4, context=3000,
               text_vocab=5, audio_vocab=7, n_audio=2, rope_theta=10000.0, eps=1e-8)
    Wqkv = np.zeros((3 * D, D))
    for h in range(H):
        Wqkv[h * dh, 2 * h] = 4.0                 # q_h[0] = 4 u[2h]
        Wqkv[D + h * dh, 2 * h + 1] = 3.0         # k_h[0] = 3 u[2h+1]
    Wqkv[2 * D:] = np.eye(D)
    alpha = np.linspace(0.6, 1.4, D)
    W = {"transformer.layers.0.norm1.alpha": alpha, "transformer.layers.0.norm2.alpha": np.ones(D),
         "transformer.layers.0.self_attn.in_proj_weight": Wqkv,
         "transformer.layers.0.self_attn.out_proj.weight": np.eye(D),
         "transformer.layers.0.gating.linear_in.weight": np.zeros((8, D)),
         "transformer.layers.0.gating.linear_out.weight": np.zeros((D, 4))}
    rng = np.random.default_rng(11)
    X = rng.standard_normal((2, D))
    X[:, :4] = [[1.5, -1.0, 0.8, 1.2], [1.1, 0.9, -1.3, 0.7]]
    return cfg, W, X, alpha


def _two_frame_qk_expected(X, alpha, pos):
    """Scalar closed form of the hand-built block above: frame 0 sees only itself (A = u_0);
    frame 1 weighs keys 0 and 1 by the softmax of s_j = q.k_j / sqrt(128), where
    q.k_j = 4 u_1[2h] * 3 u_j[2h+1] * cos(p_1 - p_j) (two pair-0 vectors rotated by their
    positions differ by the angle p_1 - p_j)."""
    D, dh = 256, 128
    U = []
    for t in range(2):
        rms = math.sqrt(sum(v * v for v in X[t]) / D + 1e-8)
        U.append([alpha[i] * X[t][i] / rms for i in range(D)])
    out0 = [X[0][i] + U[0][i] for i in range(D)]
    out1 = list(X[1])
    for h in range(2):
        s = [4.0 * U[1][2 * h] * 3.0 * U[j][2 * h + 1] * math.cos(pos[1] - pos[j]) / math.sqrt(dh)
             for j in range(2)]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        w = [v / sum(e) for v in e]
        for i in range(h * dh, (h + 1) * dh):
            out1[i] += w[0] * U[0][i] + w[1] * U[1][i]
    return np.array([out0, out1]), w


def test_two_frame_block_fixes_q_before_k_and_score_scale():
    """Fixes the Q | K | V order of the fused projection, the head split and the
    1/sqrt(d_head) score scale (audit section 3, 'One of the 32 temporal blocks' and
    'Positions, attention mask and final text head'), on both code paths."""
    cfg, W, X, alpha = _two_frame_qk_setup()
    pos = [5, 6]
    want, w = _two_frame_qk_expected(X, alpha, pos)
    assert 0.05 < w[0] < 0.95            # the two keys really compete
    got = O.block_full(X, np.array(pos), 0, W, cfg)
    assert np.allclose(got, want, atol=1e-12)
    cache = O.Cache(1)
    inc = np.stack([O.decode_step(X[t], pos[t], cache, W, cfg) for t in range(2)])
    assert np.allclose(inc, want, atol=1e-12)


@pytest.mark.parametrize("context", [3000, 4])
def test_chunk_over_history_equals_full_sequence(context):
    """A sequence split into two chunks, the second run against the history the first left
    in a cache (a prompt replayed into a live cache, audit section 9), gives the rows of
    the one full-sequence forward; with context 4 the second chunk's window also drops
    history keys."""
    cfg, W, ids = _tiny()
    cfg = synth.with_(cfg, context=context)
    full = O.forward_full(ids, W, cfg)
    c = O.Cache(cfg["n_layers"])
    a = O.forward_full(ids[:9], W, cfg, cache=c)
    b = O.forward_full(ids[9:], W, cfg, p0=9, cache=c)
    assert np.max(np.abs(a - full[:9])) < 1e-12
    assert np.max(np.abs(b - full[9:])) < 1e-12
    assert [blk[0][0] for blk in c.layers[0]] == [0, 9]   # both chunks' keys were appended


def test_chunk_over_synthetic_history_equals_incremental_decode():
    """History keys/values that no forward produced (random, as a loaded ring): a 5-frame
    chunk at positions 20..24 against a 6-key window equals frame-by-frame decode over the
    same history."""
    cfg, W, ids = _tiny()
    cfg = synth.with_(cfg, context=6)
    L, H, dh = cfg["n_layers"], cfg["n_heads"], cfg["d_head"]
    rng = np.random.default_rng(7)
    ks = [rng.standard_normal((20, H, dh)) for _ in range(L)]
    vs = [rng.standard_normal((20, H, dh)) for _ in range(L)]
    c1 = O.cache_from_blocks(ks, vs, np.arange(20), L)
    c2 = O.cache_from_blocks(ks, vs, np.arange(20), L)
    got = O.forward_full(ids[:5], W, cfg, p0=20, cache=c1)
    want = O.decode_incremental(ids[:5], W, cfg, p0=20, cache=c2)
    assert np.max(np.abs(got - want)) < 1e-12
