"""Pins of the depth-transformer oracle: closed forms with zeroed blocks, the window,
and per-position weight slicing."""

import numpy as np

from oracle import depformer as DF
from personaplex_temporal_transformer_amd import synth


def _setup(seed=0, **kw):
    cfg = synth.with_(synth.TINY_DEPTH, **kw)
    W = synth.depth_weights(cfg, seed, "fp32")
    h = synth.hidden(cfg["d_temporal"], seed + 1)
    return cfg, W, h


def test_zero_blocks_closed_form():
    """With every depth block weight zero, each block is the identity (qkv = 0 -> the
    attention output is 0; SiLU(0) * 0 = 0), so logits_q = head_q (P_q h + E(prev))."""
    cfg, W, h = _setup()
    for k in list(W):
        if k.startswith("depformer.layers.") and not k.endswith("alpha"):
            W[k] = np.zeros_like(W[k])
    forced = synth.depth_codes(cfg, 5)
    codes, logits = DF.step_logits(h, 123, forced, W, cfg)
    assert np.array_equal(codes, forced)
    for q in range(cfg["n_steps"]):
        P = W["depformer_in.%d.weight" % q].astype(np.float64)
        E = (W["depformer_text_emb.weight"][123] if q == 0
             else W["depformer_emb.%d.weight" % (q - 1)][forced[q - 1]]).astype(np.float64)
        want = W["linears.%d.weight" % q].astype(np.float64) @ (P @ h.astype(np.float64) + E)
        assert np.allclose(logits[q], want, atol=1e-12), q


def test_greedy_ties_take_lowest_index():
    cfg, W, h = _setup()
    for q in range(cfg["n_steps"]):
        W["linears.%d.weight" % q] = np.zeros_like(W["linears.%d.weight" % q])
    codes, logits = DF.step_logits(h, 7, None, W, cfg)
    assert np.all(logits == 0.0)
    assert np.all(codes == 0)


def test_window_only_matters_past_its_length():
    cfg, W, h = _setup(seed=2)
    forced = synth.depth_codes(cfg, 6)
    _, l8 = DF.step_logits(h, 9, forced, W, synth.with_(cfg, window=8))
    _, l16 = DF.step_logits(h, 9, forced, W, synth.with_(cfg, window=16))
    assert np.array_equal(l8[:8], l16[:8])
    assert np.max(np.abs(l8[8:] - l16[8:])) > 1e-6


def test_position_q_uses_slice_q():
    """Perturbing position q' weights (packed slices, FFN q', head q', projection q')
    leaves logits of positions < q' bit-unchanged and changes logits at q'."""
    cfg, W, h = _setup(seed=3)
    forced = synth.depth_codes(cfg, 8)
    _, base = DF.step_logits(h, 11, forced, W, cfg)
    D = cfg["d_model"]
    for qp in (3, 12):
        W2 = dict(W)
        for m in range(cfg["n_layers"]):
            p = "depformer.layers.%d." % m
            a = W[p + "self_attn.in_proj_weight"].copy()
            a[qp * 3 * D:(qp + 1) * 3 * D] *= 1.5
            W2[p + "self_attn.in_proj_weight"] = a
            o = W[p + "self_attn.out_proj.weight"].copy()
            o[qp * D:(qp + 1) * D] *= -1.0
            W2[p + "self_attn.out_proj.weight"] = o
        _, pert = DF.step_logits(h, 11, forced, W2, cfg)
        assert np.array_equal(base[:qp], pert[:qp])
        assert np.max(np.abs(base[qp] - pert[qp])) > 1e-6


def test_first_position_attention_sees_one_key():
    q, k, v = np.ones(4), np.arange(4.0), np.array([[2.0, -1.0, 0.5, 3.0]])
    assert np.array_equal(DF._attend(q, k[None], v), v[0])


def test_depth_consumes_hidden_and_text_token():
    cfg, W, h = _setup(seed=4)
    forced = synth.depth_codes(cfg, 1)
    _, a = DF.step_logits(h, 5, forced, W, cfg)
    _, b = DF.step_logits(h, 6, forced, W, cfg)
    _, c = DF.step_logits(h * 1.01, 5, forced, W, cfg)
    assert np.max(np.abs(a[0] - b[0])) > 1e-6
    assert np.max(np.abs(a[0] - c[0])) > 1e-6


def test_depth_window_by_uniform_attention():
    """One depth layer with Q = 0 (uniform weights over visible positions), V = u,
    W_O = I and a zero FFN: after the layer, z_q + mean{u_q' : 0 <= q - q' < window}
    with u = rmsnorm(z). With head_q = [I; 0] the logits expose that vector."""
    cfg, W, h = _setup(seed=5, n_layers=1, window=3)
    D, S = cfg["d_model"], cfg["n_steps"]
    p = "depformer.layers.0."
    qkv = np.zeros((S * 3 * D, D), np.float32)
    rng = np.random.default_rng(0)
    for q in range(S):
        qkv[q * 3 * D + D:q * 3 * D + 2 * D] = rng.standard_normal((D, D))   # K: irrelevant
        qkv[q * 3 * D + 2 * D:(q + 1) * 3 * D] = np.eye(D)                     # V = u
        W[p + "gating.%d.linear_in.weight" % q] = np.zeros_like(W[p + "gating.%d.linear_in.weight" % q])
        head = np.zeros((cfg["n_out"], D), np.float32)
        head[:D] = np.eye(D)
        W["linears.%d.weight" % q] = head
    W[p + "self_attn.in_proj_weight"] = qkv
    W[p + "self_attn.out_proj.weight"] = np.tile(np.eye(D, dtype=np.float32), (S, 1))
    forced = synth.depth_codes(cfg, 2)
    _, logits = DF.step_logits(h, 3, forced, W, cfg)
    a1 = W[p + "norm1.alpha"].astype(np.float64)
    zs, us = [], []
    for q in range(S):
        E = (W["depformer_text_emb.weight"][3] if q == 0
             else W["depformer_emb.%d.weight" % (q - 1)][forced[q - 1]]).astype(np.float64)
        z = W["depformer_in.%d.weight" % q].astype(np.float64) @ h.astype(np.float64) + E
        zs.append(z)
        us.append(a1 * z / np.sqrt(np.mean(z * z) + 1e-8))
        vis = [j for j in range(q + 1) if q - j < 3]
        want = z + sum(us[j] for j in vis) / len(vis)
        assert np.allclose(logits[q][:D], want, atol=1e-12), q
