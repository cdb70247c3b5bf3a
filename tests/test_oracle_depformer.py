"""Pins of the depth-transformer oracle: closed forms with zeroed blocks, the window,
and per-position weight slicing."""

import math

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


def _perturb(W, cfg, qp, family):
    """A copy of W with one weight family of position qp changed: the packed QKV rows or
    W_O rows of slice qp in every layer, the FFN matrices of position qp, its head or its
    projection of the temporal hidden state."""
    D = cfg["d_model"]
    W2 = dict(W)
    for m in range(cfg["n_layers"]):
        p = "depformer.layers.%d." % m
        if family == "qkv":
            a = W[p + "self_attn.in_proj_weight"].copy()
            a[qp * 3 * D:(qp + 1) * 3 * D] *= 1.5
            W2[p + "self_attn.in_proj_weight"] = a
        elif family == "out":
            o = W[p + "self_attn.out_proj.weight"].copy()
            o[qp * D:(qp + 1) * D] *= -1.0
            W2[p + "self_attn.out_proj.weight"] = o
        elif family in ("linear_in", "linear_out"):
            n = p + "gating.%d.%s.weight" % (qp, family)
            W2[n] = W[n] * -1.0
    if family == "head":
        W2["linears.%d.weight" % qp] = W["linears.%d.weight" % qp] * 0.5
    if family == "proj":
        W2["depformer_in.%d.weight" % qp] = W["depformer_in.%d.weight" % qp] * 2.0
    return W2


def test_position_q_uses_slice_q():
    """Perturbing one weight family of position q' alone -- its packed QKV slice, its W_O
    slice, its FFN input or output matrix, its head, its projection -- leaves the logits of
    positions < q' bit-unchanged and changes the logits at q' (the per-step weights:
    position q reads slice / matrix q of each family)."""
    cfg, W, h = _setup(seed=3)
    forced = synth.depth_codes(cfg, 8)
    _, base = DF.step_logits(h, 11, forced, W, cfg)
    for qp in (3, 12):
        for family in ("qkv", "out", "linear_in", "linear_out", "head", "proj"):
            _, pert = DF.step_logits(h, 11, forced, _perturb(W, cfg, qp, family), cfg)
            assert np.array_equal(base[:qp], pert[:qp]), (qp, family)
            assert np.max(np.abs(base[qp] - pert[qp])) > 1e-6, (qp, family)


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


def _z_and_u(cfg, W, h, text_tok, forced, alpha):
    """Per position: the depth input z_q = P_q h + E(prev) and its RMSNorm with scale alpha,
    in scalar math."""
    D = cfg["d_model"]
    zs, us = [], []
    for q in range(cfg["n_steps"]):
        E = (W["depformer_text_emb.weight"][text_tok] if q == 0
             else W["depformer_emb.%d.weight" % (q - 1)][forced[q - 1]]).astype(np.float64)
        z = W["depformer_in.%d.weight" % q].astype(np.float64) @ h.astype(np.float64) + E
        rms = math.sqrt(sum(v * v for v in z) / D + 1e-8)
        zs.append(z)
        us.append([alpha[i] * z[i] / rms for i in range(D)])
    return zs, us


def _identity_heads(cfg, W):
    D = cfg["d_model"]
    for q in range(cfg["n_steps"]):
        head = np.zeros((cfg["n_out"], D), np.float32)
        head[:D] = np.eye(D)
        W["linears.%d.weight" % q] = head


def test_depth_gated_ffn_halves_and_position_slice():
    """One depth layer with a zero attention (qkv = 0, so o = 0) and a nonzero gated
    feed-forward (audit section 4, 'One depth block at position q': the 2 x 2816
    projection splits into g then z, output SiLU(g) * z, with the FFN of position q).

    Position q's linear_in makes g_i = c_q v_i and z_i = v_{i+8} (i < 8, c_q = 0.5 + 0.25 q)
    and its linear_out adds SiLU(g_i) z_i to coordinate (i + 3) mod D; with head_q = [I; 0]
    the logits expose z_q + that vector, computed here with scalar math."""
    cfg, W, h = _setup(seed=7, n_layers=1)
    D, F, S = cfg["d_model"], cfg["d_ff"], cfg["n_steps"]
    p = "depformer.layers.0."
    W[p + "self_attn.in_proj_weight"] = np.zeros_like(W[p + "self_attn.in_proj_weight"])
    c = [0.5 + 0.25 * q for q in range(S)]
    for q in range(S):
        wi = np.zeros((2 * F, D), np.float32)
        wo = np.zeros((D, F), np.float32)
        for i in range(8):
            wi[i, i] = c[q]
            wi[F + i, 8 + i] = 1.0
            wo[(i + 3) % D, i] = 1.0
        W[p + "gating.%d.linear_in.weight" % q] = wi
        W[p + "gating.%d.linear_out.weight" % q] = wo
    _identity_heads(cfg, W)
    forced = synth.depth_codes(cfg, 3)
    _, logits = DF.step_logits(h, 17, forced, W, cfg)
    zs, vs = _z_and_u(cfg, W, h, 17, forced, W[p + "norm2.alpha"].astype(np.float64))
    for q in range(S):
        want = list(zs[q])
        for i in range(8):
            g, z2 = c[q] * vs[q][i], vs[q][8 + i]
            want[(i + 3) % D] += g / (1.0 + math.exp(-g)) * z2
        assert np.allclose(logits[q][:D], want, atol=1e-12), q


def test_depth_attention_scores_by_construction():
    """One depth layer with a zero feed-forward and hand-built per-position QKV slices
    (audit section 4: 16 heads x 64 in the full model, here 4 x 32; scores scaled by
    1/sqrt(d_head)). Head hd's query coordinate 0 is 3 u[hd] and its key coordinate 0 is
    2 u[4 + hd]; V = u and W_O = I, so position q's output is z_q + concat_hd of
    sum_q' softmax_q'(3 u_q[hd] 2 u_q'[4+hd] / sqrt(32)) u_q'[head hd's coordinates],
    over q' with 0 <= q - q' < window."""
    cfg, W, h = _setup(seed=8, n_layers=1, window=5)
    D, H, dh, S = cfg["d_model"], cfg["n_heads"], cfg["d_head"], cfg["n_steps"]
    p = "depformer.layers.0."
    qkv = np.zeros((S * 3 * D, D), np.float32)
    for q in range(S):
        base = q * 3 * D
        for hd in range(H):
            qkv[base + hd * dh, hd] = 3.0
            qkv[base + D + hd * dh, 4 + hd] = 2.0
        qkv[base + 2 * D:base + 3 * D] = np.eye(D)
        W[p + "gating.%d.linear_in.weight" % q] = np.zeros_like(W[p + "gating.%d.linear_in.weight" % q])
    W[p + "self_attn.in_proj_weight"] = qkv
    W[p + "self_attn.out_proj.weight"] = np.tile(np.eye(D, dtype=np.float32), (S, 1))
    _identity_heads(cfg, W)
    forced = synth.depth_codes(cfg, 4)
    _, logits = DF.step_logits(h, 21, forced, W, cfg)
    zs, us = _z_and_u(cfg, W, h, 21, forced, W[p + "norm1.alpha"].astype(np.float64))
    spread = 0.0
    for q in range(S):
        want = list(zs[q])
        vis = [j for j in range(q + 1) if q - j < 5]
        for hd in range(H):
            s = [3.0 * us[q][hd] * 2.0 * us[j][4 + hd] / math.sqrt(dh) for j in vis]
            e = [math.exp(v - max(s)) for v in s]
            w = [v / sum(e) for v in e]
            spread = max(spread, max(w) - min(w))
            for i in range(hd * dh, (hd + 1) * dh):
                want[i] += sum(w[n] * us[j][i] for n, j in enumerate(vis))
        assert np.allclose(logits[q][:D], want, atol=1e-12), q
    assert spread > 0.05                  # the scores really differ between keys
