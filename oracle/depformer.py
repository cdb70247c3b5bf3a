"""Oracle for the depth transformer ("depformer") step of one frame (fp64, NumPy, CPU).

TEST INFRASTRUCTURE ONLY -- see the package docstring. Never called by the library.

Source: "PersonaPlex native LM audit" (Clockless Inkling, personaplex-research page),
section 4 "Native depth computation: six blocks, sixteen sequential positions" (the
per-position input, the depth block, and the table of per-step weight slices), and the
same page's "Native PersonaPlex streams and output path" (depth position 0 uses the
depth text table, position q > 0 the table of position q-1 indexed by the previously
selected code; the depformer is fed the post-final-norm hidden state). Cross-checked
with the Moshi walkthrough's "Three ways to model a column" (depth input = temporal
context plus an embedding of the previous token, per-index weights).

cfg keys: n_layers (6), d_model (1024), n_heads (16), d_head (64), d_ff (2816),
n_steps (16), window, text_vocab (32001), audio_vocab (2049), n_out (2048),
d_temporal (4096), eps (1e-8).
"""

import math

import numpy as np

from .temporal import f64, rmsnorm, silu


def _attend(q, ks, vs):
    """Softmax attention of one head over the listed keys (scale 1/sqrt(d_head))."""
    s = (ks @ q) / math.sqrt(q.shape[-1])
    p = np.exp(s - np.max(s))
    return (p / np.sum(p)) @ vs


def step_logits(h, text_token, forced, W, cfg):
    """Run positions q = 0 .. n_steps-1 for one frame.

    h: temporal hidden [d_temporal] (after the final temporal RMSNorm).
    text_token: the selected agent-text token that conditions position 0.
    forced: length n_steps; forced[q] >= 0 replaces the selection at position q,
            -1 means select greedily (argmax, lowest index on ties).
    Returns (codes [n_steps] int64, logits [n_steps, n_out] fp64).

    The depth KV history starts empty for every call; position q attends to the
    positions q' of this frame with 0 <= q - q' < window."""
    def select(q, lg):
        if forced is not None and int(forced[q]) >= 0:
            return int(forced[q])
        return int(np.argmax(lg))      # first maximum = lowest index on ties
    return step_select(h, text_token, select, W, cfg)


def step_select(h, text_token, select, W, cfg):
    """The depth loop of one frame with a caller-chosen selection rule: after position q's
    logits are formed, select(q, logits_q) returns the code that position q emits, which
    is also the input of position q + 1 (the generator samples, or uses a supplied code
    where one is provided). Returns (codes [n_steps] int64, logits [n_steps, n_out])."""
    D, H, dh, F = cfg["d_model"], cfg["n_heads"], cfg["d_head"], cfg["d_ff"]
    S, L, eps, win = cfg["n_steps"], cfg["n_layers"], cfg["eps"], cfg["window"]
    h = np.asarray(h, np.float64)
    if not 0 <= int(text_token) < cfg["text_vocab"]:
        raise ValueError("text token %d out of range" % int(text_token))
    hist = [[] for _ in range(L)]          # per layer: list of (k [H, dh], v [H, dh])
    codes = np.zeros(S, np.int64)
    logits = np.zeros((S, cfg["n_out"]))
    prev = None
    for q in range(S):
        if q == 0:
            e = f64(W["depformer_text_emb.weight"][int(text_token)])
        else:
            e = f64(W["depformer_emb.%d.weight" % (q - 1)][prev])
        z = f64(W["depformer_in.%d.weight" % q]) @ h + e
        for m in range(L):
            pre = "depformer.layers.%d." % m
            u = rmsnorm(z, W[pre + "norm1.alpha"], eps)
            wqkv = f64(W[pre + "self_attn.in_proj_weight"][q * 3 * D:(q + 1) * 3 * D])
            qkv = wqkv @ u
            qh = qkv[0:D].reshape(H, dh)
            kh = qkv[D:2 * D].reshape(H, dh)
            vh = qkv[2 * D:3 * D].reshape(H, dh)
            hist[m].append((kh, vh))
            seen = [i for i in range(len(hist[m])) if 0 <= q - i < win]
            ks = np.stack([hist[m][i][0] for i in seen])          # [n, H, dh]
            vs = np.stack([hist[m][i][1] for i in seen])
            o = np.stack([_attend(qh[hd], ks[:, hd], vs[:, hd]) for hd in range(H)])
            wo = f64(W[pre + "self_attn.out_proj.weight"][q * D:(q + 1) * D])
            z = z + wo @ o.reshape(D)
            gz = f64(W[pre + "gating.%d.linear_in.weight" % q]) @ rmsnorm(z, W[pre + "norm2.alpha"], eps)
            z = z + f64(W[pre + "gating.%d.linear_out.weight" % q]) @ (silu(gz[:F]) * gz[F:])
        logits[q] = f64(W["linears.%d.weight" % q]) @ z
        prev = int(select(q, logits[q]))
        if not 0 <= prev < cfg["audio_vocab"]:
            raise ValueError("position %d selected code %d outside the audio table" % (q, prev))
        codes[q] = prev
    return codes, logits
