"""Oracle for the temporal transformer's per-frame forward (fp64, NumPy, CPU).

TEST INFRASTRUCTURE ONLY -- see the package docstring. Never called by the library.

Source: "PersonaPlex native LM audit" (Clockless Inkling, personaplex-research page),
section 3 "Native temporal computation" -- its parts "Input embedding sum",
"One of the 32 temporal blocks" and "Positions, attention mask and final text head" --
and section 6 "Three distinct caches" (temporal attention cache). Cross-checked with
"Learnings: PersonaPlex/Moshi full-duplex S2S export + real-time ORT inference"
(onnxruntime/mobius issue #369), section 1 "Architecture".

Conventions (readings of the pages where they leave a step open):
  * weights are given as NumPy arrays, either float32/float64 or uint16 holding the
    bit pattern of bfloat16; every value is widened exactly to fp64 before use;
  * linear weights use the [out_features, in_features] orientation, so y = W @ x;
  * cfg is a mapping with keys n_layers, d_model, n_heads, d_head, d_ff, context,
    text_vocab, audio_vocab, n_audio, rope_theta, eps;
  * weight names follow the constructor's parameter names (see inventory.py).
"""

import math

import numpy as np


# --------------------------------------------------------------------------- values

def f64(a):
    """Widen a weight to fp64 exactly. uint16 arrays hold bfloat16 bit patterns: a
    bfloat16 value is the float32 whose upper 16 bits are those bits."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------- embedding

def _table(W, k):
    """Stream k's table: stream 0 is agent text, streams 1..16 are audio tables 0..15
    (agent codebooks 0..7 then user codebooks 0..7) -- audit section 3, 'Input embedding sum'."""
    return W["text_emb.weight"] if k == 0 else W["emb.%d.weight" % (k - 1)]


def check_ids(ids_t, cfg):
    """Raise ValueError unless every ID is -1 (no input) or a row of its stream's table.
    -2 (the ungenerated-cache sentinel) and anything else out of range are rejected."""
    n_streams = cfg["n_audio"] + 1
    ids_t = [int(v) for v in ids_t]
    if len(ids_t) != n_streams:
        raise ValueError("expected %d stream IDs, got %d" % (n_streams, len(ids_t)))
    for k, i in enumerate(ids_t):
        vocab = cfg["text_vocab"] if k == 0 else cfg["audio_vocab"]
        if i < -1 or i >= vocab:
            raise ValueError("stream %d: ID %d outside [-1, %d)" % (k, i, vocab))


def embed(ids_t, W, cfg, precision="f64"):
    """x = sum over the 17 streams of that stream's embedding row; ID -1 contributes an
    exact zero vector (audit section 3, 'Input embedding sum').

    precision="f64": the exact sum. precision="f32": the same sum accumulated in float32
    in stream order 0..16, each addition rounded to float32 -- the fixed-order reading
    used for the bit-exact gather comparison."""
    check_ids(ids_t, cfg)
    D = cfg["d_model"]
    if precision == "f64":
        x = np.zeros(D, np.float64)
        for k, i in enumerate(ids_t):
            if int(i) != -1:
                x = x + f64(_table(W, k)[int(i)])
        return x
    if precision == "f32":
        x = np.zeros(D, np.float32)
        for k, i in enumerate(ids_t):
            if int(i) != -1:
                x = (x + f64(_table(W, k)[int(i)]).astype(np.float32)).astype(np.float32)
        return x
    raise ValueError(precision)


# --------------------------------------------------------------------------- pieces

def rmsnorm(v, alpha, eps):
    """alpha * v / sqrt(mean(v^2) + eps) over the last axis; no mean subtraction
    (audit section 3: 'RMSNorm32', eps 1e-8 inside the square root)."""
    v = np.asarray(v, np.float64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return f64(alpha) * v / np.sqrt(ms + eps)


def rope_inv_freq(d_head, theta):
    """omega_j = theta^(-2j/d_head) = exp(-ln(theta) * 2j / d_head), j = 0 .. d_head/2-1."""
    j = np.arange(d_head // 2, dtype=np.float64)
    return np.exp(-math.log(theta) * 2.0 * j / d_head)


def rope(x, pos, theta):
    """Rotate adjacent coordinate pairs (2j, 2j+1) of the last axis by angle pos*omega_j
    (audit section 3, 'Positions, attention mask and final text head').

    x: [..., d_head]; pos: a scalar or an array broadcastable to x[..., 0]."""
    x = np.asarray(x, np.float64)
    d_head = x.shape[-1]
    ang = np.asarray(pos, np.float64)[..., None] * rope_inv_freq(d_head, theta)
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def attention(q, k, v, q_pos, k_pos, window):
    """Scaled dot-product attention of one head with the causal context mask
    0 <= q_pos - k_pos < window (audit section 3; dropout 0, scale 1/sqrt(d_head)).

    q: [Tq, d], k, v: [Tk, d]; q_pos: [Tq], k_pos: [Tk]. Every query must see >= 1 key."""
    q_pos = np.asarray(q_pos)[:, None]
    k_pos = np.asarray(k_pos)[None, :]
    delta = q_pos - k_pos
    allowed = (delta >= 0) & (delta < window)
    s = (q @ k.T) / math.sqrt(q.shape[-1])
    s = np.where(allowed, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    p = p / np.sum(p, axis=-1, keepdims=True)
    return p @ v


def silu(g):
    return g / (1.0 + np.exp(-g))


def swiglu(gz, hidden):
    """ActivationGating: split the 2*hidden projection into g = first half, z = second
    half; return SiLU(g) * z (audit section 3, 'One of the 32 temporal blocks')."""
    g, z = gz[..., :hidden], gz[..., hidden:]
    return silu(g) * z


def _lw(W, l, name):
    return W["transformer.layers.%d.%s" % (l, name)]


# --------------------------------------------------------------------------- full sequence

def block_full(X, pos, l, W, cfg, cache=None):
    """One pre-norm temporal block on a whole sequence X [T, D] at absolute positions pos [T].

    cache: optional history (a Cache holding earlier positions of this sequence). Each
    query then attends to every key of the history and of the sequence inside its window
    (the same declared mask), and the sequence's post-RoPE keys and raw values are appended
    to layer l of the cache afterwards."""
    D, H, dh, F = cfg["d_model"], cfg["n_heads"], cfg["d_head"], cfg["d_ff"]
    eps, theta, C = cfg["eps"], cfg["rope_theta"], cfg["context"]
    T = X.shape[0]
    u = rmsnorm(X, _lw(W, l, "norm1.alpha"), eps)
    qkv = u @ f64(_lw(W, l, "self_attn.in_proj_weight")).T          # [T, 3D]
    Q = qkv[:, 0 * D:1 * D].reshape(T, H, dh)
    K = qkv[:, 1 * D:2 * D].reshape(T, H, dh)
    V = qkv[:, 2 * D:3 * D].reshape(T, H, dh)
    Q = rope(Q, np.asarray(pos)[:, None], theta)
    K = rope(K, np.asarray(pos)[:, None], theta)
    kpos, Ka, Va = np.asarray(pos), K, V
    if cache is not None:
        # history keys that any query of the sequence can see: 0 <= pos[-1] - p < C + T - 1
        hist = cache.visible(l, int(pos[-1]), C + T - 1)
        if hist is not None:
            kpos = np.concatenate([hist[0], kpos])
            Ka = np.concatenate([hist[1], K])
            Va = np.concatenate([hist[2], V])
        cache.add_block(l, pos, K, V)
    A = np.empty((T, H, dh))
    for h in range(H):
        A[:, h, :] = attention(Q[:, h], Ka[:, h], Va[:, h], pos, kpos, C)
    y = X + A.reshape(T, D) @ f64(_lw(W, l, "self_attn.out_proj.weight")).T
    gz = rmsnorm(y, _lw(W, l, "norm2.alpha"), eps) @ f64(_lw(W, l, "gating.linear_in.weight")).T
    return y + swiglu(gz, F) @ f64(_lw(W, l, "gating.linear_out.weight")).T


def forward_full(ids, W, cfg, p0=0, with_logits=False, after_block=None, cache=None):
    """h = final RMSNorm of the 32-block stack over frames ids [T, n_audio+1] placed at
    positions p0 .. p0+T-1 (audit section 3). Returns h [T, D] (and logits [T, V_text-1]
    from the untied text head when with_logits). after_block: optional {l: f} applied to
    every row of the residual stream after block l (a memory reader). cache: optional
    history of earlier positions (a prompt replayed into a live cache, audit section 9);
    the frames' keys and values are appended to it."""
    ids = np.asarray(ids)
    T = ids.shape[0]
    pos = np.arange(p0, p0 + T)
    X = np.stack([embed(ids[t], W, cfg) for t in range(T)])
    for l in range(cfg["n_layers"]):
        X = block_full(X, pos, l, W, cfg, cache)
        if after_block and l in after_block:
            X = np.stack([after_block[l](X[t]) for t in range(T)])
    h = rmsnorm(X, W["out_norm.alpha"], cfg["eps"])
    if with_logits:
        return h, h @ f64(W["text_linear.weight"]).T
    return h


# --------------------------------------------------------------------------- incremental

class Cache:
    """Per-layer KV history: blocks of (absolute positions [n], post-RoPE keys [n, H, dh],
    raw values [n, H, dh]); keys/values may be fp64 or bfloat16 bit patterns and are
    widened only when attended. Visibility is decided by the window 0 <= q - k < context
    alone (the declared mask), never by slot reuse."""

    def __init__(self, n_layers):
        self.layers = [[] for _ in range(n_layers)]

    def add_block(self, l, positions, k, v):
        self.layers[l].append((np.asarray(positions, np.int64), k, v))

    def visible(self, l, pos, window):
        """Positions, keys and values (fp64) of layer l inside the window of query pos, or
        None when no stored key is inside it."""
        ps, ks, vs = [], [], []
        for p, k, v in self.layers[l]:
            sel = (pos - p >= 0) & (pos - p < window)
            if np.any(sel):
                ps.append(p[sel])
                ks.append(f64(k[sel]))
                vs.append(f64(v[sel]))
        if not ps:
            return None
        return np.concatenate(ps), np.concatenate(ks), np.concatenate(vs)


def decode_step(x, pos, cache, W, cfg, after_block=None):
    """One new frame with embedding sum x [D] at absolute position pos, attending over the
    cached keys/values; appends this frame's post-RoPE key and raw value to the cache.
    Returns the residual stream after the last block (before the final norm).
    after_block: optional {l: f} applied to the residual stream after block l."""
    D, H, dh, F = cfg["d_model"], cfg["n_heads"], cfg["d_head"], cfg["d_ff"]
    eps, theta, C = cfg["eps"], cfg["rope_theta"], cfg["context"]
    x = np.asarray(x, np.float64)
    for l in range(cfg["n_layers"]):
        u = rmsnorm(x, _lw(W, l, "norm1.alpha"), eps)
        qkv = f64(_lw(W, l, "self_attn.in_proj_weight")) @ u
        q = rope(qkv[0 * D:1 * D].reshape(H, dh), pos, theta)
        k = rope(qkv[1 * D:2 * D].reshape(H, dh), pos, theta)
        v = qkv[2 * D:3 * D].reshape(H, dh)
        cache.add_block(l, [pos], k[None], v[None])
        kpos, Ks, Vs = cache.visible(l, pos, C)                   # [n], [n, H, dh] x2
        a = np.stack([attention(q[h][None], Ks[:, h], Vs[:, h], [pos], kpos, C)[0]
                      for h in range(H)])
        y = x + f64(_lw(W, l, "self_attn.out_proj.weight")) @ a.reshape(D)
        gz = f64(_lw(W, l, "gating.linear_in.weight")) @ rmsnorm(y, _lw(W, l, "norm2.alpha"), eps)
        x = y + f64(_lw(W, l, "gating.linear_out.weight")) @ swiglu(gz, F)
        if after_block and l in after_block:
            x = after_block[l](x)
    return x


def final(x, W, cfg, with_logits=False):
    h = rmsnorm(x, W["out_norm.alpha"], cfg["eps"])
    if with_logits:
        return h, f64(W["text_linear.weight"]) @ h
    return h


def decode_incremental(ids, W, cfg, p0=0, cache=None, with_logits=False, after_block=None):
    """Frame-by-frame decode of ids [T, n_audio+1] from position p0, with a KV cache
    (a separate code path from forward_full; the two must agree)."""
    ids = np.asarray(ids)
    cache = cache if cache is not None else Cache(cfg["n_layers"])
    hs, logits = [], []
    for t in range(ids.shape[0]):
        x = decode_step(embed(ids[t], W, cfg), p0 + t, cache, W, cfg, after_block)
        out = final(x, W, cfg, with_logits)
        if with_logits:
            hs.append(out[0])
            logits.append(out[1])
        else:
            hs.append(out)
    if with_logits:
        return np.stack(hs), np.stack(logits)
    return np.stack(hs)


def cache_from_blocks(k_layers, v_layers, positions, n_layers):
    """A Cache whose layer l holds post-RoPE keys k_layers[l] and values v_layers[l]
    ([n, H, dh] each, fp64 or bfloat16 bits) at absolute positions [n]."""
    cache = Cache(n_layers)
    for l in range(n_layers):
        cache.add_block(l, positions, k_layers[l], v_layers[l])
    return cache
