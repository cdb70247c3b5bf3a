"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's callers.

This module draws random numbers and nothing else: it holds none of the model's
arithmetic. Every tensor gets its own PCG64 stream, seeded from (base seed, CRC-32 of
the tensor's name), so a tensor's bytes do not depend on which other tensors were drawn.

Recipes (the pages publish no weights, codes or activations):
  * linear and embedding weights: 0.02 * N(0, 1), rounded to bfloat16 with
    round-to-nearest-even (or kept float32 for the fp32 workload);
  * RMSNorm scales: 1 + 0.02 * N(0, 1), float32;
  * stream IDs: uniform over each stream's table rows, each replaced by -1 with
    probability 0.05;
  * pre-filled cache keys/values: N(0, 1) rounded to bfloat16.

bfloat16 tensors are returned as uint16 arrays holding the bit patterns.
"""

import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# ----------------------------------------------------------------------------- shapes
# Workload shape tables (sizes named after what they are).

TINY_TEMPORAL = dict(n_layers=2, d_model=256, n_heads=4, d_head=64, d_ff=704, context=3000,
                     text_vocab=32001, audio_vocab=2049, n_audio=16, rope_theta=10000.0,
                     eps=1e-8)
FULL_TEMPORAL = dict(n_layers=32, d_model=4096, n_heads=32, d_head=128, d_ff=11264,
                     context=3000, text_vocab=32001, audio_vocab=2049, n_audio=16,
                     rope_theta=10000.0, eps=1e-8)
FULL_DEPTH = dict(n_layers=6, d_model=1024, n_heads=16, d_head=64, d_ff=2816, n_steps=16,
                  window=8, text_vocab=32001, audio_vocab=2049, n_out=2048, d_temporal=4096,
                  eps=1e-8)
TINY_DEPTH = dict(n_layers=2, d_model=128, n_heads=4, d_head=32, d_ff=352, n_steps=16,
                  window=8, text_vocab=32001, audio_vocab=2049, n_out=2048, d_temporal=256,
                  eps=1e-8)


def with_(cfg, **kw):
    out = dict(cfg)
    out.update(kw)
    return out


# ----------------------------------------------------------------------------- draws

_CHUNK = 1 << 22
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=8)
    return _POOL


def _seed_for(seed, name):
    return np.random.SeedSequence([int(seed) & 0xFFFFFFFF, zlib.crc32(name.encode())])


def normal_f32(seed, name, shape):
    """N(0, 1) float32 draws of `shape`; large tensors are drawn in fixed 4 Mi-element
    chunks, each with its own child stream, on a thread pool."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    ss = _seed_for(seed, name)
    n_chunks = (n + _CHUNK - 1) // _CHUNK
    children = ss.spawn(n_chunks)

    def fill(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(children[i]))
        out[lo:hi] = g.standard_normal(hi - lo, dtype=np.float32)

    if n_chunks == 1:
        fill(0)
    else:
        list(_pool().map(fill, range(n_chunks)))
    return out.reshape(shape)


def to_bf16_bits(a):
    """float32 -> bfloat16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def weight(seed, name, shape, wdtype):
    w = normal_f32(seed, name, shape)
    w *= np.float32(0.02)
    return to_bf16_bits(w) if wdtype == "bf16" else w


def norm_scale(seed, name, n):
    return (np.float32(1.0) + np.float32(0.02) * normal_f32(seed, name, (n,))).astype(np.float32)


# ----------------------------------------------------------------------------- model inputs

def temporal_weights(cfg, seed, wdtype="bf16", with_text_head=True, layers=None,
                     shared_layer=False):
    """Dict name -> array for the temporal model of shape table `cfg`.

    layers: iterable of layer indices to draw (default all). shared_layer: draw layer 0
    only and reuse its arrays for every layer (a full-depth stack whose blocks share one
    set of weights, for checks at full depth without drawing every layer)."""
    D, F, L = cfg["d_model"], cfg["d_ff"], cfg["n_layers"]
    W = {"text_emb.weight": weight(seed, "text_emb.weight", (cfg["text_vocab"], D), wdtype)}
    for i in range(cfg["n_audio"]):
        n = "emb.%d.weight" % i
        W[n] = weight(seed, n, (cfg["audio_vocab"], D), wdtype)
    shapes = [("self_attn.in_proj_weight", (3 * D, D)), ("self_attn.out_proj.weight", (D, D)),
              ("gating.linear_in.weight", (2 * F, D)), ("gating.linear_out.weight", (D, F))]
    todo = list(range(L)) if layers is None else list(layers)
    for l in (todo[:1] if shared_layer else todo):
        p = "transformer.layers.%d." % l
        for n, s in shapes:
            W[p + n] = weight(seed, p + n, s, wdtype)
        W[p + "norm1.alpha"] = norm_scale(seed, p + "norm1.alpha", D)
        W[p + "norm2.alpha"] = norm_scale(seed, p + "norm2.alpha", D)
    if shared_layer:
        src = "transformer.layers.%d." % todo[0]
        for l in todo[1:]:
            p = "transformer.layers.%d." % l
            for n in [s[0] for s in shapes] + ["norm1.alpha", "norm2.alpha"]:
                W[p + n] = W[src + n]
    W["out_norm.alpha"] = norm_scale(seed, "out_norm.alpha", D)
    if with_text_head:
        W["text_linear.weight"] = weight(seed, "text_linear.weight", (cfg["text_vocab"] - 1, D), wdtype)
    return W


def depth_weights(cfg, seed, wdtype="bf16"):
    """Dict name -> array for the depth transformer of shape table `cfg`."""
    D, F, S, L = cfg["d_model"], cfg["d_ff"], cfg["n_steps"], cfg["n_layers"]
    W = {}
    for q in range(S):
        n = "depformer_in.%d.weight" % q
        W[n] = weight(seed, n, (D, cfg["d_temporal"]), wdtype)
        n = "linears.%d.weight" % q
        W[n] = weight(seed, n, (cfg["n_out"], D), wdtype)
    for q in range(S - 1):
        n = "depformer_emb.%d.weight" % q
        W[n] = weight(seed, n, (cfg["audio_vocab"], D), wdtype)
    W["depformer_text_emb.weight"] = weight(seed, "depformer_text_emb.weight",
                                            (cfg["text_vocab"], D), wdtype)
    for m in range(L):
        p = "depformer.layers.%d." % m
        W[p + "self_attn.in_proj_weight"] = weight(seed, p + "self_attn.in_proj_weight", (S * 3 * D, D), wdtype)
        W[p + "self_attn.out_proj.weight"] = weight(seed, p + "self_attn.out_proj.weight", (S * D, D), wdtype)
        for q in range(S):
            n = p + "gating.%d.linear_in.weight" % q
            W[n] = weight(seed, n, (2 * F, D), wdtype)
            n = p + "gating.%d.linear_out.weight" % q
            W[n] = weight(seed, n, (D, F), wdtype)
        W[p + "norm1.alpha"] = norm_scale(seed, p + "norm1.alpha", D)
        W[p + "norm2.alpha"] = norm_scale(seed, p + "norm2.alpha", D)
    return W


def stream_ids(cfg, n_frames, seed, p_missing=0.05, batch=None):
    """int32 IDs [n_frames, n_audio+1] (or [batch, n_frames, n_audio+1])."""
    g = np.random.Generator(np.random.PCG64(_seed_for(seed, "ids")))
    shape = (n_frames,) if batch is None else (batch, n_frames)
    n_streams = cfg["n_audio"] + 1
    ids = np.empty(shape + (n_streams,), np.int32)
    ids[..., 0] = g.integers(0, cfg["text_vocab"], size=shape)
    ids[..., 1:] = g.integers(0, cfg["audio_vocab"], size=shape + (n_streams - 1,))
    ids[g.random(ids.shape) < p_missing] = -1
    return ids


def cache_frames(cfg, n_frames, seed, wdtype="bf16", batch=1):
    """Keys and values for a pre-filled cache: [n_layers, 2, batch, n_heads, n_frames, d_head],
    N(0, 1), bfloat16 bits (or float32)."""
    shape = (cfg["n_layers"], 2, batch, cfg["n_heads"], n_frames, cfg["d_head"])
    a = normal_f32(seed, "kv", shape)
    return to_bf16_bits(a) if wdtype == "bf16" else a


def hidden(n, seed, name="h"):
    return normal_f32(seed, name, (n,))


def depth_codes(cfg, seed):
    g = np.random.Generator(np.random.PCG64(_seed_for(seed, "codes")))
    return g.integers(0, cfg["n_out"], size=cfg["n_steps"]).astype(np.int32)


def reader_weights(cfg, n_readers, mem_dim, seed, wdtype="bf16", scale=0.02, zero_out=False):
    """Memory-reader weights (readers.{i}.norm / q_proj / k_proj / v_proj / out_proj):
    matrices scale * N(0, 1) (bfloat16 bits or float32), biases scale * N(0, 1) float32,
    LayerNorm weight 1 + 0.02 N(0, 1) and bias 0.02 N(0, 1); zero_out makes the output
    projection's weight and bias zero (the readers' initial state)."""
    D = cfg["d_model"]
    R = {}
    for i in range(n_readers):
        p = "readers.%d." % i
        R[p + "norm.weight"] = norm_scale(seed, p + "norm.weight", D)
        R[p + "norm.bias"] = 0.02 * normal_f32(seed, p + "norm.bias", (D,))
        for name, shape in (("q_proj", (D, D)), ("k_proj", (D, mem_dim)), ("v_proj", (D, mem_dim)),
                            ("out_proj", (D, D))):
            a = scale * normal_f32(seed, p + name + ".weight", shape)
            b = scale * normal_f32(seed, p + name + ".bias", (D,))
            if zero_out and name == "out_proj":
                a = np.zeros_like(a)
                b = np.zeros_like(b)
            R[p + name + ".weight"] = to_bf16_bits(a) if wdtype == "bf16" else a.astype(np.float32)
            R[p + name + ".bias"] = b.astype(np.float32)
    return R


def memory_bank(n, mem_dim, seed, wdtype="bf16"):
    """A memory bank [n, mem_dim] of N(0, 1) rows (the writer's output is LayerNorm-ed, so
    rows have unit scale), bfloat16 bits or float32."""
    a = normal_f32(seed, "memory", (n, mem_dim))
    return to_bf16_bits(a) if wdtype == "bf16" else a

