"""ctypes binding of libpp (include/pp.h): argument marshalling only.

Every computation happens in libpp's HIP kernels; PyTorch is used here only to hold
device memory (tensors are passed by data_ptr()) and to name the current HIP stream.
Loading fails loudly if libpp.so has not been built; there is no fallback.
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpp.so")

PP_OK, PP_E_ARG, PP_E_ID, PP_E_CAPACITY, PP_E_DEVICE, PP_E_HIP, PP_E_DTYPE = range(7)
PP_F32, PP_BF16 = 0, 1
STATUS_NAMES = {0: "PP_OK", 1: "PP_E_ARG", 2: "PP_E_ID", 3: "PP_E_CAPACITY", 4: "PP_E_DEVICE",
                5: "PP_E_HIP", 6: "PP_E_DTYPE"}

# Every entry point declared in include/pp.h.
EXPORTS = ["pp_temporal_create", "pp_temporal_destroy", "pp_kv_alloc", "pp_kv_free", "pp_kv_reset",
           "pp_kv_info", "pp_kv_load", "pp_kv_store", "pp_embed_sum", "pp_temporal_decode_step", "pp_temporal_decode_step_noalloc",
           "pp_temporal_prefill", "pp_depformer_create", "pp_depformer_destroy", "pp_depformer_step",
           "pp_last_error", "pp_temporal_set_graph", "pp_temporal_set_attn_splits", "pp_temporal_trace", "pp_temporal_trace_read",
           "pp_depformer_set_graph", "pp_kv_restore", "pp_sample_top_k", "pp_generator_create", "pp_generator_destroy",
           "pp_generator_step", "pp_generator_inspect", "pp_generator_info", "pp_generator_store",
           "pp_generator_restore", "pp_temporal_prefill_embedded", "pp_readers_attach", "pp_readers_write",
           "pp_readers_set_visible"]


class PPError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), msg))
        self.status = status


class TemporalConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("d_head", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("context", ctypes.c_int32),
                ("text_vocab", ctypes.c_int32), ("audio_vocab", ctypes.c_int32), ("n_audio", ctypes.c_int32),
                ("wdtype", ctypes.c_int32), ("rope_theta", ctypes.c_double), ("eps", ctypes.c_double)]


class TemporalWeights(ctypes.Structure):
    _fields_ = [("text_emb", ctypes.c_void_p), ("audio_emb", ctypes.POINTER(ctypes.c_void_p)),
                ("norm1", ctypes.POINTER(ctypes.c_void_p)), ("norm2", ctypes.POINTER(ctypes.c_void_p)),
                ("w_qkv", ctypes.POINTER(ctypes.c_void_p)), ("w_o", ctypes.POINTER(ctypes.c_void_p)),
                ("w_in", ctypes.POINTER(ctypes.c_void_p)), ("w_out", ctypes.POINTER(ctypes.c_void_p)),
                ("out_norm", ctypes.c_void_p), ("text_head", ctypes.c_void_p)]


class DepthConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("d_head", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("n_steps", ctypes.c_int32),
                ("window", ctypes.c_int32), ("text_vocab", ctypes.c_int32), ("audio_vocab", ctypes.c_int32),
                ("n_out", ctypes.c_int32), ("d_temporal", ctypes.c_int32), ("wdtype", ctypes.c_int32),
                ("eps", ctypes.c_double)]


class DepthWeights(ctypes.Structure):
    _fields_ = [("in_proj", ctypes.POINTER(ctypes.c_void_p)), ("text_emb", ctypes.c_void_p),
                ("audio_emb", ctypes.POINTER(ctypes.c_void_p)), ("w_qkv", ctypes.POINTER(ctypes.c_void_p)),
                ("w_o", ctypes.POINTER(ctypes.c_void_p)), ("w_in", ctypes.POINTER(ctypes.c_void_p)),
                ("w_out", ctypes.POINTER(ctypes.c_void_p)), ("norm1", ctypes.POINTER(ctypes.c_void_p)),
                ("norm2", ctypes.POINTER(ctypes.c_void_p)), ("head", ctypes.POINTER(ctypes.c_void_p))]


class GeneratorConfig(ctypes.Structure):
    _fields_ = [("n_streams", ctypes.c_int32), ("delays", ctypes.c_int32 * 32), ("text_initial", ctypes.c_int32),
                ("audio_initial", ctypes.c_int32), ("text_temperature", ctypes.c_float),
                ("text_top_k", ctypes.c_int32), ("audio_temperature", ctypes.c_float),
                ("audio_top_k", ctypes.c_int32)]


class ReaderConfig(ctypes.Structure):
    _fields_ = [("n_readers", ctypes.c_int32), ("blocks", ctypes.c_int32 * 8), ("mem_dim", ctypes.c_int32),
                ("max_slots", ctypes.c_int32), ("ln_eps", ctypes.c_double)]


class ReaderWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("ln_w", "ln_b", "w_q", "b_q", "w_k", "b_k", "w_v", "b_v", "w_o", "b_o")]


_lib = None


def load():
    """Load libpp.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libpp.so not found at %s; build it with "
                          "`python -m personaplex_temporal_transformer_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    sig = {
        "pp_temporal_create": [P(TemporalConfig), P(TemporalWeights), I32, I32, P(VP)],
        "pp_temporal_destroy": [VP],
        "pp_kv_alloc": [VP, I32, P(VP)],
        "pp_kv_free": [VP],
        "pp_kv_reset": [VP],
        "pp_kv_info": [VP, P(I64), P(ctypes.c_uint64)],
        "pp_kv_load": [VP, VP, I32, VP],
        "pp_kv_store": [VP, VP, VP],
        "pp_kv_restore": [VP, VP, I64, VP],
        "pp_embed_sum": [VP, P(I32), I32, I32, VP, VP],
        "pp_temporal_decode_step": [VP, VP, P(I32), VP, VP, VP],
        "pp_temporal_decode_step_noalloc": [VP, VP, P(I32), VP, VP, VP],
        "pp_temporal_prefill": [VP, VP, P(I32), I32, VP, VP],
        "pp_depformer_create": [P(DepthConfig), P(DepthWeights), P(VP)],
        "pp_depformer_destroy": [VP],
        "pp_depformer_step": [VP, VP, P(I32), P(I32), I32, VP, VP, VP],
        "pp_temporal_set_graph": [VP, I32],
        "pp_temporal_set_attn_splits": [VP, I32],
        "pp_depformer_set_graph": [VP, I32],
        "pp_temporal_trace": [VP, I32, I32],
        "pp_temporal_trace_read": [VP, P(I64), P(ctypes.c_double)],
        "pp_sample_top_k": [VP, I32, I32, ctypes.c_float, I32, VP, VP, VP],
        "pp_generator_create": [VP, VP, VP, P(GeneratorConfig), P(VP)],
        "pp_generator_destroy": [VP],
        "pp_generator_step": [VP, P(I32), P(ctypes.c_double), VP, P(I32), VP],
        "pp_generator_inspect": [VP, VP, VP, VP, VP, VP],
        "pp_generator_info": [VP, P(I64), P(ctypes.c_uint64)],
        "pp_generator_store": [VP, VP, VP],
        "pp_generator_restore": [VP, VP, I64, VP],
        "pp_temporal_prefill_embedded": [VP, VP, VP, I32, VP, VP],
        "pp_readers_attach": [VP, P(ReaderConfig), P(ReaderWeights)],
        "pp_readers_write": [VP, VP, I32, I32, VP],
        "pp_readers_set_visible": [VP, I32],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.pp_last_error.argtypes = []
    lib.pp_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status):
    if status != PP_OK:
        raise PPError(status, load().pp_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ids(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _ptr_array(tensors):
    arr = (ctypes.c_void_p * max(1, len(tensors)))()
    for i, t in enumerate(tensors):
        arr[i] = t.data_ptr()
    return arr


# ----------------------------------------------------------------------------- temporal

class TemporalModel:
    """pp_temporal_create over device tensors named as in the constructor
    (text_emb.weight, emb.{i}.weight, transformer.layers.{l}.*, out_norm.alpha,
    text_linear.weight). `weights` maps those names to CUDA tensors (bf16 or fp32
    matrices, fp32 norm scales); references are kept for the model's lifetime."""

    def __init__(self, cfg, weights, wdtype, max_prefill_T=0, max_batch=1):
        lib = load()
        self.cfg = dict(cfg)
        self._w = weights
        L = cfg["n_layers"]
        c = TemporalConfig(cfg["n_layers"], cfg["d_model"], cfg["n_heads"], cfg["d_head"], cfg["d_ff"],
                           cfg["context"], cfg["text_vocab"], cfg["audio_vocab"], cfg["n_audio"],
                           PP_BF16 if wdtype == "bf16" else PP_F32, cfg["rope_theta"], cfg["eps"])

        def layer(n):
            return _ptr_array([weights["transformer.layers.%d.%s" % (l, n)] for l in range(L)])

        self._arrays = dict(
            audio=_ptr_array([weights["emb.%d.weight" % i] for i in range(cfg["n_audio"])]),
            n1=layer("norm1.alpha"), n2=layer("norm2.alpha"), qkv=layer("self_attn.in_proj_weight"),
            o=layer("self_attn.out_proj.weight"), win=layer("gating.linear_in.weight"),
            wout=layer("gating.linear_out.weight"))
        a = self._arrays
        cast = lambda x: ctypes.cast(x, ctypes.POINTER(ctypes.c_void_p))
        w = TemporalWeights(weights["text_emb.weight"].data_ptr(), cast(a["audio"]), cast(a["n1"]),
                            cast(a["n2"]), cast(a["qkv"]), cast(a["o"]), cast(a["win"]), cast(a["wout"]),
                            weights["out_norm.alpha"].data_ptr(),
                            weights["text_linear.weight"].data_ptr() if "text_linear.weight" in weights else None)
        h = ctypes.c_void_p()
        _check(lib.pp_temporal_create(ctypes.byref(c), ctypes.byref(w), int(max_batch), int(max_prefill_T),
                                      ctypes.byref(h)))
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            _check(load().pp_temporal_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def kv_alloc(self, batch=1):
        return KV(self, batch)

    def embed_sum(self, ids, x_out, stream=None):
        ids = np.asarray(ids, np.int32)
        B, T = (1, 1) if ids.ndim == 1 else ((1, ids.shape[0]) if ids.ndim == 2 else ids.shape[:2])
        arr, p = _ids(ids)
        _check(load().pp_embed_sum(self.handle, p, B, T, _ptr(x_out), _stream(stream)))

    def decode_step(self, kv, ids, h_out, logits_out=None, stream=None):
        arr, p = _ids(ids)
        _check(load().pp_temporal_decode_step(self.handle, kv.handle, p, _ptr(h_out), _ptr(logits_out),
                                              _stream(stream)))

    def decode_step_noalloc(self, kv, ids, h_out, logits_out=None, stream=None):
        arr, p = _ids(ids)
        _check(load().pp_temporal_decode_step_noalloc(self.handle, kv.handle, p, _ptr(h_out), _ptr(logits_out),
                                                      _stream(stream)))

    def prefill(self, kv, ids, h_out, stream=None):
        ids = np.asarray(ids, np.int32)
        arr, p = _ids(ids)
        T = ids.shape[-2]
        _check(load().pp_temporal_prefill(self.handle, kv.handle, p, T, _ptr(h_out), _stream(stream)))

    def prefill_embedded(self, kv, x, h_out, stream=None):
        """Prefill from summed embeddings x [T, d_model] (a float32 CUDA tensor)."""
        _check(load().pp_temporal_prefill_embedded(self.handle, kv.handle, _ptr(x), int(x.shape[0]), _ptr(h_out),
                                                   _stream(stream)))

    def set_graph(self, enable):
        _check(load().pp_temporal_set_graph(self.handle, 1 if enable else 0))

    def set_attn_splits(self, splits):
        _check(load().pp_temporal_set_attn_splits(self.handle, int(splits)))

    def attach_readers(self, blocks, weights, mem_dim, max_slots, ln_eps=1e-5):
        """pp_readers_attach: reader i after block blocks[i], weights named readers.{i}.norm /
        q_proj / k_proj / v_proj / out_proj (.weight, .bias) as CUDA tensors (kept alive)."""
        self._readers = weights
        n = len(blocks)
        cfg = ReaderConfig(n, (ctypes.c_int32 * 8)(*blocks), int(mem_dim), int(max_slots), float(ln_eps))
        arr = (ReaderWeights * n)()
        for i in range(n):
            p = "readers.%d." % i
            t = lambda k: weights[p + k].data_ptr()
            arr[i] = ReaderWeights(t("norm.weight"), t("norm.bias"), t("q_proj.weight"), t("q_proj.bias"),
                                   t("k_proj.weight"), t("k_proj.bias"), t("v_proj.weight"), t("v_proj.bias"),
                                   t("out_proj.weight"), t("out_proj.bias"))
        _check(load().pp_readers_attach(self.handle, ctypes.byref(cfg), arr))

    def write_memory(self, rows, slot0=0, stream=None):
        n = rows.shape[0]
        _check(load().pp_readers_write(self.handle, _ptr(rows), int(slot0), int(n), _stream(stream)))

    def set_visible(self, n_visible):
        _check(load().pp_readers_set_visible(self.handle, int(n_visible)))

    def trace(self, layer, repeat=1):
        _check(load().pp_temporal_trace(self.handle, int(layer), int(repeat)))

    def trace_read(self):
        n, us = ctypes.c_int64(), ctypes.c_double()
        _check(load().pp_temporal_trace_read(self.handle, ctypes.byref(n), ctypes.byref(us)))
        return n.value, us.value


class KV:
    """pp_kv_alloc: the session's temporal ring."""

    def __init__(self, model, batch=1):
        self.model = model
        h = ctypes.c_void_p()
        _check(load().pp_kv_alloc(model.handle, int(batch), ctypes.byref(h)))
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            _check(load().pp_kv_free(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self):
        _check(load().pp_kv_reset(self.handle))

    def info(self):
        pos, nb = ctypes.c_int64(), ctypes.c_uint64()
        _check(load().pp_kv_info(self.handle, ctypes.byref(pos), ctypes.byref(nb)))
        return pos.value, nb.value

    def load(self, src, n_frames, stream=None):
        _check(load().pp_kv_load(self.handle, _ptr(src), int(n_frames), _stream(stream)))

    def store(self, dst, stream=None):
        _check(load().pp_kv_store(self.handle, _ptr(dst), _stream(stream)))

    def restore(self, src, position, stream=None):
        _check(load().pp_kv_restore(self.handle, _ptr(src), int(position), _stream(stream)))


# ----------------------------------------------------------------------------- depth

class Depformer:
    """pp_depformer_create over device tensors named as in the constructor
    (depformer_in.{q}.weight, depformer_text_emb.weight, depformer_emb.{q}.weight,
    depformer.layers.{m}.*, linears.{q}.weight)."""

    def __init__(self, cfg, weights, wdtype):
        lib = load()
        self.cfg = dict(cfg)
        self._w = weights
        S, L = cfg["n_steps"], cfg["n_layers"]
        c = DepthConfig(cfg["n_layers"], cfg["d_model"], cfg["n_heads"], cfg["d_head"], cfg["d_ff"],
                        cfg["n_steps"], cfg["window"], cfg["text_vocab"], cfg["audio_vocab"], cfg["n_out"],
                        cfg["d_temporal"], PP_BF16 if wdtype == "bf16" else PP_F32, cfg["eps"])
        lw = lambda n: [weights["depformer.layers.%d.%s" % (m, n)] for m in range(L)]
        a = dict(
            inp=_ptr_array([weights["depformer_in.%d.weight" % q] for q in range(S)]),
            emb=_ptr_array([weights["depformer_emb.%d.weight" % q] for q in range(S - 1)]),
            qkv=_ptr_array(lw("self_attn.in_proj_weight")), o=_ptr_array(lw("self_attn.out_proj.weight")),
            win=_ptr_array([weights["depformer.layers.%d.gating.%d.linear_in.weight" % (m, q)]
                            for m in range(L) for q in range(S)]),
            wout=_ptr_array([weights["depformer.layers.%d.gating.%d.linear_out.weight" % (m, q)]
                             for m in range(L) for q in range(S)]),
            n1=_ptr_array(lw("norm1.alpha")), n2=_ptr_array(lw("norm2.alpha")),
            head=_ptr_array([weights["linears.%d.weight" % q] for q in range(S)]))
        self._arrays = a
        cast = lambda x: ctypes.cast(x, ctypes.POINTER(ctypes.c_void_p))
        w = DepthWeights(cast(a["inp"]), weights["depformer_text_emb.weight"].data_ptr(), cast(a["emb"]),
                         cast(a["qkv"]), cast(a["o"]), cast(a["win"]), cast(a["wout"]), cast(a["n1"]),
                         cast(a["n2"]), cast(a["head"]))
        h = ctypes.c_void_p()
        _check(lib.pp_depformer_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h)))
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            _check(load().pp_depformer_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_graph(self, enable):
        _check(load().pp_depformer_set_graph(self.handle, 1 if enable else 0))

    def step(self, h, text_token, codes_out, forced=None, logits_out=None, stream=None):
        tt, tp = _ids(np.atleast_1d(np.asarray(text_token, np.int32)))
        if forced is not None:
            fa, fp = _ids(np.asarray(forced, np.int32))
        else:
            fp = None
        _check(load().pp_depformer_step(self.handle, _ptr(h), tp, fp, 1, _ptr(codes_out), _ptr(logits_out),
                                        _stream(stream)))


# ----------------------------------------------------------------------------- sampling / generator

def sample_top_k(logits, temperature, top_k, uniforms, out, stream=None):
    """pp_sample_top_k over a [rows, n] float32 CUDA tensor; uniforms: float64 CUDA tensor
    [rows] or None; out: int32 CUDA tensor [rows]."""
    rows, n = (1, logits.shape[0]) if logits.dim() == 1 else tuple(logits.shape)
    _check(load().pp_sample_top_k(_ptr(logits), int(rows), int(n), float(temperature), int(top_k),
                                  _ptr(uniforms), _ptr(out), _stream(stream)))


# Released-path generator defaults: delays per stream (text, agent codebooks 0..7, user
# codebooks 0..7), initial tokens, text and audio sampling.
GENERATOR_DEFAULTS = dict(delays=(0, 0, 1, 1, 1, 1, 1, 1, 1, 0, 1, 1, 1, 1, 1, 1, 1), text_initial=32000,
                          audio_initial=2048, text_temperature=0.7, text_top_k=25, audio_temperature=0.8,
                          audio_top_k=250)


class Generator:
    """pp_generator_create over a TemporalModel, its KV ring and a Depformer (kept alive)."""

    def __init__(self, model, kv, depformer, **overrides):
        p = dict(GENERATOR_DEFAULTS)
        p.update(overrides)
        self._keep = (model, kv, depformer)
        d = list(p["delays"])
        c = GeneratorConfig(len(d), (ctypes.c_int32 * 32)(*d), p["text_initial"], p["audio_initial"],
                            p["text_temperature"], p["text_top_k"], p["audio_temperature"], p["audio_top_k"])
        self.n = len(d)
        h = ctypes.c_void_p()
        _check(load().pp_generator_create(model.handle, kv.handle, depformer.handle, ctypes.byref(c),
                                          ctypes.byref(h)))
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            _check(load().pp_generator_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def step(self, provided=None, uniforms=None, out=None, stream=None):
        """Returns True when `out` (int32 CUDA tensor [n_streams]) received an aligned frame."""
        pp_ = None
        if provided is not None:
            pa, pp_ = _ids(np.asarray(provided, np.int32))
        up = None
        if uniforms is not None:
            ua = np.ascontiguousarray(uniforms, np.float64)
            up = ua.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
        has = ctypes.c_int32()
        _check(load().pp_generator_step(self.handle, pp_, up, _ptr(out), ctypes.byref(has), _stream(stream)))
        return bool(has.value)

    def inspect(self, inputs=None, chosen=None, text_logits=None, depth_logits=None, stream=None):
        _check(load().pp_generator_inspect(self.handle, _ptr(inputs), _ptr(chosen), _ptr(text_logits),
                                           _ptr(depth_logits), _stream(stream)))


    def info(self):
        cur, nb = ctypes.c_int64(), ctypes.c_uint64()
        _check(load().pp_generator_info(self.handle, ctypes.byref(cur), ctypes.byref(nb)))
        return cur.value, nb.value

    def store(self, dst, stream=None):
        _check(load().pp_generator_store(self.handle, _ptr(dst), _stream(stream)))

    def restore(self, src, cursor, stream=None):
        _check(load().pp_generator_restore(self.handle, _ptr(src), int(cursor), _stream(stream)))
