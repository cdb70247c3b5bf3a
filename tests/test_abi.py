"""CPU-only checks of the C ABI: the library loads, exports every entry point that
include/pp.h declares, and rejects bad arguments on the host before touching a device."""

import ctypes
import os
import re

import pytest

from personaplex_temporal_transformer_amd import pp, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "pp.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pp_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = pp.load()
    names = declared_symbols()
    assert len(names) >= 18
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(pp.EXPORTS) == names


def _cfg(**kw):
    c = dict(synth.TINY_TEMPORAL)
    c.update(kw)
    return pp.TemporalConfig(c["n_layers"], c["d_model"], c["n_heads"], c["d_head"], c["d_ff"], c["context"],
                             c["text_vocab"], c["audio_vocab"], c["n_audio"], kw.get("wdtype", pp.PP_F32),
                             c["rope_theta"], c["eps"])


@pytest.mark.parametrize("kw,status", [
    (dict(d_head=32, n_heads=8), pp.PP_E_ARG),      # unsupported head width
    (dict(n_heads=3), pp.PP_E_ARG),                 # d_model != heads * d_head
    (dict(d_ff=700), pp.PP_E_ARG),                  # not a multiple of 8
    (dict(wdtype=7), pp.PP_E_DTYPE),
    (dict(n_layers=0), pp.PP_E_ARG),
])
def test_create_rejects_bad_config_on_host(kw, status):
    lib = pp.load()
    c = _cfg(**kw)
    w = pp.TemporalWeights()
    h = ctypes.c_void_p()
    st = lib.pp_temporal_create(ctypes.byref(c), ctypes.byref(w), 1, 0, ctypes.byref(h))
    assert st == status
    assert not h.value
    assert lib.pp_last_error()


def test_null_handles_are_argument_errors():
    lib = pp.load()
    assert lib.pp_kv_reset(None) == pp.PP_E_ARG
    assert lib.pp_kv_free(None) == pp.PP_E_ARG
    assert lib.pp_temporal_destroy(None) == pp.PP_E_ARG
    assert lib.pp_temporal_decode_step(None, None, None, None, None, None) == pp.PP_E_ARG
    assert lib.pp_depformer_step(None, None, None, None, 1, None, None, None) == pp.PP_E_ARG
    assert lib.pp_temporal_trace(None, 0, 1) == pp.PP_E_ARG
    assert lib.pp_temporal_set_attn_splits(None, 0) == pp.PP_E_ARG
    assert lib.pp_temporal_decode_step_noalloc(None, None, None, None, None, None) == pp.PP_E_ARG
    assert lib.pp_temporal_trace_read(None, None, None) == pp.PP_E_ARG
    assert b"NULL" in lib.pp_last_error() or lib.pp_last_error()


def test_batch_above_one_is_rejected():
    lib = pp.load()
    c = _cfg()
    w = pp.TemporalWeights()
    h = ctypes.c_void_p()
    assert lib.pp_temporal_create(ctypes.byref(c), ctypes.byref(w), 2, 0, ctypes.byref(h)) == pp.PP_E_ARG
