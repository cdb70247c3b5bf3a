"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake -- a swapped operand, a wrong index, a dropped
term, a wrong scale or window -- in a temporary copy of the oracle package, points the
pin modules at that copy and requires at least one pin to fail. The real oracle is never
modified; the copies live under pytest's tmp_path."""

import importlib.util
import inspect
import itertools
import os
import shutil
import sys

import pytest

from tests import test_oracle_depformer as PIN_DEPTH
from tests import test_oracle_temporal as PIN_TEMPORAL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, file in oracle/, text to replace, replacement); a case may list several edits
# as (name, [(file, old, new), ...]) when the same mistake sits on both code paths.
_QK_FULL = ("temporal.py",
            "Q = qkv[:, 0 * D:1 * D].reshape(T, H, dh)\n    K = qkv[:, 1 * D:2 * D].reshape(T, H, dh)",
            "Q = qkv[:, 1 * D:2 * D].reshape(T, H, dh)\n    K = qkv[:, 0 * D:1 * D].reshape(T, H, dh)")
_QK_INC = ("temporal.py",
           "q = rope(qkv[0 * D:1 * D].reshape(H, dh), pos, theta)\n        k = rope(qkv[1 * D:2 * D]",
           "q = rope(qkv[1 * D:2 * D].reshape(H, dh), pos, theta)\n        k = rope(qkv[0 * D:1 * D]")
_WO_FULL = ("temporal.py", '@ f64(_lw(W, l, "self_attn.out_proj.weight")).T',
            '@ f64(_lw(W, l, "self_attn.out_proj.weight"))')
_WO_INC = ("temporal.py", 'f64(_lw(W, l, "self_attn.out_proj.weight")) @ a.reshape(D)',
           'f64(_lw(W, l, "self_attn.out_proj.weight")).T @ a.reshape(D)')
MUTATIONS = [
    ("Q and K sections swapped on both paths", [_QK_FULL, _QK_INC]),
    ("W_O transposed on both paths", [_WO_FULL, _WO_INC]),
    ("W_in transposed on both paths", [
        ("temporal.py", '@ f64(_lw(W, l, "gating.linear_in.weight")).T',
         '@ f64(_lw(W, l, "gating.linear_in.weight"))'),
        ("temporal.py", 'gz = f64(_lw(W, l, "gating.linear_in.weight")) @',
         'gz = f64(_lw(W, l, "gating.linear_in.weight")).T @')]),
    ("block_full: K section read as Q", "temporal.py",
     "Q = qkv[:, 0 * D:1 * D].reshape(T, H, dh)\n    K = qkv[:, 1 * D:2 * D].reshape(T, H, dh)",
     "Q = qkv[:, 1 * D:2 * D].reshape(T, H, dh)\n    K = qkv[:, 0 * D:1 * D].reshape(T, H, dh)"),
    ("decode_step: K section read as Q", "temporal.py",
     "q = rope(qkv[0 * D:1 * D].reshape(H, dh), pos, theta)\n        k = rope(qkv[1 * D:2 * D]",
     "q = rope(qkv[1 * D:2 * D].reshape(H, dh), pos, theta)\n        k = rope(qkv[0 * D:1 * D]"),
    ("temporal score scale 1/d_head", "temporal.py",
     "s = (q @ k.T) / math.sqrt(q.shape[-1])", "s = (q @ k.T) / q.shape[-1]"),
    ("temporal window off by one", "temporal.py", "(delta < window)", "(delta <= window)"),
    ("RoPE rotation sign", "temporal.py",
     "out[..., 1::2] = x0 * s + x1 * c", "out[..., 1::2] = x1 * c - x0 * s"),
    ("RoPE pairs halves instead of adjacent", "temporal.py",
     "x0, x1 = x[..., 0::2], x[..., 1::2]", "x0, x1 = x[..., :d_head // 2], x[..., d_head // 2:]"),
    ("RMSNorm eps outside the root", "temporal.py",
     "np.sqrt(ms + eps)", "(np.sqrt(ms) + eps)"),
    ("temporal SwiGLU g/z swapped", "temporal.py",
     "g, z = gz[..., :hidden], gz[..., hidden:]", "z, g = gz[..., :hidden], gz[..., hidden:]"),
    ("W_O transposed (full sequence)", "temporal.py",
     '@ f64(_lw(W, l, "self_attn.out_proj.weight")).T', '@ f64(_lw(W, l, "self_attn.out_proj.weight"))'),
    ("decode residual dropped", "temporal.py",
     'y = x + f64(_lw(W, l, "self_attn.out_proj.weight")) @ a.reshape(D)',
     'y = f64(_lw(W, l, "self_attn.out_proj.weight")) @ a.reshape(D)'),
    ("stream k reads audio table k", "temporal.py",
     'W["emb.%d.weight" % (k - 1)]', 'W["emb.%d.weight" % (k % 16)]'),
    ("chunk ignores the history", "temporal.py",
     "hist = cache.visible(l, int(pos[-1]), C + T - 1)", "hist = None"),
    ("depth FFN g/z swapped", "depformer.py",
     "(silu(gz[:F]) * gz[F:])", "(silu(gz[F:]) * gz[:F])"),
    ("depth FFN of position q+1", "depformer.py",
     'W[pre + "gating.%d.linear_in.weight" % q]',
     'W[pre + "gating.%d.linear_in.weight" % ((q + 1) % S)]'),
    ("depth score scale 1/d_head", "depformer.py",
     "s = (ks @ q) / math.sqrt(q.shape[-1])", "s = (ks @ q) / q.shape[-1]"),
    ("depth K section read as Q", "depformer.py",
     "qh = qkv[0:D].reshape(H, dh)\n            kh = qkv[D:2 * D].reshape(H, dh)",
     "qh = qkv[D:2 * D].reshape(H, dh)\n            kh = qkv[0:D].reshape(H, dh)"),
    ("depth window off by one", "depformer.py", "0 <= q - i < win", "0 <= q - i <= win"),
    ("depth input embedding of position q", "depformer.py",
     'W["depformer_emb.%d.weight" % (q - 1)][prev]', 'W["depformer_emb.%d.weight" % (q % 15)][prev]'),
]

_counter = itertools.count()


def _mutant(tmp_path, edits):
    """Import a copy of the oracle package with the text replacements `edits` applied."""
    name = "oracle_mutant_%d" % next(_counter)
    dst = os.path.join(str(tmp_path), name)
    shutil.copytree(os.path.join(ROOT, "oracle"), dst,
                    ignore=shutil.ignore_patterns("__pycache__"))
    for fname, old, new in edits:
        path = os.path.join(dst, fname)
        with open(path) as f:
            src = f.read()
        assert src.count(old) == 1, "mutation site not found exactly once in %s: %r" % (fname, old)
        with open(path, "w") as f:
            f.write(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(
        name, os.path.join(dst, "__init__.py"), submodule_search_locations=[dst])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod
    spec.loader.exec_module(mod)
    return mod


def _pins():
    for mod in (PIN_TEMPORAL, PIN_DEPTH):
        for n, f in sorted(vars(mod).items()):
            if n.startswith("test_") and callable(f) and not inspect.signature(f).parameters:
                yield "%s.%s" % (mod.__name__.split(".")[-1], n), f


def test_every_pin_passes_on_the_real_oracle():
    for _, f in _pins():
        f()


@pytest.mark.parametrize("case", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_fails_a_pin(case, tmp_path, monkeypatch):
    edits = case[1] if isinstance(case[1], list) else [case[1:]]
    mut = _mutant(tmp_path, edits)
    monkeypatch.setattr(PIN_TEMPORAL, "O", mut.temporal)
    monkeypatch.setattr(PIN_DEPTH, "DF", mut.depformer)
    for pin, f in _pins():
        try:
            f()
        except Exception:
            return                        # caught by this pin
    pytest.fail("no pin fails with the mutation planted")
