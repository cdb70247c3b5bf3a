"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake -- a swapped operand, a wrong index, a dropped
term, a wrong scale, window, delay or tie rule -- in a temporary copy of the oracle
package, points every pin module (temporal, depth, generator, reader, sampler, ring and
inventory) at that copy and requires at least one pin to fail. The real oracle is never modified; the
copies live under pytest's tmp_path."""

import importlib.util
import inspect
import itertools
import os
import shutil
import sys

import pytest

from tests import test_oracle_depformer as PIN_DEPTH
from tests import test_oracle_generator as PIN_GEN
from tests import test_oracle_inventory as PIN_INVENTORY
from tests import test_oracle_reader as PIN_READER
from tests import test_oracle_sampling as PIN_SAMPLING
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
    # temporal: RoPE frequencies, the -1 rule, norms, masks, the cache, the text head
    ("RoPE frequency j/d_head instead of 2j/d_head", "temporal.py",
     "math.log(theta) * 2.0 * j / d_head", "math.log(theta) * j / d_head"),
    ("ID -1 reads the last table row", "temporal.py",
     "            if int(i) != -1:\n                x = x + f64(",
     "            if True:\n                x = x + f64("),
    ("final norm dropped (full sequence)", "temporal.py",
     'h = rmsnorm(X, W["out_norm.alpha"], cfg["eps"])', "h = X"),
    ("final norm dropped on both paths", [
        ("temporal.py", 'h = rmsnorm(X, W["out_norm.alpha"], cfg["eps"])', "h = X"),
        ("temporal.py", 'h = rmsnorm(x, W["out_norm.alpha"], cfg["eps"])', "h = x")]),
    ("RMSNorm subtracts the mean", "temporal.py",
     "ms = np.mean(v * v, axis=-1, keepdims=True)", "ms = np.var(v, axis=-1, keepdims=True)"),
    ("causal mask excludes the query's own position", "temporal.py",
     "allowed = (delta >= 0) & (delta < window)", "allowed = (delta >= 0) & (delta < window) & (delta != 0)"),
    ("decode sees one key fewer", "temporal.py",
     "kpos, Ks, Vs = cache.visible(l, pos, C)", "kpos, Ks, Vs = cache.visible(l, pos, C - 1)"),
    ("block FFN residual dropped (full sequence)", "temporal.py",
     'return y + swiglu(gz, F) @ f64(_lw(W, l, "gating.linear_out.weight")).T',
     'return swiglu(gz, F) @ f64(_lw(W, l, "gating.linear_out.weight")).T'),
    ("norm2 takes norm1's scale on both paths", [
        ("temporal.py", 'gz = rmsnorm(y, _lw(W, l, "norm2.alpha"), eps) @',
         'gz = rmsnorm(y, _lw(W, l, "norm1.alpha"), eps) @'),
        ("temporal.py", '@ rmsnorm(y, _lw(W, l, "norm2.alpha"), eps)',
         '@ rmsnorm(y, _lw(W, l, "norm1.alpha"), eps)')]),
    ("text head on the residual before the final norm", "temporal.py",
     'return h, f64(W["text_linear.weight"]) @ h', 'return h, f64(W["text_linear.weight"]) @ x'),
    # depth: per-position slices, residuals, norms
    ("depth head of position q+1", "depformer.py",
     'W["linears.%d.weight" % q]', 'W["linears.%d.weight" % ((q + 1) % S)]'),
    ("depth in-projection of position 0 everywhere", "depformer.py",
     'W["depformer_in.%d.weight" % q]', 'W["depformer_in.%d.weight" % 0]'),
    ("depth QKV slice 0 at every position", "depformer.py",
     "[q * 3 * D:(q + 1) * 3 * D]", "[0:3 * D]"),
    ("depth W_O slice 0 at every position", "depformer.py",
     "[q * D:(q + 1) * D]", "[0:D]"),
    ("depth attention residual dropped", "depformer.py",
     "z = z + wo @ o.reshape(D)", "z = wo @ o.reshape(D)"),
    ("depth FFN residual dropped", "depformer.py",
     'z = z + f64(W[pre + "gating.%d.linear_out.weight" % q])', 'z = f64(W[pre + "gating.%d.linear_out.weight" % q])'),
    ("depth norm2 takes norm1's scale", "depformer.py",
     'rmsnorm(z, W[pre + "norm2.alpha"], eps)', 'rmsnorm(z, W[pre + "norm1.alpha"], eps)'),
    ("depth text embedding ignored", "depformer.py",
     'e = f64(W["depformer_text_emb.weight"][int(text_token)])',
     'e = 0.0 * f64(W["depformer_text_emb.weight"][int(text_token)])'),
    # generator: delays, slots, flags, draws
    ("user codebook 0 delayed", "generator.py",
     "DELAYS = (0, 0, 1, 1, 1, 1, 1, 1, 1, 0, 1,", "DELAYS = (0, 0, 1, 1, 1, 1, 1, 1, 1, 1, 1,"),
    ("aligned output ignores the stream delay", "generator.py",
     "self.tok[k, (s - MAX_DELAY + DELAYS[k]) % RING]", "self.tok[k, (s - MAX_DELAY) % RING]"),
    ("provided flags never cleared", "generator.py",
     "self.prov[:, src] = False", "pass"),
    ("text draw takes the first depth uniform", "generator.py",
     "sample_top_k(text_logits, self.tt, self.tk, u[0])", "sample_top_k(text_logits, self.tt, self.tk, u[1])"),
    ("depth position q draws with uniform q", "generator.py",
     "return sample_top_k(lg, self.at, self.ak, u[k])", "return sample_top_k(lg, self.at, self.ak, u[q])"),
    ("supplied text does not condition the depth loop", "generator.py",
     "        if self.prov[0, tgt]:\n            text = int(self.tok[0, tgt])",
     "        if False:\n            text = int(self.tok[0, tgt])"),
    ("temporal input read from the target slot", "generator.py",
     "src, tgt = (s - 1) % RING, s % RING", "src, tgt = s % RING, s % RING"),
    ("initial text token 0", "generator.py", "TEXT_INITIAL = 32000", "TEXT_INITIAL = 0"),
    # sampler
    ("temperature multiplies the logits", "sampling.py",
     "/ np.float64(np.float32(temperature))", "* np.float64(np.float32(temperature))"),
    ("ties at the cut: higher index first", "sampling.py",
     "np.lexsort((idx, -l))", "np.lexsort((-idx, -l))"),
    ("draw boundary on the other side", "sampling.py", 'side="right"', 'side="left"'),
    ("one candidate past the top k", "sampling.py",
     "order[:max(1, min(int(top_k), l.shape[0]))]", "order[:max(1, min(int(top_k) + 1, l.shape[0]))]"),
    # memory readers
    ("reader LayerNorm without the mean", "reader.py",
     "return (v - mu) / np.sqrt(var + eps) * f64(w) + f64(b)", "return v / np.sqrt(var + eps) * f64(w) + f64(b)"),
    ("reader score scale 1/d_head", "reader.py",
     "s = K[:, sl] @ q[sl] / np.sqrt(dh)", "s = K[:, sl] @ q[sl] / dh"),
    ("reader residual dropped", "reader.py", "return z + r", "return r"),
    ("reader keys from the value projection", "reader.py",
     'K = M @ f64(R[p + "k_proj.weight"]).T', 'K = M @ f64(R[p + "v_proj.weight"]).T'),
    ("reader query bias dropped", "reader.py",
     'q = f64(R[p + "q_proj.weight"]) @ x + f64(R[p + "q_proj.bias"])', 'q = f64(R[p + "q_proj.weight"]) @ x'),
    # ring slots and the parameter inventory
    ("ring slot off by one", "ring.py", "return pos % capacity", "return (pos + 1) % capacity"),
    ("stated positions one lap late", "ring.py",
     "out.append(s + ((end_offset - 1 - s) // capacity) * capacity)",
     "out.append(s + ((end_offset - s) // capacity) * capacity)"),
    ("ring mask admits the context edge", "ring.py",
     "0 <= query - p < context]", "0 <= query - p <= context]"),
    ("gated hidden width of the full feed-forward", "inventory.py",
     "return 2 * dim_feedforward // 3", "return dim_feedforward"),
    ("text head with the initial-ID row", "inventory.py",
     '("text_linear.weight", (text_vocab - 1, D))', '("text_linear.weight", (text_vocab, D))'),
    ("depth embeddings for every position", "inventory.py",
     'for q in range(n_steps - 1)]', 'for q in range(n_steps)]'),
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


# Each pin module and the names it imported from the oracle: (attribute, submodule, member).
_PIN_MODULES = [
    (PIN_TEMPORAL, "temporal.py", [("O", "temporal", None)]),
    (PIN_DEPTH, "depformer.py", [("DF", "depformer", None)]),
    (PIN_GEN, "generator.py", [("OD", "depformer", None), ("OG", "generator", None), ("OT", "temporal", None),
                               ("sample_top_k", "sampling", "sample_top_k")]),
    (PIN_READER, "reader.py", [("ORD", "reader", None), ("O", "temporal", None)]),
    (PIN_SAMPLING, "sampling.py", [("sample_top_k", "sampling", "sample_top_k"),
                                   ("top_k_order", "sampling", "top_k_order")]),
    (PIN_INVENTORY, "inventory.py", [("inventory", "inventory", None), ("ring", "ring", None)]),
]


def _calls(mod):
    """Zero-argument calls of every pin in mod: parametrized pins once per value, the
    generator pins with their weights."""
    for n, f in sorted(vars(mod).items()):
        if not (n.startswith("test_") and callable(f)):
            continue
        params = list(inspect.signature(f).parameters)
        marks = [m for m in getattr(f, "pytestmark", []) if m.name == "parametrize"]
        name = "%s.%s" % (mod.__name__.split(".")[-1], n)
        if not params:
            yield name, f
        elif params == ["weights"]:
            yield name, (lambda f=f: f(PIN_GEN.make_weights()))
        elif len(marks) == 1 and params == [marks[0].args[0]]:
            for v in marks[0].args[1]:
                yield "%s[%r]" % (name, v), (lambda f=f, v=v: f(v))
        else:
            raise AssertionError("pin %s takes arguments the mutation check cannot supply" % name)


def _pins(first_file=None):
    """Every pin, those of the module that pins first_file first."""
    mods = sorted(_PIN_MODULES, key=lambda m: m[1] != first_file and not (first_file == "ring.py" and m[0] is PIN_INVENTORY))
    for mod, _, _ in mods:
        yield from _calls(mod)


def test_every_pin_passes_on_the_real_oracle():
    for _, f in _pins():
        f()


@pytest.mark.parametrize("case", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_fails_a_pin(case, tmp_path, monkeypatch):
    edits = case[1] if isinstance(case[1], list) else [case[1:]]
    mut = _mutant(tmp_path, edits)
    for mod, _, names in _PIN_MODULES:
        for attr, sub, member in names:
            target = getattr(mut, sub)
            monkeypatch.setattr(mod, attr, getattr(target, member) if member else target)
    for pin, f in _pins(edits[0][0]):
        try:
            f()
        except Exception:
            return                        # caught by this pin
    pytest.fail("no pin fails with the mutation planted")
