"""Pins of the memory-reader oracle ("Current sequence memory: one writer, four readers",
section 6): exact identity with zero output projections or an empty memory, the
one-row closed form, softmax weights fixed by construction (which pins the 1/sqrt(d_head)
scale and the head split), LayerNorm closed forms, invariance to the order of memory rows,
and placement after the named blocks."""

import math

import numpy as np

from oracle import reader as ORD
from oracle import temporal as O
from personaplex_temporal_transformer_amd import synth

CFG = synth.TINY_TEMPORAL
H = CFG["n_heads"]
D = CFG["d_model"]
DH = D // H


def _setup(seed=0, mem_dim=32, n=9, zero_out=False, scale=0.1):
    R = synth.reader_weights(CFG, 2, mem_dim, seed, "fp32", scale=scale, zero_out=zero_out)
    M = synth.memory_bank(n, mem_dim, seed + 1, "fp32")
    z = synth.hidden(D, seed + 2)
    return R, M, z


def test_layernorm_closed_forms():
    v = np.array([1.0, -1.0] * 8)
    w, b = np.ones(16), np.zeros(16)
    got = ORD.layernorm(v, w, b)
    assert np.allclose(got, v / math.sqrt(1.0 + ORD.LN_EPS), atol=1e-15)
    g = np.random.default_rng(0)
    u = g.normal(size=64)
    w2, b2 = g.normal(size=64), g.normal(size=64)
    assert np.allclose(ORD.layernorm(u + 7.5, w2, b2), ORD.layernorm(u, w2, b2), atol=1e-12)
    assert np.allclose(ORD.layernorm(np.full(64, 3.0), w2, b2), b2, atol=1e-12)   # constant -> bias


def test_zero_output_projection_and_empty_memory_are_exact_identity():
    R, M, z = _setup(zero_out=True)
    assert np.array_equal(ORD.reader(z, M, 9, R, 0, H), z)
    R2, M2, z2 = _setup(seed=3)
    assert np.array_equal(ORD.reader(z2, M2, 0, R2, 1, H), z2)
    assert not np.allclose(ORD.reader(z2, M2, 9, R2, 1, H), z2)


def test_one_visible_row_closed_form():
    """softmax over a single row is 1: r = W_O (W_V m + b_V) + b_O whatever Q and K are."""
    R, M, z = _setup(seed=4)
    p = "readers.1."
    v = R[p + "v_proj.weight"].astype(np.float64) @ M[0] + R[p + "v_proj.bias"]
    want = z + R[p + "out_proj.weight"].astype(np.float64) @ v + R[p + "out_proj.bias"]
    assert np.allclose(ORD.reader(z, M, 1, R, 1, H), want, atol=1e-12)
    # two identical rows give the same result
    M2 = np.stack([M[0], M[0]])
    assert np.allclose(ORD.reader(z, M2, 2, R, 1, H), want, atol=1e-12)


def test_softmax_weights_by_construction():
    """Identity K/V/O maps and a fixed query: for head 0 the two rows' scores differ by
    sqrt(d_head) * ln 3 / sqrt(d_head) = ln 3 after the 1/sqrt(d_head) scale, so the output
    of head 0 is 3/4 m1 + 1/4 m2; other heads see equal scores and average."""
    R = {}
    p = "readers.0."
    R[p + "norm.weight"], R[p + "norm.bias"] = np.ones(D), np.zeros(D)
    R[p + "q_proj.weight"] = np.zeros((D, D))
    q = np.zeros(D)
    q[0] = 1.0
    R[p + "q_proj.bias"] = q
    for name in ("k_proj", "v_proj", "out_proj"):
        R[p + name + ".weight"] = np.eye(D)
        R[p + name + ".bias"] = np.zeros(D)
    g = np.random.default_rng(5)
    m1, m2 = g.normal(size=D), g.normal(size=D)
    m1[0] = m2[0] + math.sqrt(DH) * math.log(3.0)
    z = g.normal(size=D)
    out = ORD.reader(z, np.stack([m1, m2]), 2, R, 0, H) - z
    assert np.allclose(out[:DH], 0.75 * m1[:DH] + 0.25 * m2[:DH], atol=1e-12)
    assert np.allclose(out[DH:], 0.5 * (m1[DH:] + m2[DH:]), atol=1e-12)
    # values projected by 2 I, keys still by I: the weights stay 3/4, 1/4 and the output
    # doubles (keys taken from the value projection would square the odds to 9 : 1)
    R[p + "v_proj.weight"] = 2.0 * np.eye(D)
    out2 = ORD.reader(z, np.stack([m1, m2]), 2, R, 0, H) - z
    assert np.allclose(out2[:DH], 2.0 * (0.75 * m1[:DH] + 0.25 * m2[:DH]), atol=1e-12)


def test_row_order_invariance_and_prefix_visibility():
    R, M, z = _setup(seed=6)
    perm = np.random.default_rng(1).permutation(9)
    assert np.allclose(ORD.reader(z, M, 9, R, 0, H), ORD.reader(z, M[perm], 9, R, 0, H), atol=1e-12)
    # only the first n rows count: changing row 5 leaves n = 5 unchanged
    M2 = M.copy()
    M2[5] += 10.0
    assert np.array_equal(ORD.reader(z, M, 5, R, 0, H), ORD.reader(z, M2, 5, R, 0, H))
    assert not np.allclose(ORD.reader(z, M, 6, R, 0, H), ORD.reader(z, M2, 6, R, 0, H))


def test_placement_in_the_stack():
    W = synth.temporal_weights(CFG, 7, "fp32", with_text_head=False)
    ids = synth.stream_ids(CFG, 3, 8)
    R, M, _ = _setup(seed=9)
    base = O.forward_full(ids, W, CFG)
    R0, _, _ = _setup(seed=9, zero_out=True)
    assert np.array_equal(O.forward_full(ids, W, CFG, after_block=ORD.hooks([0, 1], M, 9, R0, H)), base)
    a = O.forward_full(ids, W, CFG, after_block=ORD.hooks([0], M, 9, R, H))
    b = O.forward_full(ids, W, CFG, after_block={1: ORD.hooks([1], M, 9, R, H)[1]})
    assert not np.allclose(a, base) and not np.allclose(b, base) and not np.allclose(a, b)
    # the incremental decode applies the same readers at the same places
    inc = O.decode_incremental(ids, W, CFG, after_block=ORD.hooks([0], M, 9, R, H))
    assert np.allclose(inc, a, atol=1e-12)
