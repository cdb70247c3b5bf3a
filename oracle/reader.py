"""Oracle for the memory readers inserted into the temporal stack (fp64, NumPy, CPU).

TEST INFRASTRUCTURE ONLY -- see the package docstring. Never called by the library.

Source: "Current sequence memory: one writer, four readers" (PersonaPlex + Inkling page),
sections 1 'Exact configuration' and 6 'Four independent readers': a reader sits after a
temporal block (zero-based 7, 15, 23, 31 in the released configuration) and adds to the
residual stream z

    x = LayerNorm(z)                        affine, over the model width
    Q = W_Q x + b_Q ;  K = W_K m + b_K ;  V = W_V m + b_V    for every visible memory row m
    A = softmax over the visible rows of (Q_h . K_h / sqrt(d_head))   per head h
    r = W_O concat_h(A V) + b_O ;  r = 0 when no memory row is visible
    z_out = z + r

with d_model / d_head heads (32 x 128 at full size). Readings (the page leaves them open):
the LayerNorm epsilon is 1e-5 (the value the page gives for the writer's LayerNorms);
visibility is a prefix of the bank (the first n rows); the memory bank arrives as given
(the writer that builds it is out of scope); weights are named readers.{i}.norm.weight /
.bias, .q_proj, .k_proj, .v_proj, .out_proj (.weight [out, in], .bias).
"""

import numpy as np

from .temporal import f64

LN_EPS = 1e-5


def layernorm(v, w, b, eps=LN_EPS):
    """(v - mean(v)) / sqrt(var(v) + eps) * w + b, population variance, over the last axis."""
    v = np.asarray(v, np.float64)
    mu = v.mean(axis=-1, keepdims=True)
    var = ((v - mu) ** 2).mean(axis=-1, keepdims=True)
    return (v - mu) / np.sqrt(var + eps) * f64(w) + f64(b)


def reader_kv(M, R, i):
    """Keys and values of memory rows M [n, mem_dim] for reader i: [n, D] each."""
    p = "readers.%d." % i
    M = f64(M)
    K = M @ f64(R[p + "k_proj.weight"]).T + f64(R[p + "k_proj.bias"])
    V = M @ f64(R[p + "v_proj.weight"]).T + f64(R[p + "v_proj.bias"])
    return K, V


def reader(z, M, n_visible, R, i, n_heads, eps=LN_EPS):
    """z [D] -> z + r for reader i over the first n_visible rows of the memory bank M."""
    z = np.asarray(z, np.float64)
    if n_visible <= 0:
        return z.copy()                       # empty memory adds exactly nothing
    p = "readers.%d." % i
    D = z.shape[0]
    dh = D // n_heads
    x = layernorm(z, R[p + "norm.weight"], R[p + "norm.bias"], eps)
    q = f64(R[p + "q_proj.weight"]) @ x + f64(R[p + "q_proj.bias"])
    K, V = reader_kv(np.asarray(M)[:n_visible], R, i)
    o = np.empty(D)
    for h in range(n_heads):
        sl = slice(h * dh, (h + 1) * dh)
        s = K[:, sl] @ q[sl] / np.sqrt(dh)
        w = np.exp(s - s.max())
        o[sl] = (w / w.sum()) @ V[:, sl]
    r = f64(R[p + "out_proj.weight"]) @ o + f64(R[p + "out_proj.bias"])
    return z + r


def hooks(blocks, M, n_visible, R, n_heads):
    """{block: f} for the temporal oracle's after_block argument: reader i after blocks[i]."""
    return {b: (lambda z, i=i: reader(z, M, n_visible, R, i, n_heads)) for i, b in enumerate(blocks)}
