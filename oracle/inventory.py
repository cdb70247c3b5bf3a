"""Oracle for the constructor's tensor inventory and cache sizes (integer arithmetic).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source: "PersonaPlex native LM audit" (Clockless Inkling), section 5 "Complete
constructor-derived parameter inventory" (shapes in [out, in] orientation), section 3
(gated hidden width = 2 * dim_feedforward / 3) and section 6 "Three distinct caches"
(temporal ring [2, B, 32, 3000, 128] per layer; depth cache [2, B, 16, 16, 64] per
layer). The shapes are written out from the block definitions, not from the page's
family table, so that the table's printed counts pin them.
"""


def gated_hidden(dim_feedforward):
    """ActivationGating's hidden width: 2 * dim_feedforward / 3 (exact integer)."""
    assert (2 * dim_feedforward) % 3 == 0
    return 2 * dim_feedforward // 3


def temporal_tensors(n_layers=32, d_model=4096, text_vocab=32001, audio_vocab=2049,
                     n_audio=16, dim_feedforward=16896):
    """[(name, shape)] of the temporal model: embeddings, blocks, final norm, text head."""
    D, F = d_model, gated_hidden(dim_feedforward)
    out = [("emb.%d.weight" % i, (audio_vocab, D)) for i in range(n_audio)]
    out.append(("text_emb.weight", (text_vocab, D)))
    out.append(("text_linear.weight", (text_vocab - 1, D)))   # 32000 classes: no initial-ID row
    for l in range(n_layers):
        p = "transformer.layers.%d." % l
        out += [(p + "self_attn.in_proj_weight", (3 * D, D)),
                (p + "self_attn.out_proj.weight", (D, D)),
                (p + "gating.linear_in.weight", (2 * F, D)),
                (p + "gating.linear_out.weight", (D, F)),
                (p + "norm1.alpha", (1, 1, D)),
                (p + "norm2.alpha", (1, 1, D))]
    out.append(("out_norm.alpha", (1, 1, D)))
    return out


def depth_tensors(n_steps=16, n_layers=6, d_model=1024, d_temporal=4096, text_vocab=32001,
                  audio_vocab=2049, n_out=2048, dim_feedforward=4224):
    """[(name, shape)] of the depth transformer with weights_per_step = n_steps."""
    D, F = d_model, gated_hidden(dim_feedforward)
    out = [("depformer_in.%d.weight" % q, (D, d_temporal)) for q in range(n_steps)]
    out += [("depformer_emb.%d.weight" % q, (audio_vocab, D)) for q in range(n_steps - 1)]
    out.append(("depformer_text_emb.weight", (text_vocab, D)))
    for m in range(n_layers):
        p = "depformer.layers.%d." % m
        out += [(p + "self_attn.in_proj_weight", (n_steps * 3 * D, D)),
                (p + "self_attn.out_proj.weight", (n_steps * D, D))]
        out += [(p + "gating.%d.linear_in.weight" % q, (2 * F, D)) for q in range(n_steps)]
        out += [(p + "gating.%d.linear_out.weight" % q, (D, F)) for q in range(n_steps)]
        out += [(p + "norm1.alpha", (1, 1, D)), (p + "norm2.alpha", (1, 1, D))]
    out += [("linears.%d.weight" % q, (n_out, D)) for q in range(n_steps)]
    return out


def numel(shape):
    n = 1
    for s in shape:
        n *= s
    return n


def total_params(tensors):
    return sum(numel(s) for _, s in tensors)


def temporal_kv_bytes(batch=1, n_heads=32, context=3000, d_head=128, n_layers=32, elem_bytes=2):
    """Bytes of the temporal rings: n_layers x [2, B, H, context, d_head]."""
    return n_layers * 2 * batch * n_heads * context * d_head * elem_bytes


def depth_kv_bytes(batch=1, n_heads=16, n_steps=16, d_head=64, n_layers=6, elem_bytes=2):
    """Bytes of the depth caches: n_layers x [2, B, H, n_steps, d_head]."""
    return n_layers * 2 * batch * n_heads * n_steps * d_head * elem_bytes


def kv_bytes_per_frame(d_model=4096, n_layers=32, elem_bytes=2):
    """K and V of one new position across all layers."""
    return 2 * d_model * elem_bytes * n_layers
