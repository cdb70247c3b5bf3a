"""The float16 operands of the matrix-core paths (prefill, batched decode) for weights and
activations beyond float16's range: the library scales every float16 weight copy and every
float16 activation by powers of two chosen at create time (from bounds that hold for any
input) and undoes them in float32, so these models must still meet the oracle at the bf16
bar (max |err| / max |ref| <= 2e-2).

  * large norm scales: the first norm's 1e5 makes the normalised rows entering QKV and the
    values V exceed float16's 65504 (the Q and K rows are scaled by 2^-17 so that attention
    scores stay of order one: with scores of order 1e5 the softmax is a hard argmax whose
    near-ties no 16- or 32-bit rounding reproduces); the second norm's 1e3 makes the SiLU
    products ~1e5; the output norm's 1e3 the rows entering the text head;
  * weights scaled by 2^20 (W_in: above 65504) and 2^-20 (W_out: below float16's smallest
    subnormal, 2^-24) and 2^-12 (W_QKV: inside the subnormal range)."""

import numpy as np
import pytest

from oracle import temporal as O
from personaplex_temporal_transformer_amd import pp, synth
from tests.helpers import norm_max_err, require_gpu, to_device

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


def _scaled(W, name, factor):
    """bfloat16 bits times a power of two (exact)."""
    return synth.to_bf16_bits(synth.bf16_bits_to_f32(W[name]) * np.float32(factor))


def _extreme_weights(kind):
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 150, "bf16", with_text_head=True)
    for l in range(cfg["n_layers"]):
        p = "transformer.layers.%d." % l
        if kind == "alpha":
            D = cfg["d_model"]
            W[p + "norm1.alpha"] = (W[p + "norm1.alpha"] * 1e5).astype(np.float32)
            W[p + "norm2.alpha"] = (W[p + "norm2.alpha"] * 1e3).astype(np.float32)
            qkv = synth.bf16_bits_to_f32(W[p + "self_attn.in_proj_weight"])
            qkv[:2 * D] *= np.float32(2.0 ** -17)
            W[p + "self_attn.in_proj_weight"] = synth.to_bf16_bits(qkv)
        else:
            W[p + "gating.linear_in.weight"] = _scaled(W, p + "gating.linear_in.weight", 2.0 ** 20)
            W[p + "gating.linear_out.weight"] = _scaled(W, p + "gating.linear_out.weight", 2.0 ** -20)
            W[p + "self_attn.in_proj_weight"] = _scaled(W, p + "self_attn.in_proj_weight", 2.0 ** -12)
    if kind == "alpha":
        W["out_norm.alpha"] = (W["out_norm.alpha"] * 1000.0).astype(np.float32)
    return cfg, W


@pytest.mark.parametrize("kind", ["alpha", "weights"])
def test_prefill_and_chunk_beyond_float16_range(kind):
    import torch
    require_gpu()
    cfg, W = _extreme_weights(kind)
    ids = synth.stream_ids(cfg, 200, 151)
    model = pp.TemporalModel(cfg, to_device(W), "bf16", max_prefill_T=256)
    kv = model.kv_alloc()
    h = torch.empty((200, cfg["d_model"]), device="cuda")
    model.prefill(kv, ids[:150], h[:150])
    model.prefill(kv, ids[150:], h[150:])          # a chunk over the history just written
    torch.cuda.synchronize()
    got = h.cpu().numpy()
    assert np.all(np.isfinite(got))
    want = O.forward_full(ids, W, cfg)
    e0, e1 = norm_max_err(got[:150], want[:150]), norm_max_err(got[150:], want[150:])
    print("%s: prefill err %.3g, chunk err %.3g" % (kind, e0, e1))
    assert e0 <= BF16_TOL and e1 <= BF16_TOL


@pytest.mark.parametrize("kind", ["alpha", "weights"])
def test_batched_decode_beyond_float16_range(kind):
    import torch
    require_gpu()
    cfg, W = _extreme_weights(kind)
    B, n = 4, 4
    ids = synth.stream_ids(cfg, n, 152, batch=B)
    model = pp.TemporalModel(cfg, to_device(W), "bf16", max_batch=B)
    kv = model.kv_alloc(B)
    h = torch.empty((n, B, cfg["d_model"]), device="cuda")
    lg = torch.empty((n, B, cfg["text_vocab"] - 1), device="cuda")
    for t in range(n):
        model.decode_step(kv, ids[:, t], h[t], lg[t])
    torch.cuda.synchronize()
    hn, ln = h.cpu().numpy(), lg.cpu().numpy()
    assert np.all(np.isfinite(hn)) and np.all(np.isfinite(ln))
    worst = 0.0
    for b in range(B):
        hs, lw = O.decode_incremental(ids[b], W, cfg, with_logits=True)
        worst = max(worst, norm_max_err(hn[:, b], hs), norm_max_err(ln[:, b], lw))
    print("%s: batched decode worst err %.3g" % (kind, worst))
    assert worst <= BF16_TOL


def test_non_finite_weight_rejected_for_float16_paths():
    require_gpu()
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 153, "bf16", with_text_head=False)
    w = W["transformer.layers.1.gating.linear_out.weight"].copy()
    w[3, 5] = 0x7F80                                  # bfloat16 +inf
    W["transformer.layers.1.gating.linear_out.weight"] = w
    dW = to_device(W)
    with pytest.raises(pp.PPError) as e:
        pp.TemporalModel(cfg, dW, "bf16", max_prefill_T=16)
    assert e.value.status == pp.PP_E_ARG
    pp.TemporalModel(cfg, dW, "bf16").close()         # decode alone keeps float32 activations
