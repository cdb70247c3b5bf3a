"""GPU parity of batched decode (several sessions sharing one position and every weight
byte of the step) against the oracle, through the C ABI. Each session is an independent
conversation: its outputs must equal the oracle's incremental decode of its own frames
(bf16 path tolerance: max |err| / max |ref| <= 2e-2, float16 activations into the matrix
cores as in prefill)."""

import numpy as np
import pytest

from oracle import temporal as O
from personaplex_temporal_transformer_amd import pp, synth
from tests.helpers import norm_max_err, require_gpu, to_device

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


def _run(cfg, W, B, ids, graph=True, logits=False, kv_frames=None):
    import torch
    require_gpu()
    model = pp.TemporalModel(cfg, to_device(W), "bf16", max_batch=B)
    model.set_graph(graph)
    kv = model.kv_alloc(B)
    if kv_frames is not None:
        kv.load(torch.from_numpy(kv_frames.view(np.int16)).cuda(), kv_frames.shape[-2])
    n = ids.shape[1]
    h = torch.empty((n, B, cfg["d_model"]), device="cuda")
    lg = torch.empty((n, B, cfg["text_vocab"] - 1), device="cuda") if logits else None
    for t in range(n):
        model.decode_step(kv, ids[:, t], h[t], None if lg is None else lg[t])
    torch.cuda.synchronize()
    return model, kv, h.cpu().numpy(), (lg.cpu().numpy() if logits else None)


@pytest.mark.parametrize("B", [2, 5, 8, 9, 16, 17, 40, 64])
def test_tiny_batched_matches_oracle_per_session(B):
    """B sessions of 5 frames from position 0; up to 8 sessions the QKV and W_in products
    form the row norm in their prologue (9 and more: a row-norm launch); 17, 40 and 64 (the
    maximum) sessions use 2, 3 and 4 tiles of 16."""
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 61, "bf16", with_text_head=True)
    ids = synth.stream_ids(cfg, 5, 62, batch=B)            # [B, 5, 17]
    _, kv, h, lg = _run(cfg, W, B, ids, logits=(B == 5))
    assert kv.info()[0] == 5
    worst = 0.0
    for b in range(B):
        hs, lw = O.decode_incremental(ids[b], W, cfg, with_logits=True)
        worst = max(worst, norm_max_err(h[:, b], hs))
        if lg is not None:
            worst = max(worst, norm_max_err(lg[:, b], lw))
    print("tiny batched B=%d: worst session err %.3g" % (B, worst))
    assert worst <= BF16_TOL


def test_tiny_batched_graph_equals_direct():
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 63, "bf16", with_text_head=False)
    ids = synth.stream_ids(cfg, 4, 64, batch=6)
    _, _, hg, _ = _run(cfg, W, 6, ids, graph=True)
    _, _, hd, _ = _run(cfg, W, 6, ids, graph=False)
    assert np.array_equal(hg, hd)


def test_full_width_batched_two_blocks_on_filled_rings():
    """Two 4096-wide blocks, 8 sessions, each ring pre-filled with 200 frames of its own;
    2 decode frames at positions 200, 201; sessions 0 and 7 against the oracle."""
    cfg = synth.with_(synth.FULL_TEMPORAL, n_layers=2)
    W = synth.temporal_weights(cfg, 65, "bf16", with_text_head=False, shared_layer=True)
    B, P = 8, 200
    frames = synth.cache_frames(cfg, P, 66, batch=B)       # [L, 2, B, H, P, dh] bf16 bits
    ids = synth.stream_ids(cfg, 2, 67, batch=B)
    _, kv, h, _ = _run(cfg, W, B, ids, kv_frames=frames)
    assert kv.info()[0] == P + 2
    for b in (0, 7):
        ks = [frames[l, 0, b].transpose(1, 0, 2) for l in range(2)]
        vs = [frames[l, 1, b].transpose(1, 0, 2) for l in range(2)]
        cache = O.cache_from_blocks(ks, vs, np.arange(P), 2)
        want = O.decode_incremental(ids[b], W, cfg, p0=P, cache=cache)
        err = norm_max_err(h[:, b], want)
        print("full-width batched session %d: err %.3g" % (b, err))
        assert err <= BF16_TOL


def test_batched_argument_errors():
    import torch
    require_gpu()
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 0, "fp32", with_text_head=False)
    with pytest.raises(pp.PPError):
        pp.TemporalModel(cfg, to_device(W), "fp32", max_batch=4)      # batched needs bf16
    Wb = synth.temporal_weights(cfg, 0, "bf16", with_text_head=False)
    with pytest.raises(pp.PPError):
        pp.TemporalModel(cfg, to_device(Wb), "bf16", max_batch=65)
    m = pp.TemporalModel(cfg, to_device(Wb), "bf16", max_batch=4)
    with pytest.raises(pp.PPError):
        m.kv_alloc(5)
    kv = m.kv_alloc(3)
    bad = synth.stream_ids(cfg, 1, 1, batch=3)[:, 0].copy()
    bad[2, 4] = -2
    with pytest.raises(pp.PPError) as e:
        m.decode_step(kv, bad, torch.empty((3, cfg["d_model"]), device="cuda"))
    assert e.value.status == pp.PP_E_ID
    assert kv.info()[0] == 0
