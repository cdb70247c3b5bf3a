"""GPU parity of the full-sequence (prefill) path of the temporal model against the
oracle, through the C ABI: T frames at positions 0..T-1 in one call, K/V left in ring
slots 0..T-1, decoding continuing at position T. Tolerances as for decode: max abs error
1e-4 on the fp32 path; max |err| / max |ref| <= 2e-2 on the bf16 path."""

import numpy as np
import pytest

from oracle import temporal as O
from personaplex_temporal_transformer_amd import pp, synth
from tests.helpers import max_abs_err, norm_max_err, require_gpu, to_device

pytestmark = pytest.mark.gpu

FP32_TOL = 1e-4
BF16_TOL = 2e-2


def _model(cfg, W, wdtype, max_T):
    require_gpu()
    return pp.TemporalModel(cfg, to_device(W), wdtype, max_prefill_T=max_T)


def _prefill(model, kv, ids):
    import torch
    h = torch.empty((ids.shape[0], model.cfg["d_model"]), dtype=torch.float32, device="cuda")
    model.prefill(kv, ids, h)
    torch.cuda.synchronize()
    return h.cpu().numpy()


def _ring(kv, dtype):
    import torch
    n = kv.info()[1] // (2 if dtype == "bf16" else 4)
    t = torch.empty(n, dtype=torch.int16 if dtype == "bf16" else torch.float32, device="cuda")
    kv.store(t)
    torch.cuda.synchronize()
    a = t.cpu().numpy()
    return a.view(np.uint16) if dtype == "bf16" else a


# ----------------------------------------------------------------------------- fp32, tiny

@pytest.mark.parametrize("T", [1, 37, 64, 200])
def test_tiny_fp32_prefill_matches_oracle(T):
    """T = 1 (a single frame), 37 (ragged against the 64-row tiles), 64, 200."""
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 21, "fp32", with_text_head=False)
    ids = synth.stream_ids(cfg, T, 22)
    model = _model(cfg, W, "fp32", 256)
    kv = model.kv_alloc()
    h = _prefill(model, kv, ids)
    want = O.forward_full(ids, W, cfg)
    err = max_abs_err(h, want)
    print("tiny fp32 prefill T=%d: err %.3g" % (T, err))
    assert err <= FP32_TOL
    assert kv.info()[0] == T


def test_tiny_fp32_prefill_then_decode_continues():
    """Prefill 50 frames, decode 6 more: the 56 outputs match one oracle pass over all
    56 frames, and the ring slots 0..49 hold the keys/values decoding would have written."""
    import torch
    cfg = synth.with_(synth.TINY_TEMPORAL, context=64)
    W = synth.temporal_weights(cfg, 23, "fp32", with_text_head=False)
    ids = synth.stream_ids(cfg, 56, 24)
    model = _model(cfg, W, "fp32", 64)
    kv = model.kv_alloc()
    before = _ring(kv, "fp32")
    h_pre = _prefill(model, kv, ids[:50])
    after = _ring(kv, "fp32")
    h_dec = torch.empty((6, cfg["d_model"]), device="cuda")
    for t in range(6):
        model.decode_step(kv, ids[50 + t], h_dec[t])
    torch.cuda.synchronize()
    want = O.forward_full(ids, W, cfg)
    assert max_abs_err(h_pre, want[:50]) <= FP32_TOL
    assert max_abs_err(h_dec.cpu().numpy(), want[50:]) <= FP32_TOL
    assert kv.info()[0] == 56

    L, H, C, dh = cfg["n_layers"], cfg["n_heads"], cfg["context"], cfg["d_head"]
    b = before.reshape(L, 2, 1, H, C, dh)
    a = after.reshape(L, 2, 1, H, C, dh)
    # slots >= T untouched, bit for bit (the fresh ring holds whatever the allocation held,
    # NaN patterns included, so the bits are compared, not the values)
    assert np.array_equal(a[..., 50:, :].view(np.uint32), b[..., 50:, :].view(np.uint32))
    # decoded frame by frame from an empty ring, the same 50 frames fill the same slots
    kv2 = model.kv_alloc()
    for t in range(50):
        model.decode_step(kv2, ids[t], h_dec[0])
    ref = _ring(kv2, "fp32").reshape(L, 2, 1, H, C, dh)
    assert max_abs_err(a[..., :50, :], ref[..., :50, :]) <= FP32_TOL


def test_prefill_argument_errors():
    import torch
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 0, "fp32", with_text_head=False)
    model = _model(cfg, W, "fp32", 32)
    kv = model.kv_alloc()
    h = torch.empty((64, cfg["d_model"]), device="cuda")
    ids = synth.stream_ids(cfg, 64, 1)
    with pytest.raises(pp.PPError) as e:
        model.prefill(kv, ids, h)                 # T above max_prefill_T
    assert e.value.status == pp.PP_E_CAPACITY
    bad = ids[:8].copy()
    bad[3, 2] = 2049
    with pytest.raises(pp.PPError) as e:
        model.prefill(kv, bad, h)
    assert e.value.status == pp.PP_E_ID
    assert kv.info()[0] == 0
    model.prefill(kv, ids[:8], h)
    model.prefill(kv, ids[8:16], h)               # a second chunk continues at position 8
    assert kv.info()[0] == 16
    kv.reset()
    model.prefill(kv, ids[:8], h)
    assert kv.info()[0] == 8


# ----------------------------------------------------------------------------- bf16

@pytest.mark.parametrize("T", [1, 300])
def test_tiny_bf16_prefill_matches_oracle(T):
    """Matrix-core path at d_model 256 / d_head 64; T = 300 leaves a ragged last tile of
    44 rows (128-row GEMM tiles, 128-query attention blocks)."""
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 25, "bf16", with_text_head=False)
    ids = synth.stream_ids(cfg, T, 26)
    model = _model(cfg, W, "bf16", 512)
    kv = model.kv_alloc()
    h = _prefill(model, kv, ids)
    want = O.forward_full(ids, W, cfg)
    err = norm_max_err(h, want)
    print("tiny bf16 prefill T=%d: err %.3g" % (T, err))
    assert err <= BF16_TOL


def test_full_width_bf16_prefill_two_blocks():
    """Two 4096-wide blocks (d_head 128, d_ff 11264) over T = 293 frames, then one decode
    frame at position 293 on the ring the prefill left."""
    import torch
    cfg = synth.with_(synth.FULL_TEMPORAL, n_layers=2)
    W = synth.temporal_weights(cfg, 27, "bf16", with_text_head=False, shared_layer=True)
    ids = synth.stream_ids(cfg, 294, 28)
    model = _model(cfg, W, "bf16", 512)
    kv = model.kv_alloc()
    h = _prefill(model, kv, ids[:293])
    h1 = torch.empty(cfg["d_model"], device="cuda")
    model.decode_step(kv, ids[293], h1)
    torch.cuda.synchronize()
    want = O.forward_full(ids, W, cfg)
    e_pre, e_dec = norm_max_err(h, want[:293]), norm_max_err(h1.cpu().numpy(), want[293])
    print("full-width bf16 prefill: err %.3g, decode after prefill: err %.3g" % (e_pre, e_dec))
    assert e_pre <= BF16_TOL and e_dec <= BF16_TOL


def test_full_width_bf16_short_chunk_splits_k():
    """Two 4096-wide blocks with d_ff 2048: a 300-frame prefill, then a 100-frame chunk. At
    these row counts the W_in product (32-96 output tiles) and W_O / W_out (32-96) have too
    few tiles for the GPU, so K is split over several workgroups per tile: SiLU(g)*z and the
    residual formed from float32 partials summed in split order. Against the oracle's full
    forward."""
    cfg = synth.with_(synth.FULL_TEMPORAL, n_layers=2, d_ff=2048)
    W = synth.temporal_weights(cfg, 29, "bf16", with_text_head=False, shared_layer=True)
    ids = synth.stream_ids(cfg, 400, 30)
    model = _model(cfg, W, "bf16", 300)
    kv = model.kv_alloc()
    h0 = _prefill(model, kv, ids[:300])
    h1 = _prefill(model, kv, ids[300:])
    want = O.forward_full(ids, W, cfg)
    e0, e1 = norm_max_err(h0, want[:300]), norm_max_err(h1, want[300:])
    print("full-width bf16, d_ff 2048: prefill err %.3g, 100-frame chunk err %.3g" % (e0, e1))
    assert e0 <= BF16_TOL and e1 <= BF16_TOL
