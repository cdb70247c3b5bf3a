"""GPU parity at the benchmark's full sizes, in the launch configuration bench.py times.

Full 32-block decode at context 3000: the benchmark's step (graph replay, ring full, the
new frame's slot wrapping to slot 0) against the oracle on the same inputs. The 32 blocks
share one set of weights (the full-depth computation, without drawing 13 GB on the host).

Full 32-block prefill at T = 3000: the oracle cannot run 3000 frames through 32 full-width
blocks in a test's time, so the check uses outputs it can compute one by one and
properties that hold at any size: the first rows of the prefill against the oracle (by
causality they depend only on the first frames), and the whole prefill against the
frame-by-frame decode of the same frames on the GPU (hidden rows sampled across the
sequence and the K/V it leaves in the ring). The two GPU paths round differently (the
prefill's matrix products take bf16 activations, decode keeps them fp32), so that
comparison allows the sum of two bf16-path errors, 2 x 2e-2."""

import numpy as np
import pytest

from oracle import temporal as O
from personaplex_temporal_transformer_amd import pp, synth
from tests.helpers import norm_max_err, require_gpu, to_device

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

BF16_TOL = 2e-2


def _model(cfg, W, max_T=0):
    require_gpu()
    return pp.TemporalModel(cfg, to_device(W), "bf16", max_prefill_T=max_T)


def test_full_decode_32_blocks_ctx3000_matches_oracle():
    import torch
    cfg = dict(synth.FULL_TEMPORAL)
    C, L, D = cfg["context"], cfg["n_layers"], cfg["d_model"]
    W = synth.temporal_weights(cfg, 41, "bf16", with_text_head=False, shared_layer=True)
    frames = synth.cache_frames(cfg, C, 42)                     # [L, 2, 1, H, C, dh] bf16 bits
    ids = synth.stream_ids(cfg, 2, 43)
    model = _model(cfg, W)
    model.set_graph(True)
    kv = model.kv_alloc()
    kv.load(torch.from_numpy(frames.view(np.int16)).cuda(), C)
    h = torch.empty((2, D), device="cuda")
    for t in range(2):
        model.decode_step(kv, ids[t], h[t])                     # positions 3000, 3001
    torch.cuda.synchronize()
    got = h.cpu().numpy()
    assert kv.info()[0] == C + 2

    ks = [frames[l, 0, 0].transpose(1, 0, 2) for l in range(L)]
    vs = [frames[l, 1, 0].transpose(1, 0, 2) for l in range(L)]
    cache = O.cache_from_blocks(ks, vs, np.arange(C), L)
    for t in range(2):
        want = O.final(O.decode_step(O.embed(ids[t], W, cfg), C + t, cache, W, cfg), W, cfg)
        err = norm_max_err(got[t], want)
        print("full decode, position %d: err %.3g" % (C + t, err))
        assert err <= BF16_TOL


def test_full_prefill_32_blocks_T3000():
    import torch
    cfg = dict(synth.FULL_TEMPORAL)
    C, L, D, H, dh = cfg["context"], cfg["n_layers"], cfg["d_model"], cfg["n_heads"], cfg["d_head"]
    T = C
    W = synth.temporal_weights(cfg, 44, "bf16", with_text_head=False, shared_layer=True)
    ids = synth.stream_ids(cfg, T, 45)
    model = _model(cfg, W, max_T=T)

    kv_p = model.kv_alloc()
    h_p = torch.empty((T, D), device="cuda")
    model.prefill(kv_p, ids, h_p)
    torch.cuda.synchronize()
    hp = h_p.cpu().numpy()
    assert kv_p.info()[0] == T

    # first rows against the oracle (row t depends on frames 0..t only)
    n0 = 6
    want = O.forward_full(ids[:n0], W, cfg)
    e0 = norm_max_err(hp[:n0], want)
    print("full prefill rows 0..%d vs oracle: err %.3g" % (n0 - 1, e0))
    assert e0 <= BF16_TOL

    # the whole prefill against frame-by-frame decode of the same frames
    kv_d = model.kv_alloc()
    model.set_graph(True)
    h_d = torch.empty((T, D), device="cuda")
    for t in range(T):
        model.decode_step(kv_d, ids[t], h_d[t])
    torch.cuda.synchronize()
    hd = h_d.cpu().numpy()
    rows = [0, 1, 63, 64, 127, 128, 191, 192, 1000, 1999, 2047, 2048, T - 2, T - 1]
    e1 = max(norm_max_err(hp[r], hd[r]) for r in rows)
    print("full prefill vs decode, sampled rows: err %.3g" % e1)
    assert e1 <= 2 * BF16_TOL

    n = kv_p.info()[1] // 2
    rp = torch.empty(n, dtype=torch.int16, device="cuda")
    rd = torch.empty_like(rp)
    kv_p.store(rp)
    kv_d.store(rd)
    torch.cuda.synchronize()
    ap = rp.cpu().numpy().view(np.uint16).reshape(L, 2, 1, H, C, dh)
    ad = rd.cpu().numpy().view(np.uint16).reshape(L, 2, 1, H, C, dh)
    for l in (0, L // 2, L - 1):
        for kvi in (0, 1):
            e = norm_max_err(O.f64(ap[l, kvi, 0][:, rows]), O.f64(ad[l, kvi, 0][:, rows]))
            print("ring layer %d %s: err %.3g" % (l, "KV"[kvi], e))
            assert e <= 2 * BF16_TOL
