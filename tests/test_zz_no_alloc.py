"""The allocation-free decode step (pp_temporal_decode_step_noalloc) against the ordinary
one, through the C ABI: the same frames on two rings of one model must give the same
bits, for a model and then, right after, a smaller one (whose step uses less of the
library's scratch array, so stale contents of the first must not leak in). Both are
also checked against the oracle to the bf16 bar."""

import numpy as np
import pytest

from oracle import temporal as O
from personaplex_temporal_transformer_amd import pp, synth
from tests.helpers import norm_max_err, require_gpu, to_device

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


def _pair(cfg, seed, n_frames, with_head):
    import torch
    W = synth.temporal_weights(cfg, seed, "bf16", with_text_head=with_head)
    ids = synth.stream_ids(cfg, n_frames, seed + 1)
    model = pp.TemporalModel(cfg, to_device(W), "bf16")
    kv_ref, kv_na = model.kv_alloc(), model.kv_alloc()
    D, V = cfg["d_model"], cfg["text_vocab"] - 1
    h_ref = torch.empty((n_frames, D), device="cuda")
    h_na = torch.full((n_frames, D), float("nan"), device="cuda")
    lg_ref = torch.empty((n_frames, V), device="cuda") if with_head else None
    lg_na = torch.full((n_frames, V), float("nan"), device="cuda") if with_head else None
    for t in range(n_frames):
        model.decode_step(kv_ref, ids[t], h_ref[t], lg_ref[t] if with_head else None)
        model.decode_step_noalloc(kv_na, ids[t], h_na[t], lg_na[t] if with_head else None)
    torch.cuda.synchronize()
    assert kv_na.info()[0] == n_frames
    out = dict(h_ref=h_ref.cpu().numpy(), h_na=h_na.cpu().numpy(), W=W, ids=ids)
    if with_head:
        out["lg_ref"], out["lg_na"] = lg_ref.cpu().numpy(), lg_na.cpu().numpy()
    return out


def test_noalloc_step_equals_decode_step_then_smaller_model():
    require_gpu()
    big = synth.TINY_TEMPORAL                                             # 2 blocks, 256 wide, d_ff 704
    small = synth.with_(synth.TINY_TEMPORAL, n_layers=1, d_model=128, n_heads=2, d_ff=352)
    for cfg, seed, n, head in ((big, 120, 6, True), (small, 130, 4, False)):
        r = _pair(cfg, seed, n, head)
        assert np.array_equal(r["h_na"], r["h_ref"]), cfg["d_model"]
        if head:
            assert np.array_equal(r["lg_na"], r["lg_ref"])
        want = O.forward_full(r["ids"], r["W"], cfg)
        err = norm_max_err(r["h_na"], want)
        print("allocation-free step, d_model %d: bit-identical to the ordinary step; vs oracle %.3g"
              % (cfg["d_model"], err))
        assert err <= BF16_TOL


def test_noalloc_step_rejects_what_it_cannot_hold():
    import torch
    require_gpu()
    cfg = synth.with_(synth.FULL_TEMPORAL, n_layers=1)
    W = synth.temporal_weights(cfg, 140, "bf16", with_text_head=False)
    model = pp.TemporalModel(cfg, to_device(W), "bf16", max_batch=2)
    ids = synth.stream_ids(cfg, 1, 141)
    h = torch.empty(cfg["d_model"], device="cuda")
    kv = model.kv_alloc()
    model.set_attn_splits(64)          # 32 heads x 64 splits of partials: more than 1 MiB
    with pytest.raises(pp.PPError) as e:
        model.decode_step_noalloc(kv, ids[0], h)
    assert e.value.status == pp.PP_E_CAPACITY
    assert kv.info()[0] == 0           # refused before anything was enqueued
    model.set_attn_splits(0)
    model.decode_step_noalloc(kv, ids[0], h)
    kv2 = model.kv_alloc(2)
    with pytest.raises(pp.PPError) as e:
        model.decode_step_noalloc(kv2, np.stack([ids[0], ids[0]]), torch.empty((2, cfg["d_model"]), device="cuda"))
    assert e.value.status == pp.PP_E_ARG
    torch.cuda.synchronize()
    assert kv.info()[0] == 1
