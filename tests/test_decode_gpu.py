"""GPU parity of the temporal decode path (embedding sum, blocks, final norm, text head)
against the oracle, through the C ABI. Tolerances: max abs error 1e-4 for the fp32
path; max |err| / max |ref| <= 2e-2 for the bf16 path; bit-exact for ID gathering and
cache indexing."""

import numpy as np
import pytest

from oracle import temporal as O
from personaplex_temporal_transformer_amd import pp, synth
from tests.helpers import max_abs_err, norm_max_err, require_gpu, to_device

pytestmark = pytest.mark.gpu

FP32_TOL = 1e-4
BF16_TOL = 2e-2


def _model(cfg, W, wdtype, max_T=0):
    require_gpu()
    dW = to_device(W)
    return pp.TemporalModel(cfg, dW, wdtype, max_prefill_T=max_T), dW


def _decode_all(model, kv, ids, with_logits=True):
    import torch
    T, D = ids.shape[0], model.cfg["d_model"]
    h = torch.empty((T, D), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, model.cfg["text_vocab"] - 1), dtype=torch.float32, device="cuda") if with_logits else None
    for t in range(T):
        model.decode_step(kv, ids[t], h[t], lg[t] if with_logits else None)
    torch.cuda.synchronize()
    return h.cpu().numpy(), (lg.cpu().numpy() if with_logits else None)


# ----------------------------------------------------------------------------- fp32, tiny

@pytest.mark.parametrize("context,d_ff,splits", [(3000, 704, None), (4, 704, None), (3000, 2312, None),
                                                 (3000, 704, 8), (4, 704, 3), (3000, 704, 1)])
@pytest.mark.parametrize("graph", [True, False])
def test_tiny_fp32_decode_matches_oracle(context, d_ff, splits, graph):
    """d_ff 2312 makes the W_out rows (2312 floats) longer than one 512-chunk pass, so the
    multi-pass GEMV path (x from LDS, ragged last pass) is covered at small scale; with
    <= 8 attention splits the split merge runs inside the W_O GEMV instead of a separate
    combine kernel (3 splits at context 4 also leaves splits empty; 1 split makes the
    merge a pass-through)."""
    cfg = synth.with_(synth.TINY_TEMPORAL, context=context, d_ff=d_ff)
    W = synth.temporal_weights(cfg, 0, "fp32")
    ids = synth.stream_ids(cfg, 16, 1)
    model, _ = _model(cfg, W, "fp32")
    model.set_graph(graph)
    if splits is not None:
        model.set_attn_splits(splits)
    kv = model.kv_alloc()
    h, lg = _decode_all(model, kv, ids)
    want_h, want_lg = O.forward_full(ids, W, cfg, with_logits=True)
    print("tiny fp32 C=%d F=%d graph=%s: h err %.3g, logits err %.3g" %
          (context, d_ff, graph, max_abs_err(h, want_h), max_abs_err(lg, want_lg)))
    assert max_abs_err(h, want_h) <= FP32_TOL
    assert max_abs_err(lg, want_lg) <= FP32_TOL
    assert kv.info()[0] == 16


def test_graph_and_direct_launch_are_bit_identical_and_reset_replays():
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 5, "fp32")
    ids = synth.stream_ids(cfg, 12, 6)
    model, _ = _model(cfg, W, "fp32")
    kv = model.kv_alloc()
    model.set_graph(True)
    a, _ = _decode_all(model, kv, ids, with_logits=False)
    kv.reset()
    assert kv.info()[0] == 0
    model.set_graph(False)
    b, _ = _decode_all(model, kv, ids, with_logits=False)
    assert np.array_equal(a, b)


def test_kernel_timing_repeats_leave_the_result_unchanged():
    """Timing brackets around layer 1's W_in kernel, one launch or five back to back per
    event pair: the steps' outputs are bit-identical to untimed steps (the kernel rewrites
    the same SwiGLU output from the same residual), the count is brackets x repeat, and the
    repeat count is validated."""
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 5, "fp32")
    ids = synth.stream_ids(cfg, 6, 6)
    model, _ = _model(cfg, W, "fp32")
    kv = model.kv_alloc()
    model.set_graph(True)
    want, _ = _decode_all(model, kv, ids, with_logits=False)
    for repeat in (1, 5):
        kv.reset()
        model.trace(1, repeat)
        got, _ = _decode_all(model, kv, ids, with_logits=False)
        n, us = model.trace_read()
        model.trace(-1)
        assert np.array_equal(got, want)
        assert n == ids.shape[0] * repeat and us > 0
    for bad in (0, 65):
        with pytest.raises(pp.PPError):
            model.trace(1, bad)


def test_invalid_ids_rejected_before_enqueue():
    import torch
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 0, "fp32", with_text_head=False)
    model, _ = _model(cfg, W, "fp32")
    kv = model.kv_alloc()
    h = torch.zeros(cfg["d_model"], device="cuda")
    for k, bad in ((0, -2), (0, 32001), (9, 2049), (16, -7)):
        ids = np.zeros(17, np.int32)
        ids[k] = bad
        with pytest.raises(pp.PPError) as e:
            model.decode_step(kv, ids, h)
        assert e.value.status == pp.PP_E_ID
    assert kv.info()[0] == 0
    with pytest.raises(pp.PPError) as e:
        model.decode_step(kv, np.zeros(17, np.int32), h, logits_out=h)   # no text head
    assert e.value.status == pp.PP_E_ARG


# ----------------------------------------------------------------------------- gather

@pytest.mark.parametrize("cfg_name", ["tiny", "full"])
def test_embed_sum_bit_exact(cfg_name):
    import torch
    cfg = synth.TINY_TEMPORAL if cfg_name == "tiny" else synth.with_(synth.FULL_TEMPORAL, n_layers=1)
    W = synth.temporal_weights(cfg, 11, "bf16", with_text_head=False)
    dW = to_device(W)
    model = pp.TemporalModel(cfg, dW, "bf16", max_prefill_T=64)
    ids = synth.stream_ids(cfg, 64, 12)
    ids[3] = -1                       # a frame with no input at all -> exact zeros
    ids[5, :] = [32000] + [2048] * 16  # the initial IDs are valid rows
    x = torch.empty((64, cfg["d_model"]), device="cuda")
    model.embed_sum(ids, x)
    x1 = torch.empty((cfg["d_model"],), device="cuda")
    model.embed_sum(ids[7], x1)       # single-frame path (IDs as kernel arguments)
    torch.cuda.synchronize()
    got = x.cpu().numpy()
    for t in range(64):
        want = O.embed(ids[t], W, cfg, precision="f32")
        assert np.array_equal(got[t], want), t
    assert np.all(got[3] == 0)
    assert np.array_equal(x1.cpu().numpy(), got[7])
    bad = ids.copy()
    bad[10, 4] = -2
    with pytest.raises(pp.PPError) as e:
        model.embed_sum(bad, x)
    assert e.value.status == pp.PP_E_ID


@pytest.mark.gpu
def test_embed_sum_batch_times_frames_and_capacity():
    """pp_embed_sum over batch x T frames (the ID region holds max_prefill_T x max_batch
    frames) is the fixed-order float32 gather of every frame; one frame more than that
    region is a capacity error, returned before anything is enqueued."""
    import torch
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 13, "bf16", with_text_head=False)
    model = pp.TemporalModel(cfg, to_device(W), "bf16", max_prefill_T=16, max_batch=4)
    ids = synth.stream_ids(cfg, 4 * 16, 14).reshape(4, 16, -1)
    ids[2, 5] = -1
    x = torch.full((4, 16, cfg["d_model"]), float("nan"), device="cuda")
    model.embed_sum(ids, x)
    torch.cuda.synchronize()
    got = x.cpu().numpy()
    for b in range(4):
        for t in range(16):
            assert np.array_equal(got[b, t], O.embed(ids[b, t], W, cfg, precision="f32")), (b, t)
    big = synth.stream_ids(cfg, 4 * 17, 15).reshape(4, 17, -1)
    xb = torch.empty((4, 17, cfg["d_model"]), device="cuda")
    with pytest.raises(pp.PPError) as e:
        model.embed_sum(big, xb)
    assert e.value.status == pp.PP_E_CAPACITY
    with pytest.raises(pp.PPError) as e:
        model.embed_sum(synth.stream_ids(cfg, 5, 16).reshape(5, 1, -1), xb)
    assert e.value.status == pp.PP_E_ARG
    # the region is intact: the first gather repeated gives the same bits
    model.embed_sum(ids, x)
    torch.cuda.synchronize()
    assert np.array_equal(x.cpu().numpy(), got)


@pytest.mark.gpu
@pytest.mark.parametrize("n_audio,wdt", [(2, "bf16"), (2, "fp32"), (20, "bf16"), (31, "fp32")])
def test_embed_sum_stream_counts(n_audio, wdt):
    """The gather reads 17 table slots for up to 17 streams and 32 beyond, and drops the
    slots past the stream count: with 3, 21 and 32 streams, bfloat16 and float32 tables,
    IDs from the device and as kernel arguments, it is the fixed-order float32 sum."""
    import torch
    cfg = synth.with_(synth.TINY_TEMPORAL, n_audio=n_audio, n_layers=1)
    W = synth.temporal_weights(cfg, 21, wdt, with_text_head=False)
    model = pp.TemporalModel(cfg, to_device(W), wdt, max_prefill_T=8)
    ids = synth.stream_ids(cfg, 8, 22)
    ids[2] = -1
    ids[4, 1:] = cfg["audio_vocab"] - 1
    x = torch.empty((8, cfg["d_model"]), device="cuda")
    model.embed_sum(ids, x)
    x1 = torch.empty((cfg["d_model"],), device="cuda")
    model.embed_sum(ids[5], x1)
    torch.cuda.synchronize()
    got = x.cpu().numpy()
    for t in range(8):
        assert np.array_equal(got[t], O.embed(ids[t], W, cfg, precision="f32")), t
    assert np.all(got[2] == 0)
    assert np.array_equal(x1.cpu().numpy(), got[5])


# ----------------------------------------------------------------------------- one full block

def _full_block_case(n_prefill, seed_w=2, seed_kv=3, seed_ids=4, n_layers=1):
    import torch
    cfg = synth.with_(synth.FULL_TEMPORAL, n_layers=n_layers)
    W = synth.temporal_weights(cfg, seed_w, "bf16", with_text_head=True, shared_layer=n_layers > 1)
    model, _ = _model(cfg, W, "bf16")
    kv = model.kv_alloc()
    frames = synth.cache_frames(cfg, n_prefill, seed_kv)      # [L, 2, 1, H, n, dh] bf16 bits
    src = torch.from_numpy(frames.view(np.int16)).cuda()
    kv.load(src, n_prefill)
    ids = synth.stream_ids(cfg, 2, seed_ids)
    return cfg, W, model, kv, frames, ids


def _oracle_cache(cfg, frames):
    n = frames.shape[4]
    ks = [frames[l, 0, 0].transpose(1, 0, 2) for l in range(cfg["n_layers"])]
    vs = [frames[l, 1, 0].transpose(1, 0, 2) for l in range(cfg["n_layers"])]
    return O.cache_from_blocks(ks, vs, np.arange(n), cfg["n_layers"])


def test_full_width_block_decode_bf16():
    """One 4096-wide block, ring pre-filled with 200 frames, new frame at position 200."""
    import torch
    cfg, W, model, kv, frames, ids = _full_block_case(200)
    C, H, dh = cfg["context"], cfg["n_heads"], cfg["d_head"]
    before = torch.empty(kv.info()[1] // 2, dtype=torch.int16, device="cuda")
    kv.store(before)
    h = torch.empty(cfg["d_model"], device="cuda")
    lg = torch.empty(cfg["text_vocab"] - 1, device="cuda")
    model.decode_step(kv, ids[0], h, lg)
    after = torch.empty_like(before)
    kv.store(after)
    torch.cuda.synchronize()

    cache = _oracle_cache(cfg, frames)
    x = O.decode_step(O.embed(ids[0], W, cfg), 200, cache, W, cfg)
    want_h, want_lg = O.final(x, W, cfg, with_logits=True)
    eh, el = norm_max_err(h.cpu().numpy(), want_h), norm_max_err(lg.cpu().numpy(), want_lg)
    print("full block bf16: h err %.3g, logits err %.3g" % (eh, el))
    assert eh <= BF16_TOL and el <= BF16_TOL

    b = before.cpu().numpy().view(np.uint16).reshape(1, 2, 1, H, C, dh)
    a = after.cpu().numpy().view(np.uint16).reshape(1, 2, 1, H, C, dh)
    changed = np.any(a != b, axis=-1)                    # [1, 2, 1, H, C]
    assert changed[..., 200].all()
    changed[..., 200] = False
    assert not changed.any()                             # only slot 200 was written
    _, k_new, v_new = cache.layers[0][-1]
    kk = O.f64(a[0, 0, 0, :, 200])
    vv = O.f64(a[0, 1, 0, :, 200])
    assert norm_max_err(kk, k_new[0]) <= BF16_TOL
    assert norm_max_err(vv, v_new[0]) <= BF16_TOL


def test_two_runs_are_bit_identical():
    import torch
    cfg, W, model, kv, frames, ids = _full_block_case(200)
    h1 = torch.empty(cfg["d_model"], device="cuda")
    h2 = torch.empty_like(h1)
    model.decode_step(kv, ids[0], h1)
    src = torch.from_numpy(frames.view(np.int16)).cuda()
    kv.load(src, 200)
    model.decode_step(kv, ids[0], h2)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2)
