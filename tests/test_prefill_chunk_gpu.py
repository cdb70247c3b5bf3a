"""GPU parity of prefill chunks that start past position 0 (prompt replay into a live
ring: "PersonaPlex native LM audit", section 9 'Startup prompt and clock facts') against
the oracle, through the C ABI. The plain definition of a chunk at positions p..p+T-1 is
the full causal forward over all frames 0..p+T-1 with the context window, rows p..p+T-1:
the oracle's forward_full over the whole sequence. Also: chunks whose history and own
frames together exceed the context (ring slots the chunk overwrites are still read by
its first queries), the ring a chunked prefill leaves against frame-by-frame decode, and
snapshot / restore / reset + re-prime of a session."""

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


def _chunks(model, kv, ids, sizes):
    import torch
    outs, p = [], 0
    for T in sizes:
        h = torch.empty((T, model.cfg["d_model"]), device="cuda")
        assert kv.info()[0] == p
        model.prefill(kv, ids[p:p + T], h)
        outs.append(h)
        p += T
    torch.cuda.synchronize()
    return np.concatenate([h.cpu().numpy() for h in outs]), p


def _ring(kv, dtype):
    import torch
    n = kv.info()[1] // (2 if dtype == "bf16" else 4)
    t = torch.empty(n, dtype=torch.int16 if dtype == "bf16" else torch.float32, device="cuda")
    kv.store(t)
    torch.cuda.synchronize()
    return t


@pytest.mark.parametrize("context,sizes", [(3000, [37, 64, 5, 90]), (64, [40, 50, 30, 64, 17]),
                                           (48, [1, 47, 48, 3, 20])])
def test_tiny_fp32_chunks_match_oracle(context, sizes):
    """Chunks of ragged sizes; with context 64 and 48 the history plus the chunk exceeds
    the ring, T = context fills it in one chunk, and a 1-frame chunk starts the sequence."""
    import torch
    cfg = synth.with_(synth.TINY_TEMPORAL, context=context)
    W = synth.temporal_weights(cfg, 31, "fp32", with_text_head=False)
    n = sum(sizes) + 3
    ids = synth.stream_ids(cfg, n, 32)
    model = _model(cfg, W, "fp32", max(sizes))
    kv = model.kv_alloc()
    h, p = _chunks(model, kv, ids, sizes)
    h_dec = torch.empty((3, cfg["d_model"]), device="cuda")
    for t in range(3):
        model.decode_step(kv, ids[p + t], h_dec[t])
    torch.cuda.synchronize()
    want = O.forward_full(ids, W, cfg)
    e_pre, e_dec = max_abs_err(h, want[:p]), max_abs_err(h_dec.cpu().numpy(), want[p:])
    print("tiny fp32 chunks %s ctx %d: err %.3g, decode after: %.3g" % (sizes, context, e_pre, e_dec))
    assert e_pre <= FP32_TOL and e_dec <= FP32_TOL


def test_tiny_fp32_chunked_ring_equals_decode_ring():
    """The ring after chunks across the wrap holds what frame-by-frame decode of the same
    frames leaves there."""
    import torch
    cfg = synth.with_(synth.TINY_TEMPORAL, context=64)
    W = synth.temporal_weights(cfg, 33, "fp32", with_text_head=False)
    ids = synth.stream_ids(cfg, 150, 34)
    model = _model(cfg, W, "fp32", 64)
    kv = model.kv_alloc()
    _chunks(model, kv, ids, [60, 41, 49])
    kv2 = model.kv_alloc()
    h = torch.empty(cfg["d_model"], device="cuda")
    for t in range(150):
        model.decode_step(kv2, ids[t], h)
    a, b = _ring(kv, "fp32").cpu().numpy(), _ring(kv2, "fp32").cpu().numpy()
    assert kv.info()[0] == kv2.info()[0] == 150
    assert max_abs_err(a, b) <= FP32_TOL


@pytest.mark.parametrize("context,sizes", [(256, [100, 120, 90, 200]), (3000, [300, 44, 129])])
def test_tiny_bf16_chunks_match_oracle(context, sizes):
    """Matrix-core path: history gathered into the chunk's key space (K rows, V transposed
    to float16), chunk keys at a 16-aligned offset."""
    cfg = synth.with_(synth.TINY_TEMPORAL, context=context)
    W = synth.temporal_weights(cfg, 35, "bf16", with_text_head=False)
    ids = synth.stream_ids(cfg, sum(sizes), 36)
    model = _model(cfg, W, "bf16", max(sizes))
    kv = model.kv_alloc()
    h, p = _chunks(model, kv, ids, sizes)
    want = O.forward_full(ids, W, cfg)
    errs = []
    q = 0
    for T in sizes:
        errs.append(norm_max_err(h[q:q + T], want[q:q + T]))
        q += T
    print("tiny bf16 chunks %s ctx %d: errs %s" % (sizes, context, ["%.3g" % e for e in errs]))
    assert max(errs) <= BF16_TOL


def test_tiny_bf16_chunks_after_long_history_split_keys():
    """Short chunks after a 1200-frame prefill: with few query blocks x heads the attention
    splits each query block's keys over several workgroups and a second pass combines them
    (and the small W_out products split K)."""
    cfg = synth.with_(synth.TINY_TEMPORAL, context=3000)
    sizes = [1200, 40, 7, 128]
    W = synth.temporal_weights(cfg, 37, "bf16", with_text_head=False)
    ids = synth.stream_ids(cfg, sum(sizes), 38)
    model = _model(cfg, W, "bf16", max(sizes))
    kv = model.kv_alloc()
    h, p = _chunks(model, kv, ids, sizes)
    want = O.forward_full(ids, W, cfg)
    errs = []
    q = 0
    for T in sizes:
        errs.append(norm_max_err(h[q:q + T], want[q:q + T]))
        q += T
    print("tiny bf16 chunks %s after a long history: errs %s" % (sizes, ["%.3g" % e for e in errs]))
    assert max(errs) <= BF16_TOL


def test_snapshot_restore_and_reprime_are_exact():
    """Store the ring after a prompt, decode, restore the snapshot with its position and
    decode the same frames again: identical bits. Reset and prefill the prompt again:
    identical prompt outputs and prompt slots of the ring."""
    import torch
    cfg = synth.with_(synth.TINY_TEMPORAL, context=128)
    W = synth.temporal_weights(cfg, 37, "bf16", with_text_head=False)
    ids = synth.stream_ids(cfg, 110, 38)
    model = _model(cfg, W, "bf16", 100)
    kv = model.kv_alloc()
    h1, p = _chunks(model, kv, ids, [70, 30])
    snap = _ring(kv, "bf16").clone()
    dec = lambda: [model.decode_step(kv, ids[p + t], hd[t]) for t in range(10)]
    hd = torch.empty((10, cfg["d_model"]), device="cuda")
    dec()
    torch.cuda.synchronize()
    first = hd.cpu().numpy().copy()
    kv.restore(snap, p)
    assert kv.info()[0] == p
    dec()
    torch.cuda.synchronize()
    assert np.array_equal(hd.cpu().numpy(), first)
    kv.reset()
    h2, _ = _chunks(model, kv, ids, [70, 30])
    assert np.array_equal(h1, h2)
    # slots 0..p-1 hold the prompt again; the decoded frames' slots keep their bytes
    shape = (cfg["n_layers"], 2, 1, cfg["n_heads"], cfg["context"], cfg["d_head"])
    got, ref = _ring(kv, "bf16").view(shape), snap.view(shape)
    assert torch.equal(got[..., :p, :], ref[..., :p, :])


@pytest.mark.parametrize("wdtype", ["fp32", "bf16"])
def test_prefill_from_summed_embeddings(wdtype):
    """pp_temporal_prefill_embedded (a cached prompt replayed as summed embeddings): with
    each frame's embedding sum as input (the fixed-order float32 sum the ID path's gather
    forms) it gives the token-ID prefill's rows bit for bit, as a first prompt and as a
    chunk after it; with inputs no IDs produce (the sums scaled by
    0.5) it matches the oracle's forward over those inputs."""
    import torch
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 39, wdtype, with_text_head=False)
    ids = synth.stream_ids(cfg, 90, 40)
    model = _model(cfg, W, wdtype, 64)
    X = np.stack([O.embed(ids[t], W, cfg) for t in range(90)])
    X32 = np.stack([O.embed(ids[t], W, cfg, precision="f32") for t in range(90)])   # the GPU gather's bits
    tol = 1e-4 if wdtype == "fp32" else 2e-2
    metric = max_abs_err if wdtype == "fp32" else norm_max_err
    kv = model.kv_alloc()
    h = torch.empty((90, cfg["d_model"]), device="cuda")
    model.prefill(kv, ids[:60], h[:60])
    model.prefill(kv, ids[60:], h[60:])
    kv2 = model.kv_alloc()
    h2 = torch.empty_like(h)
    x32 = torch.from_numpy(X32).cuda()
    model.prefill_embedded(kv2, x32[:60], h2[:60])
    model.prefill_embedded(kv2, x32[60:], h2[60:])
    torch.cuda.synchronize()
    assert kv2.info()[0] == 90
    assert torch.equal(h, h2)                 # the same float32 sums in: the same bits out
    xd = torch.from_numpy(X.astype(np.float32)).cuda()
    # inputs that are not embedding sums of any IDs, against the oracle's forward over them
    kv3 = model.kv_alloc()
    h3 = torch.empty((60, cfg["d_model"]), device="cuda")
    model.prefill_embedded(kv3, (0.5 * xd[:60]).contiguous(), h3)
    torch.cuda.synchronize()
    Xh = 0.5 * X[:60]
    pos = np.arange(60)
    Y = Xh
    for l in range(cfg["n_layers"]):
        Y = O.block_full(Y, pos, l, W, cfg)
    want = O.rmsnorm(Y, W["out_norm.alpha"], cfg["eps"])
    err = metric(h3.cpu().numpy(), want)
    print("prefill from summed embeddings (%s): scaled-input err %.3g" % (wdtype, err))
    assert err <= tol
