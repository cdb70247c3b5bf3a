"""GPU parity of the memory readers ("Current sequence memory: one writer, four readers",
section 6) against the oracle, through the C ABI: readers after named temporal blocks in
decode, exact identity with zero output projections or no visible memory, visibility
changes between steps under graph replay."""

import numpy as np
import pytest

from oracle import reader as ORD
from oracle import temporal as O
from personaplex_temporal_transformer_amd import pp, synth
from tests.helpers import max_abs_err, norm_max_err, require_gpu, to_device

pytestmark = pytest.mark.gpu

FP32_TOL = 1e-4
BF16_TOL = 2e-2


def _model(cfg, W, wdtype, R=None, blocks=(), mem_dim=32, max_slots=40, graph=True):
    require_gpu()
    m = pp.TemporalModel(cfg, to_device(W), wdtype)
    m.set_graph(graph)
    if R is not None:
        m.attach_readers(list(blocks), to_device(R), mem_dim, max_slots)
    return m


def _decode(m, ids, visible=None):
    import torch
    kv = m.kv_alloc()
    h = torch.empty((ids.shape[0], m.cfg["d_model"]), device="cuda")
    for t in range(ids.shape[0]):
        if visible is not None:
            m.set_visible(visible[t])
        m.decode_step(kv, ids[t], h[t])
    torch.cuda.synchronize()
    return h.cpu().numpy()


@pytest.mark.parametrize("n_visible", [1, 7, 40])
def test_tiny_fp32_readers_match_oracle(n_visible):
    import torch
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 81, "fp32", with_text_head=False)
    R = synth.reader_weights(cfg, 2, 32, 82, "fp32", scale=0.1)
    M = synth.memory_bank(40, 32, 83, "fp32")
    ids = synth.stream_ids(cfg, 4, 84)
    m = _model(cfg, W, "fp32", R, (0, 1))
    m.write_memory(torch.from_numpy(M).cuda())
    m.set_visible(n_visible)
    got = _decode(m, ids)
    want = O.decode_incremental(ids, W, cfg, after_block=ORD.hooks([0, 1], M, n_visible, R, cfg["n_heads"]))
    base = O.decode_incremental(ids, W, cfg)
    err = max_abs_err(got, want)
    print("tiny fp32 readers, %d visible rows: err %.3g (reader effect %.3g)" % (n_visible, err, max_abs_err(want, base)))
    assert err <= FP32_TOL
    assert max_abs_err(want, base) > 100 * FP32_TOL          # the readers do change the stream


def test_zero_output_and_empty_memory_are_bit_identical():
    import torch
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 85, "fp32", with_text_head=False)
    ids = synth.stream_ids(cfg, 3, 86)
    plain = _decode(_model(cfg, W, "fp32"), ids)
    R0 = synth.reader_weights(cfg, 2, 32, 87, "fp32", scale=0.1, zero_out=True)
    m = _model(cfg, W, "fp32", R0, (0, 1))
    m.write_memory(torch.from_numpy(synth.memory_bank(40, 32, 88, "fp32")).cuda())
    m.set_visible(40)
    assert np.array_equal(_decode(m, ids), plain)
    R = synth.reader_weights(cfg, 2, 32, 89, "fp32", scale=0.1)
    m2 = _model(cfg, W, "fp32", R, (1, 0))
    m2.write_memory(torch.from_numpy(synth.memory_bank(40, 32, 88, "fp32")).cuda())
    assert np.array_equal(_decode(m2, ids), plain)            # nothing visible yet


@pytest.mark.parametrize("graph", [True, False])
def test_visibility_changes_between_steps(graph):
    import torch
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 90, "fp32", with_text_head=False)
    R = synth.reader_weights(cfg, 1, 32, 91, "fp32", scale=0.1)
    M = synth.memory_bank(40, 32, 92, "fp32")
    ids = synth.stream_ids(cfg, 5, 93)
    vis = [0, 5, 5, 12, 40]
    m = _model(cfg, W, "fp32", R, (1,), graph=graph)
    m.write_memory(torch.from_numpy(M[:20]).cuda(), 0)
    m.write_memory(torch.from_numpy(M[20:]).cuda(), 20)       # rows written in two pieces
    got = _decode(m, ids, vis)
    cache = O.Cache(cfg["n_layers"])
    want = []
    for t in range(5):
        x = O.decode_step(O.embed(ids[t], W, cfg), t, cache, W, cfg,
                          after_block=ORD.hooks([1], M, vis[t], R, cfg["n_heads"]))
        want.append(O.final(x, W, cfg))
    err = max_abs_err(got, np.stack(want))
    print("visibility %s graph=%s: err %.3g" % (vis, graph, err))
    assert err <= FP32_TOL


def test_tiny_bf16_readers_match_oracle():
    import torch
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 94, "bf16", with_text_head=False)
    R = synth.reader_weights(cfg, 2, 64, 95, "bf16", scale=0.1)
    M = synth.memory_bank(100, 64, 96, "bf16")
    ids = synth.stream_ids(cfg, 4, 97)
    m = _model(cfg, W, "bf16", R, (0, 1), mem_dim=64, max_slots=128)
    m.write_memory(torch.from_numpy(M.view(np.int16)).cuda().view(torch.bfloat16))
    m.set_visible(100)
    got = _decode(m, ids)
    want = O.decode_incremental(ids, W, cfg, after_block=ORD.hooks([0, 1], M, 100, R, cfg["n_heads"]))
    err = norm_max_err(got, want)
    print("tiny bf16 readers: err %.3g" % err)
    assert err <= BF16_TOL


def test_reader_argument_errors():
    import torch
    cfg = synth.TINY_TEMPORAL
    W = synth.temporal_weights(cfg, 0, "fp32", with_text_head=False)
    R = synth.reader_weights(cfg, 2, 32, 1, "fp32")
    m = _model(cfg, W, "fp32")
    with pytest.raises(pp.PPError):
        m.set_visible(1)                                        # nothing attached
    with pytest.raises(pp.PPError):
        m.attach_readers([0, 0], to_device(R), 32, 8)           # two readers after one block
    with pytest.raises(pp.PPError):
        m.attach_readers([0, 2], to_device(R), 32, 8)           # block out of range
    m.attach_readers([0, 1], to_device(R), 32, 8)
    with pytest.raises(pp.PPError) as e:
        m.write_memory(torch.zeros((9, 32), device="cuda"))      # past max_slots
    assert e.value.status == pp.PP_E_CAPACITY
    with pytest.raises(pp.PPError):
        m.set_visible(9)
