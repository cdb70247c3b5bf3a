"""GPU parity at the benchmark's full sizes, in the launch configuration bench.py times,
against the oracle at the bf16 bar (max |err| / max |ref| <= 2e-2).

Decode: the full 32-block step at context 3000 (ring full, the new frame's slot
wrapping) against the oracle's incremental decode over the same ring.

Prefill at T = 3000: four full-width blocks with distinct weights, every row and every
ring entry against the oracle computed in the test; and the full 32-block stack (blocks
sharing one weight set) against expected rows the oracle wrote once
(tests/golden/make_prefill_T3000.py: rows at the edges of the 192- and 224-row tiles and
in the ragged last tiles, and the keys / values of layers 0 and 31 for those positions).

A 256-frame chunk at position 3000 into a ring holding 3000 synthetic frames, every row
and the overwritten ring slots against the oracle's chunk over the same history.

Batched decode at B = 4 and B = 64: sessions against the oracle's decode of their own
rings, plus every sampled session against the same session decoded alone on the GPU."""

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


def _ring(kv, cfg):
    """The ring as float32 [L, 2, 1, H, C, dh] (bf16 bits widened)."""
    import torch
    n = kv.info()[1] // 2
    r = torch.empty(n, dtype=torch.int16, device="cuda")
    kv.store(r)
    torch.cuda.synchronize()
    shape = (cfg["n_layers"], 2, 1, cfg["n_heads"], cfg["context"], cfg["d_head"])
    return r.cpu().numpy().view(np.uint16).reshape(shape)


def test_full_prefill_T3000_four_distinct_blocks_every_row():
    """Four full-width blocks with their own weights (the per-layer weight selection at
    full width), T = 3000 from position 0: every hidden row and every key / value written
    to the ring against the oracle, including the ragged last row tiles."""
    import torch
    cfg = synth.with_(synth.FULL_TEMPORAL, n_layers=4)
    T, D, L = cfg["context"], cfg["d_model"], 4
    W = synth.temporal_weights(cfg, 60, "bf16", with_text_head=False)
    ids = synth.stream_ids(cfg, T, 61)
    model = _model(cfg, W, max_T=T)
    kv = model.kv_alloc()
    h = torch.empty((T, D), device="cuda")
    model.prefill(kv, ids, h)
    torch.cuda.synchronize()
    got = h.cpu().numpy()
    ring = _ring(kv, cfg)
    cache = O.Cache(L)
    want = O.forward_full(ids, W, cfg, cache=cache)
    err = norm_max_err(got, want)
    rows = np.max(np.abs(got - want), axis=1) / np.max(np.abs(want))
    print("prefill T=3000, 4 distinct blocks: err %.3g (worst row %d, last 120 rows %.3g)"
          % (err, int(np.argmax(rows)), float(np.max(rows[2880:]))))
    assert err <= BF16_TOL
    for l in range(L):
        _, K, V = cache.layers[l][0]
        for kvi, ref in ((0, K), (1, V)):
            e = norm_max_err(O.f64(ring[l, kvi, 0]), np.asarray(ref).transpose(1, 0, 2))
            assert e <= BF16_TOL, (l, kvi, e)


def test_full_prefill_32_blocks_T3000():
    """The full 32-block stack at T = 3000 against the oracle's rows stored by
    tests/golden/make_prefill_T3000.py (same seeds: weights 44, IDs 45)."""
    import os
    import torch
    from tests.conftest import GOLDEN
    gold = np.load(os.path.join(GOLDEN, "prefill_T3000_32blocks.npz"))
    cfg = dict(synth.FULL_TEMPORAL)
    T, L, D = cfg["context"], cfg["n_layers"], cfg["d_model"]
    W = synth.temporal_weights(cfg, 44, "bf16", with_text_head=False, shared_layer=True)
    ids = synth.stream_ids(cfg, T, 45)
    model = _model(cfg, W, max_T=T)
    kv = model.kv_alloc()
    h = torch.empty((T, D), device="cuda")
    model.prefill(kv, ids, h)
    torch.cuda.synchronize()
    assert kv.info()[0] == T
    rows = gold["rows"]
    got = h.cpu().numpy()[rows]
    err = norm_max_err(got, gold["h"])
    per_row = np.max(np.abs(got - gold["h"]), axis=1) / np.max(np.abs(gold["h"]))
    print("prefill T=3000, 32 blocks: err %.3g over rows %s; worst row %d"
          % (err, list(rows), int(rows[np.argmax(per_row)])))
    assert err <= BF16_TOL
    ring = _ring(kv, cfg)
    for l in (0, L - 1):
        for kvi, name in ((0, "k%d" % l), (1, "v%d" % l)):
            g = ring[l, kvi, 0][:, rows].transpose(1, 0, 2).reshape(len(rows), D)
            e = norm_max_err(O.f64(g), gold[name])
            print("  ring layer %d %s at those positions: err %.3g" % (l, "KV"[kvi], e))
            assert e <= BF16_TOL


def test_full_generator_frames_ctx3000():
    """Generator frames at full size with the ring of keys full, as the benchmark runs them:
    every drawn code equals the oracle sampler's draw on the GPU's own logits, supplied codes
    win, the temporal input of call s is the ring slot that call s - 1 filled, and the
    aligned output takes delay-0 streams from call s - 1 and delay-1 streams from call s."""
    import torch
    from oracle import generator as OG
    from oracle.sampling import sample_top_k
    cfg, dc = dict(synth.FULL_TEMPORAL), dict(synth.FULL_DEPTH)
    C, D = cfg["context"], cfg["d_model"]
    W = synth.temporal_weights(cfg, 46, "bf16", with_text_head=True, shared_layer=True)
    model = _model(cfg, W)
    kv = model.kv_alloc()
    frames = synth.cache_frames(cfg, C, 47)
    kv.load(torch.from_numpy(frames.view(np.int16)).cuda(), C)
    del frames
    g = torch.Generator(device="cuda")
    g.manual_seed(48)
    Dd, F, S, Ld = dc["d_model"], dc["d_ff"], dc["n_steps"], dc["n_layers"]
    mat = lambda r, c: (0.02 * torch.randn((r, c), generator=g, device="cuda")).to(torch.bfloat16)
    DW = {"depformer_text_emb.weight": mat(dc["text_vocab"], Dd)}
    for q in range(S):
        DW["depformer_in.%d.weight" % q] = mat(Dd, D)
        DW["linears.%d.weight" % q] = mat(dc["n_out"], Dd)
        if q < S - 1:
            DW["depformer_emb.%d.weight" % q] = mat(dc["audio_vocab"], Dd)
    for m in range(Ld):
        p = "depformer.layers.%d." % m
        DW[p + "self_attn.in_proj_weight"] = mat(S * 3 * Dd, Dd)
        DW[p + "self_attn.out_proj.weight"] = mat(S * Dd, Dd)
        for q in range(S):
            DW[p + "gating.%d.linear_in.weight" % q] = mat(2 * F, Dd)
            DW[p + "gating.%d.linear_out.weight" % q] = mat(Dd, F)
        DW[p + "norm1.alpha"] = torch.ones(Dd, device="cuda")
        DW[p + "norm2.alpha"] = torch.ones(Dd, device="cuda")
    dep = pp.Depformer(dc, DW, "bf16")
    gen = pp.Generator(model, kv, dep)
    rng = np.random.default_rng(49)
    n = 6
    prov = np.full((n, 17), -1, np.int32)
    prov[:, 9:] = rng.integers(0, dc["n_out"], (n, 8))
    U = rng.random((n, 17))
    dly = np.array(OG.DELAYS)
    out = torch.empty(17, dtype=torch.int32, device="cuda")
    ins = torch.empty(17, dtype=torch.int32, device="cuda")
    cho = torch.empty(17, dtype=torch.int32, device="cuda")
    tl = torch.empty(cfg["text_vocab"] - 1, device="cuda")
    dl = torch.empty((S, dc["n_out"]), device="cuda")
    chosen = {}
    for s in range(n):
        has = gen.step(prov[s], U[s], out)
        if s == 0:
            assert not has
            continue
        gen.inspect(ins, cho, tl, dl)
        torch.cuda.synchronize()
        c, i, t_l, d_l = cho.cpu().numpy(), ins.cpu().numpy(), tl.cpu().numpy(), dl.cpu().numpy()
        chosen[s] = c
        assert c[0] == sample_top_k(t_l, 0.7, 25, U[s][0]), s
        for k in range(1, 9):
            assert c[k] == sample_top_k(d_l[k - 1], 0.8, 250, U[s][k]), (s, k)
        assert c[9] == prov[s][9] and np.array_equal(c[10:], prov[s - 1][10:]), s
        if s >= 2:
            assert np.array_equal(i, chosen[s - 1]), s      # the input slot is the last call's target
        assert has == (s >= 2), s
        if has:
            want = np.where(dly == 0, chosen[s - 1], c)
            assert np.array_equal(out.cpu().numpy(), want), s
    assert kv.info()[0] == C + n - 1
    print("full generator: %d calls, drawn codes equal the oracle sampler on the GPU logits" % n)


def test_full_prefill_chunk_after_full_ring():
    """A 256-frame chunk at position 3000 into a ring holding 3000 synthetic frames
    (positions 0..2999): the chunk's first queries still read keys in slots the chunk
    itself overwrites. Every row of the chunk and the ring slots it writes (layers 0, 16,
    31) against the oracle's chunk over the same history; the slots it does not write are
    left bit for bit as loaded."""
    import torch
    cfg = dict(synth.FULL_TEMPORAL)
    C, L, D, H, dh = cfg["context"], cfg["n_layers"], cfg["d_model"], cfg["n_heads"], cfg["d_head"]
    n = 256
    W = synth.temporal_weights(cfg, 50, "bf16", with_text_head=False, shared_layer=True)
    frames = synth.cache_frames(cfg, C, 52)                    # [L, 2, 1, H, C, dh] bf16 bits
    ids = synth.stream_ids(cfg, n, 51)
    model = _model(cfg, W, max_T=n)
    kv = model.kv_alloc()
    kv.load(torch.from_numpy(frames.view(np.int16)).cuda(), C)
    hc = torch.empty((n, D), device="cuda")
    model.prefill(kv, ids, hc)
    torch.cuda.synchronize()
    assert kv.info()[0] == C + n
    got = hc.cpu().numpy()
    ring = _ring(kv, cfg)
    cache = O.cache_from_blocks([frames[l, 0, 0].transpose(1, 0, 2) for l in range(L)],
                                [frames[l, 1, 0].transpose(1, 0, 2) for l in range(L)], np.arange(C), L)
    want = O.forward_full(ids, W, cfg, p0=C, cache=cache)
    err = norm_max_err(got, want)
    print("chunk of %d at position %d: rows err %.3g" % (n, C, err))
    assert err <= BF16_TOL
    for l in (0, L // 2, L - 1):
        pos, K, V = cache.layers[l][-1]
        assert pos[0] == C
        for kvi, ref in ((0, K), (1, V)):
            e = norm_max_err(O.f64(ring[l, kvi, 0][:, :n]), np.asarray(ref).transpose(1, 0, 2))
            assert e <= BF16_TOL, (l, kvi, e)
    assert np.array_equal(ring[:, :, :, :, n:], frames[:, :, :, :, n:])


@pytest.mark.parametrize("B,sessions,oracle_session", [(4, (0, 1, 2, 3), 3), (40, (0, 16, 31, 32, 39), 39),
                                                       (64, (0, 15, 16, 33, 48, 63), 33)])
def test_full_batched_decode_ctx3000(B, sessions, oracle_session):
    """B sessions decoded together (every weight byte shared, float16 activations into the
    matrix cores), rings full at 3000 random frames, 2 frames at positions 3000 and 3001
    (keys wrap). One session against the oracle's decode of its own ring (2e-2); the
    sampled sessions (tile boundaries; B = 40: 3 session tiles, the last one partial; B = 64,
    the largest batch: 4 session tiles, about 230 GB of device memory with its 100 GB of
    rings) also against the same session decoded
    alone on the GPU, which rounds differently (float32 activations), to 2 x 2e-2."""
    import gc
    import torch
    cfg = dict(synth.FULL_TEMPORAL)
    C, L, D, H, dh = cfg["context"], cfg["n_layers"], cfg["d_model"], cfg["n_heads"], cfg["d_head"]
    W = synth.temporal_weights(cfg, 70, "bf16", with_text_head=False, shared_layer=True)
    require_gpu()
    gc.collect()
    torch.cuda.empty_cache()
    model = pp.TemporalModel(cfg, to_device(W), "bf16", max_batch=B)
    g = torch.Generator(device="cuda")
    g.manual_seed(71)
    frames = torch.randn((L, 2, B, H, C, dh), generator=g, device="cuda", dtype=torch.bfloat16)
    ids = synth.stream_ids(cfg, 2, 72, batch=B)
    kv = model.kv_alloc(B)
    kv.load(frames, C)
    one = {b: frames[:, :, b:b + 1].contiguous() for b in sessions}
    del frames
    torch.cuda.empty_cache()
    hb = torch.empty((2, B, D), device="cuda")
    for t in range(2):
        model.decode_step(kv, ids[:, t], hb[t])
    torch.cuda.synchronize()
    hbn = hb.cpu().numpy()

    ring_b = one[oracle_session].view(torch.int16).cpu().numpy().view(np.uint16)   # [L, 2, 1, H, C, dh]
    cache = O.cache_from_blocks([ring_b[l, 0, 0].transpose(1, 0, 2) for l in range(L)],
                                [ring_b[l, 1, 0].transpose(1, 0, 2) for l in range(L)], np.arange(C), L)
    del ring_b
    want = O.decode_incremental(ids[oracle_session], W, cfg, p0=C, cache=cache)
    err_o = norm_max_err(hbn[:, oracle_session], want)
    print("full batched decode B=%d, session %d vs oracle: err %.3g" % (B, oracle_session, err_o))
    assert err_o <= BF16_TOL

    errs = []
    for b in sessions:
        kv1 = model.kv_alloc(1)
        kv1.load(one[b], C)
        h1 = torch.empty((2, D), device="cuda")
        for t in range(2):
            model.decode_step(kv1, ids[b, t], h1[t])
        torch.cuda.synchronize()
        errs.append(norm_max_err(hbn[:, b], h1.cpu().numpy()))
        kv1.close()
    print("full batched decode B=%d vs single sessions %s: errs %s" % (B, list(sessions), ["%.3g" % e for e in errs]))
    kv.close()
    model.close()
    assert max(errs) <= 2 * BF16_TOL


def test_full_decode_with_four_readers_matches_oracle():
    """The released reader configuration: 4 readers after zero-based blocks 7, 15, 23, 31
    of the 32-block stack, 32 heads x 128, 1024-wide memory with 1024 visible rows; one
    decode frame at position 3000 on a full ring, against the oracle (2e-2)."""
    import torch
    from oracle import reader as ORD
    cfg = dict(synth.FULL_TEMPORAL)
    C, L, D = cfg["context"], cfg["n_layers"], cfg["d_model"]
    W = synth.temporal_weights(cfg, 100, "bf16", with_text_head=False, shared_layer=True)
    R = synth.reader_weights(cfg, 4, 1024, 101, "bf16", scale=0.05)
    M = synth.memory_bank(1024, 1024, 102, "bf16")
    frames = synth.cache_frames(cfg, C, 103)
    ids = synth.stream_ids(cfg, 1, 104)
    model = _model(cfg, W)
    model.attach_readers([7, 15, 23, 31], to_device(R), 1024, 1024)
    model.write_memory(torch.from_numpy(M.view(np.int16)).cuda().view(torch.bfloat16))
    model.set_visible(1024)
    kv = model.kv_alloc()
    kv.load(torch.from_numpy(frames.view(np.int16)).cuda(), C)
    h = torch.empty(D, device="cuda")
    model.decode_step(kv, ids[0], h)
    torch.cuda.synchronize()
    ks = [frames[l, 0, 0].transpose(1, 0, 2) for l in range(L)]
    vs = [frames[l, 1, 0].transpose(1, 0, 2) for l in range(L)]
    cache = O.cache_from_blocks(ks, vs, np.arange(C), L)
    x = O.decode_step(O.embed(ids[0], W, cfg), C, cache, W, cfg,
                      after_block=ORD.hooks([7, 15, 23, 31], M, 1024, R, cfg["n_heads"]))
    err = norm_max_err(h.cpu().numpy(), O.final(x, W, cfg))
    print("full decode with 4 readers (1024 visible rows): err %.3g" % err)
    assert err <= BF16_TOL
