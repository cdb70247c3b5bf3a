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
    """A 256-frame chunk at position 3000, after a 3000-frame prefill filled the ring: its
    first queries still read keys in slots the chunk itself overwrites. Checked against
    frame-by-frame decode of the same frames from a snapshot of the same ring (hidden rows
    sampled across the chunk, and the K/V both leave in the ring), to 2 x 2e-2."""
    import torch
    cfg = dict(synth.FULL_TEMPORAL)
    C, L, D, H, dh = cfg["context"], cfg["n_layers"], cfg["d_model"], cfg["n_heads"], cfg["d_head"]
    W = synth.temporal_weights(cfg, 50, "bf16", with_text_head=False, shared_layer=True)
    ids = synth.stream_ids(cfg, C + 256, 51)
    model = _model(cfg, W, max_T=C)
    kv = model.kv_alloc()
    h0 = torch.empty((C, D), device="cuda")
    model.prefill(kv, ids[:C], h0)
    snap = torch.empty(kv.info()[1] // 2, dtype=torch.int16, device="cuda")
    kv.store(snap)
    hc = torch.empty((256, D), device="cuda")
    model.prefill(kv, ids[C:], hc)
    ring_c = torch.empty_like(snap)
    kv.store(ring_c)
    assert kv.info()[0] == C + 256
    kv.restore(snap, C)
    hd = torch.empty(D, device="cuda")
    rows = {0, 1, 100, 255}
    got_d = {}
    for t in range(256):
        model.decode_step(kv, ids[C + t], hd)
        if t in rows:
            got_d[t] = hd.cpu().numpy().copy()
    ring_d = torch.empty_like(snap)
    kv.store(ring_d)
    torch.cuda.synchronize()
    hcn = hc.cpu().numpy()
    errs = [norm_max_err(hcn[t], got_d[t]) for t in sorted(rows)]
    shape = (L, 2, 1, H, C, dh)
    rc = synth.bf16_bits_to_f32(ring_c.cpu().numpy().view(np.uint16).reshape(shape))
    rd = synth.bf16_bits_to_f32(ring_d.cpu().numpy().view(np.uint16).reshape(shape))
    ring_errs = [norm_max_err(rc[l, :, :, :, :256], rd[l, :, :, :, :256]) for l in (0, 16, 31)]
    print("full chunk at 3000: rows vs decode %s, ring %s" % (["%.3g" % e for e in errs], ["%.3g" % e for e in ring_errs]))
    assert max(errs) <= 2 * BF16_TOL and max(ring_errs) <= 2 * BF16_TOL
    assert np.array_equal(rc[:, :, :, :, 256:], rd[:, :, :, :, 256:])   # untouched slots agree bit for bit


@pytest.mark.parametrize("B,sessions", [(4, (0, 1, 2, 3)), (64, (0, 15, 16, 33, 48, 63))])
def test_full_batched_decode_ctx3000_matches_single_sessions(B, sessions):
    """B sessions decoded together (every weight byte shared, float16 activations into the
    matrix cores) against the same sessions decoded one at a time, rings full at 3000
    random frames, 2 frames at positions 3000 and 3001 (keys wrap): 2 x 2e-2. B = 64 is the
    largest batch (4 session tiles; about 230 GB of device memory with its 100 GB of rings);
    it checks the sessions at the tile boundaries."""
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
    errs = []
    for b in sessions:
        kv1 = model.kv_alloc(1)
        kv1.load(one[b], C)
        h1 = torch.empty((2, D), device="cuda")
        for t in range(2):
            model.decode_step(kv1, ids[b, t], h1[t])
        torch.cuda.synchronize()
        errs.append(norm_max_err(hb[:, b].cpu().numpy(), h1.cpu().numpy()))
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
