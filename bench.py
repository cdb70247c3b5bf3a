"""Benchmark: temporal decode ms/frame at B = 1, 32 blocks, context 3000, bf16 weights.

One step = one decode frame through libpp (embedding sum, 32 blocks, final RMSNorm) with
the ring full (3000 visible keys per head and layer). Weights are random (0.02 N(0,1),
bfloat16), drawn on the device; the ring is filled with N(0,1) bfloat16 keys/values.
Everything is resident in HBM before the timed region starts.

Prints ONE JSON line (rank 0). Extra fields: frames_per_s, achieved_GBps (whole frame,
algorithmic bytes), roofline (dominant kernel: the fused RMSNorm + W_in + SiLU-product
GEMV, timed with HIP events on the launch stream), cpu_baseline (the oracle on a bounded
sample), and optional depformer / prefill lines when those workloads are requested.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
TRACE_REPEAT = 10          # launches of the timed kernel per event pair
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "temporal decode ms/frame (B=1, 32 blocks, ctx 3000) + achieved HBM GB/s"


def frame_bytes(cfg, n_keys):
    """Algorithmic HBM bytes of one decode frame: every weight once, every visible K/V
    once, one new K/V slot, 17 embedding rows (bf16)."""
    D, F, L, H, dh = cfg["d_model"], cfg["d_ff"], cfg["n_layers"], cfg["n_heads"], cfg["d_head"]
    weights = L * (3 * D * D + D * D + 2 * F * D + D * F) * 2
    if cfg.get("_no_kv"):
        return weights
    kv_read = L * 2 * H * n_keys * dh * 2
    kv_write = L * 2 * D * 2
    emb = 17 * D * 2
    return weights + kv_read + kv_write + emb


def w_in_bytes(cfg):
    """Algorithmic bytes of one fused RMSNorm + W_in + SiLU-product launch: the
    [2F, D] bf16 matrix, the fp32 input vector and norm scale, the fp32 output."""
    D, F = cfg["d_model"], cfg["d_ff"]
    return 2 * F * D * 2 + D * 4 + D * 4 + F * 4


GEMV_SOURCES = ("device.h", "gemv_kernel.h", "gemv_swiglu.hip")  # the W_in kernel's sources


def gemv_source_hash():
    """SHA-256 over the sources the W_in kernel is compiled from."""
    import hashlib
    h = hashlib.sha256()
    for name in GEMV_SOURCES:
        h.update(open(os.path.join(ROOT, "personaplex_temporal_transformer_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the W_in kernel from the committed counter runs
    (profiles/decode_w_in_traffic.json), or None once the GEMV sources have changed since."""
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "decode_w_in_traffic.json")))
        digest = gemv_source_hash()
    except (OSError, ValueError):
        return None
    if rec.get("gemv_source_sha256") != digest:
        return None
    return rec.get("traffic_bytes_per_launch")


def make_device_weights(cfg, seed):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    D, F, L = cfg["d_model"], cfg["d_ff"], cfg["n_layers"]

    def mat(r, c):
        t = torch.empty((r, c), dtype=torch.bfloat16, device="cuda")
        for i in range(0, r, 4096):
            blk = torch.randn((min(4096, r - i), c), generator=g, device="cuda", dtype=torch.float32)
            t[i:i + blk.shape[0]] = (blk * 0.02).to(torch.bfloat16)
        return t

    def norm(n):
        return 1.0 + 0.02 * torch.randn(n, generator=g, device="cuda", dtype=torch.float32)

    W = {"text_emb.weight": mat(cfg["text_vocab"], D)}
    for i in range(cfg["n_audio"]):
        W["emb.%d.weight" % i] = mat(cfg["audio_vocab"], D)
    for l in range(L):
        p = "transformer.layers.%d." % l
        W[p + "self_attn.in_proj_weight"] = mat(3 * D, D)
        W[p + "self_attn.out_proj.weight"] = mat(D, D)
        W[p + "gating.linear_in.weight"] = mat(2 * F, D)
        W[p + "gating.linear_out.weight"] = mat(D, F)
        W[p + "norm1.alpha"] = norm(D)
        W[p + "norm2.alpha"] = norm(D)
    W["out_norm.alpha"] = norm(D)
    W["text_linear.weight"] = mat(cfg["text_vocab"] - 1, D)
    return W


def depth_frame_bytes(dc):
    """Algorithmic bytes of one depth frame: every per-step weight slice once (in_proj,
    QKV/O slices, FFN pair, head) plus one embedding row per position (bf16)."""
    D, F, S, L = dc["d_model"], dc["d_ff"], dc["n_steps"], dc["n_layers"]
    per_step = D * dc["d_temporal"] + L * (3 * D * D + D * D + 2 * F * D + D * F) + dc["n_out"] * D + D
    return S * per_step * 2


def make_depth_weights(dc, seed):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    D, F, S, L = dc["d_model"], dc["d_ff"], dc["n_steps"], dc["n_layers"]

    def mat(r, c):
        return (0.02 * torch.randn((r, c), generator=g, device="cuda")).to(torch.bfloat16)

    W = {"depformer_text_emb.weight": mat(dc["text_vocab"], D)}
    for q in range(S):
        W["depformer_in.%d.weight" % q] = mat(D, dc["d_temporal"])
        W["linears.%d.weight" % q] = mat(dc["n_out"], D)
        if q < S - 1:
            W["depformer_emb.%d.weight" % q] = mat(dc["audio_vocab"], D)
    for m in range(L):
        p = "depformer.layers.%d." % m
        W[p + "self_attn.in_proj_weight"] = mat(S * 3 * D, D)
        W[p + "self_attn.out_proj.weight"] = mat(S * D, D)
        for q in range(S):
            W[p + "gating.%d.linear_in.weight" % q] = mat(2 * F, D)
            W[p + "gating.%d.linear_out.weight" % q] = mat(D, F)
        W[p + "norm1.alpha"] = 1.0 + 0.02 * torch.randn(D, generator=g, device="cuda")
        W[p + "norm2.alpha"] = 1.0 + 0.02 * torch.randn(D, generator=g, device="cuda")
    return W


def bench_depformer(d, dc, steps, warmup):
    """Depth transformer frames (16 positions, greedy selection) at full size, bf16."""
    import torch
    S = dc["n_steps"]
    g = torch.Generator(device="cuda")
    g.manual_seed(6)
    h = torch.randn(dc["d_temporal"], generator=g, device="cuda")
    codes = torch.empty(S, dtype=torch.int32, device="cuda")
    for i in range(warmup):
        d.step(h, i % 32000, codes)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(steps):
        d.step(h, (7 * i) % 32000, codes)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    nb = depth_frame_bytes(dc)
    return {"ms_per_frame": round(ms, 4), "us_per_position": round(ms * 1000.0 / S, 2), "frame_bytes": nb,
            "achieved_GBps": round(nb / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "steps": steps,
            "workload": "depth transformer, 16 positions greedy, 6 layers x 1024, window 8, bf16"}


FRAME_BUDGET_MS = 80.0   # one 12.5 Hz audio frame


def bench_generator(model, kv, d, cfg, dc, steps, warmup):
    """Whole generator frames at full size: the code ring, the 32-block temporal step with
    the ring of keys full, the text head and a text draw (top 25, temperature 0.7), and the
    16-position depth loop drawing each code (top 250, temperature 0.8); user audio codes
    supplied every call, uniforms drawn on the host."""
    import torch
    from personaplex_temporal_transformer_amd import pp
    gen = pp.Generator(model, kv, d)
    rng = np.random.default_rng(12)
    n = warmup + steps + 1
    prov = np.full((n, 17), -1, np.int32)
    prov[:, 9:] = rng.integers(0, dc["n_out"], (n, 8))
    U = rng.random((n, 17))
    out = torch.empty(17, dtype=torch.int32, device="cuda")
    for i in range(warmup + 1):
        gen.step(prov[i], U[i], out)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(warmup + 1, n):
        gen.step(prov[i], U[i], out)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    pos, _ = kv.info()
    nb = frame_bytes(cfg, cfg["context"]) + depth_frame_bytes(dc) + (cfg["text_vocab"] - 1) * cfg["d_model"] * 2
    gen.close()
    return {"ms_per_frame": round(ms, 4), "frames_per_s": round(1000.0 / ms, 2),
            "realtime_factor": round(FRAME_BUDGET_MS / ms, 2), "frame_budget_ms": FRAME_BUDGET_MS,
            "frame_bytes": nb, "achieved_GBps": round(nb / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "steps": steps,
            "final_position": pos,
            "workload": "generator frame: code ring + 32-block temporal step (3000 visible keys) + text head "
                        "+ text draw (top 25, T 0.7) + 16-position depth loop with draws (top 250, T 0.8), bf16"}


def bench_one_block(W, cfg, steps, warmup):
    """One full-width block (layer 0's weights) as a 1-block model: ring loaded with 200
    frames, then `steps` decode steps from position 200 (201 .. 200+steps visible keys),
    each timed with its own event pair on graph replays. The step also runs the embedding
    sum and the final norm (two more launches than the block itself)."""
    import torch
    from personaplex_temporal_transformer_amd import pp, synth
    cfg1 = synth.with_(cfg, n_layers=1)
    W1 = {k: v for k, v in W.items() if not k.startswith("transformer.layers.") or k.startswith("transformer.layers.0.")}
    m1 = pp.TemporalModel(cfg1, W1, "bf16", max_prefill_T=0, max_batch=1)
    kv1 = m1.kv_alloc()
    n0 = 200
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    buf = torch.randn(2 * cfg["n_heads"] * n0 * cfg["d_head"], generator=g, device="cuda").to(torch.bfloat16)
    ids = synth.stream_ids(cfg1, warmup + steps, 4)
    h = torch.empty(cfg["d_model"], device="cuda")
    m1.set_graph(True)
    kv1.load(buf, n0)
    for i in range(warmup):
        m1.decode_step(kv1, ids[i], h)
    kv1.load(buf, n0)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        evs[i][0].record()
        m1.decode_step(kv1, ids[warmup + i], h)
        evs[i][1].record()
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1000.0 for a, b in evs)
    # the same steps back to back between one event pair (as the decode frames are timed):
    # the per-step pairs above also carry each pair's own cost
    kv1.load(buf, n0)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s0.record()
    for i in range(steps):
        m1.decode_step(kv1, ids[warmup + i], h)
    s1.record()
    torch.cuda.synchronize()
    mean_b2b = s0.elapsed_time(s1) * 1000.0 / steps
    D, F, Hh, dh = cfg["d_model"], cfg["d_ff"], cfg["n_heads"], cfg["d_head"]
    nb = (3 * D * D + D * D + 2 * F * D + D * F) * 2 + (n0 + 1) * Hh * dh * 2 * 2 + Hh * dh * 2 * 2
    med = float(np.median(us))
    kv1.close()
    m1.close()
    return {"us_per_step_median": round(med, 2), "us_per_step_min": round(us[0], 2), "steps": steps,
            "us_per_step_back_to_back": round(mean_b2b, 2),
            "hbm_frac_back_to_back": round(nb / (mean_b2b * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "step_bytes_at_201_keys": nb, "achieved_GBps": round(nb / (med * 1e-6) / 1e9, 1),
            "hbm_frac": round(nb / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "workload": "one full-width temporal block (d_model 4096, 32 x 128 heads, d_ff 11264), bf16, "
                        "ring loaded with 200 frames, steps at positions 200..%d, embedding sum and final norm "
                        "included" % (n0 + steps - 1)}


def prefill_flops(cfg, T):
    """Algorithmic FLOPs of one T-frame prefill: every linear (2 per weight per frame)
    plus causal attention (Q K^T and P V over the T (T + 1) / 2 visible pairs per head)."""
    D, F, L, H, dh = cfg["d_model"], cfg["d_ff"], cfg["n_layers"], cfg["n_heads"], cfg["d_head"]
    gemm = 2 * T * L * (3 * D * D + D * D + 2 * F * D + D * F)
    attn = 2 * 2 * dh * H * L * (T * (T + 1) // 2)
    return gemm, attn


def bench_prefill(model, cfg, T, steps, warmup):
    """Full-sequence prefill of T frames from an empty ring (its own ring), bf16 MFMA path."""
    import torch
    from personaplex_temporal_transformer_amd import synth
    kv = model.kv_alloc()
    ids = synth.stream_ids(cfg, T, 11)
    h = torch.empty((T, cfg["d_model"]), device="cuda")
    for _ in range(warmup):
        kv.reset()
        model.prefill(kv, ids, h)
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        kv.reset()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        model.prefill(kv, ids, h)
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    kv.close()
    ms = float(np.median(times))
    gemm, attn = prefill_flops(cfg, T)
    tflops = (gemm + attn) / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 3), "ms_min": round(min(times), 3), "frames": T,
            "frames_per_s": round(T / (ms * 1e-3), 1), "flop": gemm + attn, "gemm_flop": gemm,
            "attention_flop": attn, "achieved_TFLOPs": round(tflops, 1), "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
            "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "steps": steps,
            "workload": "full 32-block temporal prefill, B=1, T=%d frames from position 0, float16 matrix "
                        "cores (float16 copy of the bf16 weights; peak = the 2.5 PFLOP/s dense bf16/fp16 figure), "
                        "K/V written to ring slots 0..T-1" % T}


def bench_vendor_gemm(cfg, T, steps=10):
    """For comparison only (not the product path): the vendor library's plain float16
    products (torch.matmul, no fused epilogues) on the prefill's four GEMM shapes at M = T,
    random operands; mean us per product over `steps` back-to-back calls."""
    import torch
    D, F = cfg["d_model"], cfg["d_ff"]
    out = {}
    for name, N, K in (("QKV", 3 * D, D), ("W_O", D, D), ("W_in", 2 * F, D), ("W_out", D, F)):
        A = torch.randn(T, K, device="cuda", dtype=torch.float16)
        B = torch.randn(N, K, device="cuda", dtype=torch.float16)
        for _ in range(3):
            C = A @ B.t()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(steps):
            C = A @ B.t()
        e.record()
        torch.cuda.synchronize()
        us = s.elapsed_time(e) * 1000.0 / steps
        out[name] = {"us": round(us, 1), "M": T, "N": N, "K": K, "TFLOPs": round(2.0 * T * N * K / us / 1e6, 1)}
        del A, B, C
    out["note"] = ("vendor library (torch.matmul / hipBLASLt) plain float16 products on the same shapes, "
                   "for comparison; the library's own products carry fused epilogues")
    return out


def bench_chunk(model, kv, cfg, T, steps, warmup):
    """Prefill chunks of T frames into the live, full ring (prompt replay at position > 0):
    each chunk's queries see the 3000-key window of history plus the chunk."""
    import torch
    n = warmup + steps
    ids = synth_ids(cfg, n * T, 13)
    h = torch.empty((T, cfg["d_model"]), device="cuda")
    for i in range(warmup):
        model.prefill(kv, ids[i * T:(i + 1) * T], h)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(warmup, n):
        model.prefill(kv, ids[i * T:(i + 1) * T], h)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    D, F, L, H, dh, C = cfg["d_model"], cfg["d_ff"], cfg["n_layers"], cfg["n_heads"], cfg["d_head"], cfg["context"]
    gemm = 2.0 * T * L * (3 * D * D + D * D + 2 * F * D + D * F)
    attn = 2.0 * 2 * dh * H * L * T * C          # every query sees a full window of C keys
    tf = (gemm + attn) / (ms * 1e-3) / 1e12
    pos, _ = kv.info()
    return {"ms": round(ms, 3), "T": T, "TFLOPs": round(tf, 1), "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "frames_per_s": round(T * 1000.0 / ms, 1), "flop": gemm + attn, "steps": steps, "final_position": pos,
            "workload": "prefill chunk of %d frames into the full ring (history window 3000 keys, ring wraps), "
                        "32 blocks, bf16" % T}


def bench_batched(model, cfg, batches, steps, warmup):
    """Batched decode: B sessions at one position share every weight byte of the step;
    each session's ring is full (3000 frames, zero-filled keys/values -- the timing does
    not depend on their values), positions 3000+."""
    import torch
    out = []
    C = cfg["context"]
    for B in batches:
        kv = model.kv_alloc(B)
        buf = torch.zeros(kv.info()[1] // 2, dtype=torch.bfloat16, device="cuda")
        kv.load(buf, C)
        del buf
        ids = synth_ids(cfg, warmup + steps, 14 + B)
        h = torch.empty((B, cfg["d_model"]), device="cuda")
        rows = [np.ascontiguousarray(np.broadcast_to(ids[i], (B, ids.shape[1]))) for i in range(warmup + steps)]
        for i in range(warmup):
            model.decode_step(kv, rows[i], h)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(warmup, warmup + steps):
            model.decode_step(kv, rows[i], h)
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / steps
        nb = frame_bytes(cfg, C) + (B - 1) * (frame_bytes(cfg, C) - frame_bytes(synth_cfg_no_weights(cfg), 0))
        out.append({"B": B, "ms_per_step": round(ms, 4), "frames_per_s": round(B * 1000.0 / ms, 1),
                    "step_bytes": nb, "achieved_GBps": round(nb / (ms * 1e-3) / 1e9, 1),
                    "hbm_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)})
        kv.close()
        torch.cuda.empty_cache()
    return {"workload": "batched decode, B sessions at one position, each ring full at 3000 frames, 32 blocks, "
                        "bf16 weights, float16 activations into v_mfma_f32_16x16x32_f16", "steps": steps,
            "points": out}


def bench_readers(model, kv, cfg, slots_list, steps, warmup):
    """Decode frames with the 4 memory readers of the released configuration (after blocks
    7, 15, 23, 31; 1024-wide memory; weights drawn on the device) at several visible-memory
    sizes, on the live full ring."""
    import torch
    D, mem = cfg["d_model"], 1024
    g = torch.Generator(device="cuda")
    g.manual_seed(15)
    R = {}
    for i in range(4):
        p = "readers.%d." % i
        R[p + "norm.weight"] = 1.0 + 0.02 * torch.randn(D, generator=g, device="cuda")
        R[p + "norm.bias"] = 0.02 * torch.randn(D, generator=g, device="cuda")
        for name, k in (("q_proj", D), ("k_proj", mem), ("v_proj", mem), ("out_proj", D)):
            R[p + name + ".weight"] = (0.02 * torch.randn((D, k), generator=g, device="cuda")).to(torch.bfloat16)
            R[p + name + ".bias"] = 0.02 * torch.randn(D, generator=g, device="cuda")
    top = max(slots_list)
    model.attach_readers([7, 15, 23, 31], R, mem, top)
    model.write_memory(torch.randn((top, mem), generator=g, device="cuda").to(torch.bfloat16))
    ids = synth_ids(cfg, warmup + steps, 16)
    h = torch.empty(D, device="cuda")
    pts = []
    for n in slots_list:
        model.set_visible(n)
        for i in range(warmup):
            model.decode_step(kv, ids[i], h)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(warmup, warmup + steps):
            model.decode_step(kv, ids[i], h)
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / steps
        extra = 4 * (2 * D * D * 2 + 2 * n * D * 2)
        nb = frame_bytes(cfg, cfg["context"]) + extra
        pts.append({"visible_rows": n, "ms_per_frame": round(ms, 4), "frame_bytes": nb,
                    "reader_bytes": extra, "hbm_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)})
    model.set_visible(0)
    return {"workload": "decode frame (32 blocks, ring full) with 4 memory readers after blocks 7/15/23/31, "
                        "32 heads x 128, 1024-wide memory", "steps": steps, "points": pts}


def synth_cfg_no_weights(cfg):
    """The decode-frame byte formula with the weights taken out: frame_bytes(cfg, C) minus
    frame_bytes(this, 0) is one session's K/V read, K/V write and embedding rows."""
    c = dict(cfg)
    c["_no_kv"] = True
    return c


def synth_ids(cfg, n, seed):
    from personaplex_temporal_transformer_amd import synth
    return synth.stream_ids(cfg, n, seed)


def fill_ring(kv, cfg, seed):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    C = cfg["context"]
    per_layer = 2 * cfg["n_heads"] * C * cfg["d_head"]
    buf = torch.empty(cfg["n_layers"] * per_layer, dtype=torch.bfloat16, device="cuda")
    for l in range(cfg["n_layers"]):
        buf[l * per_layer:(l + 1) * per_layer] = torch.randn(per_layer, generator=g, device="cuda").to(torch.bfloat16)
    kv.load(buf, C)
    del buf


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count() or 1


def _host():
    """What the oracle's times ran on: CPU model, logical CPUs, BLAS threads."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "blas_threads": int(_blas_threads())}


def _timed_both(fn, n=3):
    """Best of n at the BLAS pool's threads, and once at one thread (seconds)."""
    t, _ = _best_of(fn, n)
    t1 = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t1, _ = _best_of(fn, 1)
    except ImportError:
        pass
    return t, t1


def _best_of(fn, n=3):
    times = []
    for _ in range(n):
        t0 = time.time()
        fn()
        times.append(time.time() - t0)
    return min(times), len(times)


def cpu_baselines(cfg, want_prefill=True, want_depth=True):
    """The oracle (fp64 NumPy) on bounded samples of each workload, on this host's cores:
    decode -- one frame through 2 of the 32 full-width blocks at 3000 visible keys, x16;
    prefill -- one full-width block over T = 256 frames, scaled by the FLOP ratio of the
    32-block T = 3000 prefill; depth -- 2 of the 16 positions of a depth frame (weights of a
    2-position depth stack), x8. Each is the best of 3."""
    from oracle import depformer as OD
    from oracle import temporal as O
    from personaplex_temporal_transformer_amd import synth
    cores = int(_blas_threads())
    out = {"host": _host()}
    # the tiny temporal stack (2 blocks, 256 wide, 16 frames, fp32): full sequence and
    # frame-by-frame decode
    tc = synth.TINY_TEMPORAL
    TW = synth.temporal_weights(tc, 0, "fp32")
    tids = synth.stream_ids(tc, 16, 1)
    tf, tf1 = _timed_both(lambda: O.forward_full(tids, TW, tc))
    ti, ti1 = _timed_both(lambda: O.decode_incremental(tids, TW, tc))
    out["tiny"] = {"full_sequence_ms": tf * 1e3, "incremental_ms": ti * 1e3, "cores": cores,
                   "full_sequence_ms_1thread": tf1 * 1e3 if tf1 else None,
                   "incremental_ms_1thread": ti1 * 1e3 if ti1 else None, "kind": "oracle",
                   "sample": "the whole tiny workload: 2 blocks, d_model 256, 16 frames, fp32 weights, best of 3"}
    del TW
    # one full-width block step at 201 visible keys (the one-block workload)
    oc = synth.with_(cfg, n_layers=1)
    OW = synth.temporal_weights(oc, 2, "bf16", with_text_head=False)
    ofr = synth.cache_frames(oc, 200, 3)
    oids = synth.stream_ids(oc, 1, 4)

    def block_step():
        cache = O.cache_from_blocks([ofr[0, 0, 0].transpose(1, 0, 2)], [ofr[0, 1, 0].transpose(1, 0, 2)],
                                    np.arange(200), 1)
        O.final(O.decode_step(O.embed(oids[0], OW, oc), 200, cache, OW, oc), OW, oc)

    tb, tb1 = _timed_both(block_step)
    out["one_block"] = {"value": tb * 1e3, "unit": "ms/step", "cores": cores, "kind": "oracle",
                        "value_1thread": tb1 * 1e3 if tb1 else None,
                        "sample": "the whole one-block step (embedding, one full-width block at 201 keys, final "
                                  "norm; fp64 NumPy), best of 3"}
    del OW, ofr
    n_l = 2
    sc = synth.with_(cfg, n_layers=n_l)
    W = synth.temporal_weights(sc, 8, "bf16", with_text_head=False)
    frames = synth.cache_frames(sc, cfg["context"], 9)
    ks = [frames[l, 0, 0].transpose(1, 0, 2) for l in range(n_l)]
    vs = [frames[l, 1, 0].transpose(1, 0, 2) for l in range(n_l)]
    ids = synth.stream_ids(sc, 256, 10)

    def decode_frame():
        cache = O.cache_from_blocks(ks, vs, np.arange(cfg["context"]), n_l)
        O.final(O.decode_step(O.embed(ids[0], W, sc), cfg["context"], cache, W, sc), W, sc)

    t, n = _best_of(decode_frame)
    t1 = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t1, _ = _best_of(decode_frame, 1)
    except ImportError:
        pass
    out["decode"] = {"value": t * 1000.0 * cfg["n_layers"] / n_l, "unit": "ms/frame", "cores": cores,
                     "kind": "oracle",
                     "sample": "one decode frame through 2 of 32 full-width blocks at 3000 visible keys "
                               "(fp64 NumPy), best of %d, scaled x16 to 32 blocks" % n}
    if t1 is not None:
        out["decode"]["value_1thread"] = t1 * 1000.0 * cfg["n_layers"] / n_l
    del frames, ks, vs
    if want_prefill:
        T = 256
        X = np.stack([O.embed(ids[t], W, sc) for t in range(T)])
        t, n = _best_of(lambda: O.block_full(X, np.arange(T), 0, W, sc))
        g_s, a_s = prefill_flops(synth.with_(cfg, n_layers=1), T)
        g_f, a_f = prefill_flops(cfg, cfg["context"])
        scale = (g_f + a_f) / (g_s + a_s)
        out["prefill"] = {"value": t * 1000.0 * scale, "unit": "ms per %d-frame prefill" % cfg["context"],
                          "cores": cores, "kind": "oracle",
                          "sample": "one full-width block over T=%d frames (fp64 NumPy, %.2f s), best of %d, "
                                    "scaled x%.1f by the FLOP ratio to 32 blocks at T=%d" % (T, t, n, scale, cfg["context"])}
    del W
    if want_depth:
        dc = synth.with_(synth.FULL_DEPTH, n_steps=2)
        DW = synth.depth_weights(dc, 5, "bf16")
        h = synth.hidden(dc["d_temporal"], 6)
        t, n = _best_of(lambda: OD.step_logits(h, 7, None, DW, dc))
        out["depth"] = {"value": t * 1000.0 * synth.FULL_DEPTH["n_steps"] / 2, "unit": "ms/frame", "cores": cores,
                        "kind": "oracle",
                        "sample": "2 of the 16 positions of a depth frame (fp64 NumPy, a 2-position depth stack "
                                  "of full width), best of %d, scaled x8" % n}
        from oracle.sampling import sample_top_k
        rng = np.random.default_rng(3)
        tl = rng.normal(size=cfg["text_vocab"] - 1).astype(np.float32)
        dl = rng.normal(size=(16, dc["n_out"])).astype(np.float32)
        u = rng.random(17)

        def draws():
            sample_top_k(tl, 0.7, 25, u[0])
            for q in range(16):
                sample_top_k(dl[q], 0.8, 250, u[q + 1])

        t, n = _best_of(draws)
        out["draws"] = {"value": t * 1000.0, "unit": "ms/frame"}
        Wh = synth.weight(8, "text_linear.weight", (cfg["text_vocab"] - 1, cfg["d_model"]), "bf16")
        Wf = {"out_norm.alpha": synth.norm_scale(8, "out_norm.alpha", cfg["d_model"]), "text_linear.weight": Wh}
        xv = synth.hidden(cfg["d_model"], 4)
        t, n = _best_of(lambda: O.final(xv, Wf, cfg, with_logits=True))
        out["text_head"] = {"value": t * 1000.0, "unit": "ms/frame"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", type=int, default=1, help="1: time HIP graph replays, 0: direct launches")
    ap.add_argument("--trace-layer", type=int, default=16)
    ap.add_argument("--no-depformer", action="store_true")
    ap.add_argument("--prefill-T", type=int, default=3000, help="0: skip the prefill line")
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--chunk-T", type=int, default=256, help="0: skip the prefill-chunk line")
    ap.add_argument("--batches", default="4,16,32", help="batched-decode sizes ('' to skip)")
    ap.add_argument("--reader-slots", default="1024,8192", help="visible memory rows for the reader line ('' to skip)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="also time the vendor library's plain products on the prefill GEMM shapes (comparison)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the run, copy 1 GiB device-to-device 3 times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from personaplex_temporal_transformer_amd import pp, synth

    cfg = dict(synth.FULL_TEMPORAL)
    t0 = time.time()
    W = make_device_weights(cfg, 8)
    batches = [int(b) for b in args.batches.split(",") if b.strip()]
    model = pp.TemporalModel(cfg, W, "bf16", max_prefill_T=max(args.prefill_T, 0),
                             max_batch=max(batches + [1]))
    kv = model.kv_alloc()
    fill_ring(kv, cfg, 9)
    torch.cuda.synchronize()
    print("setup %.1f s" % (time.time() - t0), file=sys.stderr, flush=True)
    ids = synth.stream_ids(cfg, args.warmup + 3 * args.steps + 4, 10)
    h = torch.empty(cfg["d_model"], device="cuda")
    C = cfg["context"]

    def run(n, first, graph, trace_layer=-1, repeat=1):
        model.set_graph(graph)
        model.trace(trace_layer, repeat)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(n):
            model.decode_step(kv, ids[first + i], h)
        end.record()
        torch.cuda.synchronize()
        tr = model.trace_read() if trace_layer >= 0 else (0, 0.0)
        model.trace(-1)
        return start.elapsed_time(end) / n, tr

    # warm-up, then K timed frames. The dominant kernel (layer `trace_layer`'s fused
    # RMSNorm + W_in + SiLU-product GEMV) is timed with HIP events on the launch stream,
    # which needs direct launches (a replayed graph cannot host per-launch events), in
    # passes after the timed one: one launch per event pair (the pair's own cost included),
    # then TRACE_REPEAT back-to-back launches per pair (the kernel is idempotent), whose
    # per-launch mean is the kernel's duration plus the dispatch gap between launches.
    run(args.warmup, 0, args.graph == 1)
    probe = {}
    def run_frames(n, first, graph):
        """n frames, each bracketed by its own event pair: per-frame ms."""
        model.set_graph(graph)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            evs[i][0].record()
            model.decode_step(kv, ids[first + i], h)
            evs[i][1].record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    if args.graph == 1:
        ms, _ = run(args.steps, args.warmup, True)
        _, (n_one, us_one) = run(args.steps, args.warmup, False, args.trace_layer)
        mode = 1
    else:
        ms, (n_one, us_one) = run(args.steps, args.warmup, False, args.trace_layer)
        mode = 0
    _, (n_tr, us_win) = run(args.steps, args.warmup, False, args.trace_layer, TRACE_REPEAT)
    per_frame = sorted(run_frames(args.steps, args.warmup + 2 * args.steps, mode == 1))
    pos, _ = kv.info()
    fb = frame_bytes(cfg, C)
    win_b = w_in_bytes(cfg)
    achieved_win = win_b / (us_win * 1e-6) / 1e9 if us_win > 0 else None
    out = {
        "metric": METRIC,
        "value": round(ms, 4),
        "unit": "ms/frame",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (random-init bf16 weights 0.02*N(0,1), ring filled with N(0,1) bf16, random IDs)",
        "config": {"workload": "full 32-block temporal decode, B=1, ring full at 3000 frames, "
                               "positions 3000+ (keys wrap), d_model 4096, 32 heads x 128, d_ff 11264",
                   "global_batch": 1, "seq_len": C, "parallelism": "none (1 GPU)",
                   "launch": "hip graph" if mode == 1 else "direct"},
        "frames_per_s": round(1000.0 / ms, 2),
        "stream_tokens_per_s": round(17 * 1000.0 / ms, 1),
        "achieved_GBps": round(fb / (ms * 1e-3) / 1e9, 1),
        "frame_bytes": fb,
        "frame_roofline_frac": round(fb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "kernel": "k_gemv RMSNorm+W_in+SiLU-product (layer %d)" % args.trace_layer,
                     "achieved": round(achieved_win, 1) if achieved_win else None, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved_win / HBM_PEAK_GBPS, 4) if achieved_win else None,
                     "traffic": measured_traffic(), "bytes_per_launch": win_b, "mean_us": round(us_win, 3),
                     "launches_timed": n_tr,
                     "timing": "HIP events on the launch stream around %d back-to-back launches of the kernel "
                               "in each of %d directly launched frames (a pass after the timed one); mean per "
                               "launch, dispatch gaps included" % (TRACE_REPEAT, args.steps),
                     "mean_us_one_launch_per_event_pair": round(us_one, 3), "launches_one_per_pair": n_one},
        "frame_ms": {"median": round(float(np.median(per_frame)), 4),
                     "p90": round(float(np.percentile(per_frame, 90)), 4),
                     "max": round(per_frame[-1], 4), "frames": len(per_frame),
                     "timing": "one event pair per frame around each replay (a separate pass after the timed one)"},
        "final_position": pos,
    }
    out["one_block"] = bench_one_block(W, cfg, 20, 5)
    # the extra workloads run after the headline decode timing (a prefill burst at full
    # matrix-core load leaves the clocks lower for a while)
    dc = dict(synth.FULL_DEPTH)
    dep = None
    if not args.no_depformer:
        DW = make_depth_weights(dc, 5)
        dep = pp.Depformer(dc, DW, "bf16")
        out["generator"] = bench_generator(model, kv, dep, cfg, dc, max(10, args.steps // 2), 3)
    slots = [int(v) for v in args.reader_slots.split(",") if v.strip()]
    if slots:
        out["readers"] = bench_readers(model, kv, cfg, slots, max(10, args.steps // 5), 3)
    if batches:
        out["batched"] = bench_batched(model, cfg, batches, max(10, args.steps // 5), 3)
    if args.chunk_T > 0 and args.prefill_T >= args.chunk_T:
        out["prefill_chunk"] = bench_chunk(model, kv, cfg, args.chunk_T, 5, 1)
    if args.prefill_T > 0:
        kv.close()
        out["prefill"] = bench_prefill(model, cfg, args.prefill_T, args.prefill_steps, 1)
    if args.vendor_gemm and args.prefill_T > 0:
        out["vendor_gemm"] = bench_vendor_gemm(cfg, args.prefill_T)
    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if dep is not None:
        out["depformer"] = bench_depformer(dep, dc, max(10, args.steps // 2), 3)
        dep.close()
    if not args.no_cpu_baseline:
        cb = cpu_baselines(cfg, want_prefill="prefill" in out, want_depth="depformer" in out)
        out["cpu_baseline"] = dict(cb["decode"], host=cb["host"], tiny=cb["tiny"])
        if "one_block" in out:
            out["one_block"]["cpu_baseline"] = cb["one_block"]
        if "prefill" in cb:
            out["prefill"]["cpu_baseline"] = cb["prefill"]
        if "depth" in cb:
            out["depformer"]["cpu_baseline"] = cb["depth"]
            g = cb["draws"]
            out["generator"]["cpu_baseline"] = {
                "value": cb["decode"]["value"] + cb["depth"]["value"] + g["value"] + cb["text_head"]["value"],
                "unit": "ms/frame", "cores": cb["decode"]["cores"], "kind": "oracle",
                "sample": "sum of the oracle's decode-frame and depth-frame samples above, the text head "
                          "(%.1f ms) and one frame's 17 draws at full vocab sizes (%.1f ms)"
                          % (cb["text_head"]["value"], g["value"])}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
