"""Write the oracle's expected values for the full-size prefill check (CPU, a few minutes).

Workload: the full temporal stack (32 blocks, d_model 4096, 32 heads x 128, d_ff 11264,
context 3000) whose blocks share one set of bf16 weights (seed 44), T = 3000 frames of
random stream IDs (seed 45) from position 0. The oracle's full-sequence forward is run
once; the hidden rows listed in ROWS and the post-RoPE keys / raw values it leaves for
those positions in layers 0 and 31 are stored (float32) in prefill_T3000_32blocks.npz.

Only the oracle and the seeded input generators are used:
    python tests/golden/make_prefill_T3000.py
"""

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import temporal as O                        # noqa: E402
from personaplex_temporal_transformer_amd import synth  # noqa: E402

OUT = os.path.join(HERE, "prefill_T3000_32blocks.npz")
SEED_W, SEED_IDS, T = 44, 45, 3000
# Rows at the edges of the prefill's row tiles (192 and 224 rows) and the ragged last
# tile (2880..2999 for 192-row tiles, 2912..2999 for 224-row tiles), plus a spread.
ROWS = [0, 1, 5, 191, 192, 223, 224, 447, 448, 1000, 1343, 1344, 1727, 1728, 2047, 2048,
        2495, 2496, 2687, 2688, 2879, 2880, 2911, 2912, 2960, 2998, 2999]


def main():
    cfg = dict(synth.FULL_TEMPORAL)
    t0 = time.time()
    W = synth.temporal_weights(cfg, SEED_W, "bf16", with_text_head=False, shared_layer=True)
    ids = synth.stream_ids(cfg, T, SEED_IDS)
    cache = O.Cache(cfg["n_layers"])
    h = O.forward_full(ids, W, cfg, cache=cache)
    rows = np.array(ROWS)
    out = {"rows": rows, "h": h[rows].astype(np.float32)}
    H, dh = cfg["n_heads"], cfg["d_head"]
    for l in (0, cfg["n_layers"] - 1):
        pos, K, V = cache.layers[l][0]
        assert np.array_equal(pos, np.arange(T))
        out["k%d" % l] = O.f64(K)[rows].reshape(len(rows), H * dh).astype(np.float32)
        out["v%d" % l] = O.f64(V)[rows].reshape(len(rows), H * dh).astype(np.float32)
    meta = dict(workload="full temporal stack, shared block weights", seed_weights=SEED_W,
                seed_ids=SEED_IDS, T=T, p0=0, layers_stored=[0, cfg["n_layers"] - 1],
                oracle_seconds=round(time.time() - t0, 1))
    out["meta"] = np.array(json.dumps(meta))
    np.savez_compressed(OUT, **out)
    print("wrote %s (%.0f s)" % (OUT, time.time() - t0))


if __name__ == "__main__":
    main()
