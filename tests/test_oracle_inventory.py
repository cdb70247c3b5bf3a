"""Pins of the oracle's shape/size arithmetic against the counts the pages print."""

import re

from oracle import inventory, ring
from tests.conftest import read_golden


def _families(tensors):
    """Group (name, shape) by family pattern: digits in names become '*'."""
    fam = {}
    for name, shape in tensors:
        if name.endswith("alpha"):
            key = ("depth" if name.startswith("depformer") else "temporal") + " norm alphas"
        else:
            key = re.sub(r"\.\d+\.", ".*.", name)
        fam.setdefault(key, []).append(shape)
    return fam


def test_param_inventory_matches_family_table():
    rows = [r.split("|") for r in read_golden("param_inventory.txt")]
    rows = {r[0].strip(): (r[1].strip(), r[2].strip(), int(r[3])) for r in rows}
    tensors = inventory.temporal_tensors() + inventory.depth_tensors()
    fam = _families(tensors)
    for key, (count, shape, params) in rows.items():
        if key.startswith("TOTAL") or key.startswith("DIFFERENCE"):
            continue
        k = key.split(" (")[0]
        assert k in fam, key
        shapes = fam[k]
        assert len(shapes) == int(count), key
        assert all(",".join(map(str, s)) == shape for s in shapes), key
        assert sum(inventory.numel(s) for s in shapes) == params, key
    assert len(tensors) == int(rows["TOTAL"][0])
    assert inventory.total_params(tensors) == rows["TOTAL"][2]


def test_param_inventory_eight_positions():
    rows = {r.split("|")[0].strip(): int(r.split("|")[3]) for r in read_golden("param_inventory.txt")}
    t16 = inventory.total_params(inventory.temporal_tensors() + inventory.depth_tensors(n_steps=16))
    t8 = inventory.total_params(inventory.temporal_tensors() + inventory.depth_tensors(n_steps=8))
    assert t8 == rows["TOTAL_8_POSITIONS"]
    assert t16 - t8 == rows["DIFFERENCE_8_POSITIONS"]


def _kv():
    out = {}
    for ln in read_golden("cache_and_width.txt"):
        k, v = ln.split("=")
        out[k.strip()] = int(v)
    return out


def test_cache_bytes():
    g = _kv()
    assert inventory.temporal_kv_bytes(n_layers=1) == g["temporal_kv_bytes_per_layer_bf16_B1"]
    assert inventory.temporal_kv_bytes() == g["temporal_kv_bytes_all_layers_bf16_B1"]
    assert inventory.depth_kv_bytes() == g["depth_kv_bytes_all_layers_bf16_B1"]
    assert inventory.kv_bytes_per_frame(n_layers=1) == g["kv_bytes_per_position_per_layer"]
    assert inventory.kv_bytes_per_frame() == g["kv_bytes_per_position_all_layers"]
    assert 3750 * inventory.kv_bytes_per_frame() // 1024 == g["kv_kilobytes_for_3750_positions"]


def test_gated_widths_and_per_layer_params():
    g = _kv()
    assert inventory.gated_hidden(16896) == g["temporal_gated_hidden_from_16896"]
    assert inventory.gated_hidden(4224) == g["depth_gated_hidden_from_4224"]
    layer0 = [s for n, s in inventory.temporal_tensors(n_layers=1) if n.startswith("transformer.")]
    by = {n.split(".")[-2] + "." + n.split(".")[-1]: s for n, s in inventory.temporal_tensors(n_layers=1)}
    attn = inventory.numel(by["self_attn.in_proj_weight"]) + inventory.numel(by["out_proj.weight"])
    mlp = inventory.numel(by["linear_in.weight"]) + inventory.numel(by["linear_out.weight"])
    assert attn == g["temporal_attention_params_per_layer"]
    assert mlp == g["temporal_gated_mlp_params_per_layer"]
    no_norm = sum(inventory.numel(s) for s in layer0 if len(s) == 2)
    assert no_norm == g["temporal_params_per_layer"]


def test_ring_examples():
    for ln in read_golden("ring_examples.txt"):
        cap, end, labels, query, n_vis = [c.strip() for c in ln.split("|")]
        cap, end, query, n_vis = int(cap), int(end), int(query), int(n_vis)
        got = ring.compat_positions(cap, end)
        if labels != "-":
            assert got == [int(x) for x in labels.split(",")]
        assert len(ring.visible(got, query, cap)) == n_vis
        # The stated mask (the library's reading) keeps every slot of a full ring usable.
        stated = ring.stated_positions(cap, end)
        assert len(ring.visible(stated, end - 1, cap)) == cap


def test_ring_mask_edges():
    """The declared mask 0 <= query - key < context on labels around both edges: with
    context 4 and query 10 the key 6 (four back) is out, 7..10 are in, 11 (future) is out;
    a full stated ring of 4 slots after positions 0..9 holds 6..9, all visible to 9 and
    three of them (7..9) to 10."""
    assert ring.visible([5, 6, 7, 8, 9, 10, 11], 10, 4) == [7, 8, 9, 10]
    assert ring.visible([None, 3, 4], 4, 1) == [4]
    stated = ring.stated_positions(4, 10)
    assert sorted(stated) == [6, 7, 8, 9]
    assert len(ring.visible(stated, 9, 4)) == 4 and sorted(ring.visible(stated, 10, 4)) == [7, 8, 9]


def test_stated_positions_brute_force():
    # Brute force: write positions 0..end-1 into slot p mod cap, remember the last writer.
    for cap in (1, 3, 4, 7):
        for end in range(0, 20):
            slots = [None] * cap
            for p in range(end):
                slots[ring.slot_of(p, cap)] = p
            assert ring.stated_positions(cap, end) == slots
