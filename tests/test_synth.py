"""The seeded input generator: determinism and recipe (CPU only)."""
import numpy as np
import torch

from moe_synth import WORKLOADS, gen, small_workload


def test_same_seed_same_bytes():
    w = small_workload("s", 4, 2, 256, 128)
    a, b = gen.make_case(w, 3), gen.make_case(w, 3)
    assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["logits"], b["logits"])
    for key in a["tensors"]:
        for f in ("codes", "scales", "lut"):
            assert np.array_equal(a["tensors"][key][f], b["tensors"][key][f])
    c = gen.make_case(w, 3, layer=1)
    assert not np.array_equal(a["tensors"][(0, 0)]["codes"], c["tensors"][(0, 0)]["codes"])


def test_subset_generation_matches_full():
    w = small_workload("s", 6, 2, 256, 128)
    full = gen.make_layer(w, 0)
    sub = gen.make_layer(w, 0, experts=[4, 1])
    assert set(sub["tensors"]) == {(e, p) for e in (1, 4) for p in range(3)}
    for key, t in sub["tensors"].items():
        assert np.array_equal(t["codes"], full["tensors"][key]["codes"])


def test_recipe_ranges():
    w = WORKLOADS["rank_share"]
    d = gen.make_layer(w, 0, experts=[0, 1])
    assert list(d["bits"][:4]) == [2, 3, 2, 3]
    for (e, p), t in d["tensors"].items():
        N, C = gen.tensor_shape(w, p)
        assert t["codes"].nbytes == N * C * t["bits"] // 8
        s = t["scales"].astype(np.float64)
        assert s.min() >= 0.0099 and s.max() <= 0.0501 and len(s) == N * C // 128
        assert len(np.unique(t["lut"])) == 1 << t["bits"]
    assert set(np.unique(d["signs_hidden"])) == {-1, 1}
    assert set(np.unique(d["signs_inter"])) == {-1, 1}


def test_mixed_bits_is_five_eighths_three_bit():
    b = gen.expert_bits(WORKLOADS["full_layer"], 0)
    assert (b == 3).sum() == 160 and (b == 2).sum() == 96
    avg = (2.0 * 96 + 3.0 * 160) / 256 + 16.0 / 128   # codes + one fp16 scale per 128
    assert avg == 2.75


def test_pack_mix_layers():
    # The pack: 43 routed layers with 3, 21 and 41 all 2-bit, then 3 MTP draft
    # layers, all 2-bit; every other layer has the 5/8 three-bit mix.
    w = WORKLOADS["pack46"]
    assert w.layers == 46 and w.max_tokens == 16
    all2 = [l for l in range(w.layers) if (gen.expert_bits(w, l) == 2).all()]
    assert all2 == [3, 21, 41, 43, 44, 45]
    for l in (0, 20, 42):
        b = gen.expert_bits(w, l)
        assert (b == 3).sum() == 160 and (b == 2).sum() == 96
    # the mixed layers are drawn per layer, not repeated
    assert not np.array_equal(gen.expert_bits(w, 0), gen.expert_bits(w, 1))


def test_bf16_rounding_matches_torch():
    a = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gen.bf16_bits_from_f32(a), ref)


def test_nvfp4_recipe():
    w = WORKLOADS["nvfp4"]
    d = gen.make_layer(w, 0, experts=[3])
    t = d["tensors"][(3, 0)]
    assert t["bits"] == 4 and t["codes"].nbytes == 2048 * 4096 // 2
    ex = (t["scales"] >> 3) & 0xF
    assert ex.min() >= 6 and ex.max() <= 8 and (t["scales"] >> 7).max() == 0
    assert 0.0032 <= float(t["tensor_scale"]) <= 0.0048


def test_zipf_bias_concentrates_routing():
    w = WORKLOADS["full_layer"]
    lg = gen.make_logits(w, 0, 24)
    top = np.argsort(-lg, axis=1)[:, :8]
    assert len(np.unique(top)) < 24 * 8 // 2
