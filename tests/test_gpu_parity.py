"""GPU path vs the CPU oracle through the C ABI (needs an MI355X).

Sizes the oracle finishes in seconds cover several tiles and ragged tails;
the full-size workloads are checked on sampled tokens (every expert FFN of
those tokens, every output element) plus exact routing for all tokens.
"""
import ctypes as C
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from bit_quantized_moe_block_amd import DeviceLayer
from moe_synth import WORKLOADS, gen, small_workload
from tests.gpu_common import (REL_TOL, check_routing, check_stats, rel_err, run_gpu, say,
                              to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def parity(case, tokens=None, max_tokens=None):
    w = case["workload"]
    m = case["x"].shape[0]
    say(f"[parity] {w.name} E={w.num_experts} k={w.top_k} H={w.hidden} I={w.inter} m={m}")
    layer = DeviceLayer.from_case(case, max_tokens=max_tokens or m)
    try:
        out = run_gpu(layer, case)
        check_routing(layer, case, m)
        check_stats(layer)
        ref = oracle.Layer.from_case(case).run(case["x"], case["logits"], tokens=tokens)
        err = rel_err(out, ref["out"], tokens)
        say(f"    rel={err:.3e}")
        assert err <= REL_TOL
        return layer, out
    finally:
        layer.close()


def test_tiny():
    parity(gen.make_case(WORKLOADS["tiny"], 1))


GRID = []
_rng = np.random.default_rng(12345)
for i in range(24):
    E = int(_rng.choice([8, 16, 32]))
    k = int(_rng.choice([1, 2, 3, 4]))
    H = int(_rng.choice([256, 512, 1024]))
    I = int(_rng.choice([128, 256, 384]))
    m = int(_rng.integers(1, 25))
    mix = str(_rng.choice(["all2", "alternate", "all3"]))
    GRID.append((small_workload(f"grid{i}", E, k, H, I, bits_mix=mix, config_id=1000 + i), m))


@pytest.mark.parametrize("w,m", GRID, ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_random_grid(w, m):
    parity(gen.make_case(w, m))


@pytest.mark.parametrize("m", [1, 4])
def test_rank_share(m):
    parity(gen.make_case(WORKLOADS["rank_share"], m))


@pytest.fixture(scope="module")
def full_layer():
    w = WORKLOADS["full_layer"]
    d = gen.make_layer(w, 0)
    d["workload"] = w
    layer = DeviceLayer.from_case(d, max_tokens=w.max_tokens)
    yield d, layer
    layer.close()


@pytest.mark.parametrize("m", [16, 24])
def test_full_layer_one_row_block_items(full_layer, m):
    # From m = 8 gate/up items span two row blocks, but only for the row
    # groups that fit in the first round of tickets (one item per resident
    # block); the later groups take one-row-block items. 34 (m = 16) and 41
    # (m = 24) row groups overflow the 32 that fit: the run's item count must
    # be that of the mixed layout, and tokens routed into the one-row-block
    # groups must match the oracle.
    d, layer = full_layer
    w = d["workload"]
    case = dict(d, m=m, x=gen.make_x(w, 0, m), logits=gen.make_logits(w, 0, m))
    say(f"[parity] full_layer one-row-block items m={m}")
    out = run_gpu(layer, case)
    info, st = layer.info(), layer.stats()
    assert st.error_word == 0 and st.items_done == st.items
    rid, _ = oracle.route(case["logits"], w.top_k)
    b = oracle.bucket(rid, w.num_experts)
    groups = [(e, g) for e in range(w.num_experts) for g in range((int(b["counts"][e]) + 15) // 16)]
    n_rb1, n_rb2 = w.inter // 128, w.hidden // 256
    ks1, ks2 = info.k_split_gate_up, info.k_split_down
    per_wide = (n_rb1 // 2) * ks1
    n_wide = min(len(groups), info.grid_blocks // per_wide)
    assert n_wide < len(groups), "the layer must overflow the first round"
    assert st.items == (n_wide * per_wide + (len(groups) - n_wide) * n_rb1 * ks1
                        + len(groups) * n_rb2 * ks2)
    late = set()
    for e, g in groups[n_wide:]:
        lo = int(b["offsets"][e]) + 16 * g
        late.update(int(t) for t in b["rows_t"][lo:min(lo + 16, int(b["offsets"][e + 1]))])
    tokens = sorted(late)[:: max(1, len(late) // 3)][:3]
    ref = oracle.Layer.from_case(case).run(case["x"], case["logits"], tokens=tokens)
    err = rel_err(out, ref["out"], tokens)
    say(f"    groups={len(groups)} wide={n_wide} items={st.items} tokens={tokens} rel={err:.3e}")
    assert err <= REL_TOL


@pytest.mark.parametrize("layer", [3, 20, 43])
def test_pack_layers_sampled(layer):
    # The pack mix at full size and the 16-row batch: an all-2-bit routed layer,
    # a mixed layer and an MTP draft layer, sampled tokens against the oracle.
    w = WORKLOADS["pack46"]
    m = 16
    case = gen.make_case(w, m, layer=layer)
    tokens = [0, 7, 15]
    say(f"[parity] pack46 layer={layer} m={m}")
    dl = DeviceLayer.from_case(case, max_tokens=m)
    try:
        out = run_gpu(dl, case)
        check_routing(dl, case, m)
        st = dl.stats()
        assert st.error_word == 0 and st.items_done == st.items
        ref = oracle.Layer.from_case(case).run(case["x"], case["logits"], tokens=tokens)
        err = rel_err(out, ref["out"], tokens)
        say(f"    rel={err:.3e} hit={st.hit_experts}")
        assert err <= REL_TOL
    finally:
        dl.close()


SHARED = [
    (small_workload("sh6a", 8, 2, 256, 128, bits_mix="alternate", config_id=311, shared_bits=6), 1),
    (small_workload("sh6b", 16, 4, 512, 256, bits_mix="alternate", config_id=312, shared_bits=6), 5),
    (small_workload("sh6c", 16, 3, 1024, 384, bits_mix="all3", config_id=313, shared_bits=6), 16),
    (small_workload("sh6d", 32, 4, 512, 256, bits_mix="alternate", config_id=314, shared_bits=6), 24),
    (small_workload("sh2", 16, 2, 512, 128, bits_mix="all2", config_id=315, shared_bits=2), 17),
    (small_workload("sh3", 8, 2, 768, 256, bits_mix="all3", config_id=316, shared_bits=3), 3),
]


@pytest.mark.parametrize("w,m", SHARED, ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_shared_expert_small(w, m):
    # The always-on shared expert (6-bit, and 2/3-bit) folded into the launch:
    # every output element against the oracle, ragged token counts (1..24,
    # one or two shared row groups).
    parity(gen.make_case(w, m))


@pytest.mark.parametrize("m", [1, 16, 24])
def test_shared_layer_sampled(m):
    w = WORKLOADS["shared_layer"]
    case = gen.make_case(w, m)
    tokens = sorted(set([0, m // 2, m - 1]))
    say(f"[parity] shared_layer m={m}")
    dl = DeviceLayer.from_case(case, max_tokens=24)
    try:
        out = run_gpu(dl, case)
        check_routing(dl, case, m)
        st = dl.stats()
        assert st.error_word == 0 and st.items_done == st.items
        ref = oracle.Layer.from_case(case).run(case["x"], case["logits"], tokens=tokens)
        err = rel_err(out, ref["out"], tokens)
        say(f"    rel={err:.3e} hit={st.hit_experts} items={st.items}")
        assert err <= REL_TOL
    finally:
        dl.close()


def test_shared_expert_bitwise_repeatable():
    w = small_workload("shrep", 16, 4, 1024, 256, bits_mix="alternate", config_id=317, shared_bits=6)
    case = gen.make_case(w, 19)
    say("[bitwise] shared expert, 6 runs")
    s = torch.cuda.Stream()
    layer = DeviceLayer.from_case(case, max_tokens=24)
    try:
        x, lg, out = to_dev(case)
        outs = []
        with torch.cuda.stream(s):
            for _ in range(6):
                out.fill_(float("nan"))
                layer.run(x, lg, out, stream=s)
                s.synchronize()
                outs.append(out.clone())
        for o in outs[1:]:
            assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))
    finally:
        layer.close()


def test_bitwise_repeatable_and_graph_replay():
    w = small_workload("rep", 16, 4, 1024, 256, bits_mix="alternate", config_id=301)
    case = gen.make_case(w, 24)
    say("[bitwise] 10 direct runs + graph replays")
    s = torch.cuda.Stream()
    layer = DeviceLayer.from_case(case, max_tokens=24)
    try:
        x, lg, out = to_dev(case)
        # a second input between the repeats: stale partial sums of another
        # run would show
        cb = gen.make_case(w, 24, layer=1)
        xb, lgb, outb = to_dev(dict(case, x=cb["x"], logits=cb["logits"]))
        outs = []
        with torch.cuda.stream(s):
            for _ in range(10):
                out.fill_(float("nan"))
                layer.run(x, lg, out, stream=s)
                s.synchronize()
                check_stats(layer)
                outs.append(out.clone())
                layer.run(xb, lgb, outb, stream=s)
                s.synchronize()
                check_stats(layer)
        for o in outs[1:]:
            assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))
        assert not torch.equal(outb, outs[0])
        g = torch.cuda.CUDAGraph()
        out_g = torch.full_like(out, float("nan"))
        with torch.cuda.graph(g, stream=s):
            layer.run(x, lg, out_g, stream=s)
        for rep in range(5):
            out_g.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out_g.view(torch.int32), outs[0].view(torch.int32)), rep
            with torch.cuda.stream(s):       # eager work between replays
                layer.run(x, lg, out, stream=s)
            s.synchronize()
            assert torch.equal(out.view(torch.int32), outs[0].view(torch.int32))
        # a fresh handle on the same inputs gives the same bytes
        layer2 = DeviceLayer.from_case(case, max_tokens=24)
        out2 = torch.full_like(out, float("nan"))
        layer2.run(x, lg, out2)
        torch.cuda.synchronize()
        assert torch.equal(out2.view(torch.int32), outs[0].view(torch.int32))
        layer2.close()
    finally:
        layer.close()


def test_zero_input_exact_zero():
    w = small_workload("zero", 8, 2, 512, 256, bits_mix="alternate", config_id=302)
    case = gen.make_case(w, 5)
    case["x"] = np.zeros_like(case["x"])
    layer = DeviceLayer.from_case(case)
    try:
        out = run_gpu(layer, case)
        assert np.all(out == 0.0)
    finally:
        layer.close()


def test_all_tokens_same_experts_hot_path():
    # Every token routes to the same k experts: R_e = m = 24 (two MFMA token
    # blocks, rows beyond 16), the largest bucket the path admits at m = 24.
    w = small_workload("hot", 32, 4, 1024, 384, bits_mix="alternate", config_id=303)
    case = gen.make_case(w, 24)
    lg = case["logits"].copy()
    lg[:, [3, 17, 8, 30]] += 50.0
    case["logits"] = lg
    layer, _ = parity(case)
    b = oracle.bucket(oracle.route(lg, 4)[0], 32)
    assert sorted(np.nonzero(b["counts"])[0].tolist()) == [3, 8, 17, 30]


def test_tied_logits():
    w = small_workload("ties", 16, 4, 256, 128, bits_mix="all3", config_id=304)
    case = gen.make_case(w, 6)
    lg = case["logits"].copy()
    lg[:, 5] = lg[:, 2]
    lg[0, :] = 0.5
    lg[1, :] = -0.0
    lg[1, 9] = 0.0
    case["logits"] = lg
    parity(case)


def test_m_zero_and_range_errors():
    import bit_quantized_moe_block_amd as B
    w = small_workload("mz", 8, 2, 256, 128, config_id=305)
    case = gen.make_case(w, 2)
    layer = DeviceLayer.from_case(case, max_tokens=2)
    try:
        x, lg, out = to_dev(case)
        out.fill_(7.0)
        layer.run(x, lg, out, m=0)
        torch.cuda.synchronize()
        assert torch.all(out == 7.0)
        # m beyond max_tokens: refused by the library (through the raw call)
        # and by the binding's shape check before it
        with pytest.raises(B.MoeDecodeError) as ei:
            B.moe_decode_run(layer.handle, x.data_ptr(), lg.data_ptr(), out.data_ptr(), 3,
                             torch.cuda.current_stream().cuda_stream)
        assert ei.value.status == B.MOE_E_INVALID and "max_tokens" in str(ei.value)
        with pytest.raises(ValueError):
            layer.run(x, lg, out, m=3)
        layer.run(x, lg, out)                # first real run binds the current stream
        torch.cuda.synchronize()
        other = torch.cuda.Stream()
        with pytest.raises(B.MoeDecodeError) as ei:
            layer.run(x, lg, out, stream=other)
        assert ei.value.status == B.MOE_E_STREAM
    finally:
        layer.close()


def test_tokens_fewer_than_max_tokens():
    # A handle sized for 24 tokens run with m = 3, then m = 11, then m = 3 again.
    w = small_workload("var", 16, 3, 512, 256, bits_mix="alternate", config_id=306)
    d = gen.make_layer(w, 0)
    d["workload"] = w
    layer = DeviceLayer.from_case(d, max_tokens=24)
    try:
        for m in (3, 11, 3):
            case = dict(d, m=m, x=gen.make_x(w, 0, m), logits=gen.make_logits(w, 0, m))
            out = run_gpu(layer, case)
            check_routing(layer, case, m)
            ref = oracle.Layer.from_case(case).run(case["x"], case["logits"])
            assert rel_err(out, ref["out"]) <= REL_TOL
    finally:
        layer.close()


NVFP4_GRID = [
    (small_workload("fp4a", 8, 2, 256, 128, fmt="nvfp4", bits_mix="nvfp4", config_id=401), 1),
    (small_workload("fp4b", 16, 4, 1024, 256, fmt="nvfp4", bits_mix="nvfp4", config_id=402), 9),
    (small_workload("fp4c", 32, 3, 512, 384, fmt="nvfp4", bits_mix="nvfp4", config_id=403), 24),
]


@pytest.mark.parametrize("w,m", NVFP4_GRID, ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_nvfp4_small(w, m):
    parity(gen.make_case(w, m))


@pytest.mark.parametrize("m", [2, 8])
def test_nvfp4_full_sampled(m):
    w = WORKLOADS["nvfp4"]
    rid, _ = oracle.route(gen.make_logits(w, 0, m), w.top_k)
    d = gen.make_layer(w, 0)
    d["workload"] = w
    case = dict(d, m=m, x=gen.make_x(w, 0, m), logits=gen.make_logits(w, 0, m))
    parity(case, tokens=sorted(set([0, m - 1])), max_tokens=8)


# Large m (prefill / batched verify, up to 512 tokens): 33 and 40 tokens on
# the persistent kernel (16-row groups), from 48 tokens on the prefill
# kernels (row groups of up to 64 rows, odd and even column-chunk counts,
# NVFP4, a 3-bit shared expert); with a 6-bit tensor the persistent kernel at
# any m. Zipf routing sends hundreds of rows to the hot experts.
LARGE_M = [
    (small_workload("lm1", 16, 4, 256, 128, bits_mix="alternate", router="zipf", config_id=401), 33),
    (small_workload("lm2", 32, 8, 512, 256, bits_mix="all3", router="zipf", config_id=402), 100),
    (small_workload("lm3", 64, 8, 512, 256, bits_mix="alternate", config_id=403), 257),
    (small_workload("lm4", 16, 2, 256, 128, bits_mix="all2", router="zipf", config_id=404), 512),
    (small_workload("lm5", 32, 4, 256, 128, bits_mix="alternate", config_id=405, shared_bits=6), 300),
    (small_workload("lm6", 16, 4, 512, 256, fmt="nvfp4", bits_mix="nvfp4", config_id=406), 200),
    (small_workload("lm7", 16, 2, 512, 256, bits_mix="all3", router="zipf", config_id=407,
                    shared_bits=3), 150),
    # the largest pair count (512 tokens x top-16 = 8192 rows, 256 experts)
    # and top-16 on the persistent kernel
    (small_workload("lm8", 256, 16, 256, 128, bits_mix="alternate", router="zipf",
                    config_id=409), 512),
    (small_workload("lm9", 32, 16, 256, 128, bits_mix="alternate", config_id=410), 40),
    # both sides of the switch between the two paths (prefill from 48 tokens)
    (small_workload("lm10", 32, 8, 512, 256, bits_mix="alternate", router="zipf",
                    config_id=411), 47),
    (small_workload("lm11", 32, 8, 512, 256, bits_mix="alternate", router="zipf",
                    config_id=411), 48),
]


@pytest.mark.parametrize("w,m", LARGE_M, ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_large_m_small_shapes(w, m):
    parity(gen.make_case(w, m))


def test_prefill_layer_sampled_and_repeatable():
    # The full 256-expert layer at m = 512: exact routing and buckets for all
    # tokens, three tokens against the oracle, and a second run bit-identical.
    w = WORKLOADS["prefill"]
    m = 512
    case = gen.make_case(w, m)
    tokens = [0, 255, 511]
    say(f"[parity] prefill m={m}")
    dl = DeviceLayer.from_case(case, max_tokens=m)
    try:
        out = run_gpu(dl, case)
        check_routing(dl, case, m)
        st = dl.stats()
        assert st.error_word == 0 and st.items_done == st.items
        out2 = run_gpu(dl, case)
        assert np.array_equal(out, out2)
        ref = oracle.Layer.from_case(case).run(case["x"], case["logits"], tokens=tokens)
        err = rel_err(out, ref["out"], tokens)
        say(f"    rel={err:.3e} hit={st.hit_experts} items={st.items}")
        assert err <= REL_TOL
    finally:
        dl.close()


def test_one_handle_both_paths_and_graph_replay():
    # One handle (max_tokens 300) alternating the prefill kernels (m = 256)
    # and the persistent kernel (m = 40): eager runs are bit-identical to
    # each other, and a graph holding both runs replays to the same bytes
    # with eager work in between; m = 256 matches the oracle.
    w = small_workload("both", 16, 4, 512, 256, bits_mix="alternate", router="zipf",
                       config_id=408)
    cases = {m: gen.make_case(w, m) for m in (256, 40)}
    say("[graph] prefill and persistent paths on one handle")
    s = torch.cuda.Stream()
    layer = DeviceLayer.from_case(cases[256], max_tokens=300)
    try:
        dev = {m: to_dev(c) for m, c in cases.items()}
        ref = {}
        with torch.cuda.stream(s):
            for rep in range(2):
                for m in (256, 40):
                    x, lg, out = dev[m]
                    out.fill_(float("nan"))
                    layer.run(x, lg, out, stream=s)
                    s.synchronize()
                    if rep == 0:
                        ref[m] = out.clone()
                    else:
                        assert torch.equal(out.view(torch.int32), ref[m].view(torch.int32)), m
        outs_g = {m: torch.full_like(dev[m][2], float("nan")) for m in dev}
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for m in (256, 40):
                layer.run(dev[m][0], dev[m][1], outs_g[m], stream=s)
        for rep in range(3):
            for o in outs_g.values():
                o.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            for m in dev:
                assert torch.equal(outs_g[m].view(torch.int32), ref[m].view(torch.int32)), (rep, m)
            with torch.cuda.stream(s):
                x, lg, out = dev[40]
                layer.run(x, lg, out, stream=s)
            s.synchronize()
            assert torch.equal(out.view(torch.int32), ref[40].view(torch.int32))
        r = oracle.Layer.from_case(cases[256]).run(cases[256]["x"], cases[256]["logits"])
        err = rel_err(ref[256].cpu().numpy(), r["out"])
        say(f"    rel={err:.3e}")
        assert err <= REL_TOL
    finally:
        layer.close()


def test_nvfp4_prefill_layer_sampled():
    # The full NVFP4 layer (256 experts, 4096 x 2048) at m = 256 on the
    # prefill kernels: exact routing, three tokens against the oracle, and a
    # second run bit-identical.
    w = WORKLOADS["nvfp4"]
    m = 256
    case = gen.make_case(w, m)
    tokens = [0, 128, 255]
    say(f"[parity] nvfp4 prefill m={m}")
    dl = DeviceLayer.from_case(case, max_tokens=m)
    try:
        out = run_gpu(dl, case)
        check_routing(dl, case, m)
        st = dl.stats()
        assert st.error_word == 0 and st.items_done == st.items
        assert np.array_equal(out, run_gpu(dl, case))
        ref = oracle.Layer.from_case(case).run(case["x"], case["logits"], tokens=tokens)
        err = rel_err(out, ref["out"], tokens)
        say(f"    rel={err:.3e} hit={st.hit_experts} items={st.items}")
        assert err <= REL_TOL
    finally:
        dl.close()


# Activations well away from N(0,1): x * 8 plus a few outliers of +-500 in
# every token. The staged x~ and h~ stay inside the fp16 range that the
# header states (|x| < 5790, |SiLU(g) u| < 5790); both expert paths.
RANGE = [
    (small_workload("rng1", 32, 4, 1024, 256, bits_mix="alternate", config_id=501), 16),
    (small_workload("rng2", 32, 4, 1024, 256, bits_mix="all3", router="zipf", config_id=502), 64),
    (small_workload("rng3", 16, 2, 512, 256, fmt="nvfp4", bits_mix="nvfp4", config_id=503), 12),
    (small_workload("rng4", 16, 2, 512, 256, fmt="nvfp4", bits_mix="nvfp4", config_id=504), 80),
]


@pytest.mark.parametrize("w,m", RANGE, ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_large_magnitude_activations(w, m):
    case = gen.make_case(w, m)
    rng = np.random.default_rng(w.config_id)
    x = rng.standard_normal((m, w.hidden)).astype(np.float32) * 8.0
    for t in range(m):
        cols = rng.choice(w.hidden, 3, replace=False)
        x[t, cols] = rng.choice([-500.0, 500.0], 3)
    case["x"] = gen.bf16_bits_from_f32(x)
    layer, out = parity(case)
    assert np.all(np.isfinite(out))
    assert np.max(np.abs(out)) > 10.0   # the scale did reach the output


# NVFP4 block scales drawn over every finite e4m3 code (either sign,
# subnormals, 448), on both expert paths.
NV_ALL = [
    (small_workload("nva1", 16, 4, 1024, 256, fmt="nvfp4", bits_mix="nvfp4", config_id=511,
                    nv_scales="all_finite", ts_scale=0.0002), 9),
    (small_workload("nva2", 32, 8, 512, 384, fmt="nvfp4", bits_mix="nvfp4", router="zipf",
                    config_id=512, nv_scales="all_finite", ts_scale=0.0002), 24),
    (small_workload("nva3", 16, 4, 512, 256, fmt="nvfp4", bits_mix="nvfp4", config_id=513,
                    nv_scales="all_finite", ts_scale=0.0002), 100),
]


@pytest.mark.parametrize("w,m", NV_ALL, ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_nvfp4_every_finite_scale_code(w, m):
    case = gen.make_case(w, m)
    codes = np.unique(np.concatenate([t["scales"] for t in case["tensors"].values()]))
    assert len(codes) == 254   # every finite code occurs
    parity(case)


@pytest.mark.parametrize("m", [8, 1])
def test_gave_up_wait_surfaces_as_device_error(monkeypatch, m):
    # A bound of zero polls makes the down items' wait for h give up at
    # once (every kernel still ends normally): the run's output must be NaN,
    # the stats query and destroy must return MOE_E_DEVICE, and a handle
    # with the normal bound must run the same inputs correctly afterwards.
    # m = 8 runs the persistent expert kernel, m = 1 the small-m kernel (its
    # 8 row groups x (512/32 + 1024/64) items fit one round of its grid).
    import bit_quantized_moe_block_amd as B
    w = small_workload("spin", 64, 8, 1024, 512, bits_mix="alternate", config_id=520)
    case = gen.make_case(w, m)
    monkeypatch.setenv("MOE_DECODE_SPIN_LIMIT", "0")
    layer = DeviceLayer.from_case(case, max_tokens=8)
    monkeypatch.delenv("MOE_DECODE_SPIN_LIMIT")
    try:
        out = run_gpu(layer, case)
        with pytest.raises(B.MoeDecodeError) as ei:
            layer.stats()
        assert ei.value.status == B.MOE_E_DEVICE
        st = B.moe_decode_stats()
        B.lib().moe_decode_query(layer.handle, B.MOE_Q_STATS, C.byref(st), C.sizeof(st))
        assert st.error_word == 1
        if m == 1:  # the small-m kernel's item count: 32-row gate/up, 64-row down items
            assert st.items == st.hit_experts * (w.inter // 32 + w.hidden // 64)
        assert np.all(np.isnan(out))
    finally:
        with pytest.raises(B.MoeDecodeError) as ei:
            layer.close()
        assert ei.value.status == B.MOE_E_DEVICE
    parity(case)
