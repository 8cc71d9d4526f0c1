"""moe_decode_run_static (the entry point that allocates nothing) against
moe_decode_run through the C ABI (needs an MI355X).

Two calls in a row on one handle, the second with fewer tokens, each
byte-identical to moe_decode_run on the same inputs; two handles of
different shapes taking turns on the one static block; a graph holding a
static run, replayed; and the refusal of a run larger than the block.
"""
import numpy as np
import pytest
import torch

import bit_quantized_moe_block_amd as B
from moe_synth import WORKLOADS, gen, small_workload
from tests.gpu_common import check_stats, device_layer, routed_case, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _pair(layer, case, m, s):
    """(run output, run_static output) on the same inputs, both checked."""
    x, lg, out = to_dev(dict(case, x=case["x"][:m], logits=case["logits"][:m]))
    out_s = torch.full_like(out, float("nan"))
    with torch.cuda.stream(s):
        layer.run(x, lg, out, stream=s)
        s.synchronize()
        check_stats(layer)
        layer.run_static(x, lg, out_s, stream=s)
        s.synchronize()
        check_stats(layer)
    return out, out_s


def test_static_matches_run_then_smaller_input():
    w = WORKLOADS["full_layer"]
    case = routed_case(w, 24)
    say("[static] full layer, m = 16 then m = 5")
    s = torch.cuda.Stream()
    layer = device_layer(case, max_tokens=24)
    try:
        for m in (16, 5):
            ref, got = _pair(layer, dict(case, x=case["x"], logits=case["logits"]), m, s)
            assert torch.all(torch.isfinite(got))
            assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), m
    finally:
        layer.close()


def test_static_two_handles_take_turns():
    # Handles of different shapes share the one static block: each static
    # run must still equal the handle's own run.
    wa = small_workload("sa", 64, 8, 1024, 512, bits_mix="alternate", router="zipf",
                        config_id=601)
    wb = small_workload("sb", 16, 2, 512, 256, bits_mix="all3", config_id=602, shared_bits=6)
    ca, cb = gen.make_case(wa, 20), gen.make_case(wb, 9)
    say("[static] two handles in turn")
    s = torch.cuda.Stream()
    la = device_layer(ca, max_tokens=24)
    lb = device_layer(cb, max_tokens=24)
    try:
        for layer, case, m in ((la, ca, 20), (lb, cb, 9), (la, ca, 7), (lb, cb, 3)):
            ref, got = _pair(layer, case, m, s)
            assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), (case["workload"].name, m)
    finally:
        la.close()
        lb.close()


def test_static_run_in_a_graph():
    w = small_workload("sg", 32, 4, 1024, 256, bits_mix="alternate", config_id=603)
    case = gen.make_case(w, 12)
    say("[static] graph replay")
    s = torch.cuda.Stream()
    layer = device_layer(case, max_tokens=12)
    try:
        ref, _ = _pair(layer, case, 12, s)
        x, lg, out = to_dev(case)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            layer.run_static(x, lg, out, stream=s)
        for rep in range(3):
            out.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), rep
            ref2, got2 = _pair(layer, case, 12, s)   # eager work between replays
            assert torch.equal(got2.view(torch.int32), ref.view(torch.int32))
    finally:
        layer.close()


def test_static_refuses_runs_beyond_its_block():
    w = WORKLOADS["full_layer"]
    case = routed_case(w, 40)
    layer = device_layer(case, max_tokens=40)
    try:
        x, lg, out = to_dev(case)
        with pytest.raises(B.MoeDecodeError) as ei:
            layer.run_static(x, lg, out)
        assert ei.value.status == B.MOE_E_UNSUPPORTED and "static scratch" in str(ei.value)
        layer.run_static(x[:39], lg[:39], out[:39])    # 39 tokens fit
        torch.cuda.synchronize()
        check_stats(layer)
    finally:
        layer.close()
