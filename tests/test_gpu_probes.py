"""The measurement probes of include/moe_probe.h on the GPU: each mode runs to
completion with valid arguments, the clocks it reports are plausible, and the
null-decode read covers a real layer's stored matrices (2-bit, 3-bit and
NVFP4). They compute nothing of the decode step, so nothing is compared with
the oracle here."""
import ctypes as C

import numpy as np
import pytest
import torch

import bench
from bit_quantized_moe_block_amd import DeviceLayer
from moe_synth import gen, small_workload
from tests.gpu_common import say

pytestmark = pytest.mark.gpu


def test_compute_rate_modes_run_and_report_a_clock():
    L = bench.probe_lib()
    clk = torch.zeros(4, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for mode in range(len(bench.COMPUTE_MODES)):
        say(f"compute_rate mode {mode}")
        assert L.moe_probe_compute_rate(mode, 256, 64, clk.data_ptr(), sink.data_ptr(), None) == 0
        torch.cuda.synchronize()
        t0, r0, t1, r1 = clk.cpu().tolist()
        assert t1 > t0 and r1 > r0
        ghz = (t1 - t0) / ((r1 - r0) / 100e6) / 1e9
        assert 0.3 < ghz < 5.0, ghz


def test_ticket_read_modes_run():
    L = bench.probe_lib()
    buf = torch.ones((4 << 20) // 4, dtype=torch.int32, device="cuda")
    ctr = torch.full((256,), 7, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for mode in range(len(bench.TICKET_MODES)):
        say(f"ticket_read mode {mode}")
        assert L.moe_probe_ticket_read(buf.data_ptr(), 4 << 20, 64, mode, ctr.data_ptr(),
                                       sink.data_ptr(), None) == 0
        torch.cuda.synchronize()
        c = ctr.cpu().numpy().reshape(8, 32)[:, 0]
        if mode == 0:
            assert np.all(c == 0)  # cleared, never claimed from
        else:
            # every unit claimed once, plus one empty claim per block
            claims = int(c.sum()) if mode == 2 else int(c[0])
            assert claims == 64 + 64, claims


@pytest.mark.parametrize("fmt,mix", [("codebook", "alternate"), ("nvfp4", "nvfp4")])
def test_null_decode_reads_a_layer(fmt, mix):
    w = small_workload("probe_" + fmt, 8, 2, 1024, 1024, fmt=fmt, bits_mix=mix, config_id=530)
    case = gen.make_case(w, 4)
    layer = DeviceLayer.from_case(case, max_tokens=4)
    try:
        say(f"null decode {fmt}")
        nd = bench.probe_null_decode(0, [layer], [np.arange(w.num_experts)],
                                     torch.cuda.current_stream(), blocks=64, reps=1)
        assert nd is not None
        # every expert's three matrices, codes and scales
        assert nd["matrices"] == 3 * w.num_experts
        assert nd["bytes_per_layer"] == sum(
            (1024 // 16) * (1024 // 128) * (256 * int(layer.descs[i].bits)
                                            + (128 if fmt == "nvfp4" else 32))
            for i in range(3 * w.num_experts))
        assert nd["gbs"] > 0
    finally:
        layer.close()
