#!/usr/bin/env python3
"""Benchmark of the routed-experts decode step on one MI355X.

Default workload: the 43-layer decode-step stack (each layer: 256 experts,
top-8, hidden 4096, expert intermediate 2048, 2/3-bit mixed codes with 62.5 %
3-bit experts, Zipf-skewed routing), m = 16 tokens (4 streams x (1 + 3
speculative tokens)), all 43 layers captured in one HIP graph on one stream.
One step = one graph replay = one pass of the whole path over all layers.
The stack streams ~11.8 GB of weights per step, far beyond the 256 MB
Infinity Cache, so every layer reads its weights cold from HBM.

Prints one JSON line. `value` is the achieved HBM throughput over the
algorithmic weight bytes of the step (stored codes + scales + codebooks of
every hit expert, each counted once per layer) divided by the step time.
`roofline` reports the dominant kernel (the expert kernel) timed alone with
HIP events recorded on its stream; its `traffic` (HBM bytes per launch) comes
from the rocprofv3 FETCH_SIZE / WRITE_SIZE summary committed under profiles/,
scaled by the counters' reading of a plain copy of known size
(`--copy-calibration`), and is null when the kernel source has changed since
those counters were taken. `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload (one whole layer: median of 5 runs on every core of
the process, plus a one-thread run on two tokens). The default run also sweeps
m = 1, 2, 4, 8, 16, 24 on the same 43 resident layers (`m_sweep`), and reports the
probes of include/moe_probe.h (`probes`): a plain streaming read of 4 GiB, the
graph-replay floor of three empty kernels per layer, the issue rates of the decode
step's decode and MFMA halves on register operands (cycles per MFMA step per SIMD,
four waves per SIMD), and a 1 GiB streaming read whose units are claimed from one
or eight shared counters against a static order, with the run's provenance.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed-MoE decode µs/launch + achieved HBM GB/s of weight bytes, m=1–24"
HBM_PEAK_GBS = 8000.0
# the device code of the decode kernels: the kernel file, then the decode step it includes
KERNEL_SRC = [os.path.join(ROOT, "bit_quantized_moe_block_amd", "csrc", f)
              for f in ("kernels.hip", "decode_step.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "expert_kernel_stack43_m16_traffic.md")


def kernel_source_sha():
    """sha256 of the decode kernels' code: the files of KERNEL_SRC in order,
    comments removed and whitespace runs collapsed (an edit to a comment
    leaves the counters of the same code valid)."""
    h = hashlib.sha256()
    for path in KERNEL_SRC:
        with open(path, encoding="utf-8") as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per expert-kernel launch from the committed counter summary,
    or None when it is missing or was taken on other kernel source."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not sha or not val or sha.group(1) != kernel_source_sha():
        return None
    return int(val.group(1))


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="stack43",
                    choices=["stack43", "pack46", "stack43_shared", "shared_layer", "full_layer",
                             "prefill", "rank_share", "nvfp4", "tiny"])
    ap.add_argument("--m", type=int, default=None, help="tokens per step (default: workload's)")
    ap.add_argument("--layers", type=int, default=None,
                    help="layers of the stack (default: the workload's, 43 for stack43)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the m = 1..24 sweep on the same layers")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the plain-read and launch-floor probes")
    ap.add_argument("--profile-passes", type=int, default=3)
    ap.add_argument("--lds-probe", action="store_true",
                    help="only run the LDS read probe over the three staging layouts and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device to device once (the known-size dispatch "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


class HipEvent:
    """A raw hipEvent_t (timing enabled) for events recorded inside the library."""
    _hip = None

    def __init__(self):
        import ctypes
        if HipEvent._hip is None:
            HipEvent._hip = ctypes.CDLL("libamdhip64.so")
        self._c = ctypes
        ev = ctypes.c_void_p()
        if HipEvent._hip.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.ptr = ev.value

    def elapsed_ms(self, end):
        ms = self._c.c_float()
        h = HipEvent._hip
        if h.hipEventSynchronize(self._c.c_void_p(end.ptr)) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        if h.hipEventElapsedTime(self._c.byref(ms), self._c.c_void_p(self.ptr),
                                 self._c.c_void_p(end.ptr)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def provenance(props):
    """Where and on what the numbers were taken."""
    import subprocess
    import torch
    try:
        git = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short=12", "HEAD"],
                             capture_output=True, text=True, timeout=10).stdout.strip() or None
    except Exception:
        git = None
    h = hashlib.sha256()
    for d in (os.path.join(ROOT, "bit_quantized_moe_block_amd", "csrc"), os.path.join(ROOT, "include")):
        for f in sorted(os.listdir(d)):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return {"git": git, "source_sha256": h.hexdigest()[:16], "device": props.name or getattr(props, "gcnArchName", ""),
            "arch": getattr(props, "gcnArchName", None), "cus": props.multi_processor_count,
            "torch": torch.__version__, "hip": torch.version.hip,
            "seeds": "numpy SeedSequence(entropy=1000+config_id, spawn_key=(layer, tag, ...)), SFC64"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


PROBE_LIB = os.path.join(ROOT, "bit_quantized_moe_block_amd", "libmoeprobe.so")
_probe = None


def _tile_stream_type():
    import ctypes as C

    class T(C.Structure):
        _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("tile_rows", C.c_int32),
                    ("groups", C.c_int32), ("bits", C.c_int32), ("units_before", C.c_int32)]
    return T


ProbeTileStream = _tile_stream_type()  # moe_probe_tile_stream of include/moe_probe.h


def probe_lib():
    """The measurement probes of include/moe_probe.h (a library of their own)."""
    global _probe
    if _probe is None:
        import ctypes as C
        L = C.CDLL(PROBE_LIB)
        L.moe_probe_stream_read.restype = C.c_int
        L.moe_probe_stream_read.argtypes = [C.c_void_p, C.c_size_t, C.c_int32, C.c_void_p,
                                            C.c_void_p]
        L.moe_probe_empty_kernels.restype = C.c_int
        L.moe_probe_empty_kernels.argtypes = [C.c_int32, C.c_void_p]
        L.moe_probe_lds_read128.restype = C.c_int
        L.moe_probe_lds_read128.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                            C.c_void_p]
        L.moe_probe_compute_rate.restype = C.c_int
        L.moe_probe_compute_rate.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                             C.c_void_p, C.c_void_p]
        L.moe_probe_tile_read.restype = C.c_int
        L.moe_probe_tile_read.argtypes = [C.POINTER(ProbeTileStream), C.c_int32, C.c_void_p,
                                          C.c_int32, C.c_void_p, C.c_void_p]
        L.moe_probe_ticket_read.restype = C.c_int
        L.moe_probe_ticket_read.argtypes = [C.c_void_p, C.c_size_t, C.c_int32, C.c_int32,
                                            C.c_void_p, C.c_void_p, C.c_void_p]
        _probe = L
    return _probe


def probe_plain_read(dev, gib=4, reps=5):
    """Achievable streaming read: one plain read of `gib` GiB of device memory
    (16-byte loads, nothing decoded), best over a few grid sizes (GB/s)."""
    import torch
    L = probe_lib()
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best, best_grid = 1e30, 0
    for grid in (1024, 2048, 4096, 8192):
        for _ in range(reps):
            e0.record(s)
            rc = L.moe_probe_stream_read(buf.data_ptr(), nbytes, grid, sink.data_ptr(),
                                         s.cuda_stream)
            e1.record(s)
            if rc:
                raise RuntimeError(f"moe_probe_stream_read: HIP error {-rc}")
            e1.synchronize()
            t = e0.elapsed_time(e1)
            if t < best:
                best, best_grid = t, grid
    del buf
    return nbytes / (best * 1e-3) / 1e9, best_grid


LDS_LAYOUTS = ("rows padded by 16 bytes (decode kernel)", "256-byte rows, xor-permuted pieces (prefill)",
               "256-byte rows, unpadded (conflicted reference)")


def probe_lds_layouts(dev, blocks=1024, iters=256):
    """LDS read rate of the MFMA activation-operand pattern per staging layout:
    one launch per layout (in LDS_LAYOUTS order) after one warm-up launch each.
    Returns [(layout, us, clocks per 16-byte read per CU at 2.4 GHz)]."""
    import torch
    L = probe_lib()
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reads_per_cu = blocks * 4 * iters * 16 / torch.cuda.get_device_properties(dev).multi_processor_count
    out = []
    for layout in range(len(LDS_LAYOUTS)):
        for timed in (False, True):
            e0.record(s)
            rc = L.moe_probe_lds_read128(layout, blocks, iters, sink.data_ptr(), s.cuda_stream)
            e1.record(s)
            if rc:
                raise RuntimeError(f"moe_probe_lds_read128: HIP error {-rc}")
            e1.synchronize()
        us = e0.elapsed_time(e1) * 1e3
        out.append((layout, us, us * 1e-6 * 2.4e9 / reads_per_cu))
    return out


COMPUTE_MODES = ("decode only (+4 VALU xor fold per step)", "MFMA only (+ group-scale FMAs)",
                 "decode into MFMA (the decode kernels' inner step)",
                 "decode into 4 v_dot2_f32_f16 (one token, no MFMA)")


def probe_compute_rates(dev, iters=2048):
    """Issue rates of the decode step's halves on register operands (3-bit
    codebook tile, 4 MFMA steps per round): one launch per mode after a
    warm-up, 4 blocks of 4 waves per CU (4 waves per SIMD, as the decode
    kernels run). Returns the shader clock (GHz, from block 0's s_memtime
    against s_memrealtime) and per mode the nanoseconds and shader cycles per
    MFMA step per SIMD."""
    import torch
    L = probe_lib()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = 4 * cus
    simds = 4 * cus
    steps_per_simd = blocks * 4 * iters * 4 / simds
    clk = torch.zeros(4, dtype=torch.int64, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = []
    for mode in range(len(COMPUTE_MODES)):
        for timed in (False, True):
            e0.record(s)
            rc = L.moe_probe_compute_rate(mode, blocks, iters, clk.data_ptr(), sink.data_ptr(),
                                          s.cuda_stream)
            e1.record(s)
            if rc:
                raise RuntimeError(f"moe_probe_compute_rate: HIP error {-rc}")
            e1.synchronize()
        c = clk.cpu().tolist()
        ghz = (c[2] - c[0]) / ((c[3] - c[1]) / 100e6) / 1e9 if c[3] > c[1] else float("nan")
        ns = e0.elapsed_time(e1) * 1e6 / steps_per_simd
        out.append({"mode": mode, "desc": COMPUTE_MODES[mode], "ns_per_step": round(ns, 3),
                    "cycles_per_step": round(ns * ghz, 1), "clock_ghz": round(ghz, 3)})
    return out


TICKET_MODES = ("static order", "one shared counter", "eight counters")


def probe_tickets(dev, mib=1024, reps=3):
    """A streaming read of `mib` MiB in 64 KiB units, the units taken in a
    static order or claimed from one or eight shared counters: best GB/s over
    a few grid sizes per mode."""
    import torch
    L = probe_lib()
    nbytes = mib << 20
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    ctr = torch.zeros(256, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = []
    for mode in range(len(TICKET_MODES)):
        best, best_grid = 1e30, 0
        for grid in (1024, 2048, 4096):
            for _ in range(reps):
                e0.record(s)
                rc = L.moe_probe_ticket_read(buf.data_ptr(), nbytes, grid, mode, ctr.data_ptr(),
                                             sink.data_ptr(), s.cuda_stream)
                e1.record(s)
                if rc:
                    raise RuntimeError(f"moe_probe_ticket_read: HIP error {-rc}")
                e1.synchronize()
                t = e0.elapsed_time(e1)
                if t < best:
                    best, best_grid = t, grid
        out.append({"mode": mode, "desc": TICKET_MODES[mode],
                    "gbs": round(nbytes / (best * 1e-3) / 1e9, 1), "grid": best_grid})
    del buf
    return out


def probe_null_decode(dev, layers, hit_lists, stream, blocks=None, reps=3):
    """The pages' null-decode measurement: the hit-expert matrices of every
    resident layer (the weight bytes of the timed step) read with the expert
    kernel's per-lane tile loads and nothing decoded, all layers in one launch
    of moe_probe_tile_read (the 32-byte-per-matrix table upload it enqueues
    first is inside the timed interval). Best of `reps` launches after one
    warm-up. None when a layer holds a code width the probe does not read."""
    import torch
    L = probe_lib()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = blocks or 4 * cus
    rows, nbytes = [], 0
    for layer, experts in zip(layers, hit_lists):
        es = list(experts) + ([layer.E] if layer.has_shared else [])
        for e in es:
            for pj in range(3):
                d = layer.descs[3 * int(e) + pj]
                bits = int(d.bits)
                if bits not in (2, 3, 4):
                    return None
                n, c = (layer.I, layer.H) if pj < 2 else (layer.H, layer.I)
                rows.append((d.codes, d.scales, n // 16, c // 128, bits))
    table = (ProbeTileStream * len(rows))()
    before = 0
    for i, (codes, scales, tr, g, bits) in enumerate(rows):
        table[i] = ProbeTileStream(codes, scales, tr, g, bits, before)
        before += (tr // 4) * (g // 8)
        nbytes += tr * g * (256 * bits + (128 if bits == 4 else 32))
    dev_tab = torch.zeros(len(rows) * 32, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = 1e30
    with torch.cuda.stream(stream):
        for i in range(reps + 1):
            e0.record(stream)
            rc = L.moe_probe_tile_read(table, len(rows), dev_tab.data_ptr(), blocks, sink.data_ptr(),
                                       stream.cuda_stream)
            e1.record(stream)
            if rc:
                raise RuntimeError(f"moe_probe_tile_read: HIP error {-rc}")
            stream.synchronize()
            if i:
                best = min(best, e0.elapsed_time(e1))
    n_layers = len(hit_lists)
    gbs = nbytes / (best * 1e-3) / 1e9
    return {"us_per_layer": round(best * 1e3 / n_layers, 2), "gbs": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_layer": int(nbytes / n_layers),
            "matrices": len(rows), "blocks": blocks}


def probe_launch_floor(dev, layers, reps=50):
    """The graph-replay floor of the step's launch structure: three empty
    kernels per layer (route, expert, combine), `layers` layers, in one graph.
    Returns microseconds per layer."""
    import torch
    L = probe_lib()
    s = torch.cuda.Stream()
    n = 3 * layers
    rc = L.moe_probe_empty_kernels(n, s.cuda_stream)
    s.synchronize()
    if rc:
        raise RuntimeError(f"moe_probe_empty_kernels: HIP error {-rc}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        rc = L.moe_probe_empty_kernels(n, s.cuda_stream)
    if rc:
        raise RuntimeError(f"moe_probe_empty_kernels: HIP error {-rc}")
    with torch.cuda.stream(s):
        for _ in range(5):
            g.replay()
    s.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        e0.record(s)
        for _ in range(reps):
            g.replay()
        e1.record(s)
    s.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps / layers


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    if args.lds_probe:
        res = probe_lds_layouts(torch.device("cuda", 0))
        for layout, us, clk in res:
            log(f"lds probe layout {layout} ({LDS_LAYOUTS[layout]}): {us:.1f} us, "
                f"{clk:.2f} clocks per 16-byte read per CU")
        print(json.dumps({"lds_probe": [{"layout": l, "desc": LDS_LAYOUTS[l], "us": round(us, 1),
                                         "clocks_per_read_per_cu": round(c, 3)}
                                        for l, us, c in res]}))
        return
    if args.copy_calibration:
        n = args.copy_calibration << 18  # float32 elements
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4}))
        return

    from bit_quantized_moe_block_amd import DeviceLayer
    import bit_quantized_moe_block_amd as B
    from moe_synth import WORKLOADS, gen

    w = WORKLOADS[args.workload]
    m = args.m or (16 if args.workload in ("stack43", "full_layer", "shared_layer") else w.max_tokens)
    n_layers = args.layers or w.layers
    stacked = n_layers > 1
    # token counts of the sweep (the metric's m = 1..24) on the same layers
    sweep = [] if (args.no_sweep or not stacked or m > 24) else [1, 2, 4, 8, 16, 24]
    max_tok = max([m] + sweep)
    dev = torch.device("cuda")
    torch.cuda.init()
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} ({props.multi_processor_count} CUs), workload {w.name}, "
        f"layers {n_layers}, m {m}")

    # ---- generate and upload every layer (weights + one batch of inputs each)
    t0 = time.time()
    layers = []
    for l in range(n_layers):
        d = gen.make_layer(w, l)
        d["workload"] = w
        layers.append(DeviceLayer.from_case(d, max_tokens=max(max_tok, 1)))
        del d
        if l % 8 == 0:
            log(f"layer {l} resident ({time.time() - t0:.1f} s)")
    info = layers[0].info()
    log(f"expert grid {info.grid_blocks} blocks ({info.blocks_per_cu}/CU), "
        f"k-splits {info.k_split_gate_up}/{info.k_split_down}")
    stream = torch.cuda.Stream()
    evs = [(HipEvent(), HipEvent()) for _ in layers]
    scrub = None if stacked else torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def measure(mm, steps, warmup, profile_passes):
        """Time the step at mm tokens: returns a dict of the figures, and the
        inputs/outputs per layer."""
        io = []
        for l in range(n_layers):
            x = torch.from_numpy(gen.make_x(w, l, mm).view(np.int16)).to(dev)
            lg = torch.from_numpy(gen.make_logits(w, l, mm)).to(dev)
            io.append((x, lg, torch.empty(mm, w.hidden, device=dev)))
        torch.cuda.synchronize()
        # one eager pass (binds handles to the stream, gives the routing)
        with torch.cuda.stream(stream):
            for layer, (x, lg, out) in zip(layers, io):
                layer.run(x, lg, out, stream=stream)
        stream.synchronize()
        wbytes, hit, hit_lists = [], [], []
        for layer in layers:
            b = layer.buckets(mm)
            experts = np.nonzero(b["counts"])[0]
            hit.append(len(experts))
            hit_lists.append(experts)
            if layer.has_shared:  # the shared expert (stored as expert E) reads its weights too
                experts = np.append(experts, layer.E)
            wbytes.append(layer.weight_bytes(experts))
            st = layer.stats()
            assert st.error_word == 0 and st.items_done == st.items, "expert kernel incomplete"
        step_bytes = float(sum(wbytes))
        if stacked:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for layer, (x, lg, out) in zip(layers, io):
                    layer.run(x, lg, out, stream=stream)
            step = g.replay
        else:
            layer0, (x0, lg0, out0) = layers[0], io[0]

            def step():
                scrub.zero_()  # 1 GiB: the weights come from HBM
                layer0.run(x0, lg0, out0, stream=stream)
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                step()
        stream.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        if stacked:
            with torch.cuda.stream(stream):
                ev0.record(stream)
                for _ in range(steps):
                    step()
                ev1.record(stream)
            torch.cuda.synchronize()
            ms = ev0.elapsed_time(ev1) / steps
        else:
            per = []
            with torch.cuda.stream(stream):
                for _ in range(steps):
                    scrub.zero_()
                    ev0.record(stream)
                    layer0.run(x0, lg0, out0, stream=stream)
                    ev1.record(stream)
                    ev1.synchronize()
                    per.append(ev0.elapsed_time(ev1))
            ms = float(np.median(per))
        wall = (time.perf_counter() - wall0) / steps * 1e3
        torch.cuda.synchronize()
        # the expert kernel alone: HIP events the library records right before
        # and after it, on its stream; every layer launched back to back per
        # pass, read after one synchronisation (graph nodes cannot be timed)
        for layer, (eb, ee) in zip(layers, evs):
            B.moe_decode_profile_events(layer.handle, eb.ptr, ee.ptr)
        kern_ms, kern_bytes = [], []
        with torch.cuda.stream(stream):
            for _ in range(profile_passes):
                for layer, (x, lg, out) in zip(layers, io):
                    if scrub is not None:
                        scrub.zero_()
                    layer.run(x, lg, out, stream=stream)
                stream.synchronize()
                for li in range(n_layers):
                    kern_ms.append(evs[li][0].elapsed_ms(evs[li][1]))
                    kern_bytes.append(wbytes[li])
        for layer in layers:
            B.moe_decode_profile_events(layer.handle, None, None)
        kern_avg_ms = float(np.mean(kern_ms))
        achieved = float(np.mean(kern_bytes)) / (kern_avg_ms * 1e-3) / 1e9
        r = {"m": mm, "ms_per_step": ms, "wall_ms": wall, "us_per_layer": ms * 1e3 / n_layers,
             "gbs": step_bytes / (ms * 1e-3) / 1e9, "step_bytes": step_bytes,
             "hit": float(np.mean(hit)), "hit_lists": hit_lists,
             "kernel_us": kern_avg_ms * 1e3, "kernel_gbs": achieved,
             "kernel_bytes": float(np.mean(kern_bytes))}
        log(f"m {mm}: step {ms:.3f} ms (wall {wall:.3f} ms), {r['us_per_layer']:.1f} us/layer, "
            f"{r['gbs']:.0f} GB/s; expert kernel {r['kernel_us']:.1f} us, {achieved:.0f} GB/s "
            f"({achieved / HBM_PEAK_GBS:.1%} of 8 TB/s), hit experts/layer {r['hit']:.1f}")
        return r, io

    # ---- the headline: the workload at m tokens, timed steps
    head, io = measure(m, args.steps, args.warmup, args.profile_passes)
    value = head["gbs"]
    ms_per_step = head["ms_per_step"]

    # ---- the m = 1..24 sweep on the same resident layers
    sweep_res = []
    for mm in sweep:
        r, _ = (head, None) if mm == m else measure(mm, args.steps, args.warmup, 1)
        sweep_res.append({"m": mm, "us_per_layer": round(r["us_per_layer"], 2),
                          "kernel_us": round(r["kernel_us"], 2),
                          "gbs": round(r["gbs"], 1), "kernel_gbs": round(r["kernel_gbs"], 1),
                          "kernel_frac": round(r["kernel_gbs"] / HBM_PEAK_GBS, 4),
                          "step_frac": round(r["gbs"] / HBM_PEAK_GBS, 4),
                          "weight_mb_per_layer": round(r["step_bytes"] / n_layers / 1e6, 1),
                          "hit_experts": round(r["hit"], 1)})

    # ---- probes: achievable streaming read, launch floor
    probes = None
    if not args.no_probes:
        gbs, grid = probe_plain_read(dev)
        floor = probe_launch_floor(dev, max(n_layers, 1))
        rates = probe_compute_rates(dev)
        tickets = probe_tickets(dev)
        nd = probe_null_decode(dev, layers, head["hit_lists"], stream)
        probes = {"plain_read_gbs": round(gbs, 1), "plain_read_frac": round(gbs / HBM_PEAK_GBS, 4),
                  "plain_read_grid": grid,
                  "launch_floor_us_per_layer": round(floor, 2),
                  "launch_floor_kernels": 3 * max(n_layers, 1),
                  "compute_rates": rates, "ticket_read": tickets, "null_decode": nd}
        log(f"probes: plain read {gbs:.0f} GB/s ({grid} blocks), launch floor "
            f"{floor:.2f} us per layer (3 empty kernels per layer in one graph)")
        for r in rates:
            log(f"probes: {r['desc']}: {r['cycles_per_step']} cycles per MFMA step per SIMD "
                f"({r['ns_per_step']} ns, clock {r['clock_ghz']} GHz)")
        for r in tickets:
            log(f"probes: streaming read, {r['desc']}: {r['gbs']} GB/s ({r['grid']} blocks)")
        if nd:
            log(f"probes: null decode (the expert kernels' weight reads, no decode) at m = {m}: "
                f"{nd['us_per_layer']} us per layer, {nd['gbs']} GB/s ({nd['frac']:.1%} of 8 TB/s)")

    # ---- CPU oracle on a bounded sample (layer 0 of the workload, all m
    # tokens when m <= 24, else the first 16): median of 5 runs after one
    # warm-up on every core of this process, then one run on one thread over
    # the first two tokens
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        tok = None if m <= 24 else list(range(16))
        rid, _ = oracle.route(gen.make_logits(w, 0, m), w.top_k)
        used = np.unique(rid if tok is None else rid[tok])
        d = gen.make_layer(w, 0, experts=used)
        d["workload"] = w
        case = dict(d, m=m, x=gen.make_x(w, 0, m), logits=gen.make_logits(w, 0, m))
        L = oracle.Layer.from_case(case)
        ex = np.append(used, layers[0].E) if layers[0].has_shared else used
        sample_bytes = layers[0].weight_bytes(ex)
        cores = len(os.sched_getaffinity(0))
        oracle.set_threads(cores)
        times, threads, r = [], 0, None
        for rep in range(6):
            t = time.perf_counter()
            r = L.run(case["x"], case["logits"], tokens=tok)
            if rep:
                times.append(time.perf_counter() - t)
            threads = int(r["threads"])
        rows = slice(None) if tok is None else tok
        got = io[0][2].cpu().numpy().astype(np.float64)[rows]
        ref = r["out"][rows]
        rel = float(np.max(np.max(np.abs(got - ref), 1) / np.max(np.abs(ref), 1)))
        t_med = float(np.median(times))
        two = [0, 1] if m >= 2 else [0]
        used2 = np.unique(rid[two])
        ex2 = np.append(used2, layers[0].E) if layers[0].has_shared else used2
        oracle.set_threads(1)
        t = time.perf_counter()
        L.run(case["x"], case["logits"], tokens=two)
        t1 = time.perf_counter() - t
        oracle.set_threads(cores)
        one_thread = layers[0].weight_bytes(ex2) / t1 / 1e9
        cpu = {"value": sample_bytes / t_med / 1e9, "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"layer 0 of {w.name}, " + (f"all {m} tokens" if tok is None else
                                                      f"tokens 0..15 of {m}")
                         + f" (hit experts only), median of 5 runs of {t_med:.2f} s after one "
                           f"warm-up; 1 thread: tokens {two}, {t1:.2f} s",
               "one_thread_value": one_thread, "cpu_model": cpu_model(),
               "rel_err_vs_gpu": rel}
        log(f"oracle {t_med:.2f} s (median of 5) on {threads} threads -> {cpu['value']:.4f} GB/s; "
            f"1 thread {one_thread:.4f} GB/s; GPU vs oracle rel {rel:.2e}")
        if rel > 2e-3:
            print(json.dumps({"error": f"GPU output differs from the oracle: rel {rel:.3e} > 2e-3"}))
            sys.exit(1)

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": (f"{w.name}: {n_layers} x MoE layer (E={w.num_experts}, top-{w.top_k}, "
                         f"hidden {w.hidden}, inter {w.inter}, {w.fmt} {w.bits_mix}, "
                         f"{w.router} routing), m={m}, "
                         + ("one HIP graph" if stacked else "1 GiB cache scrub per launch")),
            "layers": n_layers,
            "m": m,
            "us_per_launch": round(head["us_per_layer"], 2),
            "weight_bytes_per_step": int(head["step_bytes"]),
            "hit_experts_per_layer": head["hit"],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(head["kernel_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(head["kernel_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": (recorded_traffic() if args.workload == "stack43" and m == 16
                        else None),
            "kernel": "expert_kernel",
            "kernel_us_per_launch": round(head["kernel_us"], 2),
            "bytes_per_launch": int(head["kernel_bytes"]),
        },
        "cpu_baseline": cpu,
        "m_sweep": sweep_res or None,
        "probes": probes,
        "provenance": provenance(props),
    }
    print(json.dumps(res), flush=True)
    for layer in layers:
        layer.close()


if __name__ == "__main__":
    main()
