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
sample of the same workload (whole layers, about 10 s of CPU work).
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
KERNEL_SRC = os.path.join(ROOT, "bit_quantized_moe_block_amd", "csrc", "kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "expert_kernel_stack43_m16_traffic.md")


def kernel_source_sha():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


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
    ap.add_argument("--profile-passes", type=int, default=3)
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


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

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
    from moe_synth import WORKLOADS, gen

    w = WORKLOADS[args.workload]
    m = args.m or (16 if args.workload in ("stack43", "full_layer", "shared_layer") else w.max_tokens)
    n_layers = args.layers or w.layers
    stacked = n_layers > 1
    dev = torch.device("cuda")
    torch.cuda.init()
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} ({props.multi_processor_count} CUs), workload {w.name}, "
        f"layers {n_layers}, m {m}")

    # ---- generate and upload every layer (weights + one batch of inputs each)
    t0 = time.time()
    layers, inputs, routing_ids = [], [], []
    for l in range(n_layers):
        d = gen.make_layer(w, l)
        d["workload"] = w
        layer = DeviceLayer.from_case(d, max_tokens=max(m, 1))
        x = torch.from_numpy(gen.make_x(w, l, m).view(np.int16)).to(dev)
        lg = torch.from_numpy(gen.make_logits(w, l, m)).to(dev)
        out = torch.empty(m, w.hidden, device=dev)
        layers.append(layer)
        inputs.append((x, lg, out))
        del d
        if l % 8 == 0:
            log(f"layer {l} resident ({time.time() - t0:.1f} s)")
    info = layers[0].info()
    log(f"expert grid {info.grid_blocks} blocks ({info.blocks_per_cu}/CU), "
        f"k-splits {info.k_split_gate_up}/{info.k_split_down}")

    stream = torch.cuda.Stream()
    # ---- one eager pass (binds handles to the stream, gives the routing)
    with torch.cuda.stream(stream):
        for layer, (x, lg, out) in zip(layers, inputs):
            layer.run(x, lg, out, stream=stream)
    stream.synchronize()
    weight_bytes = []
    hit = []
    for layer in layers:
        b = layer.buckets(m)
        experts = np.nonzero(b["counts"])[0]
        hit.append(len(experts))
        if layer.has_shared:  # the shared expert (stored as expert E) reads its weights too
            experts = np.append(experts, layer.E)
        weight_bytes.append(layer.weight_bytes(experts))
        st = layer.stats()
        assert st.error_word == 0 and st.items_done == st.items, "expert kernel incomplete"
    step_bytes = float(sum(weight_bytes))
    log(f"weight bytes per step {step_bytes / 1e9:.3f} GB, hit experts/layer "
        f"{np.mean(hit):.1f}")

    # ---- capture the whole step in one graph
    scrub = None
    if stacked:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for layer, (x, lg, out) in zip(layers, inputs):
                layer.run(x, lg, out, stream=stream)

        def step():
            g.replay()
    else:
        # single layer: scrub 1 GiB before each launch so weights come from HBM
        scrub = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        layer, (x, lg, out) = layers[0], inputs[0]

        def step():
            scrub.zero_()
            layer.run(x, lg, out, stream=stream)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    stream.synchronize()

    # ---- timed region
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    if stacked:
        with torch.cuda.stream(stream):
            ev0.record(stream)
            for _ in range(args.steps):
                step()
            ev1.record(stream)
        torch.cuda.synchronize()
        ms_per_step = ev0.elapsed_time(ev1) / args.steps
    else:
        # time only the layer, not the scrub
        per = []
        with torch.cuda.stream(stream):
            for _ in range(args.steps):
                scrub.zero_()
                ev0.record(stream)
                layer.run(x, lg, out, stream=stream)
                ev1.record(stream)
                ev1.synchronize()
                per.append(ev0.elapsed_time(ev1))
        ms_per_step = float(np.median(per))
    wall = (time.perf_counter() - wall0) / args.steps * 1e3
    torch.cuda.synchronize()
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    us_per_layer = ms_per_step * 1e3 / n_layers
    log(f"step {ms_per_step:.3f} ms (wall {wall:.3f} ms), {us_per_layer:.1f} us/layer, "
        f"{value:.0f} GB/s")

    # ---- dominant kernel alone: HIP events recorded by the library right
    # before and after the expert kernel, on the stream it is launched on.
    # Each pass launches every layer back to back (the host enqueues far
    # faster than the layers run) and reads the events after one
    # synchronisation. (Events recorded by graph nodes cannot be timed.)
    import bit_quantized_moe_block_amd as B
    evs = [(HipEvent(), HipEvent()) for _ in layers]
    for layer, (eb, ee) in zip(layers, evs):
        B.moe_decode_profile_events(layer.handle, eb.ptr, ee.ptr)
    kern_ms, kern_bytes = [], []
    with torch.cuda.stream(stream):
        for _ in range(args.profile_passes):
            for li, (layer, (x, lg, out)) in enumerate(zip(layers, inputs)):
                if scrub is not None:
                    scrub.zero_()
                layer.run(x, lg, out, stream=stream)
            stream.synchronize()
            for li in range(len(layers)):
                kern_ms.append(evs[li][0].elapsed_ms(evs[li][1]))
                kern_bytes.append(weight_bytes[li])
    for layer in layers:
        B.moe_decode_profile_events(layer.handle, None, None)
    kern_avg_ms = float(np.mean(kern_ms))
    achieved = float(np.mean(kern_bytes)) / (kern_avg_ms * 1e-3) / 1e9
    log(f"expert kernel avg {kern_avg_ms * 1e3:.1f} us/launch, {achieved:.0f} GB/s "
        f"({achieved / HBM_PEAK_GBS:.1%} of 8 TB/s)")

    # ---- CPU oracle on a bounded sample: whole layers of the same workload
    # (all m tokens each, or the first 16 tokens when m > 24) until about
    # 10 s of CPU work, at most 4 layers
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        cpu_s, cpu_bytes, rel, threads, done_layers = 0.0, 0.0, 0.0, 0, 0
        tok = None if m <= 24 else list(range(16))
        for li in range(min(4, n_layers)):
            rid, _ = oracle.route(gen.make_logits(w, li, m), w.top_k)
            used = np.unique(rid if tok is None else rid[tok])
            d = gen.make_layer(w, li, experts=used)
            d["workload"] = w
            case = dict(d, m=m, x=gen.make_x(w, li, m), logits=gen.make_logits(w, li, m))
            L = oracle.Layer.from_case(case)
            t = time.perf_counter()
            r = L.run(case["x"], case["logits"], tokens=tok)
            cpu_s += time.perf_counter() - t
            if tok is None:
                cpu_bytes += weight_bytes[li]
            else:
                ex = np.append(used, layers[li].E) if layers[li].has_shared else used
                cpu_bytes += layers[li].weight_bytes(ex)
            threads = int(r["threads"])
            done_layers += 1
            rows = slice(None) if tok is None else tok
            ref = r["out"][rows]
            got = inputs[li][2].cpu().numpy().astype(np.float64)[rows]
            rel = max(rel, float(np.max(np.max(np.abs(got - ref), 1) / np.max(np.abs(ref), 1))))
            del L, case, d
            if cpu_s >= 10.0:
                break
        cpu = {"value": cpu_bytes / cpu_s / 1e9, "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{done_layers} layer(s) of {w.name} (layers 0..{done_layers - 1}, "
                         + (f"all {m} tokens" if tok is None else f"tokens 0..15 of {m}")
                         + f", hit experts only), {cpu_s:.1f} s of CPU time",
               "rel_err_vs_gpu": rel}
        log(f"oracle {cpu_s:.1f} s on {threads} threads over {done_layers} layer(s) -> "
            f"{cpu['value']:.4f} GB/s; GPU vs oracle rel {rel:.2e}")

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
            "us_per_launch": round(us_per_layer, 2),
            "weight_bytes_per_step": int(step_bytes),
            "hit_experts_per_layer": float(np.mean(hit)),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": (recorded_traffic() if args.workload == "stack43" and m == 16
                        else None),
            "kernel": "expert_kernel",
            "kernel_us_per_launch": round(kern_avg_ms * 1e3, 2),
            "bytes_per_launch": int(np.mean(kern_bytes)),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    for layer in layers:
        layer.close()


if __name__ == "__main__":
    main()
