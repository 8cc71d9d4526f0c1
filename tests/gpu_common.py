"""Shared helpers of the GPU tests (parity metric, device upload, cases)."""
import numpy as np
import torch

import oracle
from bit_quantized_moe_block_amd import DeviceLayer

# Worst token of max_i |y_gpu - y_ref| / max_i |y_ref| over the H outputs.
REL_TOL = 2e-3
WEIGHT_TOL = 1e-6


def rel_err(out_gpu, out_ref, tokens=None):
    g = np.asarray(out_gpu, np.float64)
    r = np.asarray(out_ref, np.float64)
    if tokens is not None:
        g, r = g[tokens], r[tokens]
    num = np.max(np.abs(g - r), axis=1)
    den = np.max(np.abs(r), axis=1)
    return float(np.max(num / np.where(den > 0, den, 1.0)))


def to_dev(case, m=None):
    x = torch.from_numpy(case["x"].view(np.int16)).cuda()
    lg = torch.from_numpy(case["logits"]).cuda()
    out = torch.full((x.shape[0], case["workload"].hidden), float("nan"), device="cuda")
    # the copies and the fill ran on the current stream; runs may use another
    torch.cuda.synchronize()
    return x, lg, out


def run_gpu(layer: DeviceLayer, case, stream=None):
    x, lg, out = to_dev(case)
    layer.run(x, lg, out, stream=stream)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def say(msg):
    print(msg, flush=True)


def check_routing(layer, case, m):
    ids, w = layer.routing(m)
    rid, rw = oracle.route(case["logits"], case["workload"].top_k)
    assert np.array_equal(ids, rid), "routing ids differ"
    assert np.max(np.abs(w.astype(np.float64) - rw)) <= WEIGHT_TOL
    b = layer.buckets(m)
    rb = oracle.bucket(rid, case["workload"].num_experts)
    assert np.array_equal(b["counts"], rb["counts"])
    assert np.array_equal(b["offsets"], rb["offsets"])
    k = case["workload"].top_k
    assert np.array_equal(b["rows"], rb["rows_t"] * k + rb["rows_j"])


def routed_case(w, m, layer=0, x=None, logits=None):
    """A case whose stored tensors cover only the experts its tokens route to
    (the oracle never reads the others; large layers generate quickly)."""
    from moe_synth import gen
    lg = gen.make_logits(w, layer, m) if logits is None else logits
    ids, _ = oracle.route(lg, w.top_k)
    d = gen.make_layer(w, layer, experts=np.unique(ids))
    d.update(workload=w, layer=layer, m=m, x=gen.make_x(w, layer, m) if x is None else x,
             logits=lg)
    return d


def device_layer(case, max_tokens=None):
    """DeviceLayer for a case that may lack unrouted experts: those point at
    one routed expert's tensors (uploaded once; the kernels never read them)."""
    w = case["workload"]
    tensors = dict(case["tensors"])
    have = sorted({e for e, _ in tensors})
    for e in range(w.num_experts):
        if e not in have:
            for p in range(3):
                tensors[(e, p)] = case["tensors"][(have[0], p)]
    c = dict(case, tensors=tensors)
    return DeviceLayer.from_case(c, max_tokens=max_tokens or case["x"].shape[0])


def check_stats(layer):
    st = layer.stats()   # raises MoeDecodeError(MOE_E_DEVICE) on a kernel error
    assert st.error_word == 0 and st.items_done == st.items, (st.error_word, st.items_done,
                                                               st.items)
    return st
