"""Seeded synthetic inputs for the routed-experts decode step.

Shared by the oracle-side tests and the GPU path. It only draws numbers: it
packs nothing, rotates nothing, routes nothing and dequantises nothing. Every
stored weight is drawn directly in its stored form:

* codebook codes: uniform random 32-bit words. Every code field of the packed
  layout then holds an i.i.d. uniform K-bit code whatever the layout is.
* codebook LUT: 2^K sorted N(0,1) draws rounded to fp16, redrawn until distinct.
* group scales: fp16 of U(0.01, 0.05).
* NVFP4 codes: uniform random bytes (two e2m1 nibbles each).
* NVFP4 block scales: e4m3fn bytes with exponent field 6..8 and any mantissa,
  i.e. values in [0.5, 3.75]; or (workload option "all_finite") uniform over
  all 254 finite e4m3fn codes of either sign, subnormals and 448 included.
* NVFP4 tensor scale: fp32 of ts_scale * U(0.8, 1.2), ts_scale 0.004 unless
  the workload says otherwise.
* activations: N(0,1) rounded to bfloat16 (round to nearest even), given as the
  raw 16-bit patterns.
* router logits: fp32 N(0,1), plus a per-expert Zipf bias -s*ln(rank) for the
  skewed workloads (rank = a seeded permutation of 1..E).
* rotation signs: +1/-1 as int8.

Seeds: numpy SeedSequence(entropy = 1000 + config_id, spawn_key = key) with
key = (layer, tag, ...). Bit generator SFC64.
"""
import concurrent.futures as _cf
import os

import numpy as np

from .configs import PACK_ALL2_LAYERS, Workload

TAG_X, TAG_LOGITS, TAG_SIGN_H, TAG_SIGN_I, TAG_ZIPF, TAG_KMIX, TAG_CODES, TAG_LUT, \
    TAG_SCALES, TAG_TSCALE = range(10)

PROJ_GATE, PROJ_UP, PROJ_DOWN = 0, 1, 2


def _rng(config_id, *key):
    ss = np.random.SeedSequence(entropy=1000 + int(config_id), spawn_key=tuple(int(k) for k in key))
    return np.random.Generator(np.random.SFC64(ss))


def _raw_words(config_id, nwords, *key):
    """nwords uniform uint32 words."""
    bg = np.random.SFC64(np.random.SeedSequence(entropy=1000 + int(config_id),
                                                spawn_key=tuple(int(k) for k in key)))
    n64 = (nwords + 1) // 2
    return bg.random_raw(n64).view(np.uint32)[:nwords].copy()


def bf16_bits_from_f32(a):
    """Round fp32 to bfloat16 (nearest even), returning uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def expert_bits(w: Workload, layer: int = 0) -> np.ndarray:
    """Bits per expert (shared by the expert's gate, up and down tensors)."""
    E = w.num_experts
    if w.bits_mix == "all2":
        return np.full(E, 2, np.int32)
    if w.bits_mix == "all3":
        return np.full(E, 3, np.int32)
    if w.bits_mix == "alternate":
        return (2 + (np.arange(E) % 2)).astype(np.int32)
    if w.bits_mix == "mix62" or (w.bits_mix == "pack" and layer not in PACK_ALL2_LAYERS):
        n3 = (E * 5) // 8
        pick = _rng(w.config_id, layer, TAG_KMIX).permutation(E)[:n3]
        b = np.full(E, 2, np.int32)
        b[pick] = 3
        return b
    if w.bits_mix == "pack":
        return np.full(E, 2, np.int32)
    if w.bits_mix == "nvfp4":
        return np.full(E, 4, np.int32)
    raise ValueError(w.bits_mix)


def make_x(w: Workload, layer: int, m: int) -> np.ndarray:
    """bf16 activations [m, hidden] as uint16 bit patterns."""
    a = _rng(w.config_id, layer, TAG_X, m).standard_normal((m, w.hidden), dtype=np.float32)
    return bf16_bits_from_f32(a)


def zipf_bias(w: Workload, layer: int) -> np.ndarray:
    rank = _rng(w.config_id, layer, TAG_ZIPF).permutation(w.num_experts) + 1
    return (-w.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)


def make_logits(w: Workload, layer: int, m: int) -> np.ndarray:
    """fp32 router logits [m, num_experts]."""
    a = _rng(w.config_id, layer, TAG_LOGITS, m).standard_normal((m, w.num_experts),
                                                                dtype=np.float32)
    if w.router == "zipf":
        a = (a + zipf_bias(w, layer)[None, :]).astype(np.float32)
    return a


def make_signs(w: Workload, layer: int, which: str) -> np.ndarray:
    n, tag = (w.hidden, TAG_SIGN_H) if which == "hidden" else (w.inter, TAG_SIGN_I)
    b = _rng(w.config_id, layer, tag).integers(0, 2, n)
    return np.where(b == 1, 1, -1).astype(np.int8)


def tensor_shape(w: Workload, proj: int):
    """(rows, cols) = (outputs, inputs) of an expert projection."""
    return (w.inter, w.hidden) if proj in (PROJ_GATE, PROJ_UP) else (w.hidden, w.inter)


def make_lut(config_id, layer, e, proj, bits):
    g = _rng(config_id, layer, TAG_LUT, e, proj)
    while True:
        v = np.sort(g.standard_normal(1 << bits)).astype(np.float16)
        if len(np.unique(v)) == len(v):
            return v


def make_tensor(w: Workload, layer: int, e: int, proj: int, bits: int) -> dict:
    """Stored form of one expert projection."""
    N, C = tensor_shape(w, proj)
    cid = w.config_id
    if w.fmt == "codebook":
        nwords = N * C * bits // 32
        codes = _raw_words(cid, nwords, layer, TAG_CODES, e, proj)
        scales = _rng(cid, layer, TAG_SCALES, e, proj).uniform(0.01, 0.05, N * C // 128)
        return dict(bits=bits, codes=codes, scales=scales.astype(np.float16),
                    lut=make_lut(cid, layer, e, proj, bits), tensor_scale=np.float32(0.0))
    # NVFP4
    nbytes = N * C // 2
    codes = _raw_words(cid, nbytes // 4, layer, TAG_CODES, e, proj).view(np.uint8)
    g = _rng(cid, layer, TAG_SCALES, e, proj)
    if w.nv_scales == "all_finite":
        # every e4m3fn byte except the two NaN codes 0x7F and 0xFF
        finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
        scales = finite[g.integers(0, len(finite), N * C // 16)]
    else:
        ex = g.integers(6, 9, N * C // 16)
        mant = g.integers(0, 8, N * C // 16)
        scales = ((ex << 3) | mant).astype(np.uint8)
    ts = np.float32(w.ts_scale * _rng(cid, layer, TAG_TSCALE, e, proj).uniform(0.8, 1.2))
    return dict(bits=4, codes=codes, scales=scales, lut=None, tensor_scale=ts)


def make_layer(w: Workload, layer: int = 0, experts=None, threads=None) -> dict:
    """All stored tensors of one layer (or of the given experts only).

    Returns dict(bits [E], tensors {(e, proj): tensor}, shared ({proj: tensor}
    or None), shared_bits, signs_hidden, signs_inter).
    """
    bits = expert_bits(w, layer)
    ex = range(w.num_experts) if experts is None else sorted(set(int(e) for e in experts))
    jobs = [(e, p) for e in ex for p in (PROJ_GATE, PROJ_UP, PROJ_DOWN)]
    threads = threads or min(16, os.cpu_count() or 1)
    with _cf.ThreadPoolExecutor(threads) as pool:
        out = list(pool.map(lambda ep: make_tensor(w, layer, ep[0], ep[1], int(bits[ep[0]])), jobs))
    tensors = {ep: t for ep, t in zip(jobs, out)}
    d = dict(bits=bits, tensors=tensors, shared=None, shared_bits=0)
    if w.shared_bits:
        # the shared expert draws as expert index E (its own seed namespace)
        d["shared"] = {p: make_tensor(w, layer, w.num_experts, p, w.shared_bits)
                       for p in (PROJ_GATE, PROJ_UP, PROJ_DOWN)}
        d["shared_bits"] = w.shared_bits
    if w.fmt == "codebook":
        d["signs_hidden"] = make_signs(w, layer, "hidden")
        d["signs_inter"] = make_signs(w, layer, "inter")
    else:
        d["signs_hidden"] = None
        d["signs_inter"] = None
    return d


def make_case(w: Workload, m: int, layer: int = 0, experts=None) -> dict:
    """One layer's weights plus one batch of m tokens."""
    d = make_layer(w, layer, experts)
    d.update(workload=w, layer=layer, m=m, x=make_x(w, layer, m), logits=make_logits(w, layer, m))
    return d
