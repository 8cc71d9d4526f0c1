"""CPU oracle of the routed-experts decode step (fp64, plain loops).

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package. The GPU library and its Python
binding never do; the two share no code.

The arithmetic lives in moe_oracle.c (built with gcc, not hipcc); this module
only marshals numpy arrays into it. See moe_oracle.c for what each function
follows on the pages.
"""
import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_ORACLE_SOURCE / MOE_ORACLE_LIBRARY: build and load another copy of the C
# source (the mutation test plants mistakes in a copy this way).
_SRC = os.environ.get("MOE_ORACLE_SOURCE") or os.path.join(_HERE, "moe_oracle.c")
_LIB = os.environ.get("MOE_ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")

FMT_CODEBOOK = 1
FMT_NVFP4 = 2


def build(force=True):
    """Compile the oracle with gcc (OpenMP, fp contraction off)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = C.CDLL(_LIB)
        P = C.c_void_p
        L.orc_f16_to_double.restype = C.c_double
        L.orc_f16_to_double.argtypes = [C.c_uint16]
        L.orc_bf16_to_double.restype = C.c_double
        L.orc_bf16_to_double.argtypes = [C.c_uint16]
        L.orc_e2m1_to_double.restype = C.c_double
        L.orc_e2m1_to_double.argtypes = [C.c_uint8]
        L.orc_e4m3fn_to_double.restype = C.c_double
        L.orc_e4m3fn_to_double.argtypes = [C.c_uint8]
        L.orc_fwht128.argtypes = [P]
        L.orc_rotate.argtypes = [C.c_int, P, P, P]
        L.orc_unrotate.argtypes = [C.c_int, P, P, P]
        L.orc_codebook_code.restype = C.c_uint32
        L.orc_codebook_code.argtypes = [C.c_int, C.c_int, C.c_int, P, C.c_int, C.c_int]
        L.orc_codebook_weight.restype = C.c_double
        L.orc_codebook_weight.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P, C.c_int, C.c_int]
        L.orc_nvfp4_code.restype = C.c_uint8
        L.orc_nvfp4_code.argtypes = [C.c_int, C.c_int, P, C.c_int, C.c_int]
        L.orc_nvfp4_weight.restype = C.c_double
        L.orc_nvfp4_weight.argtypes = [C.c_int, C.c_int, P, P, C.c_float, C.c_int, C.c_int]
        L.orc_route.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P]
        L.orc_bucket.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P, P, P, P]
        L.orc_moe_layer.restype = C.c_int
        L.orc_moe_layer.argtypes = [P, C.c_int, P, P, P, P, P, P, P]
        L.orc_dequant.argtypes = [P, C.c_int, C.c_int, C.c_int, C.c_int, P]
        L.orc_expert.argtypes = [P, C.c_int, P, P]
        L.orc_set_threads.argtypes = [C.c_int]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


class _Layer(C.Structure):
    _fields_ = [("format", C.c_int32), ("num_experts", C.c_int32), ("top_k", C.c_int32),
                ("hidden", C.c_int32), ("inter", C.c_int32), ("bits", C.c_void_p),
                ("codes", C.c_void_p), ("scales", C.c_void_p), ("luts", C.c_void_p),
                ("tscales", C.c_void_p), ("signs_hidden", C.c_void_p),
                ("signs_inter", C.c_void_p), ("has_shared", C.c_int32)]


class Layer:
    """Marshalled view of one layer's stored tensors (keeps arrays alive).

    fmt: "codebook" or "nvfp4"; tensors: {(e, proj): dict(codes, scales, lut,
    tensor_scale)}; experts missing from `tensors` must never be routed to.
    shared: None, or {proj: tensor} of the shared expert (codebook format,
    `shared_bits` bits), stored as expert E.
    """

    def __init__(self, fmt, num_experts, top_k, hidden, inter, bits, tensors,
                 signs_hidden=None, signs_inter=None, shared=None, shared_bits=0):
        E = num_experts
        self.keep = []
        self.bits = np.zeros(E + 1, np.int32)
        self.bits[:E] = np.asarray(bits, dtype=np.int32)
        self.bits[E] = shared_bits if shared else 0
        codes = (C.c_void_p * (3 * E + 3))()
        scales = (C.c_void_p * (3 * E + 3))()
        luts = (C.c_void_p * (3 * E + 3))()
        ts = np.zeros(3 * E + 3, np.float32)
        items = list(tensors.items())
        if shared:
            items += [((E, p), t) for p, t in shared.items()]
        for (e, p), t in items:
            c = np.ascontiguousarray(t["codes"])
            s = np.ascontiguousarray(t["scales"])
            self.keep += [c, s]
            codes[3 * e + p] = c.ctypes.data
            scales[3 * e + p] = s.ctypes.data
            if t.get("lut") is not None:
                lu = np.ascontiguousarray(t["lut"], dtype=np.float16)
                self.keep.append(lu)
                luts[3 * e + p] = lu.ctypes.data
            ts[3 * e + p] = np.float32(t.get("tensor_scale", 0.0))
        self.keep += [codes, scales, luts, ts]
        self.sh = None if signs_hidden is None else np.ascontiguousarray(signs_hidden, np.int8)
        self.si = None if signs_inter is None else np.ascontiguousarray(signs_inter, np.int8)
        self.s = _Layer(FMT_CODEBOOK if fmt == "codebook" else FMT_NVFP4, E, top_k, hidden, inter,
                        self.bits.ctypes.data, C.cast(codes, C.c_void_p),
                        C.cast(scales, C.c_void_p), C.cast(luts, C.c_void_p), ts.ctypes.data,
                        None if self.sh is None else self.sh.ctypes.data,
                        None if self.si is None else self.si.ctypes.data, 1 if shared else 0)
        self.fmt, self.E, self.k, self.H, self.I = fmt, E, top_k, hidden, inter

    @classmethod
    def from_case(cls, case):
        w = case["workload"]
        return cls(w.fmt, w.num_experts, w.top_k, w.hidden, w.inter, case["bits"],
                   case["tensors"], case["signs_hidden"], case["signs_inter"],
                   case.get("shared"), case.get("shared_bits", 0))

    def ptr(self):
        return C.cast(C.pointer(self.s), C.c_void_p)

    def shape(self, proj):
        return (self.I, self.H) if proj in (0, 1) else (self.H, self.I)

    def dequant(self, e, proj):
        N, Cc = self.shape(proj)
        W = np.empty((N, Cc), np.float64)
        lib().orc_dequant(self.ptr(), e, proj, N, Cc, _p(W))
        return W

    def expert(self, e, x_rot):
        x_rot = np.ascontiguousarray(x_rot, np.float64)
        y = np.empty(self.H, np.float64)
        lib().orc_expert(self.ptr(), e, _p(x_rot), _p(y))
        return y

    def run(self, x_bf16, logits, tokens=None, want_pairs=False):
        """The whole step. Returns dict(out, ids, w, threads[, y_pairs])."""
        x_bf16 = np.ascontiguousarray(x_bf16, np.uint16)
        logits = np.ascontiguousarray(logits, np.float32)
        m = x_bf16.shape[0]
        mask = None
        if tokens is not None:
            mask = np.zeros(m, np.uint8)
            mask[np.asarray(tokens, dtype=np.int64)] = 1
        out = np.full((m, self.H), np.nan)
        ids = np.empty((m, self.k), np.int32)
        w = np.empty((m, self.k), np.float64)
        yp = np.full((m, self.k, self.H), np.nan) if want_pairs else None
        thr = lib().orc_moe_layer(self.ptr(), m, _p(x_bf16), _p(logits), _p(mask), _p(out),
                                  _p(ids), _p(w), _p(yp))
        r = dict(out=out, ids=ids, w=w, threads=thr)
        if want_pairs:
            r["y_pairs"] = yp
        return r


def set_threads(n):
    """OpenMP threads of later oracle calls on this thread (timing only)."""
    lib().orc_set_threads(int(n))


# ---------------------------------------------------------------- scalars

def f16_to_double(h):
    return lib().orc_f16_to_double(int(h))


def bf16_to_double(b):
    return lib().orc_bf16_to_double(int(b))


def e2m1_to_double(n):
    return lib().orc_e2m1_to_double(int(n))


def e4m3fn_to_double(b):
    return lib().orc_e4m3fn_to_double(int(b))


def fwht128(v):
    v = np.array(v, dtype=np.float64, copy=True)
    assert v.shape == (128,)
    lib().orc_fwht128(_p(v))
    return v


def rotate(v, signs):
    v = np.ascontiguousarray(v, np.float64)
    s = np.ascontiguousarray(signs, np.int8)
    out = np.empty_like(v)
    lib().orc_rotate(len(v), _p(s), _p(v), _p(out))
    return out


def unrotate(v, signs):
    v = np.ascontiguousarray(v, np.float64)
    s = np.ascontiguousarray(signs, np.int8)
    out = np.empty_like(v)
    lib().orc_unrotate(len(v), _p(s), _p(v), _p(out))
    return out


def codebook_code(bits, N, Cc, codes, n, c):
    codes = np.ascontiguousarray(codes, np.uint32)
    return lib().orc_codebook_code(bits, N, Cc, _p(codes), n, c)


def nvfp4_code(N, Cc, codes, n, c):
    codes = np.ascontiguousarray(codes, np.uint8)
    return lib().orc_nvfp4_code(N, Cc, _p(codes), n, c)


def route(logits, k):
    logits = np.ascontiguousarray(logits, np.float32)
    m, E = logits.shape
    ids = np.empty((m, k), np.int32)
    w = np.empty((m, k), np.float64)
    lib().orc_route(m, E, k, _p(logits), _p(ids), _p(w))
    return ids, w


def bucket(ids, E):
    ids = np.ascontiguousarray(ids, np.int32)
    m, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    rt = np.empty(m * k, np.int32)
    rj = np.empty(m * k, np.int32)
    pos = np.empty(m * k, np.int32)
    lib().orc_bucket(m, E, k, _p(ids), _p(counts), _p(offsets), _p(rt), _p(rj), _p(pos))
    return dict(counts=counts, offsets=offsets, rows_t=rt, rows_j=rj, pos=pos.reshape(m, k))
