"""Device residency of one layer's stored experts, and its handle.

Uploads the stored tensors of a layer as three device blobs (codes, scales,
codebooks), fills the moe_tensor_desc table with addresses inside them and
creates the C handle. Marshalling only: no arithmetic on the values.
"""
import ctypes as C

import numpy as np
import torch

from . import (MOE_DECODE_ABI_VERSION, MOE_FMT_CODEBOOK, MOE_FMT_NVFP4, MOE_Q_BUCKETS,
               MOE_Q_INFO, MOE_Q_ROUTING, MOE_Q_STATS, moe_decode_config, moe_decode_create,
               moe_decode_destroy, moe_decode_info, moe_decode_query, moe_decode_run,
               moe_decode_run_static, moe_decode_stats, moe_tensor_desc)


def _align(n, a=256):
    return (n + a - 1) // a * a


def _blob(arrays, device):
    """Concatenate byte views at 256-byte aligned offsets into one device tensor.
    An array object passed more than once is stored once (its entries share
    the offset)."""
    offs, total, seen, first = [], 0, {}, []
    for a in arrays:
        if id(a) in seen:
            offs.append(seen[id(a)])
            continue
        seen[id(a)] = total
        offs.append(total)
        first.append((a, total))
        total += _align(a.nbytes)
    host = np.zeros(max(total, 256), np.uint8)
    for a, o in first:
        host[o:o + a.nbytes] = np.ascontiguousarray(a).view(np.uint8).reshape(-1)
    dev = torch.from_numpy(host).to(device)
    return dev, offs


class DeviceLayer:
    """One MoE layer resident on the GPU plus its moe_decode handle.

    fmt: "codebook" | "nvfp4"; tensors: {(e, proj): dict(codes, scales, lut,
    tensor_scale, bits)} for every expert; signs: int8 arrays (codebook);
    shared: None or {proj: tensor} of the always-on shared expert (stored
    after the routed experts, passed as the config's `shared` descriptors).
    """

    def __init__(self, fmt, num_experts, top_k, hidden, inter, tensors, signs_hidden=None,
                 signs_inter=None, max_tokens=24, device="cuda", shared=None):
        E = num_experts
        keys = [(e, p) for e in range(E) for p in range(3)]
        missing = [k for k in keys if k not in tensors]
        if missing:
            raise ValueError(f"missing stored tensors for {missing[:4]}...")
        n_routed = len(keys)
        if shared:
            tensors = dict(tensors)
            for p in range(3):
                tensors[(E, p)] = shared[p]
            keys = keys + [(E, p) for p in range(3)]
        self.codes, co = _blob([tensors[k]["codes"] for k in keys], device)
        self.scales, so = _blob([tensors[k]["scales"] for k in keys], device)
        luts = [tensors[k]["lut"] for k in keys]
        if fmt == "codebook":
            self.luts, lo = _blob(luts, device)
        else:
            self.luts, lo = None, [None] * len(keys)
        descs = (moe_tensor_desc * len(keys))()
        for i, k in enumerate(keys):
            t = tensors[k]
            descs[i].codes = self.codes.data_ptr() + co[i]
            descs[i].scales = self.scales.data_ptr() + so[i]
            descs[i].lut = None if self.luts is None else self.luts.data_ptr() + lo[i]
            descs[i].tensor_scale = float(t.get("tensor_scale", 0.0) or 0.0)
            descs[i].bits = int(t["bits"])
        self.descs = descs
        self.sh = self.si = None
        if signs_hidden is not None:
            self.sh = torch.from_numpy(np.ascontiguousarray(signs_hidden, np.int8)).to(device)
            self.si = torch.from_numpy(np.ascontiguousarray(signs_inter, np.int8)).to(device)
        shared_ptr = (C.cast(C.byref(descs, n_routed * C.sizeof(moe_tensor_desc)),
                             C.POINTER(moe_tensor_desc)) if shared else None)
        self.cfg = moe_decode_config(
            MOE_DECODE_ABI_VERSION, MOE_FMT_CODEBOOK if fmt == "codebook" else MOE_FMT_NVFP4,
            E, top_k, hidden, inter, max_tokens, C.cast(descs, C.POINTER(moe_tensor_desc)),
            None if self.sh is None else self.sh.data_ptr(),
            None if self.si is None else self.si.data_ptr(), shared_ptr)
        self.has_shared = bool(shared)
        self.fmt, self.E, self.k, self.H, self.I = fmt, E, top_k, hidden, inter
        self.max_tokens = max_tokens
        self.device = device
        self.handle = moe_decode_create(self.cfg)

    @classmethod
    def from_case(cls, case, max_tokens=None, device="cuda"):
        w = case["workload"]
        return cls(w.fmt, w.num_experts, w.top_k, w.hidden, w.inter, case["tensors"],
                   case["signs_hidden"], case["signs_inter"],
                   max_tokens or max(case.get("m", 1), w.max_tokens), device,
                   shared=case.get("shared"))

    def weight_bytes(self, experts):
        """Stored bytes (codes + scales + codebook) of the given experts."""
        tot = 0
        for e in experts:
            for p in range(3):
                d = self.descs[3 * int(e) + p]
                N, Cc = (self.I, self.H) if p < 2 else (self.H, self.I)
                if self.fmt == "codebook":
                    tot += N * Cc * d.bits // 8 + N * Cc // 128 * 2 + (1 << d.bits) * 2
                else:
                    tot += N * Cc // 2 + N * Cc // 16
        return tot

    def _check_args(self, x, logits, out, m):
        """Shapes, dtypes, layout and device of run()'s tensors (the C ABI
        takes raw pointers and cannot tell)."""
        if m < 0:
            raise ValueError(f"m = {m} < 0")
        want = ((x, (torch.bfloat16, torch.int16), self.H, "x"),
                (logits, (torch.float32,), self.E, "logits"),
                (out, (torch.float32,), self.H, "out"))
        for t, dtypes, cols, name in want:
            if not isinstance(t, torch.Tensor):
                raise TypeError(f"{name} must be a torch.Tensor")
            if t.dtype not in dtypes:
                raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
            if t.dim() != 2 or t.shape[1] != cols or t.shape[0] < m:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected [>= {m}, {cols}]")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous (row-major)")
        for t, _, _, name in want:
            if t.device.type != "cuda":
                raise ValueError(f"{name} is on {t.device}, expected a GPU tensor")

    def run(self, x, logits, out, m=None, stream=None):
        """x: bf16 [m, H] (or int16 bit patterns), logits fp32 [m, E], out fp32 [m, H]."""
        m = x.shape[0] if m is None else m
        self._check_args(x, logits, out, m)
        s = torch.cuda.current_stream() if stream is None else stream
        moe_decode_run(self.handle, x.data_ptr(), logits.data_ptr(), out.data_ptr(), m,
                       s.cuda_stream)

    def run_static(self, x, logits, out, m=None, stream=None):
        """run() with the per-run buffers in the library's static scratch (no
        allocation; static runs on one device must not overlap)."""
        m = x.shape[0] if m is None else m
        self._check_args(x, logits, out, m)
        s = torch.cuda.current_stream() if stream is None else stream
        moe_decode_run_static(self.handle, x.data_ptr(), logits.data_ptr(), out.data_ptr(), m,
                              s.cuda_stream)

    def info(self):
        i = moe_decode_info()
        moe_decode_query(self.handle, MOE_Q_INFO, i)
        return i

    def stats(self):
        s = moe_decode_stats()
        moe_decode_query(self.handle, MOE_Q_STATS, s)
        return s

    def routing(self, m):
        buf = np.zeros(2 * m * self.k, np.int32)
        moe_decode_query(self.handle, MOE_Q_ROUTING, buf)
        return buf[:m * self.k].reshape(m, self.k), buf[m * self.k:].view(np.float32).reshape(m, self.k)

    def buckets(self, m):
        E, np_ = self.E, m * self.k
        buf = np.zeros(2 * E + 1 + np_, np.int32)
        moe_decode_query(self.handle, MOE_Q_BUCKETS, buf)
        return dict(counts=buf[:E], offsets=buf[E:2 * E + 1], rows=buf[2 * E + 1:])

    def close(self):
        """Destroy the handle (raises MoeDecodeError if the last run reported a
        device error; the handle is gone either way)."""
        if self.handle:
            h, self.handle = self.handle, None
            moe_decode_destroy(h)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
