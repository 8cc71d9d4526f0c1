"""Python binding of libmoedecode.so (the gfx950 routed-experts decode step).

Argument marshalling only: every step of the path runs in the HIP kernels of
csrc/. PyTorch supplies device memory and streams. The functions carry the C
names of include/moe_decode.h. There is no CPU fallback: if the library is
missing or the device is not a gfx950 GPU, calls raise.
"""
import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoedecode.so")

MOE_DECODE_ABI_VERSION = 3
MOE_OK, MOE_E_INVALID, MOE_E_UNSUPPORTED, MOE_E_HIP, MOE_E_NOMEM, MOE_E_STREAM, MOE_E_DEVICE = \
    0, -1, -2, -3, -4, -5, -6
MOE_FMT_CODEBOOK, MOE_FMT_NVFP4 = 1, 2
MOE_Q_INFO, MOE_Q_ROUTING, MOE_Q_BUCKETS, MOE_Q_STATS = 1, 2, 3, 4

EXPORTED = ("moe_decode_create", "moe_decode_run", "moe_decode_run_static",
            "moe_decode_destroy", "moe_decode_last_error", "moe_decode_query",
            "moe_decode_profile_events")


class moe_tensor_desc(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("lut", C.c_void_p),
                ("tensor_scale", C.c_float), ("bits", C.c_int32)]


class moe_decode_config(C.Structure):
    _fields_ = [("abi_version", C.c_uint32), ("format", C.c_int32), ("num_experts", C.c_int32),
                ("top_k", C.c_int32), ("hidden", C.c_int32), ("inter", C.c_int32),
                ("max_tokens", C.c_int32), ("tensors", C.POINTER(moe_tensor_desc)),
                ("signs_hidden", C.c_void_p), ("signs_inter", C.c_void_p),
                ("shared", C.POINTER(moe_tensor_desc))]


class moe_decode_info(C.Structure):
    _fields_ = [("cu_count", C.c_int32), ("grid_blocks", C.c_int32),
                ("blocks_per_cu", C.c_int32), ("k_split_gate_up", C.c_int32),
                ("k_split_down", C.c_int32), ("reserved", C.c_int32),
                ("scratch_bytes", C.c_int64)]


class moe_decode_stats(C.Structure):
    _fields_ = [("m", C.c_int32), ("hit_experts", C.c_int32), ("items", C.c_int32),
                ("items_done", C.c_int32), ("error_word", C.c_int32), ("reserved", C.c_int32)]


class MoeDecodeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"moe_decode status {status}: {msg}")
        self.status = status


_lib = None


def lib():
    """Load libmoedecode.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        L.moe_decode_create.restype = C.c_int
        L.moe_decode_create.argtypes = [C.POINTER(moe_decode_config), C.POINTER(C.c_void_p)]
        L.moe_decode_run.restype = C.c_int
        L.moe_decode_run.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                                     C.c_void_p]
        L.moe_decode_run_static.restype = C.c_int
        L.moe_decode_run_static.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                            C.c_int32, C.c_void_p]
        L.moe_decode_destroy.restype = C.c_int
        L.moe_decode_destroy.argtypes = [C.c_void_p]
        L.moe_decode_last_error.restype = C.c_char_p
        L.moe_decode_last_error.argtypes = []
        L.moe_decode_query.restype = C.c_int
        L.moe_decode_query.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t]
        L.moe_decode_profile_events.restype = C.c_int
        L.moe_decode_profile_events.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p]
        _lib = L
    return _lib


def moe_decode_last_error():
    return lib().moe_decode_last_error().decode()


def _check(status):
    if status != MOE_OK:
        raise MoeDecodeError(status, moe_decode_last_error())
    return status


def moe_decode_create(cfg):
    """cfg: moe_decode_config. Returns the opaque handle (int)."""
    h = C.c_void_p()
    _check(lib().moe_decode_create(C.byref(cfg), C.byref(h)))
    return h.value


def moe_decode_run(h, x_ptr, logits_ptr, out_ptr, m, stream_ptr):
    """All pointers are device addresses (ints); stream_ptr a hipStream_t (int)."""
    return _check(lib().moe_decode_run(h, x_ptr, logits_ptr, out_ptr, m, stream_ptr))


def moe_decode_run_static(h, x_ptr, logits_ptr, out_ptr, m, stream_ptr):
    """moe_decode_run with the per-run buffers in the library's static scratch."""
    return _check(lib().moe_decode_run_static(h, x_ptr, logits_ptr, out_ptr, m, stream_ptr))


def moe_decode_destroy(h):
    return _check(lib().moe_decode_destroy(h))


def moe_decode_query(h, what, buf):
    """buf: a writable ctypes object or numpy array."""
    if hasattr(buf, "ctypes"):
        ptr, n = buf.ctypes.data, buf.nbytes
    else:
        ptr, n = C.addressof(buf), C.sizeof(buf)
    return _check(lib().moe_decode_query(h, what, ptr, n))


def moe_decode_profile_events(h, ev_begin_ptr, ev_end_ptr):
    return _check(lib().moe_decode_profile_events(h, ev_begin_ptr, ev_end_ptr))


from .device import DeviceLayer  # noqa: E402,F401
