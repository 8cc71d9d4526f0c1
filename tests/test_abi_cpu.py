"""The C ABI without a GPU: symbols, argument validation, error messages.

Every call here fails validation before the library touches the HIP runtime,
so nothing runs on a device. (CPU only.)
"""
import ctypes as C
import os
import re

import pytest

import bit_quantized_moe_block_amd as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_decode.h")

FAKE = 0x10000  # never dereferenced: validation fails first


def header_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char \*)\s*(moe_decode_\w+)\(", src,
                                 re.M)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert set(names) == set(B.EXPORTED)
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n


def test_probe_library_exports_every_declared_function():
    """include/moe_probe.h (measurement probes) against libmoeprobe.so."""
    src = open(os.path.join(ROOT, "include", "moe_probe.h")).read()
    names = sorted(set(re.findall(r"^\s*int\s+(moe_probe_\w+)\(", src, re.M)))
    assert names == ["moe_probe_compute_rate", "moe_probe_empty_kernels", "moe_probe_lds_read128",
                     "moe_probe_stream_read", "moe_probe_ticket_read", "moe_probe_tile_read"]
    L = C.CDLL(os.path.join(ROOT, "bit_quantized_moe_block_amd", "libmoeprobe.so"))
    for n in names:
        assert hasattr(L, n), n
    # validation before any HIP call: misaligned size, null pointers, no blocks
    L.moe_probe_stream_read.restype = C.c_int
    L.moe_probe_stream_read.argtypes = [C.c_void_p, C.c_size_t, C.c_int32, C.c_void_p,
                                        C.c_void_p]
    assert L.moe_probe_stream_read(FAKE, 17, 4, FAKE, None) < 0
    assert L.moe_probe_stream_read(None, 16, 4, FAKE, None) < 0
    assert L.moe_probe_stream_read(FAKE, 16, 0, FAKE, None) < 0
    L.moe_probe_compute_rate.restype = C.c_int
    L.moe_probe_compute_rate.argtypes = [C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                         C.c_void_p]
    assert L.moe_probe_compute_rate(4, 1, 1, FAKE, FAKE, None) < 0   # no such mode
    assert L.moe_probe_compute_rate(0, 0, 1, FAKE, FAKE, None) < 0   # no blocks
    assert L.moe_probe_compute_rate(0, 1, 1, None, FAKE, None) < 0   # no clock buffer
    L.moe_probe_ticket_read.restype = C.c_int
    L.moe_probe_ticket_read.argtypes = [C.c_void_p, C.c_size_t, C.c_int32, C.c_int32, C.c_void_p,
                                        C.c_void_p, C.c_void_p]
    assert L.moe_probe_ticket_read(FAKE, 65536 + 16, 4, 0, FAKE, FAKE, None) < 0  # not whole units
    assert L.moe_probe_ticket_read(FAKE, 65536, 4, 3, FAKE, FAKE, None) < 0       # no such mode
    assert L.moe_probe_ticket_read(FAKE, 65536, 4, 0, None, FAKE, None) < 0       # no counters
    import bench
    T = bench.ProbeTileStream
    assert C.sizeof(T) == 32
    L.moe_probe_tile_read.restype = C.c_int
    L.moe_probe_tile_read.argtypes = [C.POINTER(T), C.c_int32, C.c_void_p, C.c_int32, C.c_void_p,
                                      C.c_void_p]
    good = T(FAKE, FAKE, 128, 32, 3, 0)
    for bad in (T(FAKE, FAKE, 126, 32, 3, 0),   # tile rows not a multiple of 4
                T(FAKE, FAKE, 128, 12, 3, 0),   # groups not a multiple of 8
                T(FAKE, FAKE, 128, 32, 6, 0),   # a width the probe does not read
                T(None, FAKE, 128, 32, 3, 0),   # no codes
                T(FAKE, FAKE, 128, 32, 3, 5)):  # units_before not the running sum
        tab = (T * 2)(good, bad)
        tab[1].units_before = bad.units_before if bad.units_before else 32 * 4
        assert L.moe_probe_tile_read(tab, 2, FAKE, 4, FAKE, None) < 0
    assert L.moe_probe_tile_read((T * 1)(good), 0, FAKE, 4, FAKE, None) < 0        # no matrices
    assert L.moe_probe_tile_read((T * 1)(good), 1, None, 4, FAKE, None) < 0        # no device table


def test_header_constants_match_binding():
    src = open(HEADER).read()
    assert int(re.search(r"MOE_DECODE_ABI_VERSION (\d+)u", src).group(1)) == B.MOE_DECODE_ABI_VERSION
    for name, val in [("MOE_E_INVALID", -1), ("MOE_E_UNSUPPORTED", -2), ("MOE_E_HIP", -3),
                      ("MOE_E_NOMEM", -4), ("MOE_E_STREAM", -5), ("MOE_E_DEVICE", -6)]:
        assert re.search(rf"{name} = {val}", src), name
        assert getattr(B, name) == val
    assert C.sizeof(B.moe_tensor_desc) == 32
    assert C.sizeof(B.moe_decode_info) == 32
    assert C.sizeof(B.moe_decode_stats) == 24


def make_cfg(E=4, k=2, H=256, I=128, M=4, bits=2, fmt=B.MOE_FMT_CODEBOOK, **over):
    descs = (B.moe_tensor_desc * (3 * E))()
    for i in range(3 * E):
        descs[i].codes = FAKE
        descs[i].scales = FAKE
        descs[i].lut = FAKE if fmt == B.MOE_FMT_CODEBOOK else None
        descs[i].bits = bits
    cfg = B.moe_decode_config(B.MOE_DECODE_ABI_VERSION, fmt, E, k, H, I, M,
                              C.cast(descs, C.POINTER(B.moe_tensor_desc)), FAKE, FAKE)
    for key, v in over.items():
        setattr(cfg, key, v)
    cfg._keep = descs
    return cfg


def create_status(cfg):
    h = C.c_void_p()
    st = B.lib().moe_decode_create(C.byref(cfg) if cfg is not None else None, C.byref(h))
    assert h.value is None
    return st, B.moe_decode_last_error()


@pytest.mark.parametrize("over,status,msg", [
    (dict(abi_version=7), B.MOE_E_INVALID, "abi_version"),
    (dict(format=9), B.MOE_E_INVALID, "format"),
    (dict(num_experts=0), B.MOE_E_INVALID, "num_experts"),
    (dict(top_k=0), B.MOE_E_INVALID, "top_k"),
    (dict(top_k=5), B.MOE_E_INVALID, "top_k"),
    (dict(hidden=384), B.MOE_E_INVALID, "hidden"),
    (dict(inter=100), B.MOE_E_INVALID, "inter"),
    (dict(hidden=32768), B.MOE_E_UNSUPPORTED, "16384"),
    (dict(max_tokens=0), B.MOE_E_INVALID, "max_tokens"),
    (dict(max_tokens=513), B.MOE_E_UNSUPPORTED, "max_tokens"),
    (dict(signs_hidden=None), B.MOE_E_INVALID, "signs"),
])
def test_create_rejects_bad_config(over, status, msg):
    st, err = create_status(make_cfg(**over))
    assert st == status and msg in err


def test_create_rejects_too_many_experts_and_topk():
    assert create_status(make_cfg(E=300, k=2))[0] == B.MOE_E_UNSUPPORTED
    assert create_status(make_cfg(E=32, k=17))[0] == B.MOE_E_UNSUPPORTED


def test_create_rejects_bad_tensors():
    cfg = make_cfg(bits=4)
    assert create_status(cfg)[0] == B.MOE_E_INVALID
    cfg = make_cfg()
    cfg._keep[4].bits = 3           # expert 1 up differs from its gate
    st, err = create_status(cfg)
    assert st == B.MOE_E_INVALID and "different bits" in err
    cfg = make_cfg()
    cfg._keep[2].codes = None
    assert create_status(cfg)[0] == B.MOE_E_INVALID
    cfg = make_cfg()
    cfg._keep[0].lut = None
    assert "lut" in create_status(cfg)[1]
    cfg = make_cfg()
    cfg._keep[0].codes = FAKE + 4    # codes must be 16-byte aligned
    assert "misaligned" in create_status(cfg)[1]
    cfg = make_cfg(fmt=B.MOE_FMT_NVFP4, bits=4)
    cfg._keep[0].lut = FAKE
    assert "no lut" in create_status(cfg)[1]
    cfg = make_cfg()
    cfg.tensors = None
    assert create_status(cfg)[0] == B.MOE_E_INVALID


def test_null_arguments():
    L = B.lib()
    h = C.c_void_p()
    assert L.moe_decode_create(None, C.byref(h)) == B.MOE_E_INVALID
    cfg = make_cfg()
    assert L.moe_decode_create(C.byref(cfg), None) == B.MOE_E_INVALID
    assert L.moe_decode_run(None, FAKE, FAKE, FAKE, 1, None) == B.MOE_E_INVALID
    assert "handle" in B.moe_decode_last_error()
    assert L.moe_decode_destroy(None) == B.MOE_OK
    buf = (C.c_char * 64)()
    assert L.moe_decode_query(None, B.MOE_Q_INFO, buf, 64) == B.MOE_E_INVALID
    assert L.moe_decode_profile_events(None, None, None) == B.MOE_E_INVALID


def test_error_message_is_thread_local():
    import threading
    create_status(make_cfg(num_experts=0))
    seen = {}

    def other():
        seen["msg"] = B.moe_decode_last_error()
    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert "num_experts" in B.moe_decode_last_error()


def test_binding_raises_on_error():
    with pytest.raises(B.MoeDecodeError) as ei:
        B.moe_decode_create(make_cfg(top_k=0))
    assert ei.value.status == B.MOE_E_INVALID


def test_binding_is_marshalling_only():
    # The product path must not reach the CPU oracle or any fallback.
    pkg = os.path.join(ROOT, "bit_quantized_moe_block_amd")
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            src = open(os.path.join(pkg, f)).read()
            assert "oracle" not in src.replace("oracle/", ""), f
            assert "import oracle" not in src


def test_create_rejects_routed_six_bit_codes():
    # 6-bit codes are the shared expert's stored form only; a routed expert
    # with them is refused before any HIP call
    st, err = create_status(make_cfg(bits=6))
    assert st == B.MOE_E_UNSUPPORTED and "shared expert only" in err


def test_run_checks_pointer_arguments_before_the_handle():
    # The pointer checks come before the handle is read, so a handle value
    # that is never dereferenced is enough to reach them without a GPU.
    L = B.lib()
    fake_handle = C.c_void_p(FAKE)
    cases = [
        ((FAKE, FAKE, FAKE, -1), "m = -1"),
        ((None, FAKE, FAKE, 1), "NULL"),
        ((FAKE, None, FAKE, 1), "NULL"),
        ((FAKE, FAKE, None, 1), "NULL"),
        ((FAKE + 2, FAKE, FAKE, 1), "misaligned"),
        ((FAKE, FAKE + 2, FAKE, 1), "misaligned"),
        ((FAKE, FAKE, FAKE + 4, 1), "misaligned"),     # out needs 16-byte alignment
    ]
    for (x, lg, out, m), msg in cases:
        assert L.moe_decode_run(fake_handle, x, lg, out, m, None) == B.MOE_E_INVALID
        assert msg in B.moe_decode_last_error(), (x, lg, out, m)
    # m = 0 enqueues nothing and succeeds whatever the pointers
    assert L.moe_decode_run(fake_handle, None, None, None, 0, None) == B.MOE_OK


def test_device_layer_checks_run_arguments():
    import torch
    from bit_quantized_moe_block_amd import DeviceLayer
    layer = DeviceLayer.__new__(DeviceLayer)   # argument checks only: no handle, no device
    layer.H, layer.E, layer.handle = 256, 8, None
    x = torch.zeros(2, 256, dtype=torch.bfloat16)
    lg = torch.zeros(2, 8, dtype=torch.float32)
    out = torch.zeros(2, 256, dtype=torch.float32)
    with pytest.raises(TypeError, match="dtype"):
        layer._check_args(x.float(), lg, out, 2)
    with pytest.raises(TypeError, match="dtype"):
        layer._check_args(x, lg.double(), out, 2)
    with pytest.raises(ValueError, match="shape"):
        layer._check_args(x[:, :128], lg, out, 2)
    with pytest.raises(ValueError, match="shape"):
        layer._check_args(x, lg, out, 3)
    with pytest.raises(ValueError, match="contiguous"):
        layer._check_args(x, lg, torch.zeros(256, 2).t(), 2)
    with pytest.raises(ValueError, match="GPU"):
        layer._check_args(x, lg, out, 2)
    with pytest.raises(ValueError, match="< 0"):
        layer._check_args(x, lg, out, -1)
