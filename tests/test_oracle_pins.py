"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what fixes the expected value: a library routine, a closed
form, an invariant, an exhaustive search or the independent dense brute force
of tests/brute.py.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from moe_synth import WORKLOADS, gen, small_workload
from tests import brute


# ------------------------------------------------------------ number formats

def test_f16_decoder_matches_numpy_all_patterns():
    # Library: numpy's IEEE binary16, every one of the 65536 patterns.
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_double(p) for p in pats])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(ref[~both_nan], got[~both_nan])
    assert np.array_equal(np.isnan(ref), np.isnan(got))


def test_bf16_decoder_matches_torch():
    # Library: torch.bfloat16 -> float64 on a sample of finite patterns.
    pats = np.unique(np.random.default_rng(0).integers(0, 65536, 4000)).astype(np.uint16)
    pats = pats[(pats & 0x7F80) != 0x7F80]
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_double(p) for p in pats])
    assert np.array_equal(ref, got)


def test_e2m1_table_closed_form():
    # OCP MX e2m1: magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}, sign in bit 3.
    got = np.array([oracle.e2m1_to_double(i) for i in range(16)])
    assert np.array_equal(got, brute.E2M1_VALUES)
    assert np.array_equal(np.signbit(got), np.signbit(brute.E2M1_VALUES))


def test_e4m3fn_table_matches_torch_all_codes():
    # Library: torch.float8_e4m3fn, all 256 codes (bias 7, subnormals, 0x7F/0xFF NaN, max 448).
    ref = brute.e4m3fn_table()
    got = np.array([oracle.e4m3fn_to_double(i) for i in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


# ------------------------------------------------------------ Hadamard rotation

def test_fwht_equals_closed_form_columns():
    # Closed form H[i][j] = (-1)^popcount(i & j): H e_j is column j, exactly.
    Hm = brute.hadamard128()
    for j in range(128):
        e = np.zeros(128)
        e[j] = 1.0
        assert np.array_equal(oracle.fwht128(e), Hm[:, j])


def test_fwht_special_vectors_and_involution():
    e0 = np.zeros(128)
    e0[0] = 1
    assert np.array_equal(oracle.fwht128(e0), np.ones(128))            # H e0 = 1
    assert np.array_equal(oracle.fwht128(np.ones(128)), 128 * e0)      # H 1 = 128 e0
    v = np.random.default_rng(1).integers(-50, 50, 128).astype(np.float64)
    assert np.array_equal(oracle.fwht128(oracle.fwht128(v)), 128 * v)  # H H^T = 128 I
    Hm = brute.hadamard128()
    assert np.array_equal(Hm @ Hm.T, 128 * np.eye(128))


@pytest.mark.parametrize("n", [128, 256, 4096])
def test_rotation_dense_and_roundtrip(n):
    rng = np.random.default_rng(n)
    s = np.where(rng.integers(0, 2, n) == 1, 1, -1).astype(np.int8)
    v = rng.standard_normal(n)
    r = oracle.rotate(v, s)
    if n <= 256:
        assert np.allclose(r, brute.rotation_matrix(s) @ v, rtol=0, atol=1e-13)
    assert abs(np.linalg.norm(r) - np.linalg.norm(v)) < 1e-12 * np.linalg.norm(v)
    assert np.max(np.abs(oracle.unrotate(r, s) - v)) < 1e-12
    # fp32 round trip (the rotation applied in float32 arithmetic) within 1e-6.
    R = brute.rotation_matrix(s[:128]).astype(np.float32)
    v32 = v[:128].astype(np.float32)
    assert np.max(np.abs(R.T @ (R @ v32) - v32)) < 1e-6


# ------------------------------------------------------------ stored layouts

@pytest.mark.parametrize("bits", [2, 3, 6])
@pytest.mark.parametrize("shape", [(16, 128), (32, 256), (48, 384)])
def test_codebook_layout_matches_unpackbits_decoder(bits, shape):
    N, C = shape
    words = np.random.default_rng(bits * 7 + N).integers(0, 2 ** 32, N * C * bits // 32,
                                                         dtype=np.uint64).astype(np.uint32)
    ref = brute.codebook_codes(words, bits, N, C)
    rng = np.random.default_rng(3)
    for n, c in zip(rng.integers(0, N, 400), rng.integers(0, C, 400)):
        assert oracle.codebook_code(bits, N, C, words, int(n), int(c)) == ref[n, c]


def test_codebook_layout_hand_values():
    # Hand-derived from the layout definition (tiles of 16x128, slot l = row
    # l mod 16 / columns 32 (l div 16)..+31, K words per slot).
    N, C = 16, 128
    # K = 2: low bits of column kk of word d at bit 8 (kk mod 4) + 2 (kk div 4):
    # a slot word 0xFFAA5500 holds code kk mod 4 for kk = 0..15 (byte b
    # repeats code b).
    words = np.zeros(N * C * 2 // 32, np.uint32)
    words[0] = 0xFFAA5500          # slot 0 (row 0, cols 0..15)
    words[1] = 0x000000FF          # slot 0, cols 16..31: code 3 at kk = 0,4,8,12
    words[2 * 17] = 0x00000003     # slot 17 = row 1, cols 32..47: col 32 has code 3
    got = [oracle.codebook_code(2, N, C, words, 0, c) for c in range(32)]
    assert got[:16] == [c % 4 for c in range(16)]
    assert got[16:] == [3 if kk % 4 == 0 else 0 for kk in range(16)]
    assert oracle.codebook_code(2, N, C, words, 1, 32) == 3
    assert oracle.codebook_code(2, N, C, words, 1, 33) == 0
    # K = 3: word d < 3, byte b: bits 0-2 = column 8d + b, bits 3-5 = column
    # 8d + 4 + b; bits 6-7 of words 0 / 1 = low bits of columns 24 + b /
    # 28 + b, whose high bits are bits 6 / 7 of byte b of word 2.
    w3 = np.zeros(N * C * 3 // 32, np.uint32)
    w3[0] = 0x00003800             # byte 1 bits 3-5 -> column 5 = 7
    w3[1] = 0x00000040             # byte 0 bit 6 -> column 28, bit 0
    w3[2] = 0x80000007             # byte 0 bits 0-2 -> column 16 = 7; bit 31 -> column 31, bit 2
    got = [oracle.codebook_code(3, N, C, w3, 0, c) for c in range(128)]
    want = [0] * 128
    want[5], want[16], want[28], want[31] = 7, 7, 1, 4
    assert got == want
    # K = 6: column jj at bits 6 jj .. 6 jj + 5 of the slot's 192-bit string.
    # Column 0 = bits 0-5 of word 0; column 5 straddles words 0 and 1 (bits 30,
    # 31 of word 0 are its code bits 0, 1); column 31 = bits 26-31 of word 5.
    # A 6-bit tile holds words 0..2 of its 64 slots, then words 3..5: word d of
    # slot 0 is stored word (d div 3) * 192 + d mod 3.
    w6 = np.zeros(N * C * 6 // 32, np.uint32)
    w6[0] = 0x8000002A             # column 0 = 0b101010 = 42; word 0 bit 31 -> column 5 bit 1
    w6[1] = 0x00000005             # word 1 bits 0, 2 -> column 5 bits 2, 4
    w6[192 + 2] = 0xFC000000       # slot 0 word 5: column 31 = 63
    w6[3 * 17] = 0x00000001        # slot 17 (row 1, cols 32..63) word 0: col 32 = 1
    assert oracle.codebook_code(6, N, C, w6, 1, 32) == 1
    got = [oracle.codebook_code(6, N, C, w6, 0, c) for c in range(128)]
    want = [0] * 128
    want[0], want[5], want[31] = 42, 2 + 4 + 16, 63
    assert got == want


@pytest.mark.parametrize("bits", [2, 3, 6])
def test_codebook_layout_is_a_bijection(bits):
    # Every bit of a slot's K words belongs to exactly one code bit: setting
    # one stored bit changes exactly one code, by exactly one power of two.
    N, C = 16, 128
    seen = set()
    for d in range(bits):
        for bit in range(32):
            words = np.zeros(N * C * bits // 32, np.uint32)
            # word d of slot 0 (row 0, columns 0..31); a 6-bit tile stores
            # words 0..2 of its slots, then words 3..5
            at = (d // 3) * 192 + d % 3 if bits == 6 else d
            words[at] = np.uint32(1 << bit)
            codes = [oracle.codebook_code(bits, N, C, words, 0, c) for c in range(32)]
            nz = [(c, v) for c, v in enumerate(codes) if v]
            assert len(nz) == 1 and bin(nz[0][1]).count("1") == 1, (d, bit, nz)
            seen.add(nz[0])
    assert len(seen) == 32 * bits


@pytest.mark.parametrize("bits", [2, 3, 6])
def test_codebook_roundtrip_exact_weights(bits):
    # Weights that the format represents exactly: w = LUT[c] * s. Encode by
    # nearest entry, pack independently, decode with the oracle: bitwise equal.
    N, C = 32, 256
    rng = np.random.default_rng(11)
    lut = np.sort(rng.standard_normal(1 << bits)).astype(np.float16)
    sc = rng.uniform(0.01, 0.05, (N, C // 128)).astype(np.float16)
    codes = rng.integers(0, 1 << bits, (N, C))
    W = lut.astype(np.float64)[codes] * np.repeat(sc.astype(np.float64), 128, axis=1)
    enc = np.argmin(np.abs(W[..., None] / np.repeat(sc.astype(np.float64), 128, axis=1)[..., None]
                           - lut.astype(np.float64)[None, None, :]), axis=-1)
    assert np.array_equal(enc, codes)
    words = brute.pack_codebook(enc, bits)
    L = oracle.Layer("codebook", 1, 1, C, N, [bits],
                     {(0, 0): dict(codes=words, scales=brute.pack_codebook_scales(sc), lut=lut)})
    assert np.array_equal(L.dequant(0, 0), W)


@pytest.mark.parametrize("shape", [(16, 128), (32, 384)])
def test_nvfp4_layout_matches_independent_decoder(shape):
    N, C = shape
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, N * C // 2).astype(np.uint8)
    ref = brute.nvfp4_codes(codes, N, C)
    for n, c in zip(rng.integers(0, N, 400), rng.integers(0, C, 400)):
        assert oracle.nvfp4_code(N, C, codes, int(n), int(c)) == ref[n, c]
    # hand value: slot 16 (row 0, cols 32..63), byte 0 = 0x5A -> col 32 = 0xA, col 33 = 0x5
    c2 = np.zeros(N * C // 2, np.uint8)
    c2[16 * 16] = 0x5A
    assert oracle.nvfp4_code(N, C, c2, 0, 32) == 0xA
    assert oracle.nvfp4_code(N, C, c2, 0, 33) == 0x5


def test_dequant_matches_dense_decoders():
    w = small_workload("t", 4, 2, 256, 128, bits_mix="alternate")
    case = gen.make_case(w, 1)
    L = oracle.Layer.from_case(case)
    for e in range(4):
        for p in range(3):
            N, C = L.shape(p)
            assert np.array_equal(L.dequant(e, p), brute.dense_codebook(case["tensors"][(e, p)], N, C))
    wn = small_workload("n", 2, 1, 256, 128, fmt="nvfp4", bits_mix="nvfp4")
    cn = gen.make_case(wn, 1)
    Ln = oracle.Layer.from_case(cn)
    for p in range(3):
        N, C = Ln.shape(p)
        assert np.array_equal(Ln.dequant(1, p), brute.dense_nvfp4(cn["tensors"][(1, p)], N, C))


# ------------------------------------------------------------ router and buckets

def test_route_matches_subset_enumeration():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((6, 8)).astype(np.float32)
    ids, w = oracle.route(logits, 2)
    rid, rw = brute.route_enumerate(logits, 2)
    assert np.array_equal(ids, rid)
    assert np.max(np.abs(w - rw)) < 1e-12


def test_route_matches_stable_argsort_and_sums_to_one():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((24, 256)).astype(np.float32)
    logits[:, 7] = logits[:, 3]             # exact ties: lower id first
    logits[0, :] = 0.0                      # all-equal row
    ids, w = oracle.route(logits, 8)
    ref = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :8]
    assert np.array_equal(ids, ref)
    assert np.array_equal(ids[0], np.arange(8))
    assert np.max(np.abs(w.sum(1) - 1)) < 1e-12
    full = np.exp(logits.astype(np.float64) - logits.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    ren = np.take_along_axis(full, ids, 1)
    ren /= ren.sum(1, keepdims=True)
    assert np.max(np.abs(ren - w)) < 1e-12


def test_bucket_matches_numpy():
    rng = np.random.default_rng(4)
    for m, E, k in [(1, 8, 2), (24, 256, 8), (5, 16, 3), (300, 16, 4), (512, 256, 8)]:
        logits = rng.standard_normal((m, E)).astype(np.float32)
        ids, _ = oracle.route(logits, k)
        b = oracle.bucket(ids, E)
        assert np.array_equal(b["counts"], np.bincount(ids.reshape(-1), minlength=E))
        assert np.array_equal(b["offsets"], np.concatenate([[0], np.cumsum(b["counts"])]))
        tt, jj = np.meshgrid(np.arange(m), np.arange(k), indexing="ij")
        order = np.lexsort((tt.reshape(-1), ids.reshape(-1)))
        assert np.array_equal(b["rows_t"], tt.reshape(-1)[order])
        assert np.array_equal(b["rows_j"], jj.reshape(-1)[order])
        assert np.array_equal(b["pos"].reshape(-1)[order], np.arange(m * k))


# ------------------------------------------------------------ the layer

LAYER_SHAPES = [
    small_workload("cb_a", 8, 2, 256, 128, bits_mix="all2", config_id=201),
    small_workload("cb_b", 6, 3, 256, 256, bits_mix="alternate", config_id=202),
    small_workload("cb_c", 4, 2, 384, 128, bits_mix="alternate", config_id=203),
    small_workload("fp4", 6, 2, 256, 128, fmt="nvfp4", bits_mix="nvfp4", config_id=204),
    # with an always-on shared expert (6-bit, and 2-bit for a second width)
    small_workload("sh6", 6, 2, 256, 128, bits_mix="alternate", config_id=205, shared_bits=6),
    small_workload("sh2", 8, 3, 256, 256, bits_mix="all2", config_id=206, shared_bits=2),
]


@pytest.mark.parametrize("w", LAYER_SHAPES, ids=lambda w: w.name)
@pytest.mark.parametrize("m", [1, 3])
def test_layer_matches_plain_basis_brute_force(w, m):
    case = gen.make_case(w, m)
    r = oracle.Layer.from_case(case).run(case["x"], case["logits"])
    ref = brute.layer_plain(case)
    assert np.max(np.abs(r["out"] - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_tiny_workload_matches_brute_force():
    case = gen.make_case(WORKLOADS["tiny"], 1)
    r = oracle.Layer.from_case(case).run(case["x"], case["logits"])
    ref = brute.layer_plain(case)
    assert np.max(np.abs(r["out"] - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_shared_expert_adds_its_ffn_with_weight_one():
    # The shared expert's output is added with weight 1 to every token: the
    # difference between the layer with and without it is that expert's FFN,
    # here computed by the plain-basis brute force on its own.
    w = LAYER_SHAPES[4]
    case = gen.make_case(w, 3)
    with_sh = oracle.Layer.from_case(case).run(case["x"], case["logits"])["out"]
    no_sh = oracle.Layer.from_case(dict(case, shared=None, shared_bits=0)).run(
        case["x"], case["logits"])["out"]
    only = brute.shared_plain(case)
    assert np.max(np.abs((with_sh - no_sh) - only)) <= 1e-12 * np.max(np.abs(only))
    assert np.max(np.abs(only)) > 0


@pytest.mark.parametrize("fmt", ["codebook", "nvfp4"])
def test_zero_input_gives_exact_zero(fmt):
    w = LAYER_SHAPES[0] if fmt == "codebook" else LAYER_SHAPES[3]
    case = gen.make_case(w, 2)
    case["x"] = np.zeros_like(case["x"])
    r = oracle.Layer.from_case(case).run(case["x"], case["logits"])
    assert np.all(r["out"] == 0.0)


def test_token_permutation_permutes_outputs_exactly():
    w = LAYER_SHAPES[1]
    case = gen.make_case(w, 5)
    L = oracle.Layer.from_case(case)
    r = L.run(case["x"], case["logits"])
    perm = np.array([3, 0, 4, 1, 2])
    rp = L.run(case["x"][perm], case["logits"][perm])
    assert np.array_equal(rp["out"], r["out"][perm])


def test_token_subset_equals_full_run():
    w = LAYER_SHAPES[1]
    case = gen.make_case(w, 4)
    L = oracle.Layer.from_case(case)
    full = L.run(case["x"], case["logits"])
    sub = L.run(case["x"], case["logits"], tokens=[1, 3])
    assert np.array_equal(sub["out"][[1, 3]], full["out"][[1, 3]])
    assert np.all(np.isnan(sub["out"][[0, 2]]))


def test_single_expert_top1_is_textbook_swiglu():
    # k = 1 of E = 1, NVFP4 (no rotation): out = Wd (silu(Wg x) * (Wu x)).
    w = small_workload("one", 1, 1, 256, 128, fmt="nvfp4", bits_mix="nvfp4", config_id=205)
    case = gen.make_case(w, 2)
    L = oracle.Layer.from_case(case)
    r = L.run(case["x"], case["logits"])
    assert np.all(r["w"] == 1.0)
    x = brute.bf16_to_f64(case["x"])
    Wg = brute.dense_nvfp4(case["tensors"][(0, 0)], 128, 256)
    Wu = brute.dense_nvfp4(case["tensors"][(0, 1)], 128, 256)
    Wd = brute.dense_nvfp4(case["tensors"][(0, 2)], 256, 128)
    g, u = x @ Wg.T, x @ Wu.T
    ref = (g / (1 + np.exp(-g)) * u) @ Wd.T
    assert np.max(np.abs(r["out"] - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_constant_codebook_closed_form():
    # Every gate code maps to the same value c with group scale s. Then
    # g_n = c s sum_j x~_j = c s sqrt(128) sum_b s_H[128 b] x[128 b]
    # (column sums of H_128 vanish except column 0).
    w = small_workload("const", 2, 1, 512, 128, bits_mix="all2", config_id=206)
    case = gen.make_case(w, 1)
    c, s = 0.75, 0.03125
    t = case["tensors"][(0, 0)]
    t["lut"] = np.full(4, c, np.float16)
    t["scales"] = np.full_like(t["scales"], s)
    L = oracle.Layer.from_case(case)
    x = brute.bf16_to_f64(case["x"][0])
    xr = oracle.rotate(x, case["signs_hidden"])
    Wg = L.dequant(0, 0)
    g = Wg @ xr
    sh = case["signs_hidden"].astype(np.float64)
    closed = c * s * np.sqrt(128.0) * sum(sh[b] * x[b] for b in range(0, 512, 128))
    assert np.max(np.abs(g - closed)) < 1e-12 * max(1.0, abs(closed))


def test_oracle_catches_planted_mistakes():
    # The brute force must fail when the oracle's inputs are perturbed in the
    # ways a plausible bug would perturb them (sign flip, transposed signs,
    # swapped gate/up): guards that the pins above have power.
    w = LAYER_SHAPES[0]
    case = gen.make_case(w, 2)
    ref = brute.layer_plain(case)
    bad = dict(case)
    bad["signs_hidden"] = case["signs_hidden"].copy()
    bad["signs_hidden"][5] *= -1
    r = oracle.Layer.from_case(bad).run(case["x"], case["logits"])
    assert np.max(np.abs(r["out"] - ref)) > 1e-6 * np.max(np.abs(ref))
    bad = dict(case)
    bad["tensors"] = dict(case["tensors"])
    for e in range(w.num_experts):
        bad["tensors"][(e, 0)], bad["tensors"][(e, 1)] = case["tensors"][(e, 1)], case["tensors"][(e, 0)]
    r = oracle.Layer.from_case(bad).run(case["x"], case["logits"])
    assert np.max(np.abs(r["out"] - ref)) > 1e-6 * np.max(np.abs(ref))
