"""Independent numpy brute force used to pin the oracle (tests only).

Written separately from oracle/moe_oracle.c: the stored layouts are decoded
with numpy.unpackbits and index tables instead of per-element shifts, the
rotation is a dense matrix built from the closed form
H_128[i][j] = (-1)^popcount(i & j), and the layer is evaluated in the plain
basis (W_plain = W_stored R) on unrotated activations.
"""
import itertools

import numpy as np
import torch

# ----------------------------------------------------------- closed forms

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                        -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def hadamard128():
    i = np.arange(128)
    a = i[:, None] & i[None, :]
    pc = np.zeros_like(a)
    for b in range(7):
        pc += (a >> b) & 1
    return np.where(pc % 2 == 0, 1.0, -1.0)


def rotation_matrix(signs):
    """Dense R = (1/sqrt(128)) blockdiag(H_128 diag(s_block))."""
    n = len(signs)
    Hm = hadamard128()
    R = np.zeros((n, n))
    for b in range(0, n, 128):
        R[b:b + 128, b:b + 128] = Hm * np.asarray(signs[b:b + 128], np.float64)[None, :]
    return R / np.sqrt(128.0)


def e4m3fn_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------- layouts

def _byte_contents(bits):
    """What each byte of a slot holds, byte by byte: for word d and byte b,
    a list of (bit-in-byte, column, code bit). The opposite view from the
    oracle's column-by-column positions."""
    out = {}
    if bits == 6:
        # the slot as a 192-bit string: string bit q is bit q mod 8 of byte q div 8
        # (word q div 32, byte (q div 8) mod 4), and code bit q mod 6 of column q div 6
        for q in range(192):
            out.setdefault((q // 32, (q // 8) % 4), []).append((q % 8, q // 6, q % 6))
        return out
    for b in range(4):
        if bits == 3:
            for d in range(3):
                # two whole 3-bit codes: columns 8d + b and 8d + 4 + b
                out[d, b] = ([(k, 8 * d + b, k) for k in range(3)]
                             + [(3 + k, 8 * d + 4 + b, k) for k in range(3)])
            # bits 6-7: the two low bits of column 24 + b (word 0) / 28 + b
            # (word 1); word 2 keeps their high bits
            out[0, b] += [(6, 24 + b, 0), (7, 24 + b, 1)]
            out[1, b] += [(6, 28 + b, 0), (7, 28 + b, 1)]
            out[2, b] += [(6, 24 + b, 2), (7, 28 + b, 2)]
        else:
            for d in range(2):
                out[d, b] = [(2 * sh + k, 16 * d + 4 * sh + b, k) for sh in range(4) for k in range(2)]
    return out


def _slot_bit_tables(bits):
    """For slot column jj (0..31): (word, bit) of each code bit, LSB first."""
    tab = [[None] * bits for _ in range(32)]
    for (d, b), items in _byte_contents(bits).items():
        for bit_in_byte, col, sig in items:
            assert tab[col][sig] is None
            tab[col][sig] = (d, 8 * b + bit_in_byte)
    assert all(e is not None for entry in tab for e in entry)
    return tab


def _slot_words(words, bits, ntiles):
    """[tile, slot, word] view of the stored words: slot-major, except that a
    6-bit tile holds words 0..2 of its 64 slots, then words 3..5."""
    w = np.asarray(words, np.uint32)
    if bits == 6:
        return w.reshape(ntiles, 2, 64, 3).transpose(0, 2, 1, 3).reshape(ntiles, 64, 6)
    return w.reshape(ntiles, 64, bits)


def codebook_codes(words, bits, N, C):
    """Code matrix [N, C] from the tiled stored words (numpy.unpackbits)."""
    RB, G = N // 16, C // 128
    w = np.ascontiguousarray(_slot_words(words, bits, RB * G))
    b = np.unpackbits(w.view(np.uint8).reshape(RB * G, 64, bits, 4), axis=-1, bitorder="little")
    b = b.reshape(RB * G, 64, bits, 32)  # [tile, slot, word, bit]
    codes = np.zeros((RB * G, 64, 32), np.int64)
    for jj, entry in enumerate(_slot_bit_tables(bits)):
        for sig, (wd, bt) in enumerate(entry):
            codes[:, :, jj] |= b[:, :, wd, bt].astype(np.int64) << sig
    # [rb, g, q, r, jj] -> [rb, r, g, q, jj]
    codes = codes.reshape(RB, G, 4, 16, 32).transpose(0, 3, 1, 2, 4)
    return codes.reshape(N, C)


def pack_codebook(codes, bits):
    """Inverse of codebook_codes: tiled words from a code matrix [N, C]."""
    codes = np.asarray(codes, np.int64)
    N, C = codes.shape
    RB, G = N // 16, C // 128
    c5 = codes.reshape(RB, 16, G, 4, 32).transpose(0, 2, 3, 1, 4).reshape(RB * G, 64, 32)
    b = np.zeros((RB * G, 64, bits, 32), np.uint8)
    for jj, entry in enumerate(_slot_bit_tables(bits)):
        for sig, (wd, bt) in enumerate(entry):
            b[:, :, wd, bt] = (c5[:, :, jj] >> sig) & 1
    by = np.packbits(b.reshape(RB * G, 64, bits, 4, 8), axis=-1, bitorder="little")
    w = by.reshape(RB * G, 64, bits * 4).view(np.uint32)          # [tile, slot, word]
    if bits == 6:
        w = w.reshape(RB * G, 64, 2, 3).transpose(0, 2, 1, 3)     # [tile, half, slot, word]
    return np.ascontiguousarray(w).reshape(-1).copy()


def codebook_scales(scales, N, C):
    """Scale matrix [N, C // 128] (fp64) from the stored fp16 scales: per
    16 x 128 tile (tile order), the tile's 16 row scales."""
    RB, G = N // 16, C // 128
    s = np.asarray(scales, np.float16).astype(np.float64).reshape(RB, G, 16)
    return s.transpose(0, 2, 1).reshape(N, G)


def pack_codebook_scales(sc):
    """Stored order of a scale matrix [N, C // 128]."""
    N, G = sc.shape
    return np.ascontiguousarray(sc.reshape(N // 16, 16, G).transpose(0, 2, 1)).reshape(-1)


def dense_codebook(t, N, C):
    codes = codebook_codes(t["codes"], t["bits"], N, C)
    lut = np.asarray(t["lut"], np.float16).astype(np.float64)
    return lut[codes] * np.repeat(codebook_scales(t["scales"], N, C), 128, axis=1)


def nvfp4_codes(codes, N, C):
    RB, G = N // 16, C // 128
    by = np.asarray(codes, np.uint8).reshape(RB * G, 64, 16)
    nib = np.stack([by & 0xF, by >> 4], axis=-1).reshape(RB * G, 64, 32)
    return nib.reshape(RB, G, 4, 16, 32).transpose(0, 3, 1, 2, 4).reshape(N, C)


def dense_nvfp4(t, N, C):
    RB, G = N // 16, C // 128
    vals = E2M1_VALUES[nvfp4_codes(t["codes"], N, C)]
    # stored per 16 x 128 tile (tile order), a tile's 16 x 8 scales row-major
    sc = e4m3fn_table()[np.asarray(t["scales"], np.uint8)].reshape(RB, G, 16, 8)
    sc = sc.transpose(0, 2, 1, 3).reshape(N, C // 16)
    return vals * np.repeat(sc, 16, axis=1) * float(np.float32(t["tensor_scale"]))


def dense(fmt, t, N, C):
    return dense_codebook(t, N, C) if fmt == "codebook" else dense_nvfp4(t, N, C)


# ----------------------------------------------------------- router

def route_enumerate(logits, k):
    """Top-k by exhaustive subset search: the selected set maximises the sum of
    logits over all k-subsets; slots are ordered by logit (desc), then id.
    Weights: full softmax over all experts, renormalised over the set."""
    m, E = logits.shape
    ids = np.zeros((m, k), np.int64)
    w = np.zeros((m, k))
    for t in range(m):
        l = logits[t].astype(np.float64)
        best = max(itertools.combinations(range(E), k), key=lambda s: (sum(l[list(s)]), [-e for e in s]))
        order = sorted(best, key=lambda e: (-l[e], e))
        ids[t] = order
        p = np.exp(l - l.max())
        p /= p.sum()
        w[t] = p[order] / p[order].sum()
    return ids, w


# ----------------------------------------------------------- layer

def silu(z):
    return z / (1.0 + np.exp(-z))


def layer_plain(case, ids=None, w=None):
    """Whole step in the plain basis with dense fp64 matrices."""
    wl = case["workload"]
    H, I, k = wl.hidden, wl.inter, wl.top_k
    x = bf16_to_f64(case["x"])
    if ids is None:
        ids, w = route_enumerate(case["logits"], k)
    if wl.fmt == "codebook":
        RH = rotation_matrix(case["signs_hidden"])
        RI = rotation_matrix(case["signs_inter"])
    else:
        RH, RI = np.eye(H), np.eye(I)
    out = np.zeros((x.shape[0], H))
    cache = {}
    for t in range(x.shape[0]):
        for j in range(k):
            e = int(ids[t, j])
            if e not in cache:
                Wg = dense(wl.fmt, case["tensors"][(e, 0)], I, H) @ RH
                Wu = dense(wl.fmt, case["tensors"][(e, 1)], I, H) @ RH
                Wd = dense(wl.fmt, case["tensors"][(e, 2)], H, I) @ RI
                cache[e] = (Wg, Wu, Wd)
            Wg, Wu, Wd = cache[e]
            y = Wd @ (silu(Wg @ x[t]) * (Wu @ x[t]))
            out[t] += w[t, j] * y
    if case.get("shared"):
        out += shared_plain(case)
    return out


def shared_plain(case):
    """The shared expert's FFN of every token, plain basis, dense fp64."""
    wl = case["workload"]
    H, I = wl.hidden, wl.inter
    x = bf16_to_f64(case["x"])
    RH = rotation_matrix(case["signs_hidden"])
    RI = rotation_matrix(case["signs_inter"])
    sh = case["shared"]
    Wg = dense(wl.fmt, sh[0], I, H) @ RH
    Wu = dense(wl.fmt, sh[1], I, H) @ RH
    Wd = dense(wl.fmt, sh[2], H, I) @ RI
    return np.stack([Wd @ (silu(Wg @ x[t]) * (Wu @ x[t])) for t in range(x.shape[0])])
