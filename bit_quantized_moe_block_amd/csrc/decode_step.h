// The weight decode of one MFMA step (shared by the decode kernels and the
// compute-rate probe, which times exactly this instruction sequence).
// Codebook codes become fp16 through v_perm byte lookups of the per-tensor
// codebook; NVFP4 e2m1 codes through the hardware conversion.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Byte tables of the per-tensor codebook for v_perm lookups: tab[0] / tab[1]
// hold the low bytes of entries 0..3 / 4..7, tab[2] / tab[3] the high bytes.
// `raw` holds the codebook as stored (fp16 entries, little endian); a 2-bit
// codebook leaves raw[2], raw[3] zero.
__device__ __forceinline__ void lut_tables(const u32x4 raw, uint32_t (&tab)[4])
{
    tab[0] = __builtin_amdgcn_perm(raw[1], raw[0], 0x06040200u);
    tab[2] = __builtin_amdgcn_perm(raw[1], raw[0], 0x07050301u);
    tab[1] = __builtin_amdgcn_perm(raw[3], raw[2], 0x06040200u);
    tab[3] = __builtin_amdgcn_perm(raw[3], raw[2], 0x07050301u);
}

// Four codes, one per byte of t, to four fp16 values: two v_perm lookups
// give their low and high bytes, two more interleave them into fp16 pairs.
__device__ __forceinline__ void perm_lookup4(uint32_t t, const uint32_t (&tab)[4], uint32_t &o0,
                                             uint32_t &o1)
{
    const uint32_t l = __builtin_amdgcn_perm(tab[1], tab[0], t);
    const uint32_t h = __builtin_amdgcn_perm(tab[3], tab[2], t);
    o0 = __builtin_amdgcn_perm(h, l, 0x05010400u);
    o1 = __builtin_amdgcn_perm(h, l, 0x07030602u);
}

// The 8 fp16 B-operand values of MFMA step s (slot columns 8s..8s+7, natural
// order) from one lane's slot words. FMT 2 / 3: codebook bits; 4: NVFP4.
// K = 3, steps 0..2: byte b of word s holds the codes of columns 8s + b
// (bits 0-2) and 8s + 4 + b (bits 3-5); step 3: the low bits of columns
// 24 + b / 28 + b are bits 6-7 of byte b of word 0 / 1, their high bits
// bits 6 / 7 of byte b of word 2.
// K = 2: for word d = s/2 and shifts 2(s%2), 2(s%2)+1, byte b of
// t = (w_d >> 2 shift) & 3 is the code of column 16d + 4 shift + b.
// NVFP4: word s holds columns 8s..8s+7; e2m1 -> fp16 by the hardware
// conversion (unit scale), then the e4m3 block scale in fp16 (exact: at most
// 5 significant bits, inside the fp16 range).
template <int FMT, int W>
__device__ __forceinline__ half8 decode_step(const uint32_t (&w)[W], int s,
                                             const uint32_t (&tab)[4], half2v bscale)
{
    uint32_t o[4];
    if constexpr (FMT == 4) {
        const uint32_t x = w[s];
        o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 0) * bscale);
        o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 1) * bscale);
        o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 2) * bscale);
        o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 1.0f, 3) * bscale);
    } else if constexpr (FMT == 3) {
        uint32_t t0, t1;
        if (s < 3) {
            t0 = w[s] & 0x07070707u;
            t1 = (w[s] >> 3) & 0x07070707u;
        } else {
            t0 = ((w[0] >> 6) & 0x03030303u) | ((w[2] >> 4) & 0x04040404u);
            t1 = ((w[1] >> 6) & 0x03030303u) | ((w[2] >> 5) & 0x04040404u);
        }
        perm_lookup4(t0, tab, o[0], o[1]);
        perm_lookup4(t1, tab, o[2], o[3]);
    } else {
        const int d = s >> 1;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int sh = 2 * (s & 1) + hh;
            perm_lookup4((w[d] >> (2 * sh)) & 0x03030303u, tab, o[2 * hh], o[2 * hh + 1]);
        }
    }
    return __builtin_bit_cast(half8, u32x4{o[0], o[1], o[2], o[3]});
}

}  // namespace moe
