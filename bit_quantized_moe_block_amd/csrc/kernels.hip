// gfx950 kernels of the routed-experts decode step.
//
// route_kernel   one block per token: top-k on the raw logits, softmax over
//                the selected logits, block-Hadamard rotation of x (codebook)
//                or bf16->fp16 (NVFP4). The last block to finish builds the
//                per-expert row buckets and the work plan, and resets the
//                expert kernel's counters (so every run and every graph
//                replay starts clean without a memset).
// expert_kernel  persistent grid pulling work-item tickets, no grid-wide
//                barrier. Gate/up items (one hit expert, 128 rows of gate and
//                of up, one column split) write partial sums; the last split
//                of a 128-row block finishes SiLU(g)*u and the 128-point
//                rotation of h. Down items (256 rows of down, one column
//                split) wait on a per-expert counter of finished h blocks.
//                Inner loop: codes decoded in registers through v_perm byte
//                lookups of the per-tensor codebook, MFMA 16x16x32 f16 with
//                the tokens as the A operand, fp32 group-scale FMAs.
// combine_kernel out[t] = sum_j w[t][j] * y[t][j] in slot order.
//
// Page "LNA-CANON.md", section "lna2 とは": resident expert teams with
// dynamic tickets and no grid-wide barrier, small-R inner loops for
// R_e in {1,2,4,8} at m <= 24, bitwise reproducible results; page
// "lna-lab/README.md", section "2026-09-04 -- house kernel lna2".
#include "moe_internal.h"

namespace moe {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kInvSqrt128 = 0.08838834764831845f;

__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t *p, uint32_t v)
{
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_load_agent(uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_agent(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// In-wave 128-point Walsh-Hadamard transform (Sylvester order) of the pair
// (v0, v1) = elements (2 lane, 2 lane + 1): bit 0 inside the lane, bits 1..6
// across lanes with xor shuffles.
__device__ __forceinline__ void wave_fwht128(float &v0, float &v1)
{
    const int lane = threadIdx.x & 63;
    float a = v0 + v1, b = v0 - v1;
    v0 = a;
    v1 = b;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
        float p0 = __shfl_xor(v0, sh), p1 = __shfl_xor(v1, sh);
        if (lane & sh) {
            v0 = p0 - v0;
            v1 = p1 - v1;
        } else {
            v0 = v0 + p0;
            v1 = v1 + p1;
        }
    }
}

// ---------------------------------------------------------------------------
// Route
// ---------------------------------------------------------------------------

// Total order for the top-k: larger logit first, equal logits -> lower id.
// Monotone float bits in the high word, inverted id in the low word; 0 is
// below every real key and marks "not available". -0 is folded into +0.
__device__ __forceinline__ uint64_t route_key(float v, int e)
{
    if (v == 0.0f)
        v = 0.0f;
    uint32_t u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m)
{
    uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

// Exclusive block-wide scan of one int per thread (256 threads).
__device__ __forceinline__ int block_excl_scan(int v, int *tmp4, int &total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(x, off);
        if (lane >= off)
            x += y;
    }
    if (lane == 63)
        tmp4[wave] = x;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w)
        base += tmp4[w];
    total = tmp4[0] + tmp4[1] + tmp4[2] + tmp4[3];
    __syncthreads();
    return base + x - v;
}

__global__ __launch_bounds__(kThreads) void route_kernel(Params p, const uint16_t *__restrict__ x,
                                                         const float *__restrict__ logits, int m)
{
    __shared__ uint64_t red[4];
    __shared__ int sel[kMaxTopK];
    __shared__ int s_last;
    __shared__ int s_ids[kMaxPairs];
    __shared__ int tmp4[4];
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = p.E, k = p.k, H = p.H;

    // ---- top-k by k rounds of a block-wide max over route keys
    uint64_t key = 0;
    if (tid < E)
        key = route_key(logits[(size_t)t * E + tid], tid);
    for (int j = 0; j < k; ++j) {
        uint64_t b = key;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            uint64_t o = shfl_xor_u64(b, off);
            b = o > b ? o : b;
        }
        if (lane == 0)
            red[wave] = b;
        __syncthreads();
        b = red[0];
        for (int w = 1; w < 4; ++w)
            b = red[w] > b ? red[w] : b;
        const int e = (int)(0xFFFFFFFFu - (uint32_t)b);
        if (tid == 0)
            sel[j] = e;
        if (tid == e)
            key = 0;
        __syncthreads();
    }
    // ---- weights: softmax over the k selected logits, slot order
    if (tid == 0) {
        const float *l = logits + (size_t)t * E;
        const float l0 = l[sel[0]];
        float den = 0.0f;
        for (int j = 0; j < k; ++j)
            den += expf(l[sel[j]] - l0);
        for (int j = 0; j < k; ++j) {
            p.ids[t * k + j] = sel[j];
            p.wts[t * k + j] = expf(l[sel[j]] - l0) / den;
        }
    }
    // ---- activations: rotated fp16 (codebook) or plain fp16 (NVFP4)
    const uint32_t *xw = (const uint32_t *)(x + (size_t)t * H);
    half2v *xo = (half2v *)(p.xr + (size_t)t * H);
    if (p.format == kFmtCodebook) {
        for (int b = wave; b < H / 128; b += 4) {
            const int c0 = b * 128 + 2 * lane;
            const uint32_t xx = xw[c0 / 2];
            float v0 = bf16_to_f32(xx & 0xFFFFu) * (float)p.signs_h[c0];
            float v1 = bf16_to_f32(xx >> 16) * (float)p.signs_h[c0 + 1];
            wave_fwht128(v0, v1);
            xo[c0 / 2] = half2v{(_Float16)(v0 * kInvSqrt128), (_Float16)(v1 * kInvSqrt128)};
        }
    } else {
        for (int c = tid; c < H / 2; c += kThreads) {
            const uint32_t xx = xw[c];
            xo[c] = half2v{(_Float16)bf16_to_f32(xx & 0xFFFFu), (_Float16)bf16_to_f32(xx >> 16)};
        }
    }

    // ---- the last block builds buckets and the plan
    __threadfence();
    __syncthreads();
    if (tid == 0)
        s_last = atomic_add_agent(&p.ctr->route_done, 1u) == (uint32_t)(m - 1);
    __syncthreads();
    if (!s_last)
        return;
    __threadfence();
    const int np = m * k;
    for (int i = tid; i < np; i += kThreads)
        s_ids[i] = p.ids[i];
    __syncthreads();
    int cnt = 0;
    if (tid < E)
        for (int i = 0; i < np; ++i)
            cnt += s_ids[i] == tid;
    int total;
    const int off = block_excl_scan(cnt, tmp4, total);
    int nhit;
    const int u = block_excl_scan(cnt > 0 ? 1 : 0, tmp4, nhit);
    Plan *P = p.plan;
    if (tid < E) {
        p.counts[tid] = cnt;
        p.offsets[tid] = off;
        if (cnt > 0) {
            P->hit_expert[u] = tid;
            P->hit_off[u] = off;
            P->hit_rows[u] = cnt;
            int q = off;
            for (int i = 0; i < np; ++i)
                if (s_ids[i] == tid) {
                    p.rows[q] = i;
                    p.pos[i] = q;
                    ++q;
                }
        }
    }
    if (tid == 0) {
        p.offsets[E] = total;
        const int n1 = nhit * p.n_rb1 * p.ks1;
        P->m = m;
        P->n_hit = nhit;
        P->n_items1 = n1;
        P->n_items = n1 + nhit * p.n_rb2 * p.ks2;
        p.ctr->ticket = 0;
        p.ctr->items_done = 0;
        p.ctr->error_word = 0;
        p.ctr->route_done = 0;
    }
    for (int i = tid; i < nhit * p.n_rb1; i += kThreads)
        p.rb_done[i] = 0;
    for (int i = tid; i < nhit; i += kThreads)
        p.h_ready[i] = 0;
}

// ---------------------------------------------------------------------------
// Expert kernel: small-R GEMV core
// ---------------------------------------------------------------------------

// Byte tables of the per-tensor codebook for v_perm lookups: lo[i] holds the
// low bytes of entries 4i..4i+3, hi[i] the high bytes.
template <int BITS>
__device__ __forceinline__ void load_lut(const uint16_t *lut, uint32_t &lo0, uint32_t &lo1,
                                         uint32_t &hi0, uint32_t &hi1)
{
    const uint32_t *L = (const uint32_t *)lut;
    const uint32_t d0 = L[0], d1 = L[1];
    lo0 = __builtin_amdgcn_perm(d1, d0, 0x06040200u);
    hi0 = __builtin_amdgcn_perm(d1, d0, 0x07050301u);
    lo1 = hi1 = 0;
    if constexpr (BITS == 3) {
        const uint32_t d2 = L[2], d3 = L[3];
        lo1 = __builtin_amdgcn_perm(d3, d2, 0x06040200u);
        hi1 = __builtin_amdgcn_perm(d3, d2, 0x07050301u);
    }
}

// Decode one slot (32 codes of one row) into 16 packed fp16 pairs in natural
// column order: pair i holds columns 2i, 2i+1 of the slot. For word d and
// shift s, byte b of t is the code of column 16d + 4s + b; two v_perm
// lookups give its low and high bytes, two more interleave them.
template <int BITS>
__device__ __forceinline__ void decode_slot(const uint32_t (&w)[BITS], uint32_t lo0, uint32_t lo1,
                                            uint32_t hi0, uint32_t hi1, uint32_t (&out)[16])
{
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint32_t t = (w[d] >> (2 * s)) & 0x03030303u;
            if constexpr (BITS == 3)
                t |= ((w[2] >> (s + 4 * d)) & 0x01010101u) << 2;
            const uint32_t l = __builtin_amdgcn_perm(lo1, lo0, t);
            const uint32_t h = __builtin_amdgcn_perm(hi1, hi0, t);
            out[8 * d + 2 * s] = __builtin_amdgcn_perm(h, l, 0x05010400u);
            out[8 * d + 2 * s + 1] = __builtin_amdgcn_perm(h, l, 0x07030602u);
        }
}

template <int BITS>
__device__ __forceinline__ void load_slot(const uint32_t *__restrict__ codes, long tile, int lane,
                                          uint32_t (&w)[BITS])
{
    const uint32_t *src = codes + (tile * 64 + lane) * BITS;
    if constexpr (BITS == 2) {
        const u32x2 v = *(const u32x2 *)src;
        w[0] = v[0];
        w[1] = v[1];
    } else {
#pragma unroll
        for (int i = 0; i < BITS; ++i)
            w[i] = src[i];
    }
}

// One wave: 4 row blocks (64 rows) x groups [g0, g0+ng) of one codebook
// matrix with G groups per row. A: staged activations in LDS, row = token
// (R rows valid), column = input column - 128 g0, row stride astride halves.
// MFMA 16x16x32: A = tokens x 32 columns, B = 32 columns x 16 rows of W;
// lane (r = lane%16, q = lane/16) supplies token r / W row r and columns
// 32q + 8s' .. +7 of the group at step s'. Result lane layout: token
// 4(lane/16) + i, W row lane%16, so one group scale per lane.
template <int BITS, int NTB>
__device__ __forceinline__ void gemv_codebook(const DevTensor &T, int G, int rb0, int g0, int ng,
                                              const _Float16 *A, int astride, int R,
                                              floatx4 (&acc)[4][NTB])
{
    const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
    const uint32_t *codes = (const uint32_t *)T.codes;
    const uint16_t *sc = (const uint16_t *)T.scales;
    uint32_t lo0, lo1, hi0, hi1;
    load_lut<BITS>(T.lut, lo0, lo1, hi0, hi1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
            acc[i][tb] = floatx4{0.f, 0.f, 0.f, 0.f};

    uint32_t wc[4][BITS], wn[4][BITS];
    uint16_t sc_c[4], sc_n[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const long tile = (long)(rb0 + i) * G + g0;
        load_slot<BITS>(codes, tile, lane, wc[i]);
        sc_c[i] = sc[tile * 16 + r];
    }
    for (int gi = 0; gi < ng; ++gi) {
        if (gi + 1 < ng) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const long tile = (long)(rb0 + i) * G + g0 + gi + 1;
                load_slot<BITS>(codes, tile, lane, wn[i]);
                sc_n[i] = sc[tile * 16 + r];
            }
        }
        half8 a[NTB][4];
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            const int tok = tb * 16 + r;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                a[tb][s] = half8{0, 0, 0, 0, 0, 0, 0, 0};
                if (tok < R)
                    a[tb][s] = *(const half8 *)(A + tok * astride + gi * 128 + q * 32 + s * 8);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t bw[16];
            decode_slot<BITS>(wc[i], lo0, lo1, hi0, hi1, bw);
            floatx4 c[NTB];
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
                c[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const half8 b = __builtin_bit_cast(
                    half8, u32x4{bw[4 * s], bw[4 * s + 1], bw[4 * s + 2], bw[4 * s + 3]});
#pragma unroll
                for (int tb = 0; tb < NTB; ++tb)
                    c[tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[tb][s], b, c[tb], 0, 0, 0);
            }
            const float f = (float)__builtin_bit_cast(_Float16, sc_c[i]);
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
                acc[i][tb] += f * c[tb];
        }
        if (gi + 1 < ng) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int b = 0; b < BITS; ++b)
                    wc[i][b] = wn[i][b];
                sc_c[i] = sc_n[i];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Expert kernel: work items
// ---------------------------------------------------------------------------

// Stage R rows of fp16 activations into LDS: A[r][c] = src(r)[c], c < kc.
__device__ __forceinline__ void stage_rows(_Float16 *A, int astride, int R, int kc,
                                           const _Float16 *const *row_ptr)
{
    const int chunks = kc / 8;  // 16 B each
    for (int i = threadIdx.x; i < R * chunks; i += kThreads) {
        const int r = i / chunks, c = (i - r * chunks) * 8;
        *(u32x4 *)(A + r * astride + c) = *(const u32x4 *)(row_ptr[r] + c);
    }
}

template <int NTB>
__device__ __forceinline__ void run_gemv(const DevTensor &T, int G, int rb0, int g0, int ng,
                                         const _Float16 *A, int astride, int R,
                                         floatx4 (&acc)[4][NTB])
{
    if (T.bits == 2)
        gemv_codebook<2, NTB>(T, G, rb0, g0, ng, A, astride, R, acc);
    else
        gemv_codebook<3, NTB>(T, G, rb0, g0, ng, A, astride, R, acc);
}

// Gate/up item: hit expert u, 128-row block rb of gate and up, column split kq.
template <int NTB>
__device__ void gate_up_item(const Params &p, int e, int off, int R, int u, int rb, int kq,
                             _Float16 *A, const _Float16 **row_ptr, int *s_flag)
{
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int astride = p.kc1 + kLdsPadHalves;
    if (tid < R)
        row_ptr[tid] = p.xr + (size_t)(p.rows[off + tid] / p.k) * p.H + (size_t)kq * p.kc1;
    __syncthreads();
    stage_rows(A, astride, R, p.kc1, row_ptr);
    __syncthreads();

    const int proj = wave >> 1;                        // waves 0,1: gate; 2,3: up
    const DevTensor T = p.tensors[e * 3 + proj];
    const int rb0 = rb * 8 + (wave & 1) * 4;           // 16-row blocks
    floatx4 acc[4][NTB];
    run_gemv<NTB>(T, p.H / 128, rb0, kq * (p.kc1 / 128), p.kc1 / 128, A, astride, R, acc);

    // partial sums: gu_part[kq][off + tok][proj][n]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tok = tb * 16 + 4 * (lane >> 4) + j;
                if (tok < R) {
                    const size_t row = (size_t)kq * p.pair_cap + off + tok;
                    p.gu_part[(row * 2 + proj) * p.I + (rb0 + i) * 16 + (lane & 15)] = acc[i][tb][j];
                }
            }
    __threadfence();
    __syncthreads();
    if (tid == 0)
        *s_flag = atomic_add_agent(&p.rb_done[u * p.n_rb1 + rb], 1u) == (uint32_t)(p.ks1 - 1);
    __syncthreads();
    if (!*s_flag)
        return;
    __threadfence();
    // Last split of this block: h = silu(g) * u over rows rb*128..+127, then
    // h~ = (1/sqrt 128) H_128 (s_I * h), one wave per token.
    const int n = rb * 128 + 2 * lane;
    for (int tok = wave; tok < R; tok += 4) {
        float g0 = 0.f, g1 = 0.f, u0 = 0.f, u1 = 0.f;
        for (int s = 0; s < p.ks1; ++s) {
            const size_t row = (size_t)s * p.pair_cap + off + tok;
            const float *gp = p.gu_part + (row * 2 + 0) * p.I + n;
            const float *up = p.gu_part + (row * 2 + 1) * p.I + n;
            g0 += gp[0];
            g1 += gp[1];
            u0 += up[0];
            u1 += up[1];
        }
        float v0 = g0 / (1.0f + expf(-g0)) * u0 * (float)p.signs_i[n];
        float v1 = g1 / (1.0f + expf(-g1)) * u1 * (float)p.signs_i[n + 1];
        wave_fwht128(v0, v1);
        *(half2v *)(p.hr + (size_t)(off + tok) * p.I + n) =
            half2v{(_Float16)(v0 * kInvSqrt128), (_Float16)(v1 * kInvSqrt128)};
    }
    __threadfence();
    __syncthreads();
    if (tid == 0)
        atomic_add_agent(&p.h_ready[u], 1u);
}

// Down item: hit expert u, 256-row block rb of down, column split kq.
template <int NTB>
__device__ void down_item(const Params &p, int e, int off, int R, int u, int rb, int kq,
                          _Float16 *A, const _Float16 **row_ptr, int *s_flag)
{
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int astride = p.kc2 + kLdsPadHalves;
    if (tid == 0) {
        int ok = 1;
        uint32_t polls = 0;
        while (atomic_load_agent(&p.h_ready[u]) < (uint32_t)p.n_rb1) {
            __builtin_amdgcn_s_sleep(4);
            if (++polls > p.spin_limit) {
                __hip_atomic_fetch_or(&p.ctr->error_word, kErrSpinLimit, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
                ok = 0;
                break;
            }
        }
        *s_flag = ok;
    }
    if (tid < R)
        row_ptr[tid] = p.hr + (size_t)(off + tid) * p.I + (size_t)kq * p.kc2;
    __syncthreads();
    if (!*s_flag)
        return;
    __threadfence();
    stage_rows(A, astride, R, p.kc2, row_ptr);
    __syncthreads();

    const DevTensor T = p.tensors[e * 3 + 2];
    const int rb0 = rb * 16 + wave * 4;
    floatx4 acc[4][NTB];
    run_gemv<NTB>(T, p.I / 128, rb0, kq * (p.kc2 / 128), p.kc2 / 128, A, astride, R, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tok = tb * 16 + 4 * (lane >> 4) + j;
                if (tok < R) {
                    const size_t row = (size_t)kq * p.pair_cap + off + tok;
                    p.y_part[row * p.H + (rb0 + i) * 16 + (lane & 15)] = acc[i][tb][j];
                }
            }
}

__global__ __launch_bounds__(kThreads) void expert_kernel(Params p)
{
    extern __shared__ _Float16 A[];
    __shared__ const _Float16 *row_ptr[kMaxTokens];
    __shared__ int s_ticket, s_flag;
    const Plan *P = p.plan;
    const int n_items = P->n_items, n1 = P->n_items1;
    int ticket = blockIdx.x;
    uint32_t done = 0;
    while (ticket < n_items) {
        if (ticket < n1) {
            const int per_u = p.n_rb1 * p.ks1;
            const int u = ticket / per_u, rem = ticket - u * per_u;
            const int rb = rem / p.ks1, kq = rem - rb * p.ks1;
            const int e = P->hit_expert[u], off = P->hit_off[u], R = P->hit_rows[u];
            if (R <= 16)
                gate_up_item<1>(p, e, off, R, u, rb, kq, A, row_ptr, &s_flag);
            else
                gate_up_item<2>(p, e, off, R, u, rb, kq, A, row_ptr, &s_flag);
        } else {
            const int it = ticket - n1;
            const int per_u = p.n_rb2 * p.ks2;
            const int u = it / per_u, rem = it - u * per_u;
            const int rb = rem / p.ks2, kq = rem - rb * p.ks2;
            const int e = P->hit_expert[u], off = P->hit_off[u], R = P->hit_rows[u];
            if (R <= 16)
                down_item<1>(p, e, off, R, u, rb, kq, A, row_ptr, &s_flag);
            else
                down_item<2>(p, e, off, R, u, rb, kq, A, row_ptr, &s_flag);
        }
        ++done;
        __syncthreads();
        if (threadIdx.x == 0)
            s_ticket = (int)gridDim.x + (int)atomic_add_agent(&p.ctr->ticket, 1u);
        __syncthreads();
        ticket = s_ticket;
    }
    if (threadIdx.x == 0 && done)
        atomic_add_agent(&p.ctr->items_done, done);
}

// ---------------------------------------------------------------------------
// Combine
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void combine_kernel(Params p, float *__restrict__ out)
{
    const int t = blockIdx.y, i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= p.H)
        return;
    float acc = 0.0f;
    for (int j = 0; j < p.k; ++j) {
        const int pp = p.pos[t * p.k + j];
        float y = 0.0f;
        for (int s = 0; s < p.ks2; ++s)
            y += p.y_part[((size_t)s * p.pair_cap + pp) * p.H + i];
        acc += p.wts[t * p.k + j] * y;
    }
    out[(size_t)t * p.H + i] = acc;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

hipError_t launch_route(const Params &p, const uint16_t *x, const float *logits, int m,
                        hipStream_t s)
{
    route_kernel<<<dim3(m), dim3(kThreads), 0, s>>>(p, x, logits, m);
    return hipGetLastError();
}

hipError_t launch_expert(const Params &p, int grid, size_t lds_bytes, hipStream_t s)
{
    expert_kernel<<<dim3(grid), dim3(kThreads), lds_bytes, s>>>(p);
    return hipGetLastError();
}

hipError_t launch_combine(const Params &p, float *out, int m, hipStream_t s)
{
    combine_kernel<<<dim3((p.H + kThreads - 1) / kThreads, m), dim3(kThreads), 0, s>>>(p, out);
    return hipGetLastError();
}

hipError_t expert_occupancy(int *blocks_per_cu, size_t lds_bytes)
{
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, expert_kernel, kThreads,
                                                        lds_bytes);
}

}  // namespace moe
