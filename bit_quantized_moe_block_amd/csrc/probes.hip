// Measurement probes (include/moe_probe.h): a plain streaming read of a
// device buffer, an empty kernel, the LDS read pattern of the MFMA
// activation operands, the issue rates of the decode step's halves (the
// decode kernels' own decode sequence, from decode_step.h, on register
// operands: no weights, no layer) and a streaming read whose units are
// claimed from shared counters.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_probe.h"
#include "decode_step.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

// Each thread walks the buffer with a grid-wide stride, four 16-byte loads
// per round in flight, and xor-folds what it read.
__global__ __launch_bounds__(256) void stream_read(const u32x4 *__restrict__ buf, size_t n16,
                                                   uint32_t *sink)
{
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    u32x4 acc = u32x4{0, 0, 0, 0};
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride)
        acc ^= buf[i];
    const uint32_t f = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (f == 0x9E3779B9u)
        sink[0] = f;
}

__global__ void empty_kernel() {}

// The activation-operand reads of a 16x16x32 MFMA over four 16-row
// subtiles of staged fp16 rows: lane (r = lane % 16, q = lane / 16) reads the
// 16-byte piece 4q + s of row 16t + r, for steps s = 0..3 and subtiles
// t = 0..3, `iters` times. Layout 0: rows of 272 bytes (128 halves and 16
// bytes of padding); 1: rows of 256 bytes, piece p of row r stored at piece
// p ^ (r mod 16); 2: rows of 256 bytes, no padding (the 16 rows of one read
// start on the same bank).
constexpr int kLdsRows = 64, kLdsStride = 136;  // halves

__device__ __forceinline__ int lds_probe_offset(int layout, int row, int piece)
{
    if (layout == 0)
        return row * kLdsStride + piece * 8;
    if (layout == 1)
        return row * 128 + ((piece ^ row) & 15) * 8;
    return row * 128 + piece * 8;
}

__global__ __launch_bounds__(256) void lds_read128(int layout, int iters, uint32_t *sink)
{
    __shared__ __align__(16) uint16_t A[kLdsRows * kLdsStride];
    for (int i = threadIdx.x; i < kLdsRows * kLdsStride; i += 256)
        A[i] = (uint16_t)(i * 40503u);
    __syncthreads();
    const int lane = threadIdx.x & 63, r = lane & 15, q = lane >> 4;
    int off[16];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s)
            off[4 * t + s] = lds_probe_offset(layout, 16 * t + r, 4 * q + s);
    // the offsets are loop-invariant; xor-ing in (it & zero), zero = 0 at run
    // time, keeps every read inside the loop
    const int zero = iters >> 30;
    u32x4 acc = u32x4{0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
        const int z = it & zero;
#pragma unroll
        for (int k = 0; k < 16; ++k)
            acc ^= *(const u32x4 *)(A + (off[k] ^ z));
    }
    const uint32_t f = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (f == 0x9E3779B9u)
        sink[0] = f;
}

// Issue rates of one 128-column group of a 3-bit tile (4 MFMA steps of 8
// weights per lane), all operands in registers: the slot words change every
// round by an xor with the round index (one VALU op per word and round, in
// every mode). MODE 0: decode only, each step's four output words xor-folded;
// 1: MFMA only (a fixed B operand) and the group-scale FMAs; 2: decode into
// the MFMA and the group-scale FMAs (the decode kernels' inner step); 3:
// decode into four v_dot2_f32_f16 products for one token (the products on
// the VALU instead of the MFMA). Thread 0 of block 0 records the shader clock
// (s_memtime) and the 100 MHz constant clock (s_memrealtime) before and after
// its rounds in clk[0..3].
template <int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void compute_rate(int iters, uint32_t seed, unsigned long long *clk, uint32_t *sink)
{
    using namespace moe;
    const int lane = threadIdx.x & 63;
    uint32_t tab[4];
    // a codebook of eight fp16 entries of magnitude 0.25 .. 2
    lut_tables(u32x4{0xB800BC00u ^ (seed & 1u), 0x38003400u, 0xB4003C00u, 0x40003000u}, tab);
    const uint32_t w[3] = {seed * 0x9E3779B9u + (uint32_t)lane, (seed + (uint32_t)lane) * 0x85EBCA6Bu,
                           (uint32_t)lane * 0xC2B2AE35u + seed};
    half8 a[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            a[s][e] = (_Float16)(0.001f * (float)((lane + 3 * s + e) & 31));
    const half8 bconst = a[(lane >> 4) & 3];
    const float f = 0.5f + (float)(seed & 1u);
    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
    float dacc = 0.f;
    uint32_t fold = 0;
    unsigned long long t0 = 0, r0 = 0;
    const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
    if (timer) {
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    for (int it = 0; it < iters; ++it) {
        const uint32_t x[3] = {w[0] ^ (uint32_t)it, w[1] ^ (uint32_t)it, w[2] ^ (uint32_t)it};
        floatx4 cc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if constexpr (MODE == 0 || MODE == 2 || MODE == 3) {
                const half8 bv = decode_step<3>(x, s, tab, half2v{1, 1});
                if constexpr (MODE == 0) {
                    const u32x4 u = __builtin_bit_cast(u32x4, bv);
                    fold ^= u[0] ^ u[1] ^ u[2] ^ u[3];
                } else if constexpr (MODE == 2) {
                    cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[s], bv, cc, 0, 0, 0);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        dacc = __builtin_amdgcn_fdot2(
                            half2v{a[s][2 * e], a[s][2 * e + 1]}, half2v{bv[2 * e], bv[2 * e + 1]},
                            dacc, false);
                }
            } else {
                cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[s], bconst, cc, 0, 0, 0);
            }
        }
        if constexpr (MODE == 1 || MODE == 2)
            acc += f * cc;
    }
    if (timer) {
        clk[0] = t0;
        clk[1] = r0;
        clk[2] = __builtin_amdgcn_s_memtime();
        clk[3] = __builtin_amdgcn_s_memrealtime();
    }
    const uint32_t v = fold ^ __float_as_uint(dacc) ^ __float_as_uint(acc[0] + acc[1] + acc[2] + acc[3]);
    if (v == 0x9E3779B9u)
        sink[0] = v;
}

// Units of 64 KiB (4096 16-byte loads, 16 per thread, all in flight) read by
// `gridDim.x` blocks of 256 threads, one unit at a time. MODE 0: block b
// reads units b, b + G, ... (a static order); 1: each unit is claimed from
// one counter (thread 0's agent-scope atomic add, handed to the block
// through LDS); 2: from eight counters, 128 bytes apart (block b claims from
// counter b % 8, whose k-th claim is unit b % 8 + 8 k).
constexpr int kUnit16 = 4096;

template <int MODE>
__global__ __launch_bounds__(256) void ticket_read(const u32x4 *__restrict__ buf, uint32_t units,
                                                   uint32_t *ctr, uint32_t *sink)
{
    __shared__ uint32_t s_claim;
    const uint32_t nq = MODE == 2 ? 8u : 1u, q = blockIdx.x % nq;
    u32x4 acc = u32x4{0, 0, 0, 0};
    for (uint32_t k = 0;; ++k) {
        uint32_t u;
        if constexpr (MODE == 0) {
            u = blockIdx.x + k * gridDim.x;
        } else {
            if (threadIdx.x == 0)
                s_claim = __hip_atomic_fetch_add(&ctr[q * 32], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            u = q + nq * s_claim;
            __syncthreads();
        }
        if (u >= units)
            break;
        const u32x4 *p = buf + (size_t)u * kUnit16 + threadIdx.x;
        u32x4 v[kUnit16 / 256];
#pragma unroll
        for (int j = 0; j < kUnit16 / 256; ++j)
            v[j] = p[j * 256];
#pragma unroll
        for (int j = 0; j < kUnit16 / 256; ++j)
            acc ^= v[j];
    }
    const uint32_t f = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (f == 0x9E3779B9u)
        sink[0] = f;
}

// The weight reads of the decode kernels without the decode: each wave
// streams work units of one stored matrix (4 tile rows x 8 column groups of
// 16 x 128 weights: one wave's share of an expert-kernel item) in the
// kernel's order, per group the 4 tiles' slot words (one load per tile at the
// lane's slot offset, the kernel's load width for the code width) and their
// scales (one 2-byte load per tile), two groups in flight, and xor-folds what
// it read. Units are taken in a static order across the concatenated
// matrices (wave w of the grid: units w, w + W, ...).
constexpr int kMaxTileStreams = 8192;

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void tile_read(const moe_probe_tile_stream *__restrict__ st, int ns, uint32_t total_units,
               uint32_t *sink)
{
    const int lane = threadIdx.x & 63;
    const uint32_t nw = gridDim.x * 4u;
    const uint32_t gw = blockIdx.x * 4u + (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint32_t fold = 0;
    int s = 0;
    for (uint32_t U = gw; U < total_units; U += nw) {
        // the matrix holding unit U (streams in order; U only grows)
        while (s + 1 < ns && U >= (uint32_t)__builtin_amdgcn_readfirstlane(st[s + 1].units_before))
            ++s;
        const moe_probe_tile_stream T = st[s];
        const int G = __builtin_amdgcn_readfirstlane(T.groups), bits = __builtin_amdgcn_readfirstlane(T.bits);
        const uint32_t u = U - (uint32_t)__builtin_amdgcn_readfirstlane(T.units_before);
        const int per_band = G / 8;
        const int r0 = (int)(u / per_band) * 4, g0 = (int)(u % per_band) * 8;
        const uint64_t cb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)T.codes >> 32)) << 32) |
                            (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)T.codes);
        const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)T.scales >> 32)) << 32) |
                            (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)T.scales);
        const int tbytes = 256 * bits, sbytes = bits == 4 ? 128 : 32;
        const int ntiles = __builtin_amdgcn_readfirstlane(T.tile_rows) * G;
        // sized to the matrix: the bytes a 2-bit lane's 12-byte load reads
        // past the last tile read as zero, without touching memory
        const __amdgpu_buffer_rsrc_t rc =
            __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)cb, 0, ntiles * tbytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)sb, 0, ntiles * sbytes, 0x00020000);
        const int sc_lane = bits == 4 ? (lane & 15) * 8 + 2 * (lane >> 4) : (lane & 15) * 2;
        uint32_t w[2][4][4];
#pragma unroll
        for (int g = 0; g < 8 + 2; ++g) {
            if (g >= 2) {  // consume group g - 2
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    fold ^= w[g & 1][i][0] ^ w[g & 1][i][1] ^ w[g & 1][i][2] ^ w[g & 1][i][3];
            }
            if (g < 8) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tile = (r0 + i) * G + g0 + g;
                    uint32_t *d = w[g & 1][i];
                    if (bits == 4) {
                        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, lane * 16, tile * tbytes, 0);
                        d[0] = v[0]; d[1] = v[1]; d[2] = v[2];
                    } else {
                        // one 12-byte load for 2- and 3-bit tiles (the 2-bit lane's last 4 bytes unused)
                        const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rc, lane * 4 * bits, tile * tbytes, 0);
                        d[0] = v[0]; d[1] = v[1]; d[2] = v[2];
                    }
                    d[3] = __builtin_amdgcn_raw_buffer_load_b16(rs, sc_lane, tile * sbytes, 0);
                }
            }
        }
    }
    if (fold == 0x9E3779B9u)
        sink[0] = fold;
}

}  // namespace

extern "C" int moe_probe_tile_read(const moe_probe_tile_stream *streams, int32_t count,
                                   moe_probe_tile_stream *dev_streams, int32_t blocks,
                                   uint32_t *sink, void *hip_stream)
{
    if (!streams || !dev_streams || !sink || count < 1 || count > kMaxTileStreams || blocks < 1)
        return -(int)hipErrorInvalidValue;
    uint64_t units = 0;
    for (int i = 0; i < count; ++i) {
        const moe_probe_tile_stream &t = streams[i];
        const uint64_t bytes = (uint64_t)t.tile_rows * (uint64_t)t.groups * 256u * (uint64_t)t.bits;
        if (!t.codes || !t.scales || t.tile_rows < 4 || t.tile_rows % 4 || t.groups < 8 ||
            t.groups % 8 || !(t.bits == 2 || t.bits == 3 || t.bits == 4) ||
            (uint64_t)t.units_before != units || bytes > 0x7FFFFFFFu)
            return -(int)hipErrorInvalidValue;
        units += (uint64_t)(t.tile_rows / 4) * (uint64_t)(t.groups / 8);
    }
    if (units > 0x7FFFFFFFu)
        return -(int)hipErrorInvalidValue;
    const hipStream_t s = (hipStream_t)hip_stream;
    hipError_t e = hipMemcpyAsync(dev_streams, streams, sizeof(moe_probe_tile_stream) * count,
                                  hipMemcpyHostToDevice, s);
    if (e != hipSuccess)
        return -(int)e;
    tile_read<<<dim3(blocks), dim3(256), 0, s>>>(dev_streams, count, (uint32_t)units, sink);
    return -(int)hipGetLastError();
}

extern "C" int moe_probe_compute_rate(int32_t mode, int32_t blocks, int32_t iters,
                                      unsigned long long *clk, uint32_t *sink, void *hip_stream)
{
    if (mode < 0 || mode > 3 || blocks < 1 || iters < 1 || !clk || !sink)
        return -(int)hipErrorInvalidValue;
    const hipStream_t s = (hipStream_t)hip_stream;
    const dim3 g(blocks), b(256);
    const uint32_t seed = 0x2545F491u;
    switch (mode) {
    case 0: compute_rate<0><<<g, b, 0, s>>>(iters, seed, clk, sink); break;
    case 1: compute_rate<1><<<g, b, 0, s>>>(iters, seed, clk, sink); break;
    case 2: compute_rate<2><<<g, b, 0, s>>>(iters, seed, clk, sink); break;
    default: compute_rate<3><<<g, b, 0, s>>>(iters, seed, clk, sink); break;
    }
    return -(int)hipGetLastError();
}

extern "C" int moe_probe_ticket_read(const void *buf, size_t bytes, int32_t blocks, int32_t mode,
                                     uint32_t *counters, uint32_t *sink, void *hip_stream)
{
    const size_t unit = (size_t)kUnit16 * 16;
    if (!buf || !counters || !sink || ((uintptr_t)buf % 16) || bytes % unit || bytes / unit == 0 ||
        bytes / unit > 0xFFFFFFFFu || blocks < 1 || mode < 0 || mode > 2)
        return -(int)hipErrorInvalidValue;
    const hipStream_t s = (hipStream_t)hip_stream;
    hipError_t e = hipMemsetAsync(counters, 0, 8 * 32 * sizeof(uint32_t), s);
    if (e != hipSuccess)
        return -(int)e;
    const uint32_t units = (uint32_t)(bytes / unit);
    const u32x4 *p = (const u32x4 *)buf;
    const dim3 g(blocks), b(256);
    switch (mode) {
    case 0: ticket_read<0><<<g, b, 0, s>>>(p, units, counters, sink); break;
    case 1: ticket_read<1><<<g, b, 0, s>>>(p, units, counters, sink); break;
    default: ticket_read<2><<<g, b, 0, s>>>(p, units, counters, sink); break;
    }
    return -(int)hipGetLastError();
}

extern "C" int moe_probe_stream_read(const void *buf, size_t bytes, int32_t blocks, uint32_t *sink,
                                     void *hip_stream)
{
    if (!buf || !sink || bytes % 16 || ((uintptr_t)buf % 16) || blocks < 1)
        return -(int)hipErrorInvalidValue;
    stream_read<<<dim3(blocks), dim3(256), 0, (hipStream_t)hip_stream>>>((const u32x4 *)buf,
                                                                         bytes / 16, sink);
    return -(int)hipGetLastError();
}

extern "C" int moe_probe_empty_kernels(int32_t count, void *hip_stream)
{
    for (int i = 0; i < count; ++i) {
        empty_kernel<<<dim3(1), dim3(64), 0, (hipStream_t)hip_stream>>>();
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return -(int)e;
    }
    return 0;
}

extern "C" int moe_probe_lds_read128(int32_t layout, int32_t blocks, int32_t iters, uint32_t *sink,
                                     void *hip_stream)
{
    if (layout < 0 || layout > 2 || blocks < 1 || iters < 1 || iters >= (1 << 30) || !sink)
        return -(int)hipErrorInvalidValue;
    lds_read128<<<dim3(blocks), dim3(256), 0, (hipStream_t)hip_stream>>>(layout, iters, sink);
    return -(int)hipGetLastError();
}
