// gfx950 kernels of the routed-experts decode step.
//
// route_kernel   256-thread blocks. The first blocks: top-k on the raw
//                logits (one wave per token, DPP max-reductions), softmax
//                over the selected logits; the last of them to finish builds
//                the per-expert row buckets, row groups (<= 16 rows each), the
//                work plan, and resets the expert kernel's counters (so every
//                run and every graph replay starts clean without a memset).
//                The other blocks: one wave per (token, 128-column block)
//                rotates x (codebook) or converts it to fp16 (NVFP4).
// expert_kernel  persistent grid, work items assigned round robin (no shared
//                ticket counter), no grid-wide barrier. Gate/up items (one
//                row group, 128 rows of gate and of up, one column split)
//                write partial sums; the last split of a 128-row block
//                finishes SiLU(g)*u and the 128-point rotation of h. Down
//                items (256 rows of down, one column split) wait on a
//                per-group counter of finished h blocks and store their
//                partial sums under the pair index.
// small_kernel   runs of at most 4 tokens whose items fit one round of the
//                grid: gate/up items of 32 rows over all columns (whole
//                sums: SiLU(g)*u in the item), down items of 64 rows that
//                rotate h themselves after their group's h counter is full.
// combine_kernel one wave per (token, 256-row block): the down partial sums
//                of the token's k slots, in slot order, times the router
//                weights (NaN if the expert kernel reported an error).
// prefill_kernel from 48 tokens on: grouped GEMM over 64-row groups, gate/up
//                then down as two launches.
//                Inner loop: codes decoded in registers (v_perm byte lookups
//                of the per-tensor codebook, or hardware e2m1 conversion),
//                MFMA 16x16x32 f16 with the tokens as the A operand, fp32
//                group-scale FMAs; two pairs of weight groups in flight per
//                wave (ping-pong register buffers).
//
// Page "LNA-CANON.md", section "lna2 とは": resident expert teams with
// dynamic tickets and no grid-wide barrier, small-R inner loops for
// R_e in {1,2,4,8} at m <= 24, bitwise reproducible results; page
// "lna-lab/README.md", section "2026-09-04 -- house kernel lna2".
#include "moe_internal.h"
#include "decode_step.h"

namespace moe {

// Work items of one shared-expert row group in the gate/up (down = false) or
// down phase: column splits x row blocks, or x half row blocks when its items
// cover half row blocks.
__device__ __forceinline__ int shared_items(const Params &p, bool down)
{
    const int ks = down ? p.ks2 : p.ks1;
    if (p.sh_half)
        return 2 * (down ? p.n_rb2 : p.n_rb1) * ks;
    return (down ? p.n_rb2 : p.n_rb1 / p.span1) * ks;
}

constexpr float kInvSqrt128 = 0.08838834764831845f;

__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t *p, uint32_t v)
{
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_load_agent(uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Data handed between blocks of one kernel launch (gate/up partial sums ->
// the finishing block, h~ -> the down items, down partial sums -> the
// combining block) moves through agent-coherent loads and stores (sc1):
// they bypass the per-XCD L2 copies, so no L2 write-back or invalidate (what
// a device-scope fence costs on a multi-XCD part) is needed. The producer
// waits for its stores to be acknowledged (s_waitcnt) before a block barrier
// and the counter increment.
__device__ __forceinline__ void st_coherent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coherent(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte agent-coherent load (buffer_load_dwordx4 ... sc1) at byte offset
// `off` of a buffer starting at `base`.
__device__ __forceinline__ u32x4 ld_coherent16(const void *base, uint32_t off)
{
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 0x7FFFFFFF, 0x00020000);
    return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 16 /* sc1 */);
}
// All of this wave's memory operations acknowledged (stores included).
__device__ __forceinline__ void wait_stores()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Block barrier that orders LDS only: the wave's LDS accesses complete, then
// s_barrier; global loads and stores in flight stay in flight (the fences of
// __syncthreads wait for every one of them). The signal fences keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
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

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / 64;

// Monotone key of a finite float: larger value <-> larger unsigned key; -0
// is folded into +0. Key 0 is below every finite value and marks "taken".
__device__ __forceinline__ uint32_t float_key(float v)
{
    if (v == 0.0f)
        v = 0.0f;
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Maximum over the wave (DPP row shifts, then row broadcasts), as a scalar.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
    return __builtin_amdgcn_readlane(v, 63);
}

// Exclusive block-wide scan of one int per thread (kRouteThreads threads).
__device__ __forceinline__ int block_excl_scan(int v, int *tmp, int &total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off)
            x += y;
    }
    if (lane == 63)
        tmp[wave] = x;
    __syncthreads();
    int base = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kRouteWaves; ++w) {
        base += w < wave ? tmp[w] : 0;
        total += tmp[w];
    }
    __syncthreads();
    return base + x - v;
}

__device__ __forceinline__ int ld_coherent_i32(const int32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Top-k of token t by one wave; lane holds experts lane + 64 i. Each round
// takes the largest key, then the lowest expert id among equal keys (the
// lowest i with a match, then the lowest lane: one ballot per i, no second
// reduction); lane j keeps slot j. Weights: softmax over the k selected
// logits, the denominator summed in slot order. ids go out agent-coherent for
// the bucketing block, and to s_ids (if given) for a bucketing in this block.
__device__ void route_token(const Params &p, const float *__restrict__ logits, int E, int t,
                            int *s_ids)
{
    const int lane = threadIdx.x & 63;
    const int k = p.k;
    // the four loads are issued together (an expert index past E is clamped
    // and its key dropped afterwards), not one at a time under the condition
    float lv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        lv[i] = logits[(size_t)t * E + min(lane + 64 * i, E - 1)];
    uint32_t key[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        key[i] = lane + 64 * i < E ? float_key(lv[i]) : 0u;
    int my_id = 0;
    uint32_t my_key = 0;
    for (int j = 0; j < k; ++j) {
        const uint32_t kmax = wave_max_u32(max(max(key[0], key[1]), max(key[2], key[3])));
        int e = 0;
#pragma unroll
        for (int i = 3; i >= 0; --i) {
            const uint64_t hit = __ballot(key[i] == kmax);
            if (hit)
                e = 64 * i + __builtin_ctzll(hit);
        }
        e = __builtin_amdgcn_readfirstlane(e);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (e == lane + 64 * i)
                key[i] = 0u;
        if (lane == j) {
            my_id = e;
            my_key = kmax;
        }
    }
    const float l0 = key_float(__builtin_amdgcn_readlane(my_key, 0));
    const float ex = lane < k ? expf(key_float(my_key) - l0) : 0.0f;
    float den = 0.0f;
    for (int j = 0; j < k; ++j)
        den += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), j));
    if (lane < k) {
        st_coherent((uint32_t *)&p.ids[t * k + lane], (uint32_t)my_id);
        p.wts[t * k + lane] = ex / den;
        if (s_ids)
            s_ids[t * k + lane] = my_id;
    }
}

// Dynamic LDS of the route kernel: the bucketing block's per-expert token
// bitmasks and row bases, W = ceil(m / 32) words per expert each.
size_t route_lds_bytes(int E, int m)
{
    return (size_t)2 * E * ((m + 31) / 32) * sizeof(uint32_t);
}

// The last top-k block to finish builds the buckets: per-expert rows, row
// groups (<= p.group_rows rows each), the work plan, and clears the expert kernel's
// counters (every run and every graph replay starts clean without a memset).
__device__ void bucket_block(const Params &p, int m, const int *s_ids)
{
    extern __shared__ uint32_t s_route[];  // [E][W] token masks, then [E][W] row bases
    __shared__ int tmp[kRouteWaves];
    const int tid = threadIdx.x;
    const int E = p.E, k = p.k, W = (m + 31) >> 5;
    uint32_t *s_mask = s_route;
    int *s_base = (int *)(s_route + E * W);
    for (int i = tid; i < E * W; i += kRouteThreads)
        s_mask[i] = 0u;
    __syncthreads();

    // ---- buckets. Top-k picks distinct experts per token, so expert e's rows
    // are the tokens of its bitmask (bit t % 32 of word t / 32), ascending by
    // t; the rank of (t, j) inside e's bucket is the count of mask bits below t.
    const int np = m * k;
    // the first two pairs of each thread stay in registers for the ranks below
    // (m * k <= 512 needs no second load)
    int e_keep[2] = {0, 0};
    for (int i = tid; i < np; i += kRouteThreads) {
        const int t = i / k, e = s_ids ? s_ids[i] : ld_coherent_i32(&p.ids[i]);
        if (i < 2 * kRouteThreads)
            e_keep[i / kRouteThreads] = e;
        atomicOr(&s_mask[e * W + (t >> 5)], 1u << (t & 31));
    }
    __syncthreads();
    int cnt = 0;
    if (tid < E)
        for (int w = 0; w < W; ++w)
            cnt += __popc(s_mask[tid * W + w]);
    const int GR = p.group_rows;  // rows per row group: 16 (decode) or 64 (prefill)
    const int ng_e = (cnt + GR - 1) / GR;
    // one scan of (rows | groups << 16): rows <= 8192, groups <= 768
    int packed_total;
    const int packed = block_excl_scan(cnt | (ng_e << 16), tmp, packed_total);
    const int off = packed & 0xFFFF, gbase = packed >> 16;
    const int total = packed_total & 0xFFFF, ngroups = packed_total >> 16;
    Plan *P = p.plan;
    // the shared expert (if any) comes first: expert id E, bucket rows
    // m*k + t for every token t, in row groups of <= GR. It is the largest
    // expert of the layer (every token, wider codes), so its items start
    // first and its down items are not the last to find their h.
    const int ngs = p.has_shared ? (m + GR - 1) / GR : 0;
    if (tid < ngs) {
        P->g_expert[tid] = E;
        P->g_off[tid] = m * k + GR * tid;
        P->g_rows[tid] = min(GR, m - GR * tid);
    }
    if (tid < E) {
        int base = off;
        for (int w = 0; w < W; ++w) {
            s_base[tid * W + w] = base;
            base += __popc(s_mask[tid * W + w]);
        }
        p.counts[tid] = cnt;
        p.offsets[tid] = off;
        for (int g = 0; g < ng_e; ++g) {
            P->g_expert[ngs + gbase + g] = tid;
            P->g_off[ngs + gbase + g] = off + GR * g;
            P->g_rows[ngs + gbase + g] = min(GR, cnt - GR * g);
        }
    }
    __syncthreads();
    for (int i = tid; i < np; i += kRouteThreads) {
        const int e = i < 2 * kRouteThreads ? e_keep[i / kRouteThreads] : ld_coherent_i32(&p.ids[i]);
        const int t = i / k;
        const int q = s_base[e * W + (t >> 5)] + __popc(s_mask[e * W + (t >> 5)] & ((1u << (t & 31)) - 1u));
        p.rows[q] = i;
        p.pos[i] = q;
    }
    // the shared expert's rows m*k + t hold their own index: every bucket
    // row's entry is then the pair index its down partial sums go under
    if (p.has_shared)
        for (int t = tid; t < m; t += kRouteThreads)
            p.rows[np + t] = np + t;
    if (tid == 0) {
        p.offsets[E] = total;
        // gate/up items of span1 row blocks for the routed groups that fit in
        // the expert kernel's first round of tickets (one item per block);
        // the groups past them take one row block per item, so that a second
        // round costs half an item per block instead of a whole one
        const int per_wide = (p.n_rb1 / p.span1) * p.ks1;
        int n_wide = ngroups;
        if (p.span1 > 1) {
            const int room = p.egrid - ngs * shared_items(p, false);
            n_wide = min(ngroups, room > 0 ? room / per_wide : 0);
        }
        const int n1 = ngs * shared_items(p, false) + n_wide * per_wide +
                       (ngroups - n_wide) * p.n_rb1 * p.ks1;
        P->n_wide = n_wide;
        P->m = m;
        P->n_groups = ngroups + ngs;
        P->n_sgroups = ngs;
        P->n_items1 = n1;
        P->n_items = n1 + ngs * shared_items(p, true) + ngroups * p.n_rb2 * p.ks2;
        for (int i = 0; i < kDoneSlots; ++i)
            p.ctr->items_done[i] = 0;
        p.ctr->error_word = 0;
    }
    for (int i = tid; i < (ngroups + ngs) * p.n_rb1; i += kRouteThreads)
        p.rb_done[i * kCtrStride] = 0;
    for (int i = tid; i < ngroups + ngs; i += kRouteThreads)
        p.h_ready[i * kCtrStride] = 0;
}

// Blocks 0 .. ceil(m / kRouteWaves) - 1: one wave per token does its top-k;
// the last of these blocks to finish (one counter) buckets the rows. With a
// single top-k block (m <= kRouteWaves = 4) that block buckets right away
// from the ids it holds in LDS: no counter, no global round trip. (Blocks of
// 16 waves, one block for 16 tokens, measured slower at m = 16: four top-k
// waves per SIMD instead of one.) The remaining blocks: one wave per (token, 128-column
// block) rotates x (codebook) or converts it to fp16 (NVFP4).
// The scalar arguments come first: the kernel-argument preload puts them in
// scalar registers at launch, so the logit loads need not wait for the
// parameter block's loads (E is also in p; this copy is the preloaded one).
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const float *__restrict__ logits,
                                                              const uint16_t *__restrict__ x,
                                                              int m, int E, Params p)
{
    __shared__ int s_last;
    __shared__ int s_ids[kRouteWaves * kMaxTopK];
    const int nk = (m + kRouteWaves - 1) / kRouteWaves;
    const int wave = threadIdx.x >> 6;
    if (nk == 1 && blockIdx.x == 0) {
        if (wave < m)
            route_token(p, logits, E, wave, s_ids);
        __syncthreads();
        bucket_block(p, m, s_ids);
        return;
    }
    if ((int)blockIdx.x < nk) {
        const int t = blockIdx.x * kRouteWaves + wave;
        if (t < m)
            route_token(p, logits, E, t, nullptr);
        wait_stores();
        __syncthreads();
        if (threadIdx.x == 0) {
            s_last = atomic_add_agent(&p.ctr->route_done, 1u) == (uint32_t)(nk - 1);
            if (s_last)  // every top-k block has counted: clear for the next run
                __hip_atomic_store(&p.ctr->route_done, 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (s_last)
            bucket_block(p, m, nullptr);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int task = (blockIdx.x - nk) * kRouteWaves + wave;
    const int nb = p.H / 128;
    if (task >= m * nb)
        return;
    const int t = task / nb, c0 = (task - t * nb) * 128 + 2 * lane;
    const uint32_t xx = *(const uint32_t *)(x + (size_t)t * p.H + c0);
    float v0 = bf16_to_f32(xx & 0xFFFFu), v1 = bf16_to_f32(xx >> 16);
    if (p.format == kFmtCodebook) {
        // the two signs in one 16-bit load, issued before x is used
        const uint16_t sg = *(const uint16_t *)(p.signs_h + c0);
        v0 *= (float)(int8_t)(sg & 0xFF);
        v1 *= (float)(int8_t)(sg >> 8);
        wave_fwht128(v0, v1);
        v0 *= kInvSqrt128;
        v1 *= kInvSqrt128;
    }
    *(half2v *)(p.xr + (size_t)t * p.H + c0) = half2v{(_Float16)v0, (_Float16)v1};
}

// ---------------------------------------------------------------------------
// Expert kernel: the per-wave small-R GEMV core
// ---------------------------------------------------------------------------

#define GLOBAL __attribute__((address_space(1)))
typedef const uint32_t GLOBAL *gu32p;
typedef const uint16_t GLOBAL *gu16p;
typedef const uint8_t GLOBAL *gu8p;
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

// Row blocks (16 rows each) one wave computes; waves per expert-kernel block.
constexpr int kWaveRB = 4;
constexpr int kExpertThreads = 256;
constexpr int kExpertWaves = kExpertThreads / 64;

// Kernel classes: the codebook format without and with 6-bit tensors (the
// 6-bit path is compiled only into the latter, so layers without 6-bit
// tensors run code that has none of it), and NVFP4.
constexpr int kClassCb6 = 3;
template <int CLASS>
constexpr bool is_cb = CLASS != kFmtNvfp4;
template <int CLASS>
constexpr bool has6 = CLASS == kClassCb6;

// Slot words held per tile: codebook up to 3 (2-bit tensors use 2), NVFP4 4.
template <int CLASS>
struct Slot {
    static constexpr int W = is_cb<CLASS> ? 3 : 4;
};

// Wave-uniform description of the matrix part one wave computes in an item:
// row blocks rb0, rb0+1 (16 rows each) of a matrix with G 128-column groups
// per row, groups g0 .. g0+NG-1.
struct WaveJob {
    gu32p codes;
    gu8p scales;
    const uint16_t *lut;
    float ts;
    int bits;
    int G, rb0, g0;
    // entry i of a 6-bit codebook (i < 64)
    __device__ __forceinline__ _Float16 lut6(int i) const
    {
        return __builtin_bit_cast(_Float16, *(const uint16_t GLOBAL *)(lut + i));
    }
};

// One register buffer of weight data: one 128-column group of the wave's
// kWaveRB row blocks (tiles), with the lane's scales of each tile: the fp16
// group scale (codebook) or the two e4m3 block scales (NVFP4).
template <int CLASS, int NT = kWaveRB>
struct GroupBuf {
    uint32_t w[NT][Slot<CLASS>::W];
    uint32_t sc[NT];
};

// A wave-uniform value the compiler cannot prove uniform (it flows through
// loop-carried state), moved to scalar registers.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t uniform(uint64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Buffer resource over a read-only tensor (wave-uniform base).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tensor_rsrc(const void GLOBAL *base)
{
    const uint64_t b = uniform((uint64_t)(uintptr_t)base);
    return __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)b, 0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base)
{
    return tensor_rsrc((const void GLOBAL *)(uintptr_t)base);
}

// Load group j (absolute group g0 + j) of job J into b (NT tiles). KB: codebook bits
// when known at compile time, 0 to read them from the job. Buffer loads with
// the tile offset in a scalar register and one per-lane offset, so a load in
// flight holds no address registers; one VMEM instruction per tile whatever
// the bit width, so the waits the compiler places stay exact when the next
// item's width differs.
// 6-bit codes: a wave takes 2 tiles per group (kWaveRB / 2); a 6-bit tile
// stores words 0..2 of its 64 slots, then words 3..5, so a lane's half slots
// load exactly like a 3-bit slot (lane offset 12 bytes, the half in the
// scalar offset) into buffer rows 2r (columns 0..15) and 2r + 1 (16..31):
// same buffer shape, same count of loads, no extra address registers.
template <int CLASS, int KB, int NT = kWaveRB>
__device__ __forceinline__ void load_group(GroupBuf<CLASS, NT> &b, const WaveJob &J, int j, int lane,
                                           int sc_lane)
{
    const __amdgpu_buffer_rsrc_t rc = tensor_rsrc(J.codes);
    const __amdgpu_buffer_rsrc_t rsc = tensor_rsrc(J.scales);
    const bool six = has6<CLASS> && J.bits == 6;
    const int g = J.g0 + j;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int trow = six ? J.rb0 + (i >> 1) : J.rb0 + i;  // tile row block
        const int tile = trow * J.G + g;
        if constexpr (is_cb<CLASS>) {
            // one load instruction for 3-bit and 6-bit (the width only moves
            // the scalar offset): separate loads would have to be merged by
            // register copies, which wait for the loads at once
            // (the words are merged after the branch and stored once: stores
            // to different words in the two branches get merged through a
            // computed address, which sends the buffer to stack memory)
            uint32_t w0, w1, w2 = b.w[i][2];
            if (KB == 3 || (KB == 0 && (J.bits == 3 || six))) {
                const int soff = six ? tile * 1536 + (i & 1) * 768 : tile * 768;
                const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rc, lane * 12, soff, 0);
                w0 = v[0];
                w1 = v[1];
                w2 = v[2];
            } else {
                const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rc, lane * 8, tile * 512, 0);
                w0 = v[0];
                w1 = v[1];
            }
            b.w[i][0] = w0;
            b.w[i][1] = w1;
            b.w[i][2] = w2;
            // the tile's 16 row scales are contiguous (tile order): lane
            // offset 2 (lane % 16)
            b.sc[i] = __builtin_amdgcn_raw_buffer_load_b16(rsc, sc_lane, tile * 32, 0);
        } else {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, lane * 16, tile * 1024, 0);
            b.w[i][0] = v[0];
            b.w[i][1] = v[1];
            b.w[i][2] = v[2];
            b.w[i][3] = v[3];
            // the tile's 16 x 8 block scales are contiguous (tile order, row
            // major): lane offset 8 (lane % 16) + 2 (lane / 16)
            b.sc[i] = __builtin_amdgcn_raw_buffer_load_b16(rsc, sc_lane, tile * 128, 0);
        }
    }
}

// MFMA 16x16x32: A = tokens x 32 columns from the staged activations in LDS
// (row = token), B = 32 columns x 16 rows of W; lane (r = lane%16,
// q = lane/16) supplies token r / W row r and columns 32q + 8s .. +7 of the
// group at step s. Result: lane holds tokens 4(lane/16)+i of W row lane%16,
// so each lane scales by one group scale. A rows >= R (tokens the group does
// not have) only reach result rows that are never stored, so lanes r >= R
// simply read row R-1. j = group index within the item (LDS column block).
template <int CLASS, int FMT>
__device__ __forceinline__ void process_group(const GroupBuf<CLASS> &b, int j, const _Float16 *Arow,
                                              const uint32_t (&tab)[4], floatx4 (&acc)[kWaveRB])
{
    half8 a[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        a[s] = *(const half8 *)(Arow + j * 128 + s * 8);
#pragma unroll
    for (int i = 0; i < kWaveRB; ++i) {
        half2v bs_lo = half2v{1, 1}, bs_hi = half2v{1, 1};
        if constexpr (FMT == 4) {
            const _Float16 lo = (_Float16)__builtin_amdgcn_cvt_f32_fp8(b.sc[i], 0);
            const _Float16 hi = (_Float16)__builtin_amdgcn_cvt_f32_fp8(b.sc[i], 1);
            bs_lo = half2v{lo, lo};
            bs_hi = half2v{hi, hi};
        }
        floatx4 cc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const half8 bv = decode_step<FMT>(b.w[i], s, tab, s < 2 ? bs_lo : bs_hi);
            cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[s], bv, cc, 0, 0, 0);
        }
        if constexpr (FMT == 4) {
            acc[i] += cc;
        } else {
            const float f = (float)__builtin_bit_cast(_Float16, (uint16_t)b.sc[i]);
            acc[i] += f * cc;
        }
        // keep the accumulation here: sunk to the end it would keep every
        // group's MFMA result live at once
        asm volatile("" : "+v"(acc[i]));
    }
}

// Codebooks of 6-bit tensors in LDS, one per pair of waves (waves 0-1 and 2-3
// compute the same tensor in every item): 64 fp16 entries each.
constexpr int kLut6Slots = 2;
__shared__ _Float16 s_lut6[kLut6Slots * 64];

// The 8 fp16 B-operand values of step sp (0 or 1) of a 6-bit half slot: the
// half's 16 codes are bits 6c .. 6c+5 of w[0..2] read as a 96-bit
// little-endian string. Each code, shifted to bits 1-6 and or-ed with the
// wave's codebook base (lbase = 128 x slot), is the byte address of its
// fp16 entry.
__device__ __forceinline__ half8 decode6(const uint32_t (&w)[3], int sp, uint32_t lbase)
{
    const char *T = (const char *)s_lut6;
    uint32_t o[4];
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2) {
        _Float16 v[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int q = 6 * (8 * sp + 2 * c2 + e), wd = q >> 5, off = q & 31;
            uint32_t x;
            if (off == 0)
                x = w[wd] << 1;
            else if (off <= 26)
                x = w[wd] >> (off - 1);
            else
                x = __builtin_amdgcn_alignbit(w[wd + 1], w[wd], off - 1);
            v[e] = *(const _Float16 *)(T + ((x & 0x7Eu) | lbase));
        }
        o[c2] = __builtin_bit_cast(uint32_t, half2v{v[0], v[1]});
    }
    return __builtin_bit_cast(half8, u32x4{o[0], o[1], o[2], o[3]});
}

// Group j of a 6-bit item: 2 tiles; steps 0-1 of tile r come from buffer
// row 2r, steps 2-3 from row 2r + 1. Results accumulate in acc[0], acc[1].
template <int CLASS>
__device__ __forceinline__ void process_group6(const GroupBuf<CLASS> &b, int j, const _Float16 *Arow,
                                               uint32_t lbase, floatx4 (&acc)[kWaveRB])
{
    half8 a[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        a[s] = *(const half8 *)(Arow + j * 128 + s * 8);
#pragma unroll
    for (int r = 0; r < kWaveRB / 2; ++r) {
        floatx4 cc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
            cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[s], decode6(b.w[2 * r + (s >> 1)], s & 1, lbase),
                                                         cc, 0, 0, 0);
        const float f = (float)__builtin_bit_cast(_Float16, (uint16_t)b.sc[2 * r]);
        acc[r] += f * cc;
        asm volatile("" : "+v"(acc[r]));
    }
}

// Group j of the current item: the codebook bit width is a runtime property
// of the tensor, dispatched here around the decode and MFMAs only, so the
// buffers loaded outside stay in the same registers on both paths.
template <int CLASS>
__device__ __forceinline__ void process_any(const GroupBuf<CLASS> &b, int j, int bits,
                                            const _Float16 *Arow, const uint32_t (&tab)[4],
                                            uint32_t lbase, floatx4 (&acc)[kWaveRB])
{
    if constexpr (is_cb<CLASS>) {
        if (bits == 3)
            process_group<CLASS, 3>(b, j, Arow, tab, acc);
        else if (has6<CLASS> && bits == 6)
            process_group6<CLASS>(b, j, Arow, lbase, acc);
        else
            process_group<CLASS, 2>(b, j, Arow, tab, acc);
    } else {
        process_group<CLASS, 4>(b, j, Arow, tab, acc);
    }
}

// The NG groups of the current chunk from two register buffers used in turn,
// accumulated into acc. `after(j, buf)` runs once group j is consumed, with
// the buffer that held it: it loads what that buffer holds next (group j+2 of
// this chunk, or one of the first two groups of the next chunk or item).
// Wave priority (wave-uniform p, 0..3). The issue arbiter picks the highest
// priority first and the oldest wave among equals.
__device__ __forceinline__ void set_prio(int p)
{
    switch (p & 3) {
    case 0: __builtin_amdgcn_s_setprio(0); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    default: __builtin_amdgcn_s_setprio(3); break;
    }
}

// Groups 0..NG-1 of a row block. Before group j a gate/up wave takes
// priority (rot + j) mod 4, rot = the block's residency slot on its CU (0..3),
// so the four gate/up blocks of a CU take turns at each level instead of the
// oldest always going first (the arbiter's order among equal priorities);
// down items take priority 0, where the gate/up work (whose h they wait for)
// meets them a quarter of the time.
template <int CLASS, int NG, typename After>
__device__ __forceinline__ void compute_chunk(GroupBuf<CLASS> &bA, GroupBuf<CLASS> &bB, int bits,
                                              const _Float16 *Arow, const uint32_t (&tab)[4],
                                              uint32_t lbase, floatx4 (&acc)[kWaveRB], After &after,
                                              int rot, bool down)
{
#pragma unroll
    for (int j = 0; j < NG; ++j) {
        set_prio(down ? 0 : (rot + j) & 3);
        GroupBuf<CLASS> &b = (j & 1) ? bB : bA;
        process_any<CLASS>(b, j, bits, Arow, tab, lbase, acc);
        after(j, b);
    }
}

// ---------------------------------------------------------------------------
// Expert kernel: work items
// ---------------------------------------------------------------------------

// One work item: gate/up (row group u = expert e's rows off..off+R-1, 128-row
// block rb of gate and up, column split kq) or down (256-row block rb of
// down, column split kq).
// Work item: row group u (expert e, bucket rows off..off+R-1), column split
// kq, `span` consecutive row blocks from rb (128 rows each for gate/up, 256
// rows for down).
struct Item {
    int valid, down, e, off, R, u, rb, kq, span;
    int half;  // -1: whole row blocks; 0 / 1: that half of row block rb only
};

// Row-group table of the plan, cached in LDS by every block (in the dynamic
// LDS, after the staged rows, p.gcap entries each): expert, first bucket row
// and rows of group u.
struct GroupLds {
    const int *expert, *off, *rows;
};

// Ticket t of a phase (gate/up, then down) maps to a row group, a row block
// and a column split; the shared expert's groups come first. Where its items
// cover half row blocks (6-bit codes), a row block has two halves per split.
// Gate/up items of the first n_wide routed groups cover span1 row blocks, the
// later groups' items one.
__device__ __forceinline__ Item make_item(const Params &p, int n_items, int n_items1, int n_sg,
                                          int n_wide, const GroupLds &gl, int ticket)
{
    Item it{};
    it.valid = ticket < n_items;
    it.half = -1;
    if (!it.valid)
        return it;
    it.down = ticket >= n_items1;
    int t = it.down ? ticket - n_items1 : ticket;
    const int ks = it.down ? p.ks2 : p.ks1;
    const int per_s = shared_items(p, it.down);
    if (t < n_sg * per_s) {
        it.u = t / per_s;
        const int rem = t - it.u * per_s;
        const int rbh = rem / ks;  // row block (or half row block) index
        it.kq = rem - rbh * ks;
        it.span = p.sh_half ? 1 : (it.down ? 1 : p.span1);
        it.rb = p.sh_half ? rbh >> 1 : rbh * it.span;
        if (p.sh_half)
            it.half = rbh & 1;
    } else {
        t -= n_sg * per_s;
        int u0 = n_sg;
        it.span = it.down ? 1 : p.span1;
        if (!it.down && t >= n_wide * (p.n_rb1 / p.span1) * ks) {
            // past the wide groups: one row block per item
            t -= n_wide * (p.n_rb1 / p.span1) * ks;
            u0 += n_wide;
            it.span = 1;
        }
        const int per_u = (it.down ? p.n_rb2 : p.n_rb1 / it.span) * ks;
        const int v = t / per_u;
        const int rem = t - v * per_u;
        const int rbs = rem / ks;
        it.u = u0 + v;
        it.rb = rbs * it.span;
        it.kq = rem - rbs * ks;
    }
    it.e = uniform(gl.expert[it.u]);
    it.off = uniform(gl.off[it.u]);
    it.R = uniform(gl.rows[it.u]);
    return it;
}

// The stored-tensor descriptor of the matrix wave `wave` computes for item
// `it`, fetched with vector loads (they are waited on through vmcnt, in
// order with the weight prefetches, instead of sharing lgkmcnt with the LDS
// reads of the inner loop). An invalid item reads descriptor 0.
struct DescRaw {
    u32x4 d0, d1;
};

__device__ __forceinline__ int item_proj(const Item &it, int wave)
{
    // gate/up items: the first half of the waves gate, the second half up
    return it.down ? 2 : wave / (kExpertWaves / 2);
}

__device__ __forceinline__ DescRaw load_desc(const Params &p, const Item &it, int wave)
{
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<DevTensor *>(p.tensors), 0, 0x7FFFFFFF, 0x00020000);
    const int idx = it.valid ? it.e * 3 + item_proj(it, wave) : 0;
    DescRaw d;
    d.d0 = __builtin_amdgcn_raw_buffer_load_b128(r, 0, idx * (int)sizeof(DevTensor), 0);
    d.d1 = __builtin_amdgcn_raw_buffer_load_b128(r, 16, idx * (int)sizeof(DevTensor), 0);
    return d;
}

// For lane r16, bucket row q = off + min(r16, R-1) of the item's group: the
// pair index of q (t*k + j for a routed row, q itself for the shared expert's
// row m*k + t: the bucket row list holds both), under which a down item's
// partial sums are stored. Loaded one item ahead with the item's descriptor,
// unconditionally (an invalid item reads entry 0), and nothing is computed
// from it at the load: the wait for it lands where it is first used.
__device__ __forceinline__ int load_pair(const Params &p, const Item &it, int r16)
{
    const int q = it.valid ? it.off + min(r16, it.R - 1) : 0;
    return p.rows[q];
}

// The token of pair index pr (m*k = mk routed pairs, then the shared rows).
__device__ __forceinline__ int pair_token(int pr, int mk, int k)
{
    return pr < mk ? pr / k : pr - mk;
}

// The matrix part wave `wave` computes for item `it`: a gate/up item's 128
// rows of gate and of up go to the two halves of the waves, a down item's 256
// rows to all waves, kWaveRB row blocks of 16 each.
template <int CLASS, int NG>
__device__ __forceinline__ WaveJob make_job(const Params &p, const DescRaw &d, const Item &it,
                                            int wave)
{
    static_assert(sizeof(DevTensor) == 32, "descriptor layout");
    WaveJob J;
    J.codes = (gu32p)(uintptr_t)uniform(((uint64_t)d.d0[1] << 32) | d.d0[0]);
    J.scales = (gu8p)(uintptr_t)uniform(((uint64_t)d.d0[3] << 32) | d.d0[2]);
    J.lut = (const uint16_t *)(uintptr_t)uniform(((uint64_t)d.d1[1] << 32) | d.d1[0]);
    J.ts = __uint_as_float((uint32_t)uniform((int)d.d1[2]));
    J.bits = uniform((int)d.d1[3]);
    J.G = it.down ? p.I / 128 : p.H / 128;
    // a 6-bit wave takes kWaveRB / 2 tiles per row block unit (see load_group)
    const int per_wave = has6<CLASS> && J.bits == 6 ? kWaveRB / 2 : kWaveRB;
    // a half-row-block item starts at its half (16-row tiles: 8 per gate/up
    // row block, 16 per down row block)
    const int hoff = it.half > 0 ? (it.down ? 8 : 4) : 0;
    J.rb0 = it.down ? it.rb * 16 + hoff + wave * per_wave
                    : it.rb * 8 + hoff + (wave % (kExpertWaves / 2)) * per_wave;
    J.g0 = it.kq * NG;
    return J;
}

constexpr int kMaxSpan = 2;  // row blocks per gate/up item

struct Smem {
    int flag;
    int last[kMaxSpan];  // this item's split was the last of row block rb + s
};

// Last column split of a gate/up block: h = silu(g) * u over rows
// rb*128..+127 of each token, then (codebook) h~ = (1/sqrt 128) H_128 (s_I h).
// One wave per token; a wave issues the partial-sum loads of two tokens and
// four splits together.
__device__ void finish_h(const Params &p, int off, int R, int rb)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = rb * 128 + 2 * lane;
    // the signs of the lane's two columns (codebook), loaded once with the
    // first sums
    const uint16_t sg = p.format == kFmtCodebook ? *(const uint16_t *)(p.signs_i + n) : 0;
    constexpr int TPP = 2;  // tokens per pass
    for (int t0 = wave; t0 < R; t0 += TPP * kExpertWaves) {
        floatx2 g[TPP], u[TPP];
#pragma unroll
        for (int ti = 0; ti < TPP; ++ti) {
            g[ti] = floatx2{0.f, 0.f};
            u[ti] = floatx2{0.f, 0.f};
        }
        for (int s0 = 0; s0 < p.ks1; s0 += 4) {
            uint64_t vg[TPP][4], vu[TPP][4];
#pragma unroll
            for (int ti = 0; ti < TPP; ++ti)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int tok = t0 + kExpertWaves * ti;
                    vg[ti][s] = vu[ti][s] = 0;
                    if (tok < R && s0 + s < p.ks1) {
                        const size_t row = (size_t)(s0 + s) * p.pair_cap + off + tok;
                        vg[ti][s] = ld_coherent((const uint64_t *)(p.gu_part + (row * 2 + 0) * p.I + n));
                        vu[ti][s] = ld_coherent((const uint64_t *)(p.gu_part + (row * 2 + 1) * p.I + n));
                    }
                }
#pragma unroll
            for (int ti = 0; ti < TPP; ++ti)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    if (s0 + s < p.ks1) {
                        g[ti] += __builtin_bit_cast(floatx2, vg[ti][s]);
                        u[ti] += __builtin_bit_cast(floatx2, vu[ti][s]);
                    }
        }
#pragma unroll
        for (int ti = 0; ti < TPP; ++ti) {
            const int tok = t0 + kExpertWaves * ti;
            if (tok >= R)
                break;
            float v0 = g[ti][0] / (1.0f + expf(-g[ti][0])) * u[ti][0];
            float v1 = g[ti][1] / (1.0f + expf(-g[ti][1])) * u[ti][1];
            if (p.format == kFmtCodebook) {
                v0 *= (float)(int8_t)(sg & 0xFF);
                v1 *= (float)(int8_t)(sg >> 8);
                wave_fwht128(v0, v1);
                v0 *= kInvSqrt128;
                v1 *= kInvSqrt128;
            }
            st_coherent((uint32_t *)(p.hr + (size_t)(off + tok) * p.I + n),
                        __builtin_bit_cast(uint32_t, half2v{(_Float16)v0, (_Float16)v1}));
        }
    }
    // every load above complete on every path (the caller waits for the
    // stores next anyway): a load taken on one path only would otherwise
    // look pending in the next item, whose first register writes would then
    // wait for every load in flight
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

// Wait until row group u's h counter reaches `target` (bounded): every
// 128-row block of h~ written (persistent kernel), or every gate/up item of
// the group counted (small-m kernel). The pause between polls doubles up to
// about a microsecond, so waiting blocks add little traffic to the counter
// the producers increment.
__device__ __forceinline__ bool wait_h(const Params &p, int u, uint32_t target)
{
    uint32_t polls = 0;
    int pause = 1;
    while (atomic_load_agent(&p.h_ready[u * kCtrStride]) < target) {
        for (int i = 0; i < pause; ++i)
            __builtin_amdgcn_s_sleep(4);
        pause = min(2 * pause, 8);
        if (++polls > p.spin_limit) {
            __hip_atomic_fetch_or(&p.ctr->error_word, kErrSpinLimit, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
    }
    return true;
}

// Staged activations of one item, R rows x KC columns of fp16:
// gate/up items stage the rotated activations of the group's tokens, down
// items stage h~ of the group's rows. Thread tid moves 16-byte chunks
// tid, tid + kExpertThreads, ...; a wave skips the rounds that lie wholly past
// the last chunk, and inside a round indices past the end are clamped to the
// last chunk (a duplicate write of the same value). issue() starts the loads,
// commit() writes them to LDS once they are needed: loads issued in between
// (the chunk's first weight groups) stay in flight.
template <int NG>
struct Stage {
    static constexpr int KC = NG * 128;
    static constexpr int CHUNKS = KC / 8;
    static constexpr int ITERS = (kGroupRows * CHUNKS + kExpertThreads - 1) / kExpertThreads;
    static constexpr int ASTRIDE = KC + kLdsPadHalves;   // LDS row stride (halves)
    u32x4 v[ITERS];

    // tok: the token of row r16 (lane r of each wave holds row r's). The two
    // kinds of item take separate loops on a scalar branch: code shared by
    // both paths would make a load of one path look pending in the other,
    // where the compiler then waits for it before every staging load.
    // Offsets are 32-bit (the buffers are far below 2 GB).
    __device__ __forceinline__ void issue(const Params &p, const Item &it, int tok)
    {
        const int tid = threadIdx.x, last = it.R * CHUNKS - 1;
        const int wave_first = uniform(tid & ~63);
        const int col0 = it.kq * KC;
#pragma unroll
        for (int k = 0; k < ITERS; ++k)
            v[k] = u32x4{0, 0, 0, 0};
        if (uniform(it.down)) {
            // h~ rows off..off+R-1 are consecutive: one coherent buffer
            const _Float16 *base = p.hr + (size_t)uniform(it.off) * p.I + col0;
#pragma unroll
            for (int k = 0; k < ITERS; ++k) {
                if (wave_first + k * kExpertThreads > last)
                    continue;
                const int i = min(tid + k * kExpertThreads, last);
                const int r = i / CHUNKS, cc = (i - r * CHUNKS) * 8;
                v[k] = ld_coherent16(base, (uint32_t)(r * p.I + cc) * 2u);
            }
            // complete here, in their own branch (commit needs them next
            // anyway): the compiler's wait placement otherwise takes them
            // for pending at the start of the gate/up branch
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        } else {
            const __amdgpu_buffer_rsrc_t rs = buf_rsrc(p.xr + col0);
            const uint32_t hb = (uint32_t)p.H * 2u;  // bytes per activation row
#pragma unroll
            for (int k = 0; k < ITERS; ++k) {
                if (wave_first + k * kExpertThreads > last)
                    continue;
                const int i = min(tid + k * kExpertThreads, last);
                const int r = i / CHUNKS, cc = (i - r * CHUNKS) * 8;
                const uint32_t off = __umul24((uint32_t)__shfl(tok, r), hb) + (uint32_t)cc * 2u;
                v[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
            }
        }
    }
    // Every staging load is complete after the first wait below on every
    // path (they are the item's last loads, so nothing else is waited for):
    // waited for only inside the rounds a wave writes, the loads of the
    // rounds it skips would look pending past the item, and the next item's
    // first writes of these registers would wait for every load in flight.
    __device__ __forceinline__ void commit(const Item &it, _Float16 *A) const
    {
        const int tid = threadIdx.x, last = it.R * CHUNKS - 1;
        const int wave_first = uniform(tid & ~63);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
#pragma unroll
        for (int k = 0; k < ITERS; ++k) {
            if (wave_first + k * kExpertThreads > last)
                continue;
            const int i = min(tid + k * kExpertThreads, last);
            const int r = i / CHUNKS, cc = (i - r * CHUNKS) * 8;
            *(u32x4 *)(A + r * ASTRIDE + cc) = v[k];
        }
    }
};

// Store the partial sums of one row block of an item (rows rb0.. of job J).
// Gate/up partials go out agent-coherent (sc1) for the finishing block, under
// the bucket row; down partials, read only by the combine kernel after this
// kernel ends, under the row's pair index (pair: see load_pair), so that the
// combine reads them without the bucket positions. Both are written through
// (sc1): the down partials then reach memory while the kernel runs instead of
// in the write-back of dirty L2 lines at its end, ahead of the combine
// (measured 0.2-0.6 us less per layer at m = 1..24). One 32-bit offset per
// token row; the tiles differ by a constant 64 bytes.
template <int CLASS>
__device__ __forceinline__ void store_rows(const Params &p, const Item &it, const WaveJob &J,
                                           const floatx4 (&acc)[kWaveRB], int pair)
{
    const int tid = threadIdx.x;
    // the lane index, opaque to the compiler: the offsets below are
    // recomputed at each call instead of being hoisted to the kernel start
    // and held (or spilled) across the whole item loop
    int lane = tid & 63;
    asm volatile("" : "+v"(lane));
    const int ntiles = has6<CLASS> && J.bits == 6 ? kWaveRB / 2 : kWaveRB;  // 6-bit: 2 per wave
    const int q4 = 4 * (lane >> 4), R = uniform(it.R);
    const uint32_t col = (uint32_t)(J.rb0 * 16 + (lane & 15)) * 4u;  // byte offset of W row n
    if (uniform(it.down)) {
        const __amdgpu_buffer_rsrc_t rs =
            buf_rsrc(p.y_part + (size_t)uniform(it.kq) * p.pair_cap * p.H);
        const uint32_t hb = (uint32_t)p.H * 4u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t off = __umul24((uint32_t)__shfl(pair, q4 + j), hb) + col;
            if (q4 + j < R)
#pragma unroll
                for (int i = 0; i < kWaveRB; ++i)
                    if (i < ntiles)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j]), rs,
                                                              (int)off, i * 64, 16 /* sc1 */);
        }
    } else {
        const int proj = item_proj(it, tid >> 6);
        const __amdgpu_buffer_rsrc_t rs = buf_rsrc(
            p.gu_part + (((size_t)uniform(it.kq) * p.pair_cap + uniform(it.off)) * 2 + proj) * p.I);
        const uint32_t rb = (uint32_t)p.I * 8u;  // bytes per bucket row (gate and up)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t off = __umul24((uint32_t)(q4 + j), rb) + col;
            if (q4 + j < R)
#pragma unroll
                for (int i = 0; i < kWaveRB; ++i)
                    if (i < ntiles)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j]), rs,
                                                              (int)off, i * 64, 16 /* sc1 */);
        }
    }
}

// After a gate/up item's stores: once they are acknowledged, count the item's
// split in each of its row blocks; the last split of a row block finishes
// that block of h, and the group's h counter goes up by the blocks finished.
__device__ __forceinline__ void complete_item(const Params &p, const Item &it, Smem &sm)
{
    const int tid = threadIdx.x;
    if (it.down)
        return;
    __builtin_amdgcn_s_setprio(3);  // finishing h is on the down items' path
    wait_stores();
    __syncthreads();
    // a row block's arrivals: one per column split, or two (one per half)
    const uint32_t arrivals = (uint32_t)(p.ks1 << (it.half >= 0 ? 1 : 0));
    if (tid < it.span)
        sm.last[tid] = atomic_add_agent(&p.rb_done[(it.u * p.n_rb1 + it.rb + tid) * kCtrStride],
                                        1u) == arrivals - 1u;
    __syncthreads();
    int finished = 0;
    for (int s = 0; s < it.span; ++s)
        if (sm.last[s]) {
            finish_h(p, it.off, it.R, it.rb + s);
            ++finished;
        }
    if (finished) {
        wait_stores();
        __syncthreads();
        if (tid == 0)
            atomic_add_agent(&p.h_ready[it.u * kCtrStride], (uint32_t)finished);
    }
}

// The codebook of job J as stored, read through a buffer resource whose size
// is the codebook's: for a 2-bit codebook the upper 8 bytes are out of range
// and read as zero without touching memory.
__device__ __forceinline__ u32x4 load_lut_raw(const WaveJob &J)
{
    const uint64_t base = uniform((uint64_t)(uintptr_t)J.lut);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(uintptr_t)base, 0, 2 << J.bits, 0x00020000);
    const u32x2 lo = __builtin_amdgcn_raw_buffer_load_b64(r, 0, 0, 0);
    const u32x2 hi = __builtin_amdgcn_raw_buffer_load_b64(r, 8, 0, 0);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Persistent block: block b takes items b, b + G, b + 2G, ... (G = grid
// size) in order. The assignment is static: claiming items from shared
// counters puts the blocks' atomics on a few addresses, and such atomics
// serialize across the chip (measured slower than the static order here). No
// wait can deadlock: every block finishes all its gate/up items (which never
// wait) before its first down item, and every block is resident.
// An item stages its activation rows in LDS once, then for each row block of
// its span runs the 128-column weight groups through two register buffers,
// two groups in flight, the next row block's first groups loaded as the
// current one ends (same activations: no barrier in between). Nothing is
// prefetched across an item boundary: vector memory counters retire in order,
// so a load issued before the boundary would hold up the staging and the
// tail's store acknowledgements behind it. Instead the staging loads go first
// and the item's first weight groups right behind them. Four waves per SIMD (four blocks per CU, the
// 128-register budget): other blocks' groups cover each block's staging and
// tail latencies.
template <int CLASS, int NG>
__global__ __launch_bounds__(kExpertThreads) __attribute__((amdgpu_waves_per_eu(4)))
void expert_kernel(Params p)
{
    extern __shared__ __align__(16) _Float16 Abuf[];  // min(m, 16) staged rows, then the row-group table
    __shared__ Smem sm;
    using St = Stage<NG>;
    const Plan *P = p.plan;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int r16 = lane & 15, q = lane >> 4;
    // 6-bit codebook slot: the waves of one gate/up half (same tensor in every item)
    const uint32_t lut_slot = (uint32_t)(wave / (kExpertWaves / kLut6Slots));
    const int m = uniform(P->m), n_items = uniform(P->n_items), n_items1 = uniform(P->n_items1);
    const int n_sg = uniform(P->n_sgroups), n_wide = uniform(P->n_wide);

    int *s_tab = (int *)((char *)Abuf + p.lds_tab);
    const GroupLds s_grp{s_tab, s_tab + p.gcap, s_tab + 2 * p.gcap};
    // all p.gcap entries (the run's bound; entries past its groups are never
    // read): the loads need not wait for the plan's group count
    for (int i = tid; i < p.gcap; i += kExpertThreads) {
        s_tab[i] = P->g_expert[i];
        s_tab[p.gcap + i] = P->g_off[i];
        s_tab[2 * p.gcap + i] = P->g_rows[i];
    }
    __syncthreads();

    int ticket = blockIdx.x;
    // residency slot: blocks b, b + C, b + 2C, ... (C = grid / blocks per CU)
    // share a CU, dispatched in that order
    const int rot = uniform((int)(blockIdx.x / max(1u, gridDim.x / 4u))) & 3;
    Item cur = make_item(p, n_items, n_items1, n_sg, n_wide, s_grp, ticket);
    int pair = load_pair(p, cur, r16);
    uint32_t done = 0;
    if (cur.valid) {
        GroupBuf<CLASS> bA, bB;
        int sb = 0;  // row block of cur's span being computed
        WaveJob J = make_job<CLASS, NG>(p, load_desc(p, cur, wave), cur, wave);
        uint32_t tab[4] = {0, 0, 0, 0};

        while (true) {
            // 6-bit items: each row block takes two units of half the rows
            const int six = (has6<CLASS> && J.bits == 6) ? 1 : 0;
            const bool last = sb + 1 == (cur.half >= 0 ? 1 : cur.span << six);
            const int sc_lane = is_cb<CLASS> ? r16 * 2 : r16 * 8 + 2 * q;
            // after the item's last row block comes the next item: its plan
            // entries (LDS) and descriptor (vector loads)
            const int nxt_ticket = ticket + (int)gridDim.x;
            const Item nxt = make_item(p, n_items, n_items1, n_sg, n_wide, s_grp,
                                       last ? nxt_ticket : n_items);
            const DescRaw dn = load_desc(p, nxt, wave);
            const int pair_n = load_pair(p, nxt, r16);

            bool ok = true;
            if (sb == 0) {
                // the item's codebook and first two weight groups, then (down
                // items: once thread 0 has seen the group's h complete, a
                // bounded wait) its activation rows: the weights do not
                // depend on h and load during the wait
                // the item's loads leave first, at the top priority
                __builtin_amdgcn_s_setprio(3);
                u32x4 lut = u32x4{0, 0, 0, 0};
                _Float16 lut6 = 0;
                if constexpr (is_cb<CLASS>) {
                    lut = load_lut_raw(J);
                    if (has6<CLASS> && J.bits == 6)
                        lut6 = J.lut6(lane);
                }
                load_group<CLASS, 0>(bA, J, 0, lane, sc_lane);
                if constexpr (NG > 1)
                    load_group<CLASS, 0>(bB, J, 1, lane, sc_lane);
                if (cur.down) {
                    __builtin_amdgcn_s_setprio(0);  // waiting yields to the others
                    if (tid == 0)
                        sm.flag = wait_h(p, cur.u, (uint32_t)p.n_rb1);
                    lds_barrier();  // the weight groups stay in flight
                    ok = sm.flag != 0;
                }
                St st;
                st.issue(p, cur, pair_token(pair, m * p.k, p.k));
                st.commit(cur, Abuf);
                // a 6-bit codebook goes to the wave pair's LDS slot (the waves
                // sharing it write the same values)
                if (has6<CLASS> && J.bits == 6)
                    s_lut6[lut_slot * 64 + lane] = lut6;
                __syncthreads();
                if constexpr (is_cb<CLASS>)
                    lut_tables(lut, tab);
            }
            // after group j, the freed buffer takes this row block's group
            // j+2, else group j+2-NG of the span's next row block (same
            // activations and tensor: no staging in between)
            WaveJob JN = J;
            JN.rb0 += (cur.down ? 16 : 8) >> six;
            auto after = [&](int j, GroupBuf<CLASS> &b) {
                const int nx = NG == 1 ? 0 : j + 2 - NG;
                if (NG > 1 && j + 2 < NG)
                    load_group<CLASS, 0>(b, J, j + 2, lane, sc_lane);
                else if (!last && nx >= 0)
                    load_group<CLASS, 0>(b, JN, nx, lane, sc_lane);
            };
            const _Float16 *Arow = Abuf + min(r16, cur.R - 1) * St::ASTRIDE + q * 32;
            floatx4 acc[kWaveRB];
#pragma unroll
            for (int i = 0; i < kWaveRB; ++i)
                acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
            compute_chunk<CLASS, NG>(bA, bB, J.bits, Arow, tab, lut_slot * 128u, acc, after, rot,
                                     cur.down != 0);
            if constexpr (!is_cb<CLASS>)
#pragma unroll
                for (int i = 0; i < kWaveRB; ++i)
                    acc[i] *= J.ts;
            if (ok)
                store_rows<CLASS>(p, cur, J, acc, pair);
            if (!last) {
                ++sb;
                J = JN;
                continue;
            }
            if (ok)
                complete_item(p, cur, sm);
            ++done;
            // the staged rows and sm are the next item's (a down item's
            // partial-sum stores need no acknowledgement: read by the
            // combine kernel only)
            lds_barrier();
            if (!nxt.valid)
                break;
            ticket = nxt_ticket;
            cur = nxt;
            pair = pair_n;
            sb = 0;
            // every descriptor word stays live until here: one the kernel
            // does not use would free its register for a temporary, whose
            // first write then waits for the load still on its way into it
            asm volatile("" ::"v"(dn.d0), "v"(dn.d1));
            J = make_job<CLASS, NG>(p, dn, nxt, wave);
        }
    }
    if (tid == 0 && done)
        atomic_add_agent(&p.ctr->items_done[blockIdx.x % kDoneSlots], done);
}

// ---------------------------------------------------------------------------
// Small-m kernel (up to kSmallMaxTokens tokens): items by rows, all columns
// ---------------------------------------------------------------------------
// With one to four tokens the persistent kernel's column splits leave part of
// the grid idle and put a round trip between gate/up and down (partial sums,
// a split counter, the finishing block, the h counter). Here a gate/up item is
// 32 rows of gate and of up over all H columns (waves 0-1 gate, 2-3 up, one
// 16-row tile each): its sums are whole, so the item applies SiLU(g) u itself
// and stores h for its rows (fp32, not yet rotated), then counts on its row
// group's h counter. A down item is 64 rows of down over all I columns (one
// tile per wave): it loads its first kSmDepth weight groups, waits until
// every gate/up item of its group has counted, rotates h~ from h (one wave per
// token and 128-column block: the same fp32 arithmetic as the persistent
// kernel's finishing block), and writes y whole (one split). A wave streams
// its tile through kSmDepth register buffers, so a waiting down item already
// has its first groups in flight. Tickets: the gate/up items of every row
// group, then the down items; block b takes b, b + G, ... in order (no wait
// can deadlock, as in the persistent kernel). Plan, buckets, combine: shared
// with the persistent kernel.
constexpr int kSmGuRows = 32;      // rows of gate and of up per gate/up item
constexpr int kSmDnRows = 64;      // rows of down per down item
constexpr int kSmDepth = 8;        // weight groups in flight per wave
constexpr int kSmStageIters = 8;   // 16-byte staging loads per thread (R x H <= 16384)
constexpr int kSmRotBatch = 4;     // h loads a wave issues together when rotating

// Group j of one 16-row tile (buffer b) against the staged rows: as
// process_group, for one tile.
template <int CLASS, int FMT>
__device__ __forceinline__ void sm_group(const GroupBuf<CLASS, 1> &b, const _Float16 *Ag,
                                         const uint32_t (&tab)[4], floatx4 &acc)
{
    half8 a[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        a[s] = *(const half8 *)(Ag + s * 8);
    half2v bs_lo = half2v{1, 1}, bs_hi = half2v{1, 1};
    if constexpr (FMT == 4) {
        const _Float16 lo = (_Float16)__builtin_amdgcn_cvt_f32_fp8(b.sc[0], 0);
        const _Float16 hi = (_Float16)__builtin_amdgcn_cvt_f32_fp8(b.sc[0], 1);
        bs_lo = half2v{lo, lo};
        bs_hi = half2v{hi, hi};
    }
    floatx4 cc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
        cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            a[s], decode_step<FMT>(b.w[0], s, tab, s < 2 ? bs_lo : bs_hi), cc, 0, 0, 0);
    if constexpr (FMT == 4) {
        acc += cc;
    } else {
        const float f = (float)__builtin_bit_cast(_Float16, (uint16_t)b.sc[0]);
        acc += f * cc;
    }
    asm volatile("" : "+v"(acc));
}

// The wave's tile stream: group g of its tile row is tile t = rb0 * G + g of
// the tensor. Codebook tiles of either width load as one 12-byte load per
// lane at lane offset 8 (2-bit) or 12 (3-bit) bytes, through a buffer
// resource sized to the tensor (the 4 bytes a 2-bit lane reads past its own
// are not used; past the tensor's end they read as zero), so that 2- and
// 3-bit tiles issue the same instruction and the waits placed for the loads
// stay exact whichever width a wave has.
template <int CLASS>
struct SmTiles {
    __amdgpu_buffer_rsrc_t rc, rsc;
    int tile0, tbytes, voff, sc_lane;
    __device__ __forceinline__ void init(const WaveJob &J, int rows, int cols, int lane, int sc_lane_)
    {
        const int nb = is_cb<CLASS> ? J.bits : 4;  // bits per weight
        const uint64_t cb = uniform((uint64_t)(uintptr_t)J.codes);
        rc = __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)cb, 0,
                                               (int)((long)rows * cols / 8 * nb), 0x00020000);
        rsc = tensor_rsrc(J.scales);
        tile0 = J.rb0 * J.G;
        tbytes = 256 * nb;  // 16 x 128 weights
        voff = lane * 4 * nb;  // 8, 12 or 16 bytes per lane
        sc_lane = sc_lane_;
    }
    __device__ __forceinline__ void load(GroupBuf<CLASS, 1> &b, int g) const
    {
        const int tile = tile0 + g;
        if constexpr (is_cb<CLASS>) {
            const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rc, voff, tile * tbytes, 0);
            b.w[0][0] = v[0];
            b.w[0][1] = v[1];
            b.w[0][2] = v[2];
            b.sc[0] = __builtin_amdgcn_raw_buffer_load_b16(rsc, sc_lane, tile * 32, 0);
        } else {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, voff, tile * 1024, 0);
            b.w[0][0] = v[0];
            b.w[0][1] = v[1];
            b.w[0][2] = v[2];
            b.w[0][3] = v[3];
            b.sc[0] = __builtin_amdgcn_raw_buffer_load_b16(rsc, sc_lane, tile * 128, 0);
        }
    }
};

// All G groups of the wave's tile: buffer d holds groups d, d + D, ... and
// is refilled with the group D ahead once used (clamped to the last group,
// so that every load is unconditional), except in the last round. The
// buffers arrive holding groups 0 .. D-1 (clamped likewise). Clamped loads
// that no group uses are waited for at the end: left pending they would be
// waited for inside the next item's loop, where the wait takes every load in
// flight with it. FMT: the code width (2, 3) or 4 (NVFP4), fixed per instance.
template <int CLASS, int FMT>
__device__ __forceinline__ void sm_stream(const SmTiles<CLASS> &T, int G, const _Float16 *Arow,
                                          const uint32_t (&tab)[4],
                                          GroupBuf<CLASS, 1> (&buf)[kSmDepth], floatx4 &acc)
{
    int g0 = 0;
    for (; g0 + kSmDepth < G; g0 += kSmDepth) {
#pragma unroll
        for (int d = 0; d < kSmDepth; ++d) {
            sm_group<CLASS, FMT>(buf[d], Arow + (g0 + d) * 128, tab, acc);
            T.load(buf[d], min(g0 + d + kSmDepth, G - 1));
        }
    }
#pragma unroll
    for (int d = 0; d < kSmDepth; ++d)
        if (g0 + d < G)
            sm_group<CLASS, FMT>(buf[d], Arow + (g0 + d) * 128, tab, acc);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

template <int CLASS>
__global__ __launch_bounds__(kExpertThreads) __attribute__((amdgpu_waves_per_eu(4)))
void small_kernel(Params p)
{
    static_assert(!has6<CLASS>, "6-bit codes run on the persistent kernel");
    extern __shared__ __align__(16) _Float16 Abuf[];  // staged rows (R x (cols + pad) halves), then the row-group table
    __shared__ float s_u[2][16][16];    // up results of a gate/up item: [tile][row][token]
    __shared__ int s_flag;
    const Plan *P = p.plan;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int r16 = lane & 15, q = lane >> 4;
    const int m = uniform(P->m), ngr = uniform(P->n_groups);
    int *s_tab = (int *)((char *)Abuf + p.lds_tab);
    const GroupLds s_grp{s_tab, s_tab + p.gcap, s_tab + 2 * p.gcap};
    for (int i = tid; i < p.gcap; i += kExpertThreads) {
        s_tab[i] = P->g_expert[i];
        s_tab[p.gcap + i] = P->g_off[i];
        s_tab[2 * p.gcap + i] = P->g_rows[i];
    }
    __syncthreads();
    const int nsl = p.I / kSmGuRows, ndn = p.H / kSmDnRows;
    const int n_gu = ngr * nsl, n_all = n_gu + ngr * ndn;
    const int sc_lane = is_cb<CLASS> ? r16 * 2 : r16 * 8 + 2 * q;
    float *const h_pre = p.gu_part;  // [bucket row][I]: SiLU(g) u, before the rotation
    uint32_t done = 0;
    for (int t = blockIdx.x; t < n_all; t += gridDim.x) {
        Item it{};
        it.valid = 1;
        it.half = -1;
        it.span = 1;
        it.down = t >= n_gu;
        const int tt = it.down ? t - n_gu : t;
        const int per = it.down ? ndn : nsl;
        it.u = tt / per;
        const int sl = tt - it.u * per;  // row slice of the item
        it.e = uniform(s_grp.expert[it.u]);
        it.off = uniform(s_grp.off[it.u]);
        it.R = uniform(s_grp.rows[it.u]);
        const int pair = load_pair(p, it, r16);
        const DevTensor d = p.tensors[it.e * 3 + (it.down ? 2 : wave >> 1)];
        WaveJob J;
        J.codes = (gu32p)(uintptr_t)uniform((uint64_t)(uintptr_t)d.codes);
        J.scales = (gu8p)(uintptr_t)uniform((uint64_t)(uintptr_t)d.scales);
        J.lut = (const uint16_t *)(uintptr_t)uniform((uint64_t)(uintptr_t)d.lut);
        J.ts = __uint_as_float((uint32_t)uniform((int)__float_as_uint(d.tensor_scale)));
        J.bits = uniform(d.bits);
        J.G = it.down ? p.I / 128 : p.H / 128;
        J.rb0 = it.down ? sl * (kSmDnRows / 16) + wave : sl * (kSmGuRows / 16) + (wave & 1);
        J.g0 = 0;
        const int cols = it.down ? p.I : p.H;
        const int astr = cols + kLdsPadHalves;  // LDS row stride (halves)
        SmTiles<CLASS> T;
        T.init(J, it.down ? p.H : p.I, cols, lane, sc_lane);

        GroupBuf<CLASS, 1> buf[kSmDepth];
        u32x4 lut = u32x4{0, 0, 0, 0};
        bool ok = true;
        if (!it.down) {
            // the activation rows first (their commit then waits for them
            // only), then the codebook and the first D weight groups
            const int cpr = cols / 8, last = it.R * cpr - 1;
            // the thread index, opaque to the compiler: the chunk offsets
            // are recomputed per item instead of being hoisted to the kernel
            // start and held (or spilled) across the item loop
            int ti = tid;
            asm volatile("" : "+v"(ti));
            const int tok = pair_token(pair, m * p.k, p.k);
            const __amdgpu_buffer_rsrc_t rx = buf_rsrc(p.xr);
            u32x4 v[kSmStageIters];
#pragma unroll
            for (int k = 0; k < kSmStageIters; ++k) {
                const int i = min(ti + k * kExpertThreads, last);
                const int r = i / cpr;
                const uint32_t off = __umul24((uint32_t)__shfl(tok, r), (uint32_t)p.H * 2u) +
                                     (uint32_t)(i - r * cpr) * 16u;
                v[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0);
            }
            if constexpr (is_cb<CLASS>)
                lut = load_lut_raw(J);
#pragma unroll
            for (int k = 0; k < kSmDepth; ++k)
                T.load(buf[k], min(k, J.G - 1));
            // every chunk is written, the clamped ones again with the same
            // value: a write skipped on some path would leave its load's wait
            // pending into the loop below, where it would wait for every load
#pragma unroll
            for (int k = 0; k < kSmStageIters; ++k) {
                const int i = min(ti + k * kExpertThreads, last);
                const int r = i / cpr;
                *(u32x4 *)(Abuf + r * astr + (i - r * cpr) * 8) = v[k];
            }
        } else {
            // the weights first: they do not depend on h and load during the wait
            if constexpr (is_cb<CLASS>)
                lut = load_lut_raw(J);
#pragma unroll
            for (int k = 0; k < kSmDepth; ++k)
                T.load(buf[k], min(k, J.G - 1));
            if (tid == 0)
                s_flag = wait_h(p, it.u, (uint32_t)nsl);
            lds_barrier();  // the weight groups stay in flight
            ok = s_flag != 0;
            // h~ = (1/sqrt 128) H_128 (s_I h) per token and 128-column block
            // (codebook; NVFP4 stages h as it is), task c = (row c / nb,
            // block c % nb) by wave c % 4, kSmRotBatch tasks' loads at a time
            const int nb = p.I / 128, ntask = it.R * nb;
            for (int c0 = wave; c0 < ntask; c0 += kExpertWaves * kSmRotBatch) {
                uint64_t hv[kSmRotBatch];
                uint16_t sg[kSmRotBatch];  // the signs of the lane's two columns
#pragma unroll
                for (int j = 0; j < kSmRotBatch; ++j) {
                    const int c = min(c0 + kExpertWaves * j, ntask - 1), r = c / nb, b = c - r * nb;
                    hv[j] = ld_coherent((const uint64_t *)(h_pre + (size_t)(it.off + r) * p.I + b * 128 + 2 * lane));
                    sg[j] = 0;
                    if constexpr (is_cb<CLASS>)
                        sg[j] = *(const uint16_t *)(p.signs_i + b * 128 + 2 * lane);
                }
#pragma unroll
                for (int j = 0; j < kSmRotBatch; ++j) {
                    // clamped tasks are done again (same values, same place),
                    // so that every load is consumed on every path
                    const int c = min(c0 + kExpertWaves * j, ntask - 1);
                    const int r = c / nb, b = c - r * nb, n = b * 128 + 2 * lane;
                    const floatx2 hh = __builtin_bit_cast(floatx2, hv[j]);
                    float v0 = hh[0], v1 = hh[1];
                    if constexpr (is_cb<CLASS>) {
                        v0 *= (float)(int8_t)(sg[j] & 0xFF);
                        v1 *= (float)(int8_t)(sg[j] >> 8);
                        wave_fwht128(v0, v1);
                        v0 *= kInvSqrt128;
                        v1 *= kInvSqrt128;
                    }
                    *(half2v *)(Abuf + r * astr + n) = half2v{(_Float16)v0, (_Float16)v1};
                }
            }
        }
        lds_barrier();  // staged rows written; the weight groups stay in flight
        uint32_t tab[4] = {0, 0, 0, 0};
        if constexpr (is_cb<CLASS>) {
            lut_tables(lut, tab);
            // computed once here, not recomputed from the codebook inside
            // the loop (where its loads look pending to the wait placement)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                asm volatile("" : "+v"(tab[i]));
        }
        floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
        const _Float16 *Arow = Abuf + min(r16, it.R - 1) * astr + q * 32;
        // the instance for the wave's code width (wave-uniform: the gate and
        // up tensors of a block may differ); no barrier inside
        if constexpr (!is_cb<CLASS>)
            sm_stream<CLASS, 4>(T, J.G, Arow, tab, buf, acc);
        else if (J.bits == 3)
            sm_stream<CLASS, 3>(T, J.G, Arow, tab, buf, acc);
        else
            sm_stream<CLASS, 2>(T, J.G, Arow, tab, buf, acc);
        if constexpr (!is_cb<CLASS>)
            acc *= J.ts;
        // result: lane holds rows (tokens) 4q + j of W row r16 of the tile;
        // y is written through (sc1), as the persistent kernel's down partials
        if (it.down) {
            const __amdgpu_buffer_rsrc_t ry = buf_rsrc(p.y_part);
            const uint32_t col = (uint32_t)(J.rb0 * 16 + r16) * 4u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // pair index of row 4q + j (see load_pair)
                const uint32_t off = __umul24((uint32_t)__shfl(pair, 4 * q + j), (uint32_t)p.H * 4u) + col;
                if (ok && 4 * q + j < it.R)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[j]), ry, (int)off, 0,
                                                          16 /* sc1 */);
            }
        } else {
            // the up waves hand their results to the gate waves
            if (wave >= 2)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (4 * q + j < it.R)
                        s_u[wave & 1][r16][4 * q + j] = acc[j];
            lds_barrier();
            if (wave < 2) {
                const int n = sl * kSmGuRows + wave * 16 + r16;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (4 * q + j < it.R) {
                        const float g = acc[j], u = s_u[wave][r16][4 * q + j];
                        st_coherent(&h_pre[(size_t)(it.off + 4 * q + j) * p.I + n],
                                    g / (1.0f + expf(-g)) * u);
                    }
            }
            wait_stores();
            __syncthreads();
            if (tid == 0)
                atomic_add_agent(&p.h_ready[it.u * kCtrStride], 1u);
        }
        ++done;
        lds_barrier();  // the staged rows and s_u are the next item's
    }
    if (tid == 0 && done)
        atomic_add_agent(&p.ctr->items_done[blockIdx.x % kDoneSlots], done);
}

// ---------------------------------------------------------------------------
// Combine
// ---------------------------------------------------------------------------

// out[t][n] = sum_j w[t][j] * sum_s y_part[s][t*k + j][n], slots j in
// order, splits s in order (no float atomics: bitwise reproducible), plus
// the shared expert's row (weight 1) when there is one. Block
// (rb, t) covers rows rb*256 .. +255 of token t; runs after the expert
// kernel, so plain loads see its partial sums.
// Loads in rounds of up to 8 slots: a round's weights and partial sums of
// the first two splits (and, before the first round, the shared expert's row
// and the error word) are issued before any is used (further splits, where a
// layer has more than two, follow separately); then that round's sums, in
// the order above. Every load of a round is issued whatever k and the split
// count (indices past them are clamped to the last slot / split and their
// values not used), so that the compiler can keep them all in flight. KMAX:
// 8 or 16 slots (one or two rounds). The scalar arguments come first:
// the kernel-argument preload puts them in scalar registers at launch, so
// the loads need not wait for the parameter block (they are also in p).
template <int KMAX>
__global__ __launch_bounds__(64) void combine_kernel(const float *__restrict__ y_part,
                                                     const float *__restrict__ wts,
                                                     const Counters *ctr, int k, int ks2,
                                                     int pair_cap, int H, int has_shared, Params p)
{
    const int t = blockIdx.y, row = blockIdx.x * 256 + 4 * threadIdx.x;
    const bool shared = has_shared != 0;
    const uint32_t err = ctr->error_word;
    const int s1 = ks2 > 1 ? 1 : 0;
    auto part = [&](int s, size_t q) { return *(const floatx4 *)(y_part + ((size_t)s * pair_cap + q) * H + row); };
    // the shared expert's row of token t: bucket row m*k + t (a routed row
    // when there is no shared expert: loaded, not used)
    const size_t qsh = shared ? (size_t)gridDim.y * k + t : (size_t)t * k;
    const floatx4 vsh0 = part(0, qsh), vsh1 = part(s1, qsh);
    floatx4 o = floatx4{0.f, 0.f, 0.f, 0.f};
    // slots in rounds of up to 8: one round's loads all issue before its sums;
    // a 16-slot round's arrays would be too large to stay in registers
    constexpr int CH = KMAX < 8 ? KMAX : 8;
#pragma unroll
    for (int j0 = 0; j0 < KMAX; j0 += CH) {
        if (j0 >= k)
            break;
        float wj[CH];
        floatx4 v[CH][2];
#pragma unroll
        for (int jj = 0; jj < CH; ++jj) {
            const size_t q = (size_t)t * k + min(j0 + jj, k - 1);  // partials are stored by pair index
            wj[jj] = wts[q];
            v[jj][0] = part(0, q);
            v[jj][1] = part(s1, q);
        }
#pragma unroll
        for (int jj = 0; jj < CH; ++jj) {
            const int j = j0 + jj;
            if (j >= k)
                break;
            floatx4 y = v[jj][0];
            if (ks2 > 1)
                y += v[jj][1];
            for (int s = 2; s < ks2; ++s)
                y += part(s, (size_t)t * k + j);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                o[c] += wj[jj] * y[c];
        }
    }
    if (shared) {
        // weight 1, after the routed slots
        floatx4 ysh = vsh0;
        if (ks2 > 1)
            ysh += vsh1;
        for (int s = 2; s < ks2; ++s)
            ysh += part(s, qsh);
        o += ysh;
    }
    // a dependency wait of the expert kernel gave up (some down partial
    // sums are stale): the failure shows in the output instead of a
    // plausible wrong value
    if (__builtin_amdgcn_readfirstlane(err) != 0u)
        o = floatx4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    *(floatx4 *)(p.out + (size_t)t * H + row) = o;
}

// ---------------------------------------------------------------------------
// Prefill / batched verify (more than 32 tokens): grouped GEMM over buckets
// ---------------------------------------------------------------------------
// With many tokens an expert has tens to hundreds of rows. The buckets are
// cut into row groups of up to 64 rows, and each decoded weight step feeds
// one MFMA per 16-row subtile of the group (up to four): the decode, the VALU
// cost of these formats, is paid once per 64 rows instead of once per 16. A block
// covers one row group and 128 output rows (of gate and of up: four waves
// of two 16-row tiles each) or 256 (down: eight waves), over all input
// columns, so there are no column splits
// and no partial sums. The gate/up block finishes SiLU(g) u and the h
// rotation of its 128 rows itself (exactly one rotation block); the down
// block writes y; the combine kernel sums the slots. The down kernel runs
// after the gate/up kernel in stream order.

constexpr int kPfThreads = 512;                   // 8 waves: 4 per projection (gate/up)
constexpr int kPfWaves = kPfThreads / 64;
constexpr int kPfNT = 2;                          // 16-row tiles per wave
constexpr int kPfProjWaves = 8 / kPfNT;           // gate/up: waves per projection (128 rows)
constexpr int kPfRows = 64;                       // rows of a prefill row group
constexpr int kPfSub = kPfRows / 16;              // MFMA subtiles per row group
// Staged chunk rows are 256 bytes (128 halves) unpadded; the 16-byte piece p
// of row r sits at piece p ^ (r mod 16) of its row, so that the 16 rows one
// MFMA operand read spans (row r16 of lane r16, pieces 4q + s) and the 16
// pieces one row's staging write covers each fall on distinct LDS banks.
constexpr int kPfAStride = 128;                   // staged chunk row stride (halves)
constexpr int kPfHStride = 128 + 4;               // epilogue buffer row stride (floats)
constexpr size_t kPfLds = 2 * kPfRows * kPfAStride * sizeof(_Float16) > kPfRows * kPfHStride * sizeof(float)
                              ? 2 * kPfRows * kPfAStride * sizeof(_Float16)
                              : kPfRows * kPfHStride * sizeof(float);
__device__ __forceinline__ int pf_piece(int row, int piece) { return row * kPfAStride + ((piece ^ row) & 15) * 8; }

// One 128-column chunk of the first ROWS activation rows of the group (the
// rows of its NSUB subtiles, ROWS = 16 NSUB): ROWS x 128 fp16 = 16 ROWS
// 16-byte pieces, piece i by thread i mod 512; rows past R repeat row R-1
// (their results are never stored). A piece index past the end skips whole
// waves (256 pieces = 4 waves). Gate/up rows are tokens: lane r of every
// wave holds the token of row r. Down rows off .. off+R-1 of h~ are
// consecutive. A thread's rows are the same in every chunk: their element
// offsets (row x row length, below 2^31) are computed once.
template <int ROWS>
struct PfStage {
    static constexpr int PIECES = ROWS * 16;
    static constexpr int ITERS = (PIECES + kPfThreads - 1) / kPfThreads;
    u32x4 v[ITERS];
    int rowoff[ITERS];
    __device__ __forceinline__ void init(const Params &p, bool down, int off, int R, int tok)
    {
        const int tid = threadIdx.x;
#pragma unroll
        for (int k = 0; k < ITERS; ++k) {
            const int row = min((tid + k * kPfThreads) >> 4, R - 1);
            rowoff[k] = down ? (off + row) * p.I : __shfl(tok, row) * p.H;
        }
    }
    __device__ __forceinline__ void issue(const Params &p, bool down, int c)
    {
        const int tid = threadIdx.x;
        const _Float16 *base = down ? p.hr : p.xr;
#pragma unroll
        for (int k = 0; k < ITERS; ++k) {
            const int i = tid + k * kPfThreads;
            if (PIECES % kPfThreads != 0 && i >= PIECES)
                continue;
            const _Float16 *src = base + rowoff[k] + c * 128 + (i & 15) * 8;
            v[k] = *(const u32x4 GLOBAL *)src;
        }
    }
    __device__ __forceinline__ void commit(_Float16 *A) const
    {
        const int tid = threadIdx.x;
#pragma unroll
        for (int k = 0; k < ITERS; ++k) {
            const int i = tid + k * kPfThreads;
            if (PIECES % kPfThreads != 0 && i >= PIECES)
                continue;
            *(u32x4 *)(A + pf_piece(i >> 4, i & 15)) = v[k];
        }
    }
};

// Two fp16 values packed in w, each times f (fp16). The word comes in as a
// value: a bit cast applied to a vector element in place has been compiled
// to read the vector's first element.
__device__ __forceinline__ uint32_t scale_pair(uint32_t w, _Float16 f)
{
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, w) * half2v{f, f});
}

// One 128-column group of the wave's kPfNT tiles against the first NSUB
// staged 16-row subtiles (A, B and result layouts as in process_group;
// subtile t = rows 16t .. 16t+15; NSUB = ceil(R / 16), fixed per loop
// instance: per-subtile branches inside the loop cost more issue slots than
// the MFMAs they skip). Per step: one decode per tile, then per subtile its A
// operand and one MFMA per tile (each A operand read from LDS feeds kPfNT
// MFMAs); staged rows past R repeat row R-1 and their results are never
// stored. Codebook: the group's MFMA sums are scaled by the fp16
// group scale in fp32 and added to the accumulators, as in the decode kernel
// (the scaled weight is never rounded). NVFP4: the e4m3 block scale is exact
// in the fp16 operand, so the MFMAs accumulate directly.
template <int CLASS, int FMT, int NSUB>
__device__ __forceinline__ void pf_group(const GroupBuf<CLASS, kPfNT> &b, const _Float16 *A,
                                         const uint32_t (&tab)[4], floatx4 (&acc)[kPfNT][NSUB])
{
    const int lane = threadIdx.x & 63, r16 = lane & 15, q = lane >> 4;
    floatx4 cc[kPfNT][NSUB];
    if constexpr (FMT != 4)
#pragma unroll
        for (int i = 0; i < kPfNT; ++i)
#pragma unroll
            for (int t = 0; t < NSUB; ++t)
                cc[i][t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        half8 bv[kPfNT];
#pragma unroll
        for (int i = 0; i < kPfNT; ++i) {
            half2v bs = half2v{1, 1};
            if constexpr (FMT == 4) {
                const _Float16 v = (_Float16)(s < 2 ? __builtin_amdgcn_cvt_f32_fp8(b.sc[i], 0)
                                                    : __builtin_amdgcn_cvt_f32_fp8(b.sc[i], 1));
                bs = half2v{v, v};
            }
            bv[i] = decode_step<FMT>(b.w[i], s, tab, bs);
        }
#pragma unroll
        for (int t = 0; t < NSUB; ++t) {
            const half8 a = *(const half8 *)(A + pf_piece(16 * t + r16, 4 * q + s));
#pragma unroll
            for (int i = 0; i < kPfNT; ++i) {
                if constexpr (FMT == 4)
                    acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bv[i], acc[i][t], 0, 0, 0);
                else
                    cc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bv[i], cc[i][t], 0, 0, 0);
            }
        }
    }
    if constexpr (FMT != 4)
#pragma unroll
        for (int i = 0; i < kPfNT; ++i) {
            const float f = (float)__builtin_bit_cast(_Float16, (uint16_t)b.sc[i]);
#pragma unroll
            for (int t = 0; t < NSUB; ++t) {
                acc[i][t] += f * cc[i][t];
                asm volatile("" : "+v"(acc[i][t]));
            }
        }
}

// The main loop and epilogue of a prefill block, for one code format: FMT =
// codebook bits (2 or 3, the row group's expert) or 4 (NVFP4). One decode
// path per instance keeps the loop inside the register budget.
template <int CLASS, bool DOWN, int FMT, int NSUB>
__device__ __forceinline__ void pf_run(const Params &p, _Float16 *pf_lds, const WaveJob &J, int off,
                                       int R, int tok, int rb, int wave, int sc_lane)
{
    constexpr int KB = FMT == 4 ? 0 : FMT;
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, q = lane >> 4;
    u32x4 lut = u32x4{0, 0, 0, 0};
    if constexpr (is_cb<CLASS>)
        lut = load_lut_raw(J);
    // every load below is unconditional (a chunk index past the end reloads
    // the last chunk): a load under a branch would merge with the buffer's
    // old value, and the register copies that merge takes wait for every
    // load in flight
    GroupBuf<CLASS, kPfNT> bA, bB;
    PfStage<16 * NSUB> st;
    const int G1 = J.G - 1;
    st.init(p, DOWN, off, R, tok);
    st.issue(p, DOWN, 0);
    load_group<CLASS, KB, kPfNT>(bA, J, 0, lane, sc_lane);
    st.commit(pf_lds);
    load_group<CLASS, KB, kPfNT>(bB, J, min(1, G1), lane, sc_lane);
    // the codebook's byte tables for the v_perm lookups (unscaled entries)
    uint32_t tab[4] = {0, 0, 0, 0};
    if constexpr (is_cb<CLASS>)
        lut_tables(lut, tab);
    __syncthreads();

    floatx4 acc[kPfNT][NSUB];
#pragma unroll
    for (int i = 0; i < kPfNT; ++i)
#pragma unroll
        for (int t = 0; t < NSUB; ++t)
            acc[i][t] = floatx4{0.f, 0.f, 0.f, 0.f};
    _Float16 *const half0 = pf_lds, *const half1 = pf_lds + kPfRows * kPfAStride;
    // chunk c: weights from buffer c % 2 (refilled with chunk c + 2),
    // activations from LDS half c % 2
    auto step = [&](int c, GroupBuf<CLASS, kPfNT> &b) {
        const _Float16 *A = (c & 1) ? half1 : half0;
        _Float16 *Anext = (c & 1) ? half0 : half1;
        st.issue(p, DOWN, min(c + 1, G1));
        if (c < J.G)
            pf_group<CLASS, FMT, NSUB>(b, A, tab, acc);
        load_group<CLASS, KB, kPfNT>(b, J, min(c + 2, G1), lane, sc_lane);
        st.commit(Anext);
        __syncthreads();
    };
    for (int c = 0; c < J.G; c += 2) {
        step(c, bA);
        step(c + 1, bB);
    }
    if constexpr (!is_cb<CLASS>)
#pragma unroll
        for (int i = 0; i < kPfNT; ++i)
#pragma unroll
            for (int t = 0; t < NSUB; ++t)
                acc[i][t] *= J.ts;

    // result layout: lane holds rows 16t + 4q + j (j = 0..3) of subtile t,
    // output row 16i + r16 of the wave's tile i
    if constexpr (DOWN) {
        // y goes out under each row's pair index (t*k + j for a routed row,
        // the bucket row itself for the shared expert's), as the combine reads it
        const int n0 = rb * 256 + wave * (kPfNT * 16);
        const int mk = uniform(p.plan->m) * p.k;
        int pair[NSUB][4];
#pragma unroll
        for (int t = 0; t < NSUB; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int qr = off + min(16 * t + 4 * q + j, R - 1);
                pair[t][j] = qr < mk ? p.rows[qr] : qr;
            }
#pragma unroll
        for (int i = 0; i < kPfNT; ++i)
#pragma unroll
            for (int t = 0; t < NSUB; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 16 * t + 4 * q + j;
                    if (row < R)
                        p.y_part[(size_t)pair[t][j] * p.H + n0 + 16 * i + r16] = acc[i][t][j];
                }
    } else {
        // h = silu(g) u through LDS (the up waves' u, then the gate waves'
        // h in place), then each wave rotates the h of rows wave, wave + 8, ...
        float *hb = (float *)pf_lds;  // [64 rows][kPfHStride]
        const int lr0 = (wave % kPfProjWaves) * (kPfNT * 16);
        if (wave >= kPfProjWaves)
#pragma unroll
            for (int i = 0; i < kPfNT; ++i)
#pragma unroll
                for (int t = 0; t < NSUB; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int row = 16 * t + 4 * q + j;
                        if (row < R)
                            hb[row * kPfHStride + lr0 + 16 * i + r16] = acc[i][t][j];
                    }
        __syncthreads();
        if (wave < kPfProjWaves)
#pragma unroll
            for (int i = 0; i < kPfNT; ++i)
#pragma unroll
                for (int t = 0; t < NSUB; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int row = 16 * t + 4 * q + j;
                        if (row < R) {
                            float *hp = hb + row * kPfHStride + lr0 + 16 * i + r16;
                            const float g = acc[i][t][j];
                            *hp = g / (1.0f + expf(-g)) * *hp;
                        }
                    }
        __syncthreads();
        const int n = rb * 128 + 2 * lane;
        // the lane's two signs (codebook), once rather than per row
        const uint16_t sg = p.format == kFmtCodebook ? *(const uint16_t *)(p.signs_i + n) : 0;
        for (int row = wave; row < R; row += kPfWaves) {
            float v0 = hb[row * kPfHStride + 2 * lane], v1 = hb[row * kPfHStride + 2 * lane + 1];
            if (p.format == kFmtCodebook) {
                v0 *= (float)(int8_t)(sg & 0xFF);
                v1 *= (float)(int8_t)(sg >> 8);
                wave_fwht128(v0, v1);
                v0 *= kInvSqrt128;
                v1 *= kInvSqrt128;
            }
            *(half2v *)(p.hr + (size_t)(off + row) * p.I + n) = half2v{(_Float16)v0, (_Float16)v1};
        }
    }
}

// The loop instance for the group's code width and subtile count.
template <int CLASS, bool DOWN, int NSUB>
__device__ __forceinline__ void pf_dispatch(const Params &p, _Float16 *pf_lds, const WaveJob &J,
                                            int off, int R, int tok, int rb, int wave, int sc_lane)
{
    if constexpr (!is_cb<CLASS>)
        pf_run<CLASS, DOWN, 4, NSUB>(p, pf_lds, J, off, R, tok, rb, wave, sc_lane);
    else if (J.bits == 3)
        pf_run<CLASS, DOWN, 3, NSUB>(p, pf_lds, J, off, R, tok, rb, wave, sc_lane);
    else
        pf_run<CLASS, DOWN, 2, NSUB>(p, pf_lds, J, off, R, tok, rb, wave, sc_lane);
}

// Block b: row group u = b / RB, output row block rb = b % RB (RB = I / 128
// gate/up blocks, H / 256 down blocks); blocks past the run's groups exit.
// The chunks of the activations go through two LDS halves and the weight
// groups through two register buffers: chunk c+1's activations and weight
// group c+2 load while chunk c is computed.
template <int CLASS, bool DOWN>
// two blocks per CU (four waves per SIMD, at most 128 VGPRs): one block's
// barrier waits are covered by the other block's work
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(4)))
void prefill_kernel(Params p)
{
    extern __shared__ __align__(16) _Float16 pf_lds[];  // [2][64][kPfAStride]; the gate/up epilogue reuses it
    const Plan *P = p.plan;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int r16 = lane & 15, q = lane >> 4;
    const int RB = DOWN ? p.H / 256 : p.n_rb1;
    const int u = blockIdx.x / RB, rb = blockIdx.x - u * RB;
    if (u >= uniform(P->n_groups))
        return;
    const int e = uniform(P->g_expert[u]), off = uniform(P->g_off[u]), R = uniform(P->g_rows[u]);
    const int m = uniform(P->m);
    int tok = 0;  // gate/up: token of row `lane` of the group
    if (!DOWN) {
        const int qrow = off + min(lane, R - 1);
        tok = qrow < m * p.k ? p.rows[qrow] / p.k : qrow - m * p.k;
    }
    const DevTensor d = p.tensors[e * 3 + (DOWN ? 2 : wave / kPfProjWaves)];
    WaveJob J;
    J.codes = (gu32p)(uintptr_t)uniform((uint64_t)(uintptr_t)d.codes);
    J.scales = (gu8p)(uintptr_t)uniform((uint64_t)(uintptr_t)d.scales);
    J.lut = (const uint16_t *)(uintptr_t)uniform((uint64_t)(uintptr_t)d.lut);
    J.ts = __uint_as_float((uint32_t)uniform((int)__float_as_uint(d.tensor_scale)));
    J.bits = uniform(d.bits);
    J.G = DOWN ? p.I / 128 : p.H / 128;
    J.rb0 = DOWN ? rb * 16 + wave * kPfNT : rb * 8 + (wave % kPfProjWaves) * kPfNT;
    J.g0 = 0;
    const int sc_lane = is_cb<CLASS> ? r16 * 2 : r16 * 8 + 2 * q;

    // one MFMA subtile per 16 rows of the group: groups of up to 16 rows are
    // most experts at Zipf routing, 17 .. 48 rows the tails of hot experts
    if (R <= 16)
        pf_dispatch<CLASS, DOWN, 1>(p, pf_lds, J, off, R, tok, rb, wave, sc_lane);
    else if (R <= 32)
        pf_dispatch<CLASS, DOWN, 2>(p, pf_lds, J, off, R, tok, rb, wave, sc_lane);
    else if (R <= 48)
        pf_dispatch<CLASS, DOWN, 3>(p, pf_lds, J, off, R, tok, rb, wave, sc_lane);
    else
        pf_dispatch<CLASS, DOWN, kPfSub>(p, pf_lds, J, off, R, tok, rb, wave, sc_lane);
    if (tid == 0)
        atomic_add_agent(&p.ctr->items_done[blockIdx.x % kDoneSlots], 1u);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

hipError_t launch_route(const Params &p, const uint16_t *x, const float *logits, int m,
                        hipStream_t s)
{
    const int tasks = m * (p.H / 128);
    const int blocks = (m + kRouteWaves - 1) / kRouteWaves + (tasks + kRouteWaves - 1) / kRouteWaves;
    route_kernel<<<dim3(blocks), dim3(kRouteThreads), route_lds_bytes(p.E, m), s>>>(logits, x, m, p.E, p);
    return hipGetLastError();
}

template <int CLASS, int NG>
static void *expert_fn()
{
    return (void *)expert_kernel<CLASS, NG>;
}

// The expert kernel specialised for the format class (codebook with or
// without 6-bit tensors, NVFP4) and the groups per column split (1, 2, 4, 8).
static void *expert_kernel_for(int format, int ng, bool six)
{
    if (format == kFmtCodebook && six) {
        switch (ng) {
        case 8: return expert_fn<kClassCb6, 8>();
        case 4: return expert_fn<kClassCb6, 4>();
        case 2: return expert_fn<kClassCb6, 2>();
        default: return expert_fn<kClassCb6, 1>();
        }
    }
    if (format == kFmtCodebook) {
        switch (ng) {
        case 8: return expert_fn<kFmtCodebook, 8>();
        case 4: return expert_fn<kFmtCodebook, 4>();
        case 2: return expert_fn<kFmtCodebook, 2>();
        default: return expert_fn<kFmtCodebook, 1>();
        }
    }
    switch (ng) {
    case 8: return expert_fn<kFmtNvfp4, 8>();
    case 4: return expert_fn<kFmtNvfp4, 4>();
    case 2: return expert_fn<kFmtNvfp4, 2>();
    default: return expert_fn<kFmtNvfp4, 1>();
    }
}

// The two prefill kernels: grid_groups row groups (a bound on the run's
// groups; blocks past them exit).
hipError_t launch_prefill(const Params &p, int grid_groups, hipStream_t s)
{
    void *gu = p.format == kFmtCodebook ? (void *)prefill_kernel<kFmtCodebook, false>
                                        : (void *)prefill_kernel<kFmtNvfp4, false>;
    void *dn = p.format == kFmtCodebook ? (void *)prefill_kernel<kFmtCodebook, true>
                                        : (void *)prefill_kernel<kFmtNvfp4, true>;
    void *args[] = {const_cast<Params *>(&p)};
    hipError_t err = hipLaunchKernel(gu, dim3(grid_groups * p.n_rb1), dim3(kPfThreads), args,
                                     kPfLds, s);
    if (err != hipSuccess)
        return err;
    return hipLaunchKernel(dn, dim3(grid_groups * (p.H / 256)), dim3(kPfThreads), args, kPfLds, s);
}

hipError_t launch_combine(const Params &p, int m, hipStream_t s)
{
    if (p.k <= 8)
        combine_kernel<8><<<dim3(p.n_rb2, m), dim3(64), 0, s>>>(p.y_part, p.wts, p.ctr, p.k, p.ks2,
                                                                p.pair_cap, p.H, p.has_shared, p);
    else
        combine_kernel<kMaxTopK><<<dim3(p.n_rb2, m), dim3(64), 0, s>>>(
            p.y_part, p.wts, p.ctr, p.k, p.ks2, p.pair_cap, p.H, p.has_shared, p);
    return hipGetLastError();
}

static void *small_kernel_for(int format)
{
    return format == kFmtCodebook ? (void *)small_kernel<kFmtCodebook>
                                  : (void *)small_kernel<kFmtNvfp4>;
}

hipError_t launch_small(const Params &p, int grid, size_t lds_bytes, hipStream_t s)
{
    void *args[] = {const_cast<Params *>(&p)};
    return hipLaunchKernel(small_kernel_for(p.format), dim3(grid), dim3(kExpertThreads), args,
                           lds_bytes, s);
}

hipError_t small_occupancy(int format, int *blocks_per_cu, size_t lds_bytes)
{
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, small_kernel_for(format),
                                                        kExpertThreads, lds_bytes);
}

hipError_t launch_expert(const Params &p, int grid, size_t lds_bytes, hipStream_t s)
{
    void *fn = expert_kernel_for(p.format, p.kc1 / 128, p.has6 != 0);
    void *args[] = {const_cast<Params *>(&p)};
    return hipLaunchKernel(fn, dim3(grid), dim3(kExpertThreads), args, lds_bytes, s);
}

hipError_t expert_occupancy(int format, int ng, bool six, int *blocks_per_cu, size_t lds_bytes)
{
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu,
                                                        expert_kernel_for(format, ng, six),
                                                        kExpertThreads, lds_bytes);
}

}  // namespace moe
