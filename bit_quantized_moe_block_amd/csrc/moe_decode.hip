// Host side of the C ABI declared in include/moe_decode.h.
//
// create() validates the configuration before touching the HIP runtime,
// copies the descriptor table to the device, allocates one scratch block per
// handle and sizes the persistent expert grid per token count from the
// occupancy calculator (no autotuning: page "lna-lab/README.md", "The three
// traps", item 2 -- a tuner running under graph capture broke decode).
// run() only enqueues kernels, so it can be captured into a HIP graph.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe_decode.h"
#include "moe_internal.h"

using namespace moe;

struct moe_decode_s {
    Params p{};
    int device = 0;
    int cu_count = 0;
    int max_tokens = 0;
    void *scratch = nullptr;
    size_t scratch_bytes = 0;
    DevTensor *dev_tensors = nullptr;
    std::vector<int> grid;       // [m] persistent grid of the expert kernel
    std::vector<int> bpc;        // [m] resident blocks per CU
    std::vector<size_t> lds;     // [m] dynamic LDS bytes
    std::vector<int> span1;      // [m] 128-row blocks per gate/up item
    std::vector<int> gcap;       // [m] row-group table entries (bound on the groups)
    std::vector<int> prefill;    // [m] 1: the prefill kernels (64-row groups) run this m
    std::vector<int> lds_tab;    // [m] byte offset of the group table in the dynamic LDS
    std::vector<int> small;      // [m] 1: the small-m kernel runs this m
    std::vector<int> sgrid;      // [m] its persistent grid
    std::vector<size_t> slds;    // [m] its dynamic LDS bytes
    std::vector<int> slds_tab;   // [m] byte offset of its group table
    bool bound = false;
    hipStream_t stream = nullptr;
    bool ran = false;
    int last_m = 0;
    int last_path = 0;           // kernels of the last run: 0 persistent, 1 prefill, 2 small-m
    Params last{};               // parameters of the last run (its buffers: queries read them)
    hipEvent_t ev_begin = nullptr, ev_end = nullptr;
};

static thread_local std::string g_err;

static moe_status fail(moe_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
static moe_status fail(moe_status s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

#define HIP_TRY(call)                                                                       \
    do {                                                                                    \
        hipError_t e_ = (call);                                                             \
        if (e_ != hipSuccess)                                                               \
            return fail(MOE_E_HIP, "%s failed: %s", #call, hipGetErrorString(e_));          \
    } while (0)

static bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Columns per split, shared by the gate/up (hidden) and down (inter) GEMVs:
// 128 x the largest power of two d <= 8 dividing both H/128 and I/128 (the
// expert kernel is specialised for 1, 2, 4 or 8 groups per split).
static int split_cols(int H, int I)
{
    int best = 1;
    for (int d = 1; d <= 8; d *= 2)
        if ((H / 128) % d == 0 && (I / 128) % d == 0)
            best = d;
    return 128 * best;
}

// Upper bound on the row groups of a run with m tokens: an expert with R
// rows has ceil(R / 16) <= R / 16 + 1 groups, at most min(E, m k) experts
// are hit, and the shared expert adds ceil(m / 16).
static int group_cap(const Params &p, int m, int rows = kGroupRows)
{
    const int np = m * p.k;
    return std::min(p.E, np) + (np + rows - 1) / rows + (p.has_shared ? (m + rows - 1) / rows : 0);
}

// From this many tokens on the prefill kernels run (64-row groups, one decode
// per 64 rows), unless a tensor has 6-bit codes (the persistent kernel serves
// those at every m). Below it the persistent kernel is faster: measured on the
// 4096 x 2048 layer with Zipf routing, per layer, persistent vs prefill:
// m = 16 103 vs 114 us, 24 148 vs 161, 32 161 vs 169, 48 193 vs 184,
// 64 227 vs 212, 96 293 vs 251.
constexpr int kPrefillFrom = 48;

// Byte offsets of the per-run buffers in one scratch block, for runs of up to
// `tokens` tokens with `pc` bucket rows and `gmax` row groups (256-byte
// aligned pieces). The counters come first: handles of different shapes that
// share one block (the static scratch below) find them at the same place.
struct Layout {
    size_t ctr, rbdone, hready, ids, wts, counts, offsets, rows, pos, plan, xr, gu, hr, y, end;
};

static Layout scratch_layout(const Params &p, size_t tokens, size_t pc, size_t gmax)
{
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) & ~size_t(255);
        return o;
    };
    const size_t E = p.E, H = p.H, I = p.I;
    const size_t ctr_b = 4 * kCtrStride;  // one counter per 128-byte line
    L.ctr = take(sizeof(Counters));
    L.rbdone = take(ctr_b * gmax * p.n_rb1);
    L.hready = take(ctr_b * gmax);
    L.ids = take(4 * pc);
    L.wts = take(4 * pc);
    L.counts = take(4 * E);
    L.offsets = take(4 * (E + 1));
    L.rows = take(4 * pc);
    L.pos = take(4 * pc);
    L.plan = take(sizeof(Plan));
    L.xr = take(2 * tokens * H);
    L.gu = take(4 * (size_t)p.ks1 * pc * 2 * I);
    L.hr = take(2 * pc * I);
    L.y = take(4 * (size_t)p.ks2 * pc * H);
    L.end = off;
    return L;
}

// Point the per-run buffers of p into the block at `base` laid out by L.
static void bind_scratch(Params &p, char *base, const Layout &L)
{
    p.ctr = (Counters *)(base + L.ctr);
    p.rb_done = (uint32_t *)(base + L.rbdone);
    p.h_ready = (uint32_t *)(base + L.hready);
    p.ids = (int32_t *)(base + L.ids);
    p.wts = (float *)(base + L.wts);
    p.counts = (int32_t *)(base + L.counts);
    p.offsets = (int32_t *)(base + L.offsets);
    p.rows = (int32_t *)(base + L.rows);
    p.pos = (int32_t *)(base + L.pos);
    p.plan = (Plan *)(base + L.plan);
    p.xr = (_Float16 *)(base + L.xr);
    p.gu_part = (float *)(base + L.gu);
    p.hr = (_Float16 *)(base + L.hr);
    p.y_part = (float *)(base + L.y);
}

// Static scratch of moe_decode_run_static(): one block per device (each GPU
// holds its own copy of this array from the library's load until the process
// ends). Every static run on a device uses it, so runs that overlap on one
// device race. Host code uses the address that hipGetSymbolAddress gives for
// the current device, never the array's name (a host-side stand-in).
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
static std::mutex g_static_mu;
static void *g_static_ptr[kMaxDevices] = {};

// Once per device, with that device current (called by create): the device
// address of its static scratch, and its counters cleared (the route kernel's
// top-k hand-off counter must start at zero; every run leaves it at zero, and
// each run writes every other buffer before reading it).
static moe_status static_scratch_init(int device)
{
    if (device < 0 || device >= kMaxDevices)
        return fail(MOE_E_UNSUPPORTED, "device %d beyond the %d supported", device, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_static_mu);
    if (g_static_ptr[device])
        return MOE_OK;
    void *ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
        return fail(MOE_E_HIP, "hipGetSymbolAddress(static scratch) failed: %s", hipGetErrorString(e));
    e = hipMemset(ptr, 0, sizeof(Counters));
    if (e == hipSuccess)
        e = hipDeviceSynchronize();
    if (e != hipSuccess)
        return fail(MOE_E_HIP, "clearing the static scratch failed: %s", hipGetErrorString(e));
    g_static_ptr[device] = ptr;
    return MOE_OK;
}

static moe_status validate(const moe_decode_config *c)
{
    if (!c)
        return fail(MOE_E_INVALID, "cfg is NULL");
    if (c->abi_version != MOE_DECODE_ABI_VERSION)
        return fail(MOE_E_INVALID, "abi_version %u, library is %u", c->abi_version,
                    MOE_DECODE_ABI_VERSION);
    if (c->format != MOE_FMT_CODEBOOK && c->format != MOE_FMT_NVFP4)
        return fail(MOE_E_INVALID, "unknown format %d", c->format);
    if (c->num_experts < 1)
        return fail(MOE_E_INVALID, "num_experts %d < 1", c->num_experts);
    if (c->num_experts > kMaxExperts)
        return fail(MOE_E_UNSUPPORTED, "num_experts %d > %d", c->num_experts, kMaxExperts);
    if (c->top_k < 1 || c->top_k > c->num_experts)
        return fail(MOE_E_INVALID, "top_k %d not in 1..num_experts", c->top_k);
    if (c->top_k > kMaxTopK)
        return fail(MOE_E_UNSUPPORTED, "top_k %d > %d", c->top_k, kMaxTopK);
    if (c->hidden < 256 || c->hidden % 256)
        return fail(MOE_E_INVALID, "hidden %d is not a positive multiple of 256", c->hidden);
    if (c->inter < 128 || c->inter % 128)
        return fail(MOE_E_INVALID, "inter %d is not a positive multiple of 128", c->inter);
    if (c->hidden > 16384 || c->inter > 16384)
        return fail(MOE_E_UNSUPPORTED, "hidden/inter above 16384");
    if (c->max_tokens < 1)
        return fail(MOE_E_INVALID, "max_tokens %d < 1", c->max_tokens);
    if (c->max_tokens > kMaxTokens)
        return fail(MOE_E_UNSUPPORTED, "max_tokens %d > %d", c->max_tokens, kMaxTokens);
    if (!c->tensors)
        return fail(MOE_E_INVALID, "tensors is NULL");
    const bool cb = c->format == MOE_FMT_CODEBOOK;
    if (cb && (!c->signs_hidden || !c->signs_inter))
        return fail(MOE_E_INVALID, "codebook format needs signs_hidden and signs_inter");
    if (c->shared && !cb)
        return fail(MOE_E_UNSUPPORTED, "a shared expert needs the codebook format");
    const int n_exp = c->num_experts + (c->shared ? 1 : 0);
    for (int e = 0; e < n_exp; ++e) {
        // expert e == num_experts is the shared expert
        const moe_tensor_desc *td = e < c->num_experts ? c->tensors + 3 * e : c->shared;
        const int b0 = td[0].bits;
        for (int p = 0; p < 3; ++p) {
            const moe_tensor_desc &t = td[p];
            if (!t.codes || !t.scales)
                return fail(MOE_E_INVALID, "expert %d projection %d: NULL codes or scales", e, p);
            if (t.bits != b0)
                return fail(MOE_E_INVALID, "expert %d: projections have different bits", e);
            if (cb) {
                if (t.bits != 2 && t.bits != 3 && t.bits != 6)
                    return fail(MOE_E_INVALID, "expert %d projection %d: bits %d not 2, 3 or 6", e,
                                p, t.bits);
                // 6-bit codes are the stored form of the shared expert only (the
                // pack's dense linears); routed experts are 2/3-bit
                if (t.bits == 6 && e < c->num_experts)
                    return fail(MOE_E_UNSUPPORTED,
                                "expert %d: 6-bit codes are supported for the shared expert only", e);
                if (!t.lut)
                    return fail(MOE_E_INVALID, "expert %d projection %d: NULL lut", e, p);
                if (!aligned(t.codes, 16) || !aligned(t.scales, 16) || !aligned(t.lut, 4))
                    return fail(MOE_E_INVALID, "expert %d projection %d: misaligned pointer", e, p);
            } else {
                if (t.bits != 4)
                    return fail(MOE_E_INVALID, "expert %d projection %d: NVFP4 needs bits 4", e, p);
                if (t.lut)
                    return fail(MOE_E_INVALID, "expert %d projection %d: NVFP4 takes no lut", e, p);
                if (!aligned(t.codes, 16))
                    return fail(MOE_E_INVALID, "expert %d projection %d: misaligned codes", e, p);
            }
        }
    }
    return MOE_OK;
}

extern "C" const char *moe_decode_last_error(void) { return g_err.c_str(); }

extern "C" moe_status moe_decode_create(const moe_decode_config *cfg, moe_decode_t *out)
{
    if (!out)
        return fail(MOE_E_INVALID, "out is NULL");
    *out = nullptr;
    moe_status st = validate(cfg);
    if (st != MOE_OK)
        return st;

    moe_decode_s *h = new moe_decode_s();
    Params &p = h->p;
    p.format = cfg->format;
    p.E = cfg->num_experts;
    p.k = cfg->top_k;
    p.H = cfg->hidden;
    p.I = cfg->inter;
    p.max_tokens = cfg->max_tokens;
    p.kc1 = p.kc2 = split_cols(p.H, p.I);
    p.ks1 = p.H / p.kc1;
    p.ks2 = p.I / p.kc2;
    p.span1 = 1;
    p.n_rb1 = p.I / 128;
    p.n_rb2 = p.H / 256;
    p.has_shared = cfg->shared ? 1 : 0;
    p.has6 = 0;
    for (int i = 0; i < 3 * p.E; ++i)
        p.has6 |= cfg->tensors[i].bits == 6;
    for (int i = 0; cfg->shared && i < 3; ++i)
        p.has6 |= cfg->shared[i].bits == 6;
    p.sh_half = cfg->shared && cfg->shared[0].bits == 6;
    p.pair_cap = p.max_tokens * (p.k + p.has_shared);
    p.spin_limit = 2u * 1000u * 1000u;  // polls of up to ~1 us: a ~2 s bound
    // Test hook: MOE_DECODE_SPIN_LIMIT=<polls> shortens the bound of the
    // dependency waits, so that a test can make them give up (every kernel
    // still ends normally; the failure then shows as MOE_E_DEVICE and NaN
    // outputs). It changes no result of a run that completes.
    if (const char *sl = getenv("MOE_DECODE_SPIN_LIMIT"))
        p.spin_limit = (uint32_t)strtoul(sl, nullptr, 10);
    p.signs_h = cfg->signs_hidden;
    p.signs_i = cfg->signs_inter;
    h->max_tokens = cfg->max_tokens;

    auto cleanup = [&](moe_status s) {
        if (h->scratch)
            (void)hipFree(h->scratch);
        delete h;
        return s;
    };
    hipError_t err = hipGetDevice(&h->device);
    if (err != hipSuccess)
        return cleanup(fail(MOE_E_HIP, "hipGetDevice failed: %s", hipGetErrorString(err)));
    hipDeviceProp_t prop;
    err = hipGetDeviceProperties(&prop, h->device);
    if (err != hipSuccess)
        return cleanup(fail(MOE_E_HIP, "hipGetDeviceProperties failed: %s", hipGetErrorString(err)));
    h->cu_count = prop.multiProcessorCount;
    {
        const moe_status ss = static_scratch_init(h->device);
        if (ss != MOE_OK)
            return cleanup(ss);
    }

    // The handle's scratch: the per-run buffers for max_tokens, then the
    // device copy of the descriptor table.
    const size_t E = p.E, M = p.max_tokens;
    const Layout L = scratch_layout(p, M, p.pair_cap, group_cap(p, p.max_tokens));
    const size_t o_tensors = L.end;
    const size_t total = o_tensors + sizeof(DevTensor) * (E * 3 + 3);
    h->scratch_bytes = total;
    err = hipMalloc(&h->scratch, total);
    if (err != hipSuccess)
        return cleanup(fail(MOE_E_NOMEM, "hipMalloc(%zu) failed: %s", total, hipGetErrorString(err)));
    char *base = (char *)h->scratch;
    h->dev_tensors = (DevTensor *)(base + o_tensors);
    p.tensors = h->dev_tensors;
    bind_scratch(p, base, L);

    std::vector<DevTensor> tab(E * 3 + 3, DevTensor{});
    for (size_t i = 0; i < E * 3 + (cfg->shared ? 3 : 0); ++i) {
        const moe_tensor_desc &t = i < E * 3 ? cfg->tensors[i] : cfg->shared[i - E * 3];
        tab[i] = DevTensor{t.codes, t.scales, (const uint16_t *)t.lut, t.tensor_scale, t.bits};
    }
    err = hipMemcpy(h->dev_tensors, tab.data(), sizeof(DevTensor) * (E * 3 + 3),
                    hipMemcpyHostToDevice);
    if (err == hipSuccess)  // counters (rb_done and h_ready are reset by every run)
        err = hipMemset(base + L.ctr, 0, L.ids - L.ctr);
    if (err == hipSuccess)
        err = hipDeviceSynchronize();
    if (err != hipSuccess)
        return cleanup(fail(MOE_E_HIP, "scratch initialisation failed: %s", hipGetErrorString(err)));

    // Per token count: the persistent grid (resident blocks per CU x CUs) and
    // the 128-row blocks per gate/up item. With m >= 8 tokens (many row
    // groups) a gate/up item covers two row blocks of one column split: one
    // staging of the activations serves both, and there are about as many
    // gate/up items as resident blocks. Fewer tokens keep one row block per
    // item so that the few groups still spread over the grid.
    const int kc = p.kc1;
    h->grid.assign(M + 1, 0);
    h->bpc.assign(M + 1, 0);
    h->lds.assign(M + 1, 0);
    h->span1.assign(M + 1, 1);
    h->gcap.assign(M + 1, 0);
    h->prefill.assign(M + 1, 0);
    h->lds_tab.assign(M + 1, 0);
    h->small.assign(M + 1, 0);
    h->sgrid.assign(M + 1, 0);
    h->slds.assign(M + 1, 0);
    h->slds_tab.assign(M + 1, 0);
    for (int m = 1; m <= (int)M; ++m) {
        h->span1[m] = (m >= 8 && p.n_rb1 % 2 == 0) ? 2 : 1;
        // dynamic LDS: the staged rows (min(m, 16) x kc halves, padded), then
        // the row-group table (3 ints per group)
        const size_t stage = ((size_t)std::min(m, kGroupRows) * (kc + kLdsPadHalves) *
                                  sizeof(_Float16) + 15) & ~size_t(15);
        h->gcap[m] = group_cap(p, m);
        h->prefill[m] = m >= kPrefillFrom && !p.has6;
        h->lds_tab[m] = (int)stage;
        const size_t lds = stage + 3 * sizeof(int) * (size_t)h->gcap[m];
        int bpc = 0;
        err = expert_occupancy(p.format, p.kc1 / 128, p.has6 != 0, &bpc, lds);
        if (err != hipSuccess || bpc < 1)
            return cleanup(fail(MOE_E_UNSUPPORTED, "expert kernel cannot be resident with %zu B LDS",
                                lds));
        h->bpc[m] = bpc;
        h->lds[m] = lds;
        h->grid[m] = bpc * h->cu_count;
        // the small-m kernel: up to kSmallMaxTokens tokens, no 6-bit codes,
        // staged rows R x max(H, I) within its per-thread staging loads, at
        // least two resident blocks per CU, and every item of the run in one
        // round of the grid (at most one row group per hit expert, plus the
        // shared expert's): with a second round the down items of the late
        // gate/up items wait behind them, and the persistent kernel is faster
        // (stack43: m = 1 33.8 vs 35.3 us, m = 2 45.5 vs 40.5, m = 4 56.5 vs
        // 52.5 expert-kernel us)
        const int R = std::min(m, kGroupRows), wide = std::max(p.H, p.I);
        const long worst_items = (long)(std::min(p.E, m * p.k) + (p.has_shared ? 1 : 0)) *
                                 (p.I / 32 + p.H / 64);
        if (m <= kSmallMaxTokens && !p.has6 && (long)R * wide <= kSmallStageElems) {
            const size_t sstage = ((size_t)R * (wide + kLdsPadHalves) * sizeof(_Float16) + 15) &
                                  ~size_t(15);
            const size_t slds = sstage + 3 * sizeof(int) * (size_t)h->gcap[m];
            int sb = 0;
            if (small_occupancy(p.format, &sb, slds) == hipSuccess && sb >= 2 &&
                worst_items <= (long)sb * h->cu_count) {
                h->small[m] = 1;
                h->sgrid[m] = sb * h->cu_count;
                h->slds[m] = slds;
                h->slds_tab[m] = (int)sstage;
            }
            (void)hipGetLastError();
        }
    }
    if (getenv("MOE_DECODE_LOG"))
        fprintf(stderr,
                "[moe_decode] ACTIVE: gfx950 routed-experts decode, E=%d k=%d H=%d I=%d "
                "max_tokens=%d, %d CUs, grid(max)=%d, scratch=%zu B\n",
                p.E, p.k, p.H, p.I, p.max_tokens, h->cu_count, h->grid[M], h->scratch_bytes);
    *out = h;
    return MOE_OK;
}

// Arguments of a run, checked before the handle is read. *skip is set for
// m = 0 (nothing to enqueue).
static moe_status check_run_args(moe_decode_t h, const void *x_bf16, const float *logits,
                                 float *out, int32_t m, bool *skip)
{
    *skip = false;
    if (!h)
        return fail(MOE_E_INVALID, "handle is NULL");
    if (m < 0)
        return fail(MOE_E_INVALID, "m = %d < 0", m);
    if (m == 0) {
        *skip = true;
        return MOE_OK;
    }
    if (!x_bf16 || !logits || !out)
        return fail(MOE_E_INVALID, "NULL x, logits or out");
    // the kernels read x as bf16 pairs and logits as fp32, and write out in
    // 16-byte pieces
    if (!aligned(x_bf16, 4) || !aligned(logits, 4) || !aligned(out, 16))
        return fail(MOE_E_INVALID, "misaligned x (needs 4 B), logits (4 B) or out (16 B)");
    if (m > h->max_tokens)
        return fail(MOE_E_INVALID, "m = %d not in 0..max_tokens (%d)", m, h->max_tokens);
    return MOE_OK;
}

// Bind the handle to its stream on the first run; another stream later is
// refused.
static moe_status bind_stream(moe_decode_t h, hipStream_t s)
{
    if (h->bound && s != h->stream)
        return fail(MOE_E_STREAM, "handle is bound to another stream");
    h->bound = true;
    h->stream = s;
    return MOE_OK;
}

// The per-run fields of the kernels' parameters for m tokens.
static void run_params(const moe_decode_t h, Params &p, float *out, int m)
{
    p.out = out;
    p.span1 = h->span1[m];
    p.gcap = h->gcap[m];
    p.lds_tab = h->small[m] ? h->slds_tab[m] : h->lds_tab[m];
    p.egrid = h->grid[m];
    p.group_rows = h->prefill[m] ? kPrefillRows : kGroupRows;
}

// Enqueue the kernels of one run (route; the persistent expert kernel, the
// small-m kernel or the two prefill kernels; combine) with the buffers p
// points at.
static moe_status enqueue(moe_decode_t h, Params p, const void *x_bf16, const float *logits,
                          int m, hipStream_t s)
{
    const int path = h->prefill[m] ? 1 : h->small[m] ? 2 : 0;
    HIP_TRY(launch_route(p, (const uint16_t *)x_bf16, logits, m, s));
    if (h->ev_begin)
        HIP_TRY(hipEventRecord(h->ev_begin, s));
    if (path == 1) {
        HIP_TRY(launch_prefill(p, group_cap(p, m, kPrefillRows), s));
        p.ks2 = 1;  // y written whole: one split for the combine
    } else if (path == 2) {
        HIP_TRY(launch_small(p, h->sgrid[m], h->slds[m], s));
        p.ks2 = 1;
    } else {
        HIP_TRY(launch_expert(p, h->grid[m], h->lds[m], s));
    }
    if (h->ev_end)
        HIP_TRY(hipEventRecord(h->ev_end, s));
    HIP_TRY(launch_combine(p, m, s));
    h->ran = true;
    h->last_m = m;
    h->last_path = path;
    h->last = p;
    return MOE_OK;
}

extern "C" moe_status moe_decode_run(moe_decode_t h, const void *x_bf16, const float *logits,
                                     float *out, int32_t m, void *hip_stream)
{
    bool skip;
    moe_status st = check_run_args(h, x_bf16, logits, out, m, &skip);
    if (st != MOE_OK || skip)
        return st;
    hipStream_t s = (hipStream_t)hip_stream;
    if ((st = bind_stream(h, s)) != MOE_OK)
        return st;
    Params p = h->p;
    run_params(h, p, out, m);
    return enqueue(h, p, x_bf16, logits, m, s);
}

extern "C" moe_status moe_decode_run_static(moe_decode_t h, const void *x_bf16,
                                            const float *logits, float *out, int32_t m,
                                            void *hip_stream)
{
    bool skip;
    moe_status st = check_run_args(h, x_bf16, logits, out, m, &skip);
    if (st != MOE_OK || skip)
        return st;
    void *base = g_static_ptr[h->device];  // set by create for this device
    if (!base)
        return fail(MOE_E_INVALID, "no static scratch on device %d", h->device);
    Params p = h->p;
    run_params(h, p, out, m);
    // the buffers sized for this run: m tokens, m (k + shared) bucket rows
    p.pair_cap = m * (p.k + p.has_shared);
    const Layout L = scratch_layout(p, m, p.pair_cap, group_cap(p, m));
    if (L.end > kStaticScratchBytes)
        return fail(MOE_E_UNSUPPORTED,
                    "a run of %d tokens needs %zu bytes of static scratch, more than its %zu", m,
                    L.end, kStaticScratchBytes);
    hipStream_t s = (hipStream_t)hip_stream;
    if ((st = bind_stream(h, s)) != MOE_OK)
        return st;
    bind_scratch(p, (char *)base, L);
    return enqueue(h, p, x_bf16, logits, m, s);
}

extern "C" moe_status moe_decode_destroy(moe_decode_t h)
{
    if (!h)
        return MOE_OK;
    hipError_t err = hipSuccess;
    uint32_t error_word = 0;
    if (h->scratch) {
        if (h->bound)
            err = hipStreamSynchronize(h->stream);
        if (err == hipSuccess && h->ran)
            err = hipMemcpy(&error_word, &h->last.ctr->error_word, sizeof error_word,
                            hipMemcpyDeviceToHost);
        hipError_t e2 = hipFree(h->scratch);
        if (err == hipSuccess)
            err = e2;
    }
    delete h;
    if (err != hipSuccess)
        return fail(MOE_E_HIP, "destroy: %s", hipGetErrorString(err));
    if (error_word)
        return fail(MOE_E_DEVICE, "destroy: the last run reported error word 0x%x", error_word);
    return MOE_OK;
}

extern "C" moe_status moe_decode_query(moe_decode_t h, int32_t what, void *host_buf, size_t bytes)
{
    if (!h)
        return fail(MOE_E_INVALID, "handle is NULL");
    if (!host_buf)
        return fail(MOE_E_INVALID, "host_buf is NULL");
    const Params &p = h->p;
    if (what == MOE_Q_INFO) {
        if (bytes < sizeof(moe_decode_info))
            return fail(MOE_E_INVALID, "buffer too small for moe_decode_info");
        moe_decode_info info{};
        info.cu_count = h->cu_count;
        info.grid_blocks = h->grid[h->max_tokens];
        info.blocks_per_cu = h->bpc[h->max_tokens];
        info.k_split_gate_up = p.ks1;
        info.k_split_down = p.ks2;
        info.scratch_bytes = (int64_t)h->scratch_bytes;
        memcpy(host_buf, &info, sizeof info);
        return MOE_OK;
    }
    if (what != MOE_Q_ROUTING && what != MOE_Q_BUCKETS && what != MOE_Q_STATS)
        return fail(MOE_E_INVALID, "unknown query item %d", what);
    if (!h->ran)
        return fail(MOE_E_INVALID, "no run yet");
    const Params &r = h->last;  // the buffers of the last run
    const int m = h->last_m, np = m * p.k;
    size_t need = what == MOE_Q_ROUTING  ? (size_t)np * 8
                  : what == MOE_Q_BUCKETS ? (size_t)(2 * p.E + 1 + np) * 4
                                          : sizeof(moe_decode_stats);
    if (bytes < need)
        return fail(MOE_E_INVALID, "buffer too small (%zu < %zu)", bytes, need);
    HIP_TRY(hipStreamSynchronize(h->stream));
    char *dst = (char *)host_buf;
    if (what == MOE_Q_ROUTING) {
        HIP_TRY(hipMemcpy(dst, r.ids, 4 * np, hipMemcpyDeviceToHost));
        HIP_TRY(hipMemcpy(dst + 4 * np, r.wts, 4 * np, hipMemcpyDeviceToHost));
    } else if (what == MOE_Q_BUCKETS) {
        HIP_TRY(hipMemcpy(dst, r.counts, 4 * p.E, hipMemcpyDeviceToHost));
        HIP_TRY(hipMemcpy(dst + 4 * p.E, r.offsets, 4 * (p.E + 1), hipMemcpyDeviceToHost));
        HIP_TRY(hipMemcpy(dst + 4 * (2 * p.E + 1), r.rows, 4 * np, hipMemcpyDeviceToHost));
    } else {
        Plan plan;
        Counters c;
        HIP_TRY(hipMemcpy(&plan, r.plan, sizeof plan, hipMemcpyDeviceToHost));
        HIP_TRY(hipMemcpy(&c, r.ctr, sizeof c, hipMemcpyDeviceToHost));
        moe_decode_stats st{};
        st.m = plan.m;
        std::vector<int32_t> counts(p.E);
        HIP_TRY(hipMemcpy(counts.data(), r.counts, 4 * p.E, hipMemcpyDeviceToHost));
        st.hit_experts = 0;
        for (int32_t c : counts)
            st.hit_experts += c > 0;
        // prefill: one item per (row group, output row block) of each kernel;
        // small-m: 32-row gate/up and 64-row down items per row group
        st.items = h->last_path == 1   ? plan.n_groups * (p.n_rb1 + p.H / 256)
                   : h->last_path == 2 ? plan.n_groups * (p.I / 32 + p.H / 64)
                                       : plan.n_items;
        uint32_t done = 0;
        for (int i = 0; i < kDoneSlots; ++i)
            done += c.items_done[i];
        st.items_done = (int32_t)done;
        st.error_word = (int32_t)c.error_word;
        memcpy(dst, &st, sizeof st);
        if (c.error_word)
            return fail(MOE_E_DEVICE, "the last run reported error word 0x%x (1: a dependency "
                        "wait gave up; that run's output is NaN)", c.error_word);
    }
    return MOE_OK;
}

extern "C" moe_status moe_decode_profile_events(moe_decode_t h, void *ev_begin, void *ev_end)
{
    if (!h)
        return fail(MOE_E_INVALID, "handle is NULL");
    if ((ev_begin == nullptr) != (ev_end == nullptr))
        return fail(MOE_E_INVALID, "pass both events or neither");
    h->ev_begin = (hipEvent_t)ev_begin;
    h->ev_end = (hipEvent_t)ev_end;
    return MOE_OK;
}
