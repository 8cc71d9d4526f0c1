/*
 * moe_decode.h -- C ABI of the routed-experts decode step of a bit-quantized
 * mixture-of-experts layer on AMD Instinct MI355X (gfx950).
 *
 * One call of moe_decode_run() performs the whole step for m <= max_tokens
 * tokens: top-k routing, per-expert row buckets, block-Hadamard rotation of
 * the activations, the fused gate/up GEMV of every hit expert on its rows,
 * SiLU(gate)*up, the down GEMV, and the per-token combine with the router
 * weights in slot order. This is the routed-experts decode kernel of page
 * "LNA-CANON.md", section "lna2 とは" (rows per expert R_e in {1,2,4,8} at
 * m <= 24, resident expert teams with dynamic tickets and no grid-wide
 * barrier, one scratch per device, one stream at a time, bitwise reproducible)
 * and of page "lna-lab/README.md", section "2026-09-04 -- house kernel lna2".
 *
 * Conventions (all entry points):
 *  - Device pointers are plain device addresses (e.g. torch tensor data_ptr()).
 *    Host pointers are marked "host".
 *  - Return value: MOE_OK or a negative moe_status. No exception crosses the
 *    boundary. moe_decode_last_error() gives a thread-local message about the
 *    last failing call on the calling thread.
 *  - Argument validation happens before any HIP call, so invalid arguments are
 *    reported the same way with or without a GPU.
 *  - There is no fallback path: an unsupported configuration fails at create
 *    (page "LNA-CANON.md", section "教訓": a silent fallback passes the gate).
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_DECODE_ABI_VERSION 3u

typedef struct moe_decode_s *moe_decode_t; /* opaque handle, owned by the library */

typedef enum {
    MOE_OK = 0,
    MOE_E_INVALID = -1,     /* bad argument (null pointer, bad shape, m out of range) */
    MOE_E_UNSUPPORTED = -2, /* valid but not supported by this build (reported at create) */
    MOE_E_HIP = -3,         /* a HIP runtime call failed (message names it) */
    MOE_E_NOMEM = -4,       /* device scratch allocation failed */
    MOE_E_STREAM = -5,      /* run() on a stream other than the one the handle is bound to */
    MOE_E_DEVICE = -6       /* a kernel reported an error (see MOE_Q_STATS.error_word) */
} moe_status;

typedef enum { MOE_FMT_CODEBOOK = 1, MOE_FMT_NVFP4 = 2 } moe_format;

/*
 * One stored expert projection (gate, up or down). All pointers are device
 * pointers BORROWED by the handle: the memory must stay allocated and
 * unmodified until moe_decode_destroy().
 *
 * Matrix W has N rows (outputs) and C columns (inputs): gate and up are
 * inter x hidden, down is hidden x inter. It is stored as tiles of 16 rows x
 * 128 columns, tile (rb, g) at index rb*(C/128)+g, tiles in index order; a
 * tile has 64 slots, slot l covering row 16rb + (l mod 16) and the columns
 * 128g + 32(l div 16) + jj, jj = 0..31, slots in order.
 *
 * MOE_FMT_CODEBOOK (bits = 2, 3 or 6): stand-in for the 2/3-bit codes of the
 * routed experts and the 6-bit codes of the dense linears that the pages
 * name but do not define (page "lna-lab/README.md", "What is in the pack").
 * Routed experts take bits 2 or 3 (6 fails create with MOE_E_UNSUPPORTED);
 * the shared expert takes 2, 3 or 6.
 * Weights live in the rotated basis (see signs_* below).
 *   codes  : uint32 words, bits words per slot (tile = 64*bits words),
 *            4-byte aligned. Column jj of a slot, code bits LSB first:
 *            bits = 2 (d = jj/16, kk = jj%16): word d, bits 8(kk%4) + 2(kk/4)
 *            and +1. bits = 3, jj < 24 (d = jj/8, i = jj%8): word d, bits
 *            8(i%4) + 3(i/4) + 0..2; jj >= 24 (i = jj-24): bits 0 and 1 at
 *            word i/4, bits 8(i%4) + 6 and + 7, bit 2 at word 2, bit
 *            8(i%4) + 6 + i/4. bits = 6: bits 6jj .. 6jj+5 of the slot's six
 *            words read as one 192-bit little-endian string; a 6-bit tile
 *            stores words 0..2 of its 64 slots (in slot order), then words
 *            3..5.
 *   scales : fp16, one per (row, 128-column group), stored per tile in the
 *            tile order: the 16 scales of tile (rb, g) in row order,
 *            scales[(rb*(C/128) + g)*16 + n%16] for row n = 16rb + n%16.
 *            16-byte aligned.
 *   lut    : fp16[2^bits] codebook. W[n][c] = lut[code] * scale.
 *   tensor_scale: ignored.
 * MOE_FMT_NVFP4 (bits = 4): page "V100 換引擎", sections 4.0 and 7.1.
 *   codes  : bytes, 16 per slot; column jj in byte jj/2, low nibble for even jj
 *            (OCP e2m1). 16-byte aligned.
 *   scales : OCP e4m3fn bytes, one per (row, 16-column block), stored per
 *            tile in the tile order, a tile's 16 x 8 scales row-major:
 *            scales[(rb*(C/128) + g)*128 + (n%16)*8 + (c%128)/16]. 16-byte
 *            aligned.
 *   lut    : must be NULL.
 *   tensor_scale: fp32 host value, copied at create.
 *   W[n][c] = e2m1(code) * e4m3(scale) * tensor_scale.
 * The three projections of one expert must have the same bits.
 */
typedef struct {
    const void *codes;
    const void *scales;
    const void *lut;
    float tensor_scale;
    int32_t bits;
} moe_tensor_desc;

typedef struct {
    uint32_t abi_version;            /* MOE_DECODE_ABI_VERSION */
    int32_t format;                  /* moe_format */
    int32_t num_experts;             /* E, 1..256 */
    int32_t top_k;                   /* k, 1..min(16, E) */
    int32_t hidden;                  /* H, multiple of 256, <= 16384 */
    int32_t inter;                   /* I, multiple of 128, <= 16384 */
    int32_t max_tokens;              /* largest m passed to run(), 1..512. Decode is m <= 24;
                                        larger m (prefill, batched verify) run the same
                                        kernels on more row groups. The scratch grows
                                        linearly with max_tokens (about 0.9 MiB per token
                                        at top-8, H = 4096, I = 2048) */
    const moe_tensor_desc *tensors;  /* host [E*3]: expert e -> gate, up, down at 3e, 3e+1, 3e+2;
                                        copied at create */
    const int8_t *signs_hidden;      /* device int8 [H] of +1/-1 (codebook; NULL for NVFP4) */
    const int8_t *signs_inter;       /* device int8 [I] of +1/-1 (codebook; NULL for NVFP4) */
    const moe_tensor_desc *shared;   /* host [3] gate, up, down of an always-on shared expert
                                        (codebook format, any codebook bits, the routed
                                        experts' shapes), or NULL; copied at create. Every
                                        token runs it; its output is added with weight 1
                                        after the k routed terms. The pages' MoE block has
                                        shared experts stored 6-bit with the dense linears
                                        (page "lna-lab/README.md", "What is in the pack"). */
} moe_decode_config;

/*
 * Create a handle for one layer on the current HIP device. Validates the
 * configuration, copies the descriptor table to the device, allocates the
 * handle's scratch (routing buffers, partial sums, counters) and zeroes its
 * counters. Errors: MOE_E_INVALID (null cfg/out/tensors/pointers, shapes not
 * multiples, bits mismatch, wrong abi_version), MOE_E_UNSUPPORTED (sizes over
 * the limits above), MOE_E_HIP, MOE_E_NOMEM. On error *out is set to NULL.
 */
moe_status moe_decode_create(const moe_decode_config *cfg, moe_decode_t *out);

/*
 * Enqueue one decode step on `hip_stream` (a hipStream_t; NULL = default
 * stream). Asynchronous: no allocation, no host synchronisation, no tuning;
 * safe to capture into a HIP graph.
 *   x_bf16 : device bf16 [m][hidden], row-major, 4-byte aligned.
 *   logits : device fp32 [m][num_experts], row-major, 4-byte aligned; must be
 *            finite.
 *   out    : device fp32 [m][hidden], row-major, 16-byte aligned; fully
 *            overwritten.
 * Activation range: x~ (the rotated x) and h~ (the rotated h = SiLU(g)*u)
 * are staged in fp16; products and sums are fp32. Results match the fp64
 * definition within 2e-3 (per token, relative to the token's largest output)
 * while every staged value stays below the fp16 maximum 65504. A rotated
 * 128-block holds values of at most sqrt(128) times the block's largest
 * input, so it suffices that |x| < 5790 and |SiLU(g)*u| < 5790 (codebook
 * format; NVFP4 rotates nothing: |x|, |SiLU(g)*u| < 65504). g and u scale
 * with x, so h grows with the square of the activations' scale. Staged
 * values beyond the range become inf.
 * The expert kernel is persistent: its grid is the number of its blocks
 * that fit on the device at once, and its down work waits (bounded) for
 * gate/up work of other blocks. It therefore assumes every block of its grid
 * becomes resident; work of other streams or processes that holds compute
 * units for the whole run can keep some blocks from starting. If a wait
 * gives up (about 2 s), the run writes NaN to `out` and the next
 * moe_decode_query(MOE_Q_STATS) or moe_decode_destroy() returns
 * MOE_E_DEVICE.
 *   m      : 0..max_tokens. m = 0 returns MOE_OK and enqueues nothing.
 * The handle binds to the first stream it runs on; a different stream later
 * returns MOE_E_STREAM (page "LNA-CANON.md", "lna2 とは": concurrent streams
 * are forbidden; page "lna-lab/README.md", "The three traps", item 3: two
 * streams sharing one lock buffer deadlocked). Results are bitwise identical
 * for identical inputs (same m). From m = 48 on (without 6-bit tensors) the
 * step runs grouped-GEMM prefill kernels instead of the persistent decode
 * kernel (page "LNA-CANON.md", section "起動": prefill batches of up to 512
 * tokens); a token's output then differs from a run at smaller m in rounding
 * only. With very few tokens (at most 4, and only where every work item of
 * the run fits in one round of a persistent grid: one token at top-8 on the
 * 4096 x 2048 layer) a small-m kernel replaces the persistent one: its
 * gate/up items cover 32 rows over all columns, so no split sums cross
 * blocks; it is persistent too (the residency note above applies), and a
 * token's output differs from the other kernels' in rounding only.
 * Errors: MOE_E_INVALID, MOE_E_STREAM, MOE_E_HIP (launch failure).
 * Device faults surface at the caller's next sync.
 */
moe_status moe_decode_run(moe_decode_t h, const void *x_bf16, const float *logits, float *out,
                          int32_t m, void *hip_stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as moe_decode_run(), same arguments, same kernels and bitwise the
 * same results, with every per-run buffer (routing, buckets, work plan,
 * counters, rotated activations, partial sums) in the library's static
 * scratch instead of the handle's: one 32 MiB block per device, held from
 * the library's load until the process ends, whose address create() looks
 * up once per device. It allocates nothing and calls no allocating routine.
 * Every static run on a device uses that one block (page "LNA-CANON.md",
 * section "lna2 とは": one scratch per device), so static runs that overlap
 * on one device race: runs of any handles must be ordered (one stream).
 * A run whose buffers exceed the block (at 256 experts, top-8, hidden 4096,
 * inter 2048: more than 39 tokens, or 35 with a shared expert) fails with
 * MOE_E_UNSUPPORTED before anything is enqueued. Queries
 * after a static run read the block, so they see that run only until the
 * next static run on the device. Errors: as moe_decode_run().
 */
moe_status moe_decode_run_static(moe_decode_t h, const void *x_bf16, const float *logits,
                                 float *out, int32_t m, void *hip_stream);

/* Free the handle's scratch and the handle (after synchronising its stream).
 * NULL is accepted. Graphs that captured runs of the handle must not be
 * replayed afterwards. Returns MOE_E_DEVICE (after freeing) if the last run
 * reported a kernel error. */
moe_status moe_decode_destroy(moe_decode_t h);

/* Thread-local message of the last failing call on this thread ("" if none). */
const char *moe_decode_last_error(void);

/* Query items (moe_decode_query `what`). All synchronise the bound stream. */
enum {
    MOE_Q_INFO = 1,    /* moe_decode_info */
    MOE_Q_ROUTING = 2, /* int32 ids[m*k] then fp32 weights[m*k] of the last run */
    MOE_Q_BUCKETS = 3, /* int32 counts[E], offsets[E+1], rows[m*k] (entry t*k+j) of the last run */
    MOE_Q_STATS = 4    /* moe_decode_stats of the last run */
};

typedef struct {
    int32_t cu_count;        /* compute units of the device */
    int32_t grid_blocks;     /* workgroups of the expert kernel at max_tokens */
    int32_t blocks_per_cu;   /* resident workgroups per CU at max_tokens */
    int32_t k_split_gate_up; /* column splits of the gate/up GEMV */
    int32_t k_split_down;    /* column splits of the down GEMV */
    int32_t reserved;
    int64_t scratch_bytes;   /* device scratch owned by the handle */
} moe_decode_info;

typedef struct {
    int32_t m;              /* tokens of the last run */
    int32_t hit_experts;    /* experts with at least one row */
    int32_t items;          /* work items (tickets) of the last run */
    int32_t items_done;     /* work items the expert kernel completed */
    int32_t error_word;     /* 0, or a bit set by a kernel (1 = spin-wait limit reached) */
    int32_t reserved;
} moe_decode_stats;

/* Copy the requested item into host_buf (host, `bytes` long). Errors:
 * MOE_E_INVALID (unknown item, NULL buffer, buffer too small, no run yet for
 * ROUTING/BUCKETS/STATS), MOE_E_HIP, MOE_E_DEVICE (MOE_Q_STATS only: the
 * stats are copied, and error_word of the last run is nonzero). */
moe_status moe_decode_query(moe_decode_t h, int32_t what, void *host_buf, size_t bytes);

/*
 * Observability: record the hipEvent_t `ev_begin` immediately before and
 * `ev_end` immediately after the expert kernel of every subsequent run (both
 * on the run's stream), so callers can time that kernel alone. Pass NULL,NULL
 * to stop. The events are borrowed. Errors: MOE_E_INVALID (only one NULL).
 */
moe_status moe_decode_profile_events(moe_decode_t h, void *ev_begin, void *ev_end);

#ifdef __cplusplus
}
#endif
#endif /* MOE_DECODE_H */
