/*
 * moe_probe.h -- measurement probes that bench.py reports beside the decode
 * step's numbers on AMD Instinct MI355X (gfx950): the achievable HBM read
 * bandwidth of a plain streaming read, the launch floor of near-empty
 * kernels, the LDS read rate of the MFMA operand pattern per staging
 * layout, the issue rates of the decode step's decode and MFMA halves on
 * register operands, and a streaming read whose work units are claimed from
 * shared counters. None of them computes a layer. The pages bound their
 * own kernel by the cold-read rate of their card, measured with a variant
 * that reads the weights without decoding them (page "LNA-CANON.md",
 * section "lna2 とは").
 *
 * Conventions: device pointers are plain device addresses; `hip_stream` is a
 * hipStream_t (NULL = default stream). Functions only enqueue work (kernels,
 * and for moe_probe_ticket_read a memset of the caller's counters) and return
 * 0, or a negative HIP error code from the launch. No allocation.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes at device address `buf` (16-byte aligned, bytes a
 * multiple of 16) once, with `blocks` blocks of 256 threads, each thread
 * keeping four 16-byte loads in flight; the words are xor-folded and
 * `sink` (device, 4 bytes) is written only if the fold equals a value the
 * caller's data does not produce (so the loads cannot be removed).
 */
int moe_probe_stream_read(const void *buf, size_t bytes, int32_t blocks, uint32_t *sink,
                          void *hip_stream);

/* Enqueue `count` empty kernels (one block of 64 threads each). */
int moe_probe_empty_kernels(int32_t count, void *hip_stream);

/*
 * The LDS reads of the MFMA activation operands alone: `blocks` blocks of
 * 256 threads each read four 16-row subtiles of a staged 64-row fp16 chunk
 * (one 16-byte ds_read per lane and subtile-step, 16 per round) `iters`
 * times, in the staging layout `layout`: 0 = 272-byte rows (16 bytes of
 * padding per row: the bank pattern of the decode kernel's staged rows,
 * which are 16 bytes past a multiple of 256), 1 = 256-byte rows with the 16-byte
 * pieces of row r permuted by xor with r mod 16 (the prefill kernels'),
 * 2 = 256-byte rows unpadded (all rows of one read start on the same bank:
 * the conflicted reference). `sink` (device, 4 bytes) as for
 * moe_probe_stream_read. Returns -hipErrorInvalidValue for a layout outside
 * 0..2, blocks < 1, iters outside 1 .. 2^30 - 1 or a NULL sink.
 */
int moe_probe_lds_read128(int32_t layout, int32_t blocks, int32_t iters, uint32_t *sink,
                          void *hip_stream);

/*
 * Issue rates of the decode step's halves, on register operands only (no
 * memory traffic): `blocks` blocks of 256 threads (4 waves), each wave
 * running `iters` rounds of one 128-column group of a 3-bit codebook tile
 * (4 MFMA 16x16x32 steps of 8 weights per lane) with the decode kernels' own
 * decode instruction sequence. mode 0: decode only (each step's output
 * xor-folded: 4 more VALU ops per step); 1: MFMA only (fixed B operand) and
 * the group-scale FMAs; 2: decode into the MFMA and the group-scale FMAs (the
 * decode kernels' inner step); 3: decode into four v_dot2_f32_f16 per step
 * for one token (products on the VALU instead of the MFMA, the R = 1
 * alternative). Every mode also changes the slot words each round (3 VALU
 * ops). `clk` (device, 4 x u64): block 0's shader clock (s_memtime) and 100 MHz
 * constant clock (s_memrealtime) before and after its rounds, from which the
 * caller derives the clock rate; `sink` as for moe_probe_stream_read.
 * Returns -hipErrorInvalidValue for a mode outside 0..3, blocks < 1,
 * iters < 1 or a NULL clk or sink.
 */
int moe_probe_compute_rate(int32_t mode, int32_t blocks, int32_t iters, unsigned long long *clk,
                           uint32_t *sink, void *hip_stream);

/*
 * The cost of claiming work from shared counters: `bytes` bytes at `buf`
 * (16-byte aligned, a positive multiple of 64 KiB) read once in 64 KiB
 * units by `blocks` blocks of 256 threads, one unit at a time (16 loads of
 * 16 bytes per thread, all in flight). mode 0: block b reads units b, b + G,
 * ... (static order); 1: every unit claimed from one counter (an agent-scope
 * atomic add by the block's first thread, handed on through LDS); 2: from
 * eight counters 128 bytes apart (block b claims from counter b % 8).
 * `counters` (device, 1 KiB) is cleared by an enqueued memset before the
 * kernel; `sink` as for moe_probe_stream_read. Returns -hipErrorInvalidValue
 * for a bad size, alignment, mode or pointer.
 */
int moe_probe_ticket_read(const void *buf, size_t bytes, int32_t blocks, int32_t mode,
                          uint32_t *counters, uint32_t *sink, void *hip_stream);

/* One stored matrix for moe_probe_tile_read (the layout of the decode step's
 * stored formats: tiles of 16 rows x 128 columns, `tile_rows` x `groups`
 * tiles in row-block-major order, 256 * bits bytes each; scales per tile,
 * 32 bytes (codebook) or 128 bytes (NVFP4, bits = 4)). */
typedef struct moe_probe_tile_stream {
    const void *codes;     /* device address of the matrix's first tile */
    const void *scales;    /* device address of its first tile's scales */
    int32_t tile_rows;     /* rows / 16, a positive multiple of 4 */
    int32_t groups;        /* columns / 128, a positive multiple of 8 */
    int32_t bits;          /* 2 or 3 (codebook codes), 4 (NVFP4) */
    int32_t units_before;  /* work units of the matrices before this one
                              (a unit: 4 tile rows x 8 groups) */
} moe_probe_tile_stream;

/*
 * The decode kernels' weight reads without the decode (the pages' null-decode
 * measurement, "LNA-CANON.md" §"lna2 とは"): `count` (1..8192) stored
 * matrices, described in the host array `streams`, read once by `blocks`
 * blocks of 4 waves. Each wave takes units of 4 tile rows x 8 column groups
 * (one wave's share of an expert-kernel item) in a static order across the
 * matrices and reads them as the expert kernel does: per group one load of
 * the lane's slot words per tile (12 bytes for 2- and 3-bit tiles, 16 for
 * NVFP4) and one 2-byte scale load per tile, two groups in flight; the words
 * are xor-folded. The table is copied (enqueued) to `dev_streams` (device,
 * count x 32 bytes); `sink` as for moe_probe_stream_read. Returns
 * -hipErrorInvalidValue for a bad count, block count, pointer, shape, width,
 * units_before (must be the running sum) or a matrix of 2 GiB or more.
 */
int moe_probe_tile_read(const moe_probe_tile_stream *streams, int32_t count,
                        moe_probe_tile_stream *dev_streams, int32_t blocks, uint32_t *sink,
                        void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_PROBE_H */
