/*
 * moe_probe.h -- measurement probes that bench.py reports beside the decode
 * step's numbers on AMD Instinct MI355X (gfx950): the achievable HBM read
 * bandwidth of a plain streaming read, the launch floor of near-empty
 * kernels, and the LDS read rate of the MFMA operand pattern per staging
 * layout. They compute nothing of the decode step. The pages bound their
 * own kernel by the cold-read rate of their card, measured with a variant
 * that reads the weights without decoding them (page "LNA-CANON.md",
 * section "lna2 とは").
 *
 * Conventions: device pointers are plain device addresses; `hip_stream` is a
 * hipStream_t (NULL = default stream). Functions only enqueue work and return
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

#ifdef __cplusplus
}
#endif
#endif /* MOE_PROBE_H */
