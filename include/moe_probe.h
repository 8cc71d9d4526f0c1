/*
 * moe_probe.h -- measurement probes that bench.py reports beside the decode
 * step's numbers on AMD Instinct MI355X (gfx950): the achievable HBM read
 * bandwidth of a plain streaming read, and the launch floor of near-empty
 * kernels. They compute nothing of the decode step. The pages bound their
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

#ifdef __cplusplus
}
#endif
#endif /* MOE_PROBE_H */
