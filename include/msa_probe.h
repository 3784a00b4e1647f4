/*
 * msa_probe.h - peak-rate probes of the MI355X (gfx950) for the measurement of
 * libmsa: a plain streaming read of device memory and a dense bf16 MFMA loop.
 * They give the practical ceilings the kernels' roofline fractions are also
 * quoted against (next to the published peaks: 8 TB/s HBM3E, 2.5 PFLOP/s dense
 * bf16). Built as libmsa_probe.so; not part of the attention path.
 *
 * Conventions as in msa.h: device pointers, the caller owns every buffer, each
 * call only enqueues one kernel on `stream` and returns; the caller times it
 * (HIP events on the same stream).
 */
#ifndef MSA_PROBE_H_
#define MSA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` of `buf` once with 16-byte non-temporal loads (8 in flight per
 * thread, grid-stride over `groups` work-groups of 256 threads) and writes one
 * word per work-group to sink[groups] so that nothing is optimised away.
 * bytes must be a positive multiple of 32768 and buf 16-byte aligned; groups in
 * [1, 65536]. Returns 0, or -1 on a bad argument (nothing enqueued), or the
 * launch's hipError_t. */
int msa_probe_stream_read(const void *buf, size_t bytes, int groups, uint32_t *sink,
                          void *stream);

/* Dense bf16 MFMA issue: `groups` work-groups of 256 threads (4 waves); every
 * wave runs `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 chains on
 * register operands (no memory traffic in the loop) and writes one word to
 * sink[groups * 4]. Floating-point work: groups * 4 * iters * 8 * 32768 flop.
 * groups in [1, 65536], iters >= 1. Returns as msa_probe_stream_read. */
int msa_probe_mfma_bf16(int groups, int iters, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_PROBE_H_ */
