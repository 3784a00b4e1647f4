/*
 * msa_probe.h - peak-rate probes of the MI355X (gfx950) for the measurement of
 * libmsa: a plain streaming read of device memory, a plain device copy, dense
 * bf16 MFMA loops on constant and on random operands, and MFMA next to fp32 VALU
 * work on one SIMD.
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

/* Copies `bytes` from src to dst (device buffers that do not overlap) with 16-byte
 * loads, 8 in flight per thread, and 16-byte stores, grid-stride over `groups`
 * work-groups of 256 threads: the rate of a plain copy, the ceiling of a kernel
 * that writes as many bytes as it reads. bytes a positive multiple of 16, both
 * pointers 16-byte aligned; groups in [1, 65536]. Returns as msa_probe_stream_read. */
int msa_probe_copy(const void *src, void *dst, size_t bytes, int groups, void *stream);

/* Dense bf16 MFMA issue: `groups` work-groups of 256 threads (4 waves); every
 * wave runs `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 chains on
 * register operands (no memory traffic in the loop) and writes one word to
 * sink[groups * 4]. Floating-point work: groups * 4 * iters * 8 * 32768 flop.
 * groups in [1, 65536], iters >= 1. Returns as msa_probe_stream_read. */
int msa_probe_mfma_bf16(int groups, int iters, float *sink, void *stream);

/* As msa_probe_mfma_bf16 with random operands: every lane holds 8 operand pairs
 * uniform in (-1.7, 1.7) that use all bf16 mantissa bits (the MFMA rate depends on
 * the data: small constant operands run faster). Same flop count and sink. */
int msa_probe_mfma_bf16_random(int groups, int iters, float *sink, void *stream);

/* MFMA and fp32 VALU work of two waves on one SIMD: `groups` work-groups of 8
 * waves holding 128 KiB of LDS each (one per CU; waves w and w + 4 share a SIMD).
 * mode 1: waves 0-3 run `iters` rounds of 16 random-operand 32x32x16 bf16 MFMAs
 * (groups * 4 * iters * 16 * 32768 flop); mode 2: waves 4-7 run `iters` rounds of
 * a softmax tile's fp32 work on 16 values per lane (max3 tree, 16 x (fma, exp2,
 * add), 8 bf16 packs); mode 3: both at once. Comparing the three times shows how
 * much of the smaller one the SIMD hides. Writes sink[groups * 8]. groups in [1,
 * 32768], iters >= 1, mode in {1, 2, 3}. Returns as msa_probe_stream_read. */
int msa_probe_mfma_valu(int groups, int iters, int mode, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_PROBE_H_ */
