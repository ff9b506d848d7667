/*
 * mlora_probes.h -- measured ceilings of the MI355X this library runs on, for
 * reporting achieved rates against the machine as it behaves, beside the
 * published peaks.  Not part of the layer: libmlora_probes.so, separate
 * from libmlora.so.  Every call enqueues one kernel on `stream` (a
 * hipStream_t as void*, NULL = null stream) and returns the hipError_t of
 * the launch as an int (0 = success); a malformed call returns
 * hipErrorInvalidValue (1) and launches nothing.
 */
#ifndef MLORA_PROBES_H
#define MLORA_PROBES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Pure-MFMA loop: n_wg workgroups of four waves, one per SIMD; each wave
 * keeps sixteen 32x32 fp32 accumulators and issues `iters` rounds of
 * sixteen independent v_mfma_f32_32x32x16_bf16 (the base GEMM's
 * instruction and operand pattern, without memory traffic).  Work =
 * n_wg * 4 * iters * 16 * 32768 flops.  operands: device, at least 8192
 * bytes of bf16 values (random ones draw the power a real GEMM draws; zeros
 * let the clock run higher); out: device, n_wg * 256 floats (a sum of the
 * accumulators, so the loop is not removed).  n_wg in [1, 2^20], iters in
 * [1, 2^24].
 */
int mlora_probe_mfma(int64_t n_wg, int64_t iters, const void *operands, float *out, void *stream);

/* The same loop on the MXFP8 instruction (v_mfma_scale_f32_32x32x64_f8f6f4,
 * E4M3 x E4M3, unit scales): work = n_wg * 4 * iters * 16 * 131072 flops;
 * operands: at least 8192 bytes (E4M3 codes: random bytes draw realistic
 * power, though some codes are NaN). */
int mlora_probe_mfma8(int64_t n_wg, int64_t iters, const void *operands, float *out, void *stream);

/* Streaming copy dst[i] = src[i] of `bytes` bytes (a multiple of 16, both
 * 16-byte aligned, not overlapping) with 16-byte loads and stores: HBM
 * traffic = 2 * bytes. */
int mlora_probe_copy(const void *src, void *dst, int64_t bytes, void *stream);

/* Streaming read of `bytes` bytes (a multiple of 16, 16-byte aligned) with
 * 16-byte loads; each of the 2048 * 256 threads writes one float of its sum
 * to out (device, 524288 floats): HBM traffic = bytes + 2 MiB. */
int mlora_probe_read(const void *src, int64_t bytes, float *out, void *stream);

/* Operand blocks from L2 into LDS: n_wg workgroups (one per CU: each holds
 * 160 KiB of LDS) each stream their own 64 KiB slab `iters` times, 16 KiB
 * per wave per pass, by one of three paths:
 *   MLORA_L2L_DIRECT  global_load_lds_dwordx4 (the base GEMM's copies);
 *   MLORA_L2L_STAGED  global_load_dwordx4 into registers one pass ahead,
 *                     then ds_write_b128;
 *   MLORA_L2L_VGPR    the same loads into registers only.
 * Bytes moved = n_wg * iters * 65536.  src: device, 16-byte aligned, at
 * least (n_wg + 1) * 65536 bytes (slab b at byte 65536 b; the staged and
 * register paths read 16 bytes past their slab on odd passes); with n_wg
 * up to 32 per XCD the slabs stay in L2.  out: device, n_wg * 256 uint32 (a
 * digest of LDS, so no load is removed).  path in [0, 2], n_wg in
 * [1, 4096], iters in [2, 2^20]. */
#define MLORA_L2L_DIRECT 0
#define MLORA_L2L_STAGED 1
#define MLORA_L2L_VGPR 2
int mlora_probe_l2_to_lds(int path, int64_t n_wg, int64_t iters, const void *src, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MLORA_PROBES_H */
