/*
 * fa_calib.h -- calibration kernels for measuring the attention kernels, exported
 * by the same library (libfa.so).  They are not part of the attention method:
 * they tell what the chip sustains for the two resources the attention kernels
 * are priced against, in the same process, so that a fraction of the published
 * peak can be read next to a fraction of what this chip delivers under the same
 * clock and power conditions, and so that hardware counters can be turned into
 * utilisation (MFMA busy at a known full load; HBM bytes per counter unit).
 * Error codes are those of fa.h.  Calls are asynchronous on `stream`.
 */
#ifndef FA_CALIB_H_
#define FA_CALIB_H_

#include <stdint.h>

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_calib_mfma -- `workgroups` workgroups of 4 wavefronts, each wavefront running
 * `iters` rounds of 4 independent dense MFMAs (32x32 output blocks) and nothing
 * else.  kind 0: v_mfma_f32_32x32x16_bf16, 32768 FLOP per instruction; kind 1:
 * v_mfma_scale_f32_32x32x64_f8f6f4 on e4m3 operands with unit block scales, 131072
 * FLOP per instruction.  FLOP per launch = workgroups * 4 * iters * 4 * (FLOP per
 * instruction).
 *   out: float32 [workgroups * 256] (device), one sum per thread (keeps the work live).
 * Errors: FA_ERR_UNSUPPORTED (kind), FA_ERR_SHAPE (workgroups outside 1..2^20,
 * iters outside 1..2^24), FA_ERR_NULL, FA_ERR_HIP.
 */
int fa_calib_mfma(int kind, int64_t workgroups, int64_t iters, float* out, void* stream);

/*
 * fa_calib_copy -- dst[0 .. bytes) = src[0 .. bytes) (device memory) by 16-byte
 * loads and stores, each byte read once and written once: `bytes` of HBM reads and
 * `bytes` of HBM writes per launch.
 * Errors: FA_ERR_SHAPE (bytes negative or not a multiple of 16), FA_ERR_NULL,
 * FA_ERR_UNSUPPORTED (a pointer not 16-byte aligned), FA_ERR_ALIAS (the ranges
 * overlap), FA_ERR_HIP.
 */
int fa_calib_copy(const void* src, void* dst, int64_t bytes, void* stream);

/*
 * fa_calib_read -- reads src[0 .. bytes) (device memory) once by 16-byte loads and
 * writes one 32-bit XOR of what each thread read into out: `bytes` of HBM reads
 * per launch (and a few KiB of writes).
 *   out: uint32 [min(ceil(bytes / 16384), 16384) * 256] (device); at most
 *   FA_CALIB_READ_OUT_WORDS words.
 * Errors: as fa_calib_copy (FA_ERR_ALIAS: out overlaps src).
 */
#define FA_CALIB_READ_OUT_WORDS (16384 * 256)
int fa_calib_read(const void* src, int64_t bytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_CALIB_H_ */
