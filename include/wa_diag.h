/*
 * wa_diag.h -- measurement probes beside the Whisper attention library.
 *
 * Not part of the attention path: these calls exist so that a measured
 * throughput can be set against what this GPU sustains at the moment it is
 * measured (matrix-core rate and shader clock under load), not only against
 * the published peak.  They live in their own library, libwa_diag.so.
 */
#ifndef WA_DIAG_H
#define WA_DIAG_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "wa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { WA_DIAG_BF16 = 0, WA_DIAG_FP8 = 1 } wa_diag_dtype;

/*
 * wa_diag_mfma_ceiling -- back-to-back dense matrix-core products.
 *
 * What: n_blocks blocks of 4 waves; every wave issues iters x 4 products on
 *   four independent accumulators, nothing else: v_mfma_f32_32x32x16_bf16
 *   (32*32*16*2 = 32768 flop each) for WA_DIAG_BF16, or the fp8 (E4M3)
 *   v_mfma_f32_32x32x64_f8f6f4 (131072 flop each) for WA_DIAG_FP8.  The
 *   call's flop count is n_blocks * 4 * iters * 4 * that figure; the caller
 *   times it (events on `stream`).  Use at least 2 blocks per compute unit.
 * ticks      device uint64 [n_blocks][2]: per block, the shader-clock cycles
 *            (s_memtime) and the 100 MHz constant-clock ticks
 *            (s_memrealtime) its first wave spent in the loop; their ratio
 *            times the constant clock's rate (wa_diag_wall_clock_khz) is
 *            the shader clock under this load.
 * Errors: null ticks, n_blocks or iters outside [1, 2^20], or a bad dtype ->
 *   WA_ERR_INVALID_ARGUMENT; a launch failure -> WA_ERR_HIP.
 */
wa_status wa_diag_mfma_ceiling(wa_diag_dtype dtype, int n_blocks, int iters, uint64_t *ticks,
                               hipStream_t stream);

/*
 * wa_diag_sclk_probe -- the shader clock right now.
 *
 * What: n_blocks blocks of one wave; each reads the shader clock
 *   (s_memtime) and the 100 MHz constant clock (s_memrealtime) while it
 *   spins for `spin` constant-clock ticks (bounded by a read count as well,
 *   so it always ends).  Launched on `stream` right after a kernel, it reads
 *   the clock that kernel left the GPU at: the power management changes it
 *   over much longer times than the probe takes (a spin of 500 is 5 us).
 * ticks      device uint64 [n_blocks][2]: shader-clock cycles and
 *            constant-clock ticks of each block's spin; their ratio times
 *            wa_diag_wall_clock_khz is the shader clock.
 * Errors: null ticks, n_blocks outside [1, 2^16] or spin outside [1, 10^5]
 *   -> WA_ERR_INVALID_ARGUMENT; a launch failure -> WA_ERR_HIP.
 */
wa_status wa_diag_sclk_probe(int n_blocks, int spin, uint64_t *ticks, hipStream_t stream);

/*
 * wa_diag_wall_clock_khz -- the rate of the constant clock that
 * s_memrealtime counts on the current device, in kHz, into *khz (host).
 * Errors: null khz -> WA_ERR_INVALID_ARGUMENT; HIP failure -> WA_ERR_HIP.
 */
wa_status wa_diag_wall_clock_khz(int *khz);

#ifdef __cplusplus
}
#endif

#endif /* WA_DIAG_H */
