/*
 * mxfp4_probe.h - measurement probes of the MI355X (gfx950) MXFP4 library.
 *
 * Not part of the GEMM path.  They measure the two ceilings the GEMM kernels
 * are compared against, on the machine at hand, next to the published peaks:
 *   - the rate at which the matrix cores retire block-scaled MFMAs (FP4 x FP4,
 *     or FP4 x FP8 as in the W4A8 GEMM) when a kernel does nothing else (the
 *     clock they sustain under that load sets it, not only the unit counts);
 *   - the HBM read rate of a plain streaming kernel.
 * Both live in libmxfp4.so and follow the conventions of mxfp4.h: device
 * pointers on the current device, caller-owned buffers, stream-ordered
 * asynchronous launches, host-side argument checks that launch nothing on
 * failure, and mxfp4_last_error() for details.
 */
#ifndef MXFP4_PROBE_H_
#define MXFP4_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "mxfp4.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * MFMA probe: `blocks` workgroups of 8 waves (the occupancy of the 256x256
 * GEMM tile kernel); every wave runs `iters` iterations of 8 independent
 * v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands (a 128x64 accumulator
 * block per wave, like a wave of the tile kernel), with no memory traffic in
 * the loop.  Operand registers start from `seed` and change every iteration,
 * so the matrix cores switch as they do on real data.
 *   seed  device, >= MXFP4_PROBE_SEED_BYTES bytes, 16-byte aligned (any bytes);
 *   out   device float[blocks * 512], 16-byte aligned (per-thread sums that keep
 *         the work live; their values mean nothing);
 *   1 <= blocks <= 65536, 1 <= iters <= 2^24.
 * mxfp4_probe_mfma_flops() gives the floating-point operations one call does.
 */
#define MXFP4_PROBE_SEED_BYTES 6144
mxfp4_status_t mxfp4_probe_mfma(const void* seed, void* out, int32_t blocks, int32_t iters, void* stream);
double mxfp4_probe_mfma_flops(int32_t blocks, int32_t iters);

/*
 * The same probe with the MFMA's second operand in FP8 E4M3 (the W4A8
 * GEMM's A operand), built from the same seed with NaN codes masked off;
 * same arguments, same flop count (mxfp4_probe_mfma_flops).
 */
mxfp4_status_t mxfp4_probe_mfma_w4a8(const void* seed, void* out, int32_t blocks, int32_t iters, void* stream);

/*
 * Read probe: `blocks` workgroups of 256 threads read `bytes` bytes of `src`
 * once, 16 bytes per load, 16 loads in flight per thread, and write one
 * 32-bit value per thread to `out` (the XOR of what it read).
 *   src   device, 16-byte aligned, bytes a positive multiple of 16, <= 2^40;
 *   out   device uint32[blocks * 256], 4-byte aligned;
 *   1 <= blocks <= 65536.
 */
mxfp4_status_t mxfp4_probe_read(const void* src, int64_t bytes, void* out, int32_t blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_PROBE_H_ */
