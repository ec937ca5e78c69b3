/*
 * w4a8_peaks.h — on-device peak probes that the W4A8 measurements are set
 * against, next to the datasheet peaks (HBM 8 TB/s; dense int8 matrix cores
 * 5.0 POP/s at 2.4 GHz).
 *
 * "The 4-bit CPU path", its commit message: every measured figure is reported
 * with its spread and the baseline it is compared with.  A datasheet peak
 * assumes the full engine clock and an ideal access pattern; these two
 * kernels measure what this device reaches in the same run, so a kernel's
 * fraction can be stated against both.
 *
 * Conventions are those of include/w4a8.h: caller-owned device buffers,
 * asynchronous on `stream` (a hipStream_t as void*), 0 or a negative W4A8
 * status, all checks on the host before any launch, w4a8_last_error() for
 * the detail.
 */
#ifndef W4A8_PEAKS_H
#define W4A8_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * w4a8_peak_stream_read — reads `bytes` of device memory once with 16-byte
 * loads (every lane of a wavefront reads consecutive 16-byte pieces, a grid
 * of `blocks` 256-thread workgroups strides over the buffer) and folds what
 * it read into a value that is stored only when it equals a constant no
 * input reaches in practice, so the loads cannot be removed and almost
 * nothing is written.
 *   buf   device, `bytes` bytes, 16-byte aligned; bytes % 16 == 0, > 0
 *   sink  device uint32 [blocks] (written only in the unlikely case above)
 *   blocks  1 .. 65536 workgroups
 * A buffer larger than the 256 MB last-level cache measures HBM.
 */
int w4a8_peak_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks,
                          void* stream);

/*
 * w4a8_peak_mfma_i8 — every wavefront runs `iters` rounds of eight
 * independent v_mfma_i32_16x16x64_i8 (32768 int8 operations each) on
 * operands drawn from its lane index, in `blocks` workgroups of 256 threads
 * (pass 2 x compute units for two wavefronts per SIMD).  Integer operations
 * per launch: iters * 8 * 32768 * blocks * 4.
 *   sink    device int32 [blocks * 256]: each thread's folded accumulators
 *   clocks  device uint64 [2 * blocks] or NULL: per workgroup, the shader
 *           clock cycles (s_memtime) and the 100 MHz constant clock ticks
 *           (s_memrealtime) that its first wavefront saw across the loop;
 *           their ratio gives the engine clock the MFMAs ran at
 *   iters   1 .. 2^20
 */
int w4a8_peak_mfma_i8(int32_t iters, int32_t* sink, uint64_t* clocks, int32_t blocks,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A8_PEAKS_H */
