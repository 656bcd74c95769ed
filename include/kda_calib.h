/* kda_calib.h -- a kernel of known instruction count, for scaling hardware counters.
 *
 * Not part of the KDA computation.  The profiler's MFMA-busy counter
 * (SQ_VALU_MFMA_BUSY_CYCLES) has no documented unit; a dispatch of this kernel issues a
 * known number of v_mfma_f32_16x16x32_bf16 instructions, so the counter's value for it
 * gives the busy cycles per instruction, and its duration the sustained MFMA rate, by
 * which the counters of the KDA kernels are read.  The same role as the plain device
 * copy that scales the HBM byte counters.
 */
#ifndef KDA_CALIB_H
#define KDA_CALIB_H

#ifdef __cplusplus
extern "C" {
#endif

/* Launches n_workgroups workgroups of 256 threads (4 waves) on `stream` (a hipStream_t,
 * NULL for the default stream).  Every wave issues a dependent chain of `iters`
 * v_mfma_f32_16x16x32_bf16 instructions (16 * 16 * 32 multiply-adds each; the waves that
 * share a SIMD overlap their chains), then writes one float per thread to
 * out[n_workgroups * 256] (device memory, caller-owned), so that the products are not
 * discarded.  Total MFMA instructions: n_workgroups * 4 * iters.
 * Returns 0, or 1 for n_workgroups or iters below 1 or a null out (nothing launched), or
 * the HIP error code of the launch plus 1000. */
int kda_calib_mfma(int n_workgroups, int iters, float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif
