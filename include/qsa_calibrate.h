/*
 * qsa_calibrate.h -- C ABI of libqsa_calib.so, the two calibration kernels the QSA
 * measurements are reported against (not part of the QSA path; libqsa.so does not use it).
 *
 * Both enqueue one kernel on `stream` and return at once: 0 on success, 1 for an invalid
 * argument (nothing enqueued), 3 when the launch failed.  Pointers are DEVICE pointers owned
 * by the caller.  Timing is the caller's (events around the call on the same stream).
 */
#ifndef QSA_CALIBRATE_H_
#define QSA_CALIBRATE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads every byte of src[0 .. bytes) once with 16-byte loads (bytes a multiple of 16,
 * src 16-byte aligned), `blocks` workgroups of 256 lanes in a grid-stride loop with eight
 * loads in flight per lane; writes one XOR checksum per workgroup to sink[0 .. blocks). */
int qsa_calib_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks,
                          hipStream_t stream);

/* `blocks` workgroups of 8 waves (two per SIMD when blocks is a multiple of the CU count),
 * each wave issuing iters x 4 dense v_mfma_f32_32x32x16_bf16 on register operands (four
 * independent accumulators).  Writes the algorithmic flop count of the launch to *flops (a
 * HOST pointer) and one float per lane to sink[0 .. qsa_calib_mfma_sink_floats(blocks)). */
int qsa_calib_mfma_bf16(int iters, int blocks, float* sink, double* flops, hipStream_t stream);

/* Floats of sink that qsa_calib_mfma_bf16 writes for `blocks` workgroups. */
int qsa_calib_mfma_sink_floats(int blocks);

#ifdef __cplusplus
}
#endif

#endif /* QSA_CALIBRATE_H_ */
