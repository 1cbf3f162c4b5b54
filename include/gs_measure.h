/*
 * gs_measure.h -- C ABI of libgs_measure.so, the two calibration kernels a
 * benchmark times beside the rasterizer (gfx950).  They compute nothing of the
 * method: their rates are the HBM and fp32 figures this GPU actually delivers,
 * quoted next to its published peaks as a second roofline denominator.
 *
 * Conventions as in gs.h: device pointers, a hipStream_t passed as void*, the
 * calls only enqueue work, GS_OK (0) or a negative gs.h error code.
 */
#ifndef GS_MEASURE_MI355X_H
#define GS_MEASURE_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * gs_stream_copy -- dst[i] = src[i] for i < count (float32, count a multiple
 * of 4, both arrays 16-byte aligned, not overlapping), read and written with
 * non-temporal 16-byte accesses: 8 count bytes of HBM traffic.
 * -1: count negative or not a multiple of 4, or a null pointer; -2: misaligned.
 */
int gs_stream_copy(const float* src, float* dst, int64_t count, void* stream);

/*
 * gs_fma_loop -- `blocks` blocks of 256 lanes, each running 8 independent
 * chains f <- f a + b (fp32 FMA), 8 steps of each chain per iteration for
 * `iters` iterations, then writing the sum of its chains to
 * out[block * 256 + lane] (out holds blocks * 256 floats):
 * blocks * 256 * iters * 128 flops.  With a = 1, b = 0 each lane writes
 * 8 lane + 28 exactly.  -1: blocks < 1, iters < 0 or out null.
 */
int gs_fma_loop(int32_t blocks, int32_t iters, float a, float b, float* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif
