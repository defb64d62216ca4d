/*
 * Measurement probes of libbfp8_probes.so (not part of the GEMM path). The benchmark runs them
 * to report the GEMM kernels against ceilings measured on the same device in the same run,
 * next to the vendor peaks (dense FP8 matrix throughput, HBM bandwidth).
 *
 * All calls enqueue one kernel on `stream` (a hipStream_t passed as void*; NULL = the null
 * stream) and return 0 when it was enqueued, 1 for invalid arguments (nothing launched), 2
 * when the launch failed. Pointers are device pointers owned by the caller.
 */
#ifndef BFP8_PROBES_H_
#define BFP8_PROBES_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * FP8 matrix-core loop: `workgroups` workgroups of 8 waves; every wave issues `iters` steps of
 * 8 independent 16x16x128 e4m3 MFMAs (gfx950 v_mfma_f32_16x16x128_f8f6f4) on register operands,
 * no memory traffic. mode 0: each MFMA accumulates into its chain (C = the chain's previous
 * result); mode 1: each MFMA starts from a zero accumulator and its product is scaled into a
 * float32 sum with four FMAs (the per-128-block promotion acc += P * (As * Bs) of the blockwise
 * method); mode 2: zero accumulator, one element of each product added to a sum. Other modes
 * return 1. out: workgroups * 512 floats (one result per lane, written so the work is not dead).
 */
int bfp8_probe_mfma_loop(float* out, int workgroups, int iters, int mode, void* stream);

/* FLOPs of one bfp8_probe_mfma_loop launch (2 * 16 * 16 * 128 per MFMA). */
double bfp8_probe_mfma_loop_flops(int workgroups, int iters);

/*
 * The same loop with 4 independent 32x32x64 e4m3 MFMAs per step (gfx950
 * v_mfma_f32_32x32x64_f8f6f4, whose K of 64 is one group of the 1x64 layout). mode 0: each MFMA
 * accumulates into its chain; mode 1: each starts from a zero accumulator and its 16 results are
 * scaled into float32 sums with 16 FMAs (the promotion of the 1x64 method). Other modes return 1.
 */
int bfp8_probe_mfma32_loop(float* out, int workgroups, int iters, int mode, void* stream);

/* FLOPs of one bfp8_probe_mfma32_loop launch (2 * 32 * 32 * 64 per MFMA). */
double bfp8_probe_mfma32_loop_flops(int workgroups, int iters);

/*
 * Streaming read of `bytes` bytes (a multiple of 16) at src (16-byte aligned) by `workgroups`
 * workgroups of 256 threads, 16-byte loads, eight in flight per thread, each byte read once.
 * out: workgroups * 256 words (one per thread, so the loads are not dead).
 */
int bfp8_probe_stream_read(const void* src, size_t bytes, uint32_t* out, int workgroups, void* stream);

/*
 * Global -> LDS copy throughput: `workgroups` workgroups of 8 waves; every wave issues `iters`
 * copies of 8 rows x 128 bytes (8 lanes per row, 16 bytes per lane) of a [rows][4096]-byte
 * matrix at src, keeping `inflight` (4, 8 or 16; iters a multiple of it) of them in flight.
 * dma 1: the direct-to-LDS load; dma 0: a load into registers and an LDS write; dma 2, 3 or 4
 * (inflight 8 only): the direct-to-LDS load with 16, 32 or 64 lanes per row, i.e. 4 rows of
 * 256, 2 of 512 or 1 of 1024 bytes per copy. Copy c reads row group c % groups (groups a power
 * of two; src must hold groups * 8 rows of 4096 bytes) at column block (c / groups) % 32.
 * Bytes moved: workgroups * 8 * iters * 1024. out: workgroups * 512 words.
 */
int bfp8_probe_copy_lds(const void* src, uint32_t groups, int iters, int inflight, int dma, uint32_t* out,
                        int workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BFP8_PROBES_H_ */
