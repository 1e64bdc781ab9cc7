/*
 * tidar_ceilings.h - measurement kernels of libtidar: the machine ceilings
 * that the decode step's rooflines are stated against (HBM streaming read,
 * bf16 MFMA rate, LDS read rate, fp32 exponential and FMA issue rates, one
 * empty kernel).
 * They compute nothing of the method; bench.py times them with HIP events on
 * the stream they are enqueued on.
 *
 * Conventions as in tidar.h: device pointers, enqueue only, no allocation,
 * no synchronisation. Return 0 on success, -1 for a bad argument (nothing is
 * launched), -5 when the launch fails.
 */
#ifndef TIDAR_CEILINGS_H_
#define TIDAR_CEILINGS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a positive multiple of 16; src 16-byte aligned) once with a
 * grid of `grid` 256-thread workgroups, 16-byte loads. `sink` is one device
 * uint32 that is written only with a value the data cannot produce. */
int tidar_ceiling_hbm_read(const void* src, size_t bytes, int grid, uint32_t* sink, void* stream);

/* `grid` workgroups of 4 waves; each wave issues 4 * iters
 * v_mfma_f32_32x32x16_bf16 (32768 flops each) on four independent chains:
 * grid * 4 * 4 * iters * 32768 flops in all. `sink`: one device float. */
int tidar_ceiling_mfma_bf16(int grid, int iters, float* sink, void* stream);

/* `grid` workgroups of 256 threads, each with a 64 KB LDS buffer (two fit
 * on a CU): every wave issues 8 * iters LDS reads, ds_read_b128 (16 bytes per
 * lane: grid * 256 * 8 * iters * 16 bytes in all) or the transposing
 * ds_read_b64_tr_b16 (8 bytes per lane). `sink`: one device uint32. */
int tidar_ceiling_lds_read_b128(int grid, int iters, uint32_t* sink, void* stream);
int tidar_ceiling_lds_read_tr16(int grid, int iters, uint32_t* sink, void* stream);

/* `grid` workgroups of 256 threads; each thread evaluates 8 * iters fp32
 * base-2 exponentials (v_exp_f32) on eight independent chains. */
int tidar_ceiling_exp_f32(int grid, int iters, float* sink, void* stream);

/* Same shape with fp32 FMAs (v_fma_f32) instead of exponentials. */
int tidar_ceiling_fma_f32(int grid, int iters, float* sink, void* stream);

/* An empty kernel of `grid` workgroups of 64 threads (launch and kernel
 * boundary cost). */
int tidar_ceiling_empty(int grid, void* stream);

/* Per-workgroup timestamps of the last attention launch made with the
 * environment variable TIDAR_ATTN_STAMPS=1 set when tidar_attn_step was
 * called (it selects a timestamped instantiation of the bf16 main kernel
 * that computes exactly what the plain one does; only the head_dim-128,
 * single-sequence-plan launch without an LSE output has one, other launches
 * run unstamped). Copies the records of the first `max_workgroups`
 * workgroups (at most 4096) into host memory `dst`, 8 uint64 each:
 * shader-clock counter (s_memtime) at entry, the 100 MHz reference
 * (s_memrealtime) at entry, s_memtime once tile 0's scores are in registers,
 * s_memtime after the tile loop, s_memtime and s_memrealtime after the
 * output stores are acknowledged, HW_ID | XCC_ID << 32, and tiles | split
 * << 16 | grid size << 32. Synchronous: waits for the device copy. Returns
 * 0, -1 for a bad argument, -5 when the copy fails. */
int tidar_attn_stamps(uint64_t* dst, int max_workgroups);

#ifdef __cplusplus
}
#endif

#endif /* TIDAR_CEILINGS_H_ */
