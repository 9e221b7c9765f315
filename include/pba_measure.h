/*
 * pba_measure.h -- measurement helpers of libpba (gfx950), not operations of
 * packed attention.  They run fixed instruction loops whose timings give the
 * sustained unit rates (bf16 MFMA, LDS reads, vector ALU and exp) that the
 * attention kernels' rooflines are argued from.  Conventions (device memory
 * from the caller, no allocation or synchronisation, work enqueued on
 * `stream`, host argument errors returned synchronously) and return codes
 * are those of pba.h.
 */
#ifndef PBA_MEASURE_H
#define PBA_MEASURE_H

#include "pba.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueues n_blocks workgroups of 256 threads that each run `iters` iterations of 16 bf16
 * MFMAs (v_mfma_f32_32x32x16_bf16, 32768 FLOP each) per wave, i.e.
 * n_blocks * 4 * iters * 16 * 32768 FLOP, and write one float per thread
 * to `out` (device, caller-allocated, n_blocks * 256 floats).  Timing it
 * gives the sustained MFMA rate of the device.  Returns PBA_OK,
 * PBA_ERR_NULL, PBA_ERR_SHAPE (n_blocks outside 1..2^20 or iters < 1) or
 * PBA_ERR_DEVICE. */
PBA_API int pba_mfma_probe(float* out, int n_blocks, int iters, void* stream);

/* n_blocks workgroups of 512 threads, each filling a
 * 64 KB LDS array and then reading `iters` x 16 times 16 bytes per thread
 * from it (lane-contiguous, no bank conflicts), i.e.
 * n_blocks * 512 * 256 * iters bytes of LDS reads; one float per thread to
 * `out` (device, n_blocks * 512 floats).  Timing it gives the sustained LDS
 * read bandwidth.  Errors as pba_mfma_probe. */
PBA_API int pba_lds_probe(float* out, int n_blocks, int iters, void* stream);

/* n_blocks workgroups of 256 threads, each thread
 * running `iters` x 16 independent fp32 FMAs (exp2 = 0), or 16 times
 * v_exp_f32 followed by one multiply (exp2 = 1); one float per thread to
 * `out` (device, n_blocks * 256 floats).  Timing it gives the vector-ALU
 * and the transcendental issue rates.  Errors as pba_mfma_probe
 * (PBA_ERR_SHAPE also for exp2 outside {0, 1}). */
PBA_API int pba_valu_probe(float* out, int n_blocks, int iters, int exp2, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PBA_MEASURE_H */
