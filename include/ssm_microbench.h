/*
 * ssm_microbench.h -- measurement-only microbenchmarks (libssm_microbench.so).
 *
 * They measure, on the current HIP device, the rates that bound the scan and
 * SSD kernels, to set measured ceilings next to the published peaks.  Nothing
 * in the product path calls them.  Each function allocates its own small
 * buffers, runs on the null stream, synchronises, frees what it allocated and
 * returns the best of three timed runs after one warm-up, or a negative value
 * when a HIP call fails.
 */
#ifndef SSM_MICROBENCH_H
#define SSM_MICROBENCH_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* fp32 FMA lane-operations per second (v_fma_f32, 8 independent chains per lane). */
double ssm_mb_fma_rate(void);
/* v_exp_f32 lane-operations per second (8 independent chains per lane). */
double ssm_mb_exp_rate(void);
/* Scan recurrence elements per second: one v_exp_f32 and six dependent VALU
 * ops per element (the per-(token, channel, state) work of the selective scan),
 * 8 independent chains per lane. */
double ssm_mb_scan_element_rate(void);
/* Dense bf16 matrix FLOP/s of v_mfma_f32_16x16x32_bf16 (8 independent accumulators per wave). */
double ssm_mb_mfma_bf16_flops(void);
/* HBM copy: bytes read plus bytes written per second for two device buffers of
 * `bytes` each (float4 grid-stride copy). */
double ssm_mb_copy_bytes_per_s(size_t bytes);

#ifdef __cplusplus
}
#endif

#endif
