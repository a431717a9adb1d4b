/*
 * rpa_probes.h -- measurement probes of the MI355X (gfx950) that give the
 * attention kernels' roofline figures a measured ceiling next to the
 * published peaks: HBM streaming bandwidth, dense bf16 MFMA throughput with
 * the shader clock it runs at, and the issue rate of the VALU instructions the
 * softmax is made of (v_exp_f32, v_rcp_f32, v_fma_f32).
 *
 * Library librpa_probes.so (separate from librpa.so; nothing in the attention
 * path uses it).  Every pointer is a caller-owned DEVICE pointer; each call
 * enqueues one kernel on `stream` (a hipStream_t, NULL = default stream) and
 * returns 0 or a HIP error code.  The caller times the launch (events on the
 * same stream) and converts it with the work counts stated below.
 */
#ifndef RPA_PROBES_H_
#define RPA_PROBES_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads n16 16-byte words of src once, with non-temporal loads spread over
 * `blocks` workgroups of 256 threads (grid-stride), and writes one 32-bit word
 * per thread to sink (blocks * 256 words) so the loads are kept.  Bytes moved:
 * 16 * n16 read (sink writes are negligible).  src must be 16-byte aligned. */
int rpa_probe_read(const void* src, size_t n16, uint32_t* sink, int blocks, void* stream);

/* Copies n16 16-byte words src -> dst (non-temporal loads and stores), over
 * `blocks` workgroups of 256 threads.  Bytes moved: 32 * n16. */
int rpa_probe_copy(const void* src, void* dst, size_t n16, int blocks, void* stream);

/* Dense bf16 MFMA burn: every wave of `blocks` workgroups of 256 threads runs
 * 4 independent accumulation chains of v_mfma_f32_32x32x16_bf16 for `iters`
 * steps (4 * iters MFMAs per wave, 32 * 32 * 16 * 2 FLOPs each), then stores
 * its accumulators to sink (blocks * 256 * 16 floats).  Lane 0 of each wave
 * also writes clocks[2 * wave] = shader clock cycles (s_memtime) and
 * clocks[2 * wave + 1] = constant-rate (100 MHz) ticks (s_memrealtime) it
 * spent, so the shader clock under full matrix load is
 * 100 MHz * clocks[0] / clocks[1].  clocks holds 2 * blocks * 4 int64. */
int rpa_probe_mfma(float* sink, int64_t* clocks, int iters, int blocks, void* stream);

/* VALU issue rate: every lane of `blocks` workgroups of 256 threads runs 8
 * independent chains of one instruction for `iters` steps (8 * iters
 * instructions per lane) and stores its chain values to sink (blocks * 256 * 8
 * floats).  op 0: v_exp_f32, 1: v_rcp_f32, 2: v_fma_f32.  Lane-operations
 * per launch: blocks * 256 * 8 * iters. */
int rpa_probe_valu(float* sink, int op, int iters, int blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RPA_PROBES_H_ */
