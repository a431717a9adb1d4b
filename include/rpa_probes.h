/*
 * rpa_probes.h -- measurement probes of the MI355X (gfx950) that give the
 * attention kernels' roofline figures a measured ceiling next to the
 * published peaks: HBM streaming bandwidth, dense bf16 MFMA throughput with
 * the shader clock it runs at, the issue rate of the VALU instructions the
 * softmax is made of (v_exp_f32, v_rcp_f32, v_fma_f32), and the LDS and
 * global -> LDS rates the prefill kernel's block pipeline depends on.
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

/* LDS throughput: every wave of `blocks` workgroups of 256 threads (32 KiB of
 * LDS each) runs `iters` rounds of 8 LDS instructions over its own 8 KiB, at
 * contiguous (conflict-free) lane addresses.  op 0: ds_read_b128 (1 KiB per
 * instruction and wave), 1: ds_read_b64_tr_b16 (512 B), 2: ds_write_b128
 * (1 KiB).  Bytes per launch: blocks * 4 * iters * 8 * (1024, 512, 1024).
 * sink receives blocks * 256 words; clocks as for rpa_probe_mfma (2 * blocks
 * * 4 int64). */
int rpa_probe_lds(uint32_t* sink, int64_t* clocks, int op, int iters, int blocks, void* stream);

/* Global -> LDS copy rate (global_load_lds_dwordx4): every wave of `blocks`
 * workgroups of 256 threads copies 8 KiB per round (8 instructions of 1 KiB)
 * into its own 8 KiB of LDS and waits for them, for `iters` rounds, walking
 * a source window of window_bytes (a multiple of 1024, at least 8192) from a
 * per-wave starting point.  A window that fits in L2 measures the L2 -> LDS
 * path.  Bytes per launch: blocks * 4 * iters * 8192.  sink and clocks as for
 * rpa_probe_lds. */
int rpa_probe_dma(const void* src, size_t window_bytes, uint32_t* sink, int64_t* clocks, int iters,
                  int blocks, void* stream);

/* MFMA beside VALU work in the same wave: every wave of `blocks` workgroups of
 * 256 threads runs `iters` rounds of 4 independent v_mfma_f32_32x32x16_bf16
 * chains, each MFMA followed by nv (0..4) VALU pairs on chains of their own:
 * v_fma_f32 then v_exp_f32 (exp = 1) or two v_fma_f32 (exp = 0).  4 * iters
 * MFMAs per wave; sink: blocks * 256 * 16 floats; clocks as for
 * rpa_probe_mfma.  The MFMA rate against rpa_probe_mfma's shows how much of
 * that VALU work runs under the matrix cores. */
int rpa_probe_mix(float* sink, int64_t* clocks, int nv, int exp, int iters, int blocks,
                  void* stream);

/* rpa_probe_mix built with the MFMA accumulators in VGPRs (the form the
 * attention kernels' MFMAs take, since their VALU code reads the
 * accumulators) rather than AGPRs, where the compiler puts them in
 * rpa_probe_mix.  Same arguments and work. */
int rpa_probe_mix_vgpr_acc(float* sink, int64_t* clocks, int nv, int exp, int iters, int blocks,
                           void* stream);

/* MFMA fed from LDS, in the prefill kernel's operand patterns: every wave of
 * `blocks` workgroups of 256 threads (32 KiB of LDS each) runs `iters` rounds
 * of 16 v_mfma_f32_32x32x16_bf16.  mode 0: A operand from one ds_read_b128
 * issued two MFMAs ahead, 2 accumulators in turn (the q.k pattern); 1: A
 * from two ds_read_b64_tr_b16 issued one MFMA ahead, 4 accumulators (the p.v
 * pattern); 2: mode 0 with A from registers; 3: mode 0 with 4 accumulators.
 * 16 * iters MFMAs per wave; sink: blocks * 256 * 16 floats; clocks as for
 * rpa_probe_mfma. */
int rpa_probe_lds_mfma(float* sink, int64_t* clocks, int mode, int iters, int blocks,
                       void* stream);

/* LDS reads beside global -> LDS copies: in every workgroup of 256 threads,
 * waves 0 and 1 run rounds of 8 ds_read_b128 over their own 8 KiB of LDS
 * (mode bit 0; 8 KiB per round) and waves 2 and 3 rounds of 8 KiB of
 * global -> LDS copies from a window of window_bytes (as for rpa_probe_dma;
 * mode bit 1), until `ticks` of the 100 MHz constant clock have passed.
 * counts[2 w] = rounds of wave w, counts[2 w + 1] = its shader clocks
 * (2 * blocks * 4 int64); sink: blocks * 256 words.  Mode 1 or 2 runs one
 * kind alone, 3 both side by side. */
int rpa_probe_lds_dma(const void* src, size_t window_bytes, uint32_t* sink, int64_t* counts,
                      int mode, int64_t ticks, int blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RPA_PROBES_H_ */
