/*
 * fa_ceilings.h — C ABI of libfa_ceilings: measured ceilings of the GPU the
 * attention kernels of libfa run on.  The kernels' rooflines use the
 * published peaks of the part (dense bf16 matrix cores 2.5 PFLOP/s at
 * 2.4 GHz, HBM 8 TB/s); these entry points measure what this part actually
 * delivers at the clock it holds: matrix-core throughput of
 * v_mfma_f32_32x32x16_bf16 (the instruction every bf16 attention kernel is
 * built on), a streaming HBM read, the LDS read rate of the two read forms the
 * kernels use, and the core clock under matrix-core load.  No entry point
 * defines anything of the attention method itself.
 *
 * Conventions: pointers are DEVICE pointers; the caller owns every buffer;
 * each call only enqueues one kernel on `stream` (a hipStream_t, NULL = the
 * default stream) and the caller times it (HIP events on that stream).  The
 * return value is 0 (hipSuccess) or a hipError_t code; invalid arguments
 * return hipErrorInvalidValue (1) before anything is enqueued.
 */
#ifndef FA_CEILINGS_H
#define FA_CEILINGS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Compute units, constant-rate counter frequency (kHz, the rate of the wall
 * ticks recorded below) and the part's peak core clock (kHz) of the current
 * device. */
int fa_ceil_device(int* ncu, int* wall_clock_khz, int* peak_clock_khz);

/* workgroups x 4 waves each run iters rounds of 4 independent
 * v_mfma_f32_32x32x16_bf16 (32768 FLOP each): 4 * 32768 * iters FLOP per wave.
 * sink: float[4 * workgroups] (written; keeps the products alive).
 * stamps: uint64[16 * workgroups]: per wave (core cycles before, after; wall
 * ticks before, after), written by lane 0. */
int fa_ceil_mfma_bf16(float* sink, unsigned long long* stamps, int workgroups, int iters, void* stream);

/* Reads `bytes` (a multiple of 16, buf 16-byte aligned) once with 16-byte
 * non-temporal loads spread over `workgroups` of 256 lanes, each lane keeping
 * loads_in_flight (4, 8 or 16) loads in flight.  sink: 16 * 256 * workgroups
 * bytes, 16-byte aligned; written only if the xor of the data hits a fixed
 * 64-bit pattern (never, for data the caller plants), so the launch is the
 * read alone. */
int fa_ceil_hbm_read(const void* buf, size_t bytes, void* sink, int workgroups, int loads_in_flight,
                     void* stream);

/* Streaming read through direct-to-LDS loads (global_load_lds_dwordx4), the
 * load form the decode streams its cache with: `workgroups` one-wave
 * workgroups each read a contiguous share of buf (16-byte aligned) in 1 KB
 * instructions into a private LDS ring of `stages` (2..4) stages of
 * `stage_kb` (4, 8 or 16) KB, at most stages - 1 stages in flight, with the
 * default (nontemporal = 0) or the non-temporal (1) cache policy.  The bytes
 * read are fa_ceil_hbm_read_lds_bytes(bytes, workgroups, stage_kb) (each share
 * rounded down to whole stages); that function returns 0 for arguments the
 * read refuses. */
long long fa_ceil_hbm_read_lds_bytes(size_t bytes, int workgroups, int stage_kb);
int fa_ceil_hbm_read_lds(const void* buf, size_t bytes, int workgroups, int stage_kb, int stages, int nontemporal,
                         void* stream);

/* LDS read rate: each of `workgroups` (256 lanes, 64 KB of LDS each) fills its
 * LDS, then each of its 4 waves reads 4 * iters times: mode 0 ds_read_b128
 * (1 KB per read, conflict-free consecutive slots), mode 1 ds_read_b64_tr_b16
 * (512 B per read, the attention kernels' transposed-fragment addressing of a
 * swizzled 256-byte-row tile), mode 2 ds_read_b64 (512 B per read,
 * consecutive slots), mode 3 ds_read_b64_tr_b16 of the same tile without the
 * swizzle.  sink: uint32[256 * workgroups] (written only
 * for one data pattern that does not occur).  stamps as fa_ceil_mfma_bf16, per
 * wave, around the read loop. */
int fa_ceil_lds_read(void* sink, unsigned long long* stamps, int mode, int workgroups, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_CEILINGS_H */
