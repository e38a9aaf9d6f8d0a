/*
 * qkra_phase_stamps -- the profiling build of the attention library
 * (libqknorm_rope_attn_stamps.so, the same sources compiled with
 * -DQKRA_PHASE_STAMPS).  Its bf16 prefill attention kernels record, for every
 * workgroup below QKRA_STAMP_WGS and each of its QKRA_STAMP_WAVES
 * wavefronts, the 100 MHz constant clock (s_memrealtime) at the points below
 * and where the workgroup ran.  The attention itself is unchanged
 * (Code Walkthrough "Chapter 3 Forward Pass and Generation", section 3.3),
 * and so is every entry point of qknorm_rope_attn.h; the normal library
 * exports none of the symbols declared here.
 *
 * Record layout: uint64 stamps[QKRA_STAMP_WGS][QKRA_STAMP_WAVES][QKRA_STAMP_SLOTS]
 * indexed by the hardware workgroup id (blockIdx.x).  A later launch
 * overwrites the records of the workgroups it runs; a workgroup that ran no
 * work item (past the items, or the other softmax kernel's) leaves
 * QKRA_STAMP_END untouched, so clear the records before the launch to tell
 * them apart.  Slot QKRA_STAMP_WHERE holds HW_ID bits 0-15 (wave, SIMD, CU,
 * shader array, shader engine), XCC_ID bits 16-19, the item's K/V tile count
 * at bits 20-35 and its logical item index at bits 36-62.  In the fused
 * mixed-step kernel the workgroups of the decode role stamp only
 * QKRA_STAMP_ENTRY and QKRA_STAMP_END, and set bit 63 of QKRA_STAMP_WHERE.
 */
#ifndef QKRA_PHASE_STAMPS_H
#define QKRA_PHASE_STAMPS_H

#include <stddef.h>
#include <stdint.h>

#define QKRA_STAMP_WGS 16384
#define QKRA_STAMP_WAVES 8
#define QKRA_STAMP_SLOTS 8

#define QKRA_STAMP_ENTRY 0      /* first instruction */
#define QKRA_STAMP_ISSUED 1     /* item decoded, tile 0 and Q loads issued, softmax path taken */
#define QKRA_STAMP_Q_READY 2    /* Q normalised, rotated and in MFMA operand registers */
#define QKRA_STAMP_LOOP 3       /* tile 0 in LDS and scored: the tile loop starts */
#define QKRA_STAMP_FIRST_STEP 4 /* the loop's first step done */
#define QKRA_STAMP_LOOP_END 5   /* the tile loop done */
#define QKRA_STAMP_END 6        /* the output rows issued */
#define QKRA_STAMP_WHERE 7

#ifdef __cplusplus
extern "C" {
#endif

#define QKRA_STAMPS_API __attribute__((visibility("default")))

/* Copies the first `bytes` of the record array (at most its size) into the
 * HOST buffer `dst` (synchronous).  Returns 0, or 1 for a bad argument, 6 for
 * a HIP error. */
QKRA_STAMPS_API int32_t qkra_phase_stamps_read(void* dst, size_t bytes);

/* Zeroes every record on `hip_stream` (a hipStream_t, NULL = the default
 * stream).  Returns 0, or 6 for a HIP error. */
QKRA_STAMPS_API int32_t qkra_phase_stamps_clear(void* hip_stream);

/* The size of the record array in bytes. */
QKRA_STAMPS_API size_t qkra_phase_stamps_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* QKRA_PHASE_STAMPS_H */
