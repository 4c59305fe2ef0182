/*
 * mpgemm_timeline.h -- per-workgroup timeline of the pipelined GEMM kernel,
 * exported only by the timeline build of the library
 * (libmpgemm_timeline.so: the product source compiled with
 * -DMPGEMM_TIMELINE; every mpgemm.h entry point is there too and computes
 * the same results).  The product library exports none of this.
 *
 * It answers where a launch's time goes -- workgroup start skew, the wait
 * for the first K tile, the interval between K tiles, the epilogue -- which
 * whole-kernel timers and counters cannot.  The pages read per-kernel
 * profiler figures ("Capstone 4: a tensor-core GEMM", section "Results");
 * this is the per-workgroup view beneath them.
 *
 * Every launch of the pipelined kernel overwrites the records of its first
 * 4096 workgroups (workgroup b at entries 48*b .. 48*b + 47 of the device
 * array; launches of the other kernels record nothing).  The stamps of one
 * workgroup are taken by its thread 0:
 *   [0]       constant 100 MHz clock (s_memrealtime) at the start
 *   [1]       shader clock (s_memtime) at the start
 *   [2 + t]   shader clock right after K tile t was published to the
 *             workgroup (its copies landed, the barrier passed), t < 41
 *   [43]      number of K tiles of the launch
 *   [44]      shader clock when the K loop (and the K tail step) ended
 *   [45]      shader clock after the epilogue's stores were issued
 *   [46]      constant 100 MHz clock at the end
 *   [47]      (XCC_ID << 32) | HW_ID of the wave (XCD, shader engine, CU)
 * Records of a later launch with fewer workgroups leave the others as they
 * were: clear before a launch whose records are read.  Calls are synchronous
 * (they wait for the device) and are not for use under graph capture.
 */
#ifndef MPGEMM_TIMELINE_H
#define MPGEMM_TIMELINE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of uint64 entries of the record array (4096 * 48). */
int64_t mpgemm_timeline_entries(void);

/* Copies the first `entries` records (at most mpgemm_timeline_entries())
 * of the current device into host memory at `out`.  Waits for the device.
 * MPGEMM_ENULL for NULL, MPGEMM_EDIM for entries < 0 or too many,
 * MPGEMM_ELAUNCH if the copy fails. */
int mpgemm_timeline_read(uint64_t *out, int64_t entries);

/* Zeroes every record on the current device.  Waits for the device.
 * MPGEMM_ELAUNCH if the fill fails. */
int mpgemm_timeline_clear(void);

#ifdef __cplusplus
}
#endif

#endif /* MPGEMM_TIMELINE_H */
