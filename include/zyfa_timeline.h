/*
 * zyfa_timeline.h -- the timeline build of the library (libzyfa_timeline.so), a profiling
 * tool: the same entry points as libzyfa.so (include/zyfa.h), with the attention kernels
 * built to record, for every workgroup of the eight-wave prefill kernels (contiguous and
 * packed-batch layouts; not the paged or decode ones), when it ran and where. The records
 * show how a launch's time splits into each workgroup's prologue (loading Q and the first
 * key/value tiles), its loop over key tiles, its epilogue, the dispatcher's gaps between
 * workgroups on a compute unit, and the idle tail of each XCD. libzyfa.so is built without
 * them and is unaffected.
 *
 * Record of workgroup w (its blockIdx.x, w < ZYFA_TIMELINE_WORKGROUPS), written by its first
 * thread at the kernel's last launch that reached it, ZYFA_TIMELINE_FIELDS 64-bit fields:
 *   0  wall clock at entry            (s_memrealtime: a 100 MHz constant clock)
 *   1  wall clock before the first key-tile iteration
 *   2  wall clock after the last iteration, before the last tile's P·V
 *   3  wall clock after the output stores are issued
 *   4  the wave's HW_ID register (CU, SIMD, shader array and engine ids)
 *   5  the wave's XCC_ID register (bits 0-3: the XCD)
 *   6  key tiles the workgroup iterates over
 *   7  unused (0)
 * A workgroup with no visible key (fields 1-3 and 6 stay 0) or that a packed batch leaves
 * unwritten records its entry and ids only.
 */
#ifndef ZYFA_TIMELINE_H
#define ZYFA_TIMELINE_H

#ifdef __cplusplus
extern "C" {
#endif

#define ZYFA_TIMELINE_WORKGROUPS 65536
#define ZYFA_TIMELINE_FIELDS 8

/* Zero every record, enqueued on `stream` (a hipStream_t, NULL = the null stream) of the
 * current device. Returns a hipError_t code (0 on success). */
int zyfa_timeline_clear(void* stream);

/* Copy the records of workgroups 0 .. n_workgroups - 1 of the current device to host
 * memory `host` (n_workgroups * ZYFA_TIMELINE_FIELDS values; synchronous). Returns a
 * hipError_t code: hipErrorInvalidValue (1) for a null host pointer or n_workgroups
 * outside [0, ZYFA_TIMELINE_WORKGROUPS]. */
int zyfa_timeline_read(unsigned long long* host, long long n_workgroups);

#ifdef __cplusplus
}
#endif

#endif /* ZYFA_TIMELINE_H */
