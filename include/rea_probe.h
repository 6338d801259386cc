/*
 * rea_probe.h - a measurement aid exported by librea.so; not part of the
 * method.  It streams a device buffer through the GPU with the load the
 * decode scoring kernel uses (non-temporal 16-byte loads, each wave
 * instruction covering 1 KB of contiguous memory) and nothing else, so the
 * rate it reaches is the HBM read rate the scoring pass can be held against.
 */
#ifndef REA_PROBE_H
#define REA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` bytes of device memory at `buf` once (both 16-byte aligned;
 * bytes a multiple of 1024).  The buffer is cut into wg_per_cu * (CU count)
 * contiguous slices, one per 256-thread workgroup; each wave keeps
 * `loads_in_flight` (4, 8 or 16) 1 KB load instructions in flight.  Every
 * workgroup writes the XOR of what it read to sink[workgroup] (device array of
 * wg_per_cu * CU count words), so no load can be dropped.  Enqueued on
 * `stream` (a hipStream_t, NULL = the null stream).
 * Returns 0, or 1 for invalid arguments, or 2 if the launch failed.
 */
int rea_probe_stream_read(const void *buf, size_t bytes, int wg_per_cu, int loads_in_flight,
                          uint32_t *sink, void *stream);

/* Number of compute units of the current device (0 if none). */
int rea_probe_cu_count(void);

#ifdef __cplusplus
}
#endif

#endif /* REA_PROBE_H */
