/*
 * pa_read_probe.h -- C ABI of libpa_read_probe.so, a measuring aid beside the
 * decode library (not part of it).
 *
 * The flash-decoding-bench design note, rationale section, treats a decode
 * step as bound by reading the KV cache once; the time of a plain read of the
 * same bytes, with the decode kernel's load shape and nothing else, is the
 * ceiling a decode kernel is measured against.
 *
 * pa_probe_read reads `bytes` bytes at device address `src` (16-byte
 * aligned) once: `workgroups` workgroups of 4 waves, workgroup g taking the
 * g-th contiguous slice of ceil(bytes / workgroups) bytes rounded up to 1 KB,
 * each wave with `depth` 16-byte non-temporal loads per lane in flight
 * (depth 16 = 16 KB per wave, the decode kernel's two tiles of K and V rows;
 * 8 and 32 are also built).  It writes one 32-bit word per workgroup to
 * `sink` (device memory of `workgroups` words), which keeps the loads from
 * being optimised away.  Enqueue only, on `stream` (a hipStream_t, NULL = the
 * null stream).  Returns 0, -1 (NULL pointer), -2 (negative size or no
 * workgroup), -3 (depth not built, or a slice of 2^31 bytes or more) or -7
 * (launch failed).
 */
#ifndef PA_READ_PROBE_H
#define PA_READ_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

int pa_probe_read(const void *src, long long bytes, int workgroups, int depth, unsigned *sink,
                  void *stream);

/*
 * pa_probe_stamp enqueues on `stream` a one-thread kernel that writes the
 * device's constant-rate clock (s_memrealtime, a 100 MHz counter shared by
 * the compute units) to dst[0] (device memory).  Captured at the two ends of a
 * sequence of steps in one HIP graph, the difference of two stamps is the
 * time those steps took on the device, without the graph's launch overhead
 * that events recorded around the graph would include.  Returns 0, -1 (NULL)
 * or -7 (launch failed).
 */
int pa_probe_stamp(unsigned long long *dst, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_READ_PROBE_H */
