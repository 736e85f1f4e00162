/*
 * pa_timeline.h -- the timeline library libpa_decode_timeline.so: the decode
 * library built with per-workgroup time stamps (PA_TIMELINE=1), a tracing aid
 * beside it.  It exports everything include/pa_decode.h declares, computing
 * the same results, plus the two calls below; libpa_decode.so has neither.
 *
 * The stamps show where a decode step's time goes between the reads of the
 * KV cache (which the flash-decoding-bench design note, rationale section,
 * treats as the step's cost) and the split's merge (its implementations
 * section): when each workgroup starts, ends its streaming, publishes its
 * partial sums, learns its place in the merge, and ends its merge.
 *
 * pa_timeline_enable(n) allocates (with hipMalloc, synchronising the device
 * when it replaces an earlier buffer) room for the first n workgroups of each
 * decode launch, zeroed; every later launch overwrites the slots of its
 * workgroups 0 .. n - 1 (numbered x + gridDim.x * (y + gridDim.y * z) on the
 * grid (Hkv, sequences, partitions[ x 2 V slices])).  pa_timeline_copy(host,
 * n) copies the slots of the last launch to host memory (n * 16 uint64),
 * synchronously.  Slots of workgroup w (host[16 w + i]), times from
 * s_memrealtime (100 MHz):
 *   0       entry
 *   1 .. 4  end of the streaming loop of waves 0 .. 3
 *   13      wave 0's four row groups merged (after its loop)
 *   14      every wave's sums in LDS (after the barrier)
 *   6       thread 0's share of the output or of the partial record issued
 *   15      the record's stores acknowledged (after the wait and the barrier)
 *   7       ticket returned (and, for a waiting merger, the wait ended)
 *   8       bits 0..7: merge role + 1 (0 = does not merge), bits 8..39: the
 *           ticket's arrival count, bits 40..47: workgroups sharing the merge
 *   9       end of its merge
 *   10      XCC (XCD) id, 11 the raw HW_ID register
 *   12      1 = wrote its output directly, 2 = published partial sums,
 *           3 = had no tile
 * Unused slots are 0.  Returns PA_OK, PA_ERR_VALUE (n out of range),
 * PA_ERR_NULL or PA_ERR_HIP.
 */
#ifndef PA_TIMELINE_H
#define PA_TIMELINE_H

#ifdef __cplusplus
extern "C" {
#endif

int pa_timeline_enable(int workgroups);
int pa_timeline_copy(unsigned long long *host, int workgroups);

#ifdef __cplusplus
}
#endif

#endif /* PA_TIMELINE_H */
