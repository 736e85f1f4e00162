/*
 * pa_read_probe.h -- C ABI of libpa_read_probe.so, measuring aids beside the
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

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int pa_probe_read(const void *src, long long bytes, int workgroups, int depth, unsigned *sink,
                  void *stream);

/*
 * pa_probe_gather reads, once, exactly the K and V rows one decode step
 * reads, the way the decode kernel gathers them, and does nothing else: no
 * scores, no softmax, no merge.  Its time is what the kernel's own access
 * pattern costs, the bound the kernel's arithmetic and merge add to.  (The
 * lookup of each token's block through the block table is the docs page's
 * block table mechanics; the deal of the context over partitions is the
 * design note's split into chunks.)
 *
 * Arguments as in pa_decode (include/pa_decode.h): k_cache and v_cache are
 * [pool][block_size][Hkv][row_bytes / element size] (device memory, 16-byte
 * aligned), block_tables [B][max_blocks] and context_lens [B] int32 (device
 * memory); row_bytes = d * element size, 128, 256 or 512.  The grid is
 * (Hkv, B, partitions * v_slices) workgroups of 4 waves; with v_slices = 2,
 * as in the decode kernel's V-split launches, two workgroups serve each
 * partition (z = 2 partition + slice), both reading all of K and each one
 * half of every V row.  A sequence's 16-token tiles are
 * dealt in runs of two to the partitions * 4 (partition, wave) lanes in turn
 * (every partition takes part, whatever the length), each wave keeping two
 * tiles in flight, one scalar table read per tile, and one buffer descriptor
 * per tile over its live rows of the kv head, so rows past the context
 * (lengths clamped to [0, max_blocks * block_size]) and -1 entries read as
 * zeros without a memory access; every other entry used must be a valid pool
 * block.  Loads are 16 bytes per lane, non-temporal, each instruction
 * covering whole rows.  Workgroup (x, y, z) writes to sink[(z * B + y) * Hkv
 * + x] (device memory of B * Hkv * partitions * v_slices words) the xor of
 * every 32-bit word it read, so the xor of the whole sink is that of every
 * live K row of every (sequence, kv head) read v_slices times and every live
 * V row read once.  Enqueue only, on `stream`.  Returns 0, -1 (NULL pointer),
 * -2 (negative or zero size), -3 (row_bytes, block_size, partitions or
 * v_slices outside the supported set, B or Hkv above 65535, or the size
 * limits of pa_decode) or -7 (launch failed).
 */
int pa_probe_gather(const void *k_cache, const void *v_cache, const int32_t *block_tables,
                    const int32_t *context_lens, int B, int Hkv, int row_bytes, int block_size,
                    int max_blocks, int partitions, int v_slices, unsigned *sink,
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
