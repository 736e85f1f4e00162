// pa_internal.h -- what the host launcher (pa_decode.hip) and the kernel
// translation units (pa_kernels_*.hip) share: the kernel parameter blocks,
// the launch constants, the table of built shapes and the launcher entry
// points, one instantiation per element type.
#ifndef PA_INTERNAL_H
#define PA_INTERNAL_H

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_decode.h"

namespace pa_detail {

constexpr int kWave = 64;
// The kernels walk a sequence in tiles of 16 tokens, the row count of one MFMA
// tile.  A physical block of block_size tokens (a power of two from 16 to 256)
// holds block_size / 16 tiles; each tile lies inside one block.
constexpr int kTile = 16;
constexpr int kMaxBlockSize = 256;

#ifndef PA_WAVES_PER_GROUP
#define PA_WAVES_PER_GROUP 4
#endif
constexpr int kWavesPerGroup = PA_WAVES_PER_GROUP;  // waves per workgroup

// What a workgroup does with its merged (M, L, O).  kFusedLate is kFused
// with the query loaded only once a partition knows it has tiles: used when
// most partitions of a launch are empty (units covering the device, long
// sequences only splitting), so that those leave without loading it.
// kSingleSplitV is the single pass with the head dim of V cut in two: two
// workgroups per (kv head, sequence) (grid z = 2), each reading all of K for
// the scores and one half of every V row, and writing that half of the
// output.  It spreads a single pass that would leave at least half of the
// compute units idle over twice as many; the second K read of a pair mostly
// hits the XCD's L2, since both workgroups run on one XCD at the same time.
// kFusedSplitV does the same for the fused split (grid z = 2 P, z = 2 part +
// slice): each slice stores its half of a partition's sums (slice 0 also the
// (max, sum) pair), a unit's ticket counts the arrivals of both slices, and
// the last of them merges the whole head dim.  kPartialsSplitV is kPartials
// split the same way, for the shapes built only with V split
// (v_split_only); its partials have the layout of kPartials.
enum Mode {
    kSingle = 0,
    kPartials = 1,
    kFused = 2,
    kFusedLate = 3,
    kSingleSplitV = 4,
    kFusedSplitV = 5,
    kPartialsSplitV = 6
};
constexpr int v_slices(int mode) {
    return mode == kSingleSplitV || mode == kFusedSplitV || mode == kPartialsSplitV ? 2 : 1;
}

// The V-split modes are built for head dims of at least 128 (a half row then still
// gives each lane whole 8- or 16-byte V loads).
constexpr bool split_v_built(int d) { return d >= 128; }

struct Params {
    const char *q;
    const char *k;
    const char *v;
    const int32_t *table;
    const int32_t *lens;
    void *out;          // [B][H][d] dtype (single pass, fused merge)
    float2 *part_ml;    // [B][H][P] (max, sum)
    float *part_acc;    // [B][H][P][d]
    int *counters;      // [B][Hkv][kTicketStride] arrival tickets (fused mode, the
                        // first int of each), zero between calls
    long long blk_bytes;  // bytes per physical block: block_size * Hkv * d * esize
    unsigned pool_limit;  // table entries >= pool_limit (as unsigned: -1 too) are skipped
    int tok_bytes;        // bytes between tokens of a block: Hkv * d * esize
    int B, H, Hkv, max_blocks, P;
    int b0;               // first sequence of this launch (grid y covers b0 ..)
    int tiles_log2;       // log2(block_size / 16): tiles per physical block
    int max_tiles;        // max_blocks * block_size / 16
    int part_tiles_log2;  // a sequence of n tiles uses min(P, ceil(n / 2^this)) partitions,
    int solo_tiles;       // or one when n <= solo_tiles
    int merge_ways;       // fused merge shared by the last 1, 2, 4, 8 or 16 arrivals (1
                          // unless every workgroup of the launch can be resident at once)
    int cus;              // compute units of the device (the launcher's bound on waiters)
    float qk_scale;       // scale * log2(e)
    // Timeline build only (PA_TIMELINE=1): kTimelineSlots stamps per
    // workgroup for the first timeline_cap workgroups of a launch; else null.
    unsigned long long *timeline;
    unsigned timeline_cap;
    // Breakdown build only (PA_BREAKDOWN=1): where a fused split stops, for
    // timing -- 0 the whole step, 1 after the stream (no epilogue), 2 after
    // the waves' sums are combined (nothing stored), 3 after the partial sums
    // are stored (no ticket, no merge); 0 in the library.
    int stop_after;
};

// Stamps per workgroup in the timeline build (pa_timeline.h gives the layout).
constexpr int kTimelineSlots = 16;

struct MergeParams {
    const float2 *part_ml;
    const float *part_acc;
    void *out;
    int B, H, P, d;
};

// The (dtype, head dim, group size) combinations with a kernel: head dims
// 64, 128 and 256, groups of 1 to 16 query heads per kv head.
constexpr bool shape_built(int dtype, int d, int G) {
    (void)dtype;
    if (d != 64 && d != 128 && d != 256) return false;
    return G == 1 || G == 2 || G == 4 || G == 8 || G == 16;
}

// The shapes built only in the V-split modes.  One workgroup keeps the fp32
// accumulators of all G heads of its group in registers (G * DV / 16 per lane,
// DV the head dim of V it serves) next to the tiles in flight: with d = 256
// and G = 16 (or G >= 8 for fp32) the whole head dim would spill to scratch
// memory, half of it fits.  For these the launcher always splits V's head dim
// over two workgroups.
constexpr bool v_split_only(int dtype, int d, int G) {
    return d == 256 && (dtype == PA_DTYPE_F32 ? G >= 8 : G >= 16);
}

// Whether the kernel of (dtype, d, G) is built in `mode`.  kPartialsSplitV
// only for the V-split-only shapes (the others use kPartials).
constexpr bool mode_built(int dtype, int d, int G, int mode) {
    if (!shape_built(dtype, d, G)) return false;
    if (mode == kPartialsSplitV) return v_split_only(dtype, d, G);
    if (v_slices(mode) > 1) return split_v_built(d);
    return !v_split_only(dtype, d, G);
}

// Ints between the arrival tickets of two (sequence, kv head) units, so that
// each ticket has a cache line of its own: the workgroups of a launch take
// their tickets at about the same time, and atomics on one line queue behind
// each other (adjacent tickets measured ~0.3 us slower on a launch of 256
// workgroups).
#ifndef PA_TICKET_STRIDE
#define PA_TICKET_STRIDE 32
#endif
constexpr int kTicketStride = PA_TICKET_STRIDE;

// At most this many workgroups share a fused merge (p.merge_ways; the kernel
// builds the merge for 1, 2, 4, 8 and 16 slices of the head dim).
#ifndef PA_MERGE_WAYS
#define PA_MERGE_WAYS 16
#endif
constexpr int kMergeWays = PA_MERGE_WAYS;
// Rounds a merger waits for the generation of its ticket to move on before it
// writes NaN instead (a launch whose workgroups cannot all be resident; never
// reached otherwise).
constexpr int kMaxPollRounds = 1 << 22;

// Sequences per decode launch: the grid's y extent.
constexpr int kMaxGridY = 65535;

// Launch the decode kernel for element type DT on a (Hkv, nseq, P) grid of
// kWavesPerGroup-wave workgroups covering sequences p.b0 .. p.b0 + nseq - 1
// (mode_built(DT, d, G, mode) must hold), or the merge kernel on one wave per
// (b, h).  Return the launch's hipGetLastError().
template <int DT>
hipError_t launch_decode(const Params &p, int d, int G, int mode, int nseq,
                         hipStream_t stream);
template <int DT>
hipError_t launch_merge(const MergeParams &mp, int groups, hipStream_t stream);

extern template hipError_t launch_decode<PA_DTYPE_F32>(const Params &, int, int, int, int,
                                                       hipStream_t);
extern template hipError_t launch_decode<PA_DTYPE_BF16>(const Params &, int, int, int, int,
                                                        hipStream_t);
extern template hipError_t launch_decode<PA_DTYPE_F16>(const Params &, int, int, int, int,
                                                       hipStream_t);
extern template hipError_t launch_merge<PA_DTYPE_F32>(const MergeParams &, int, hipStream_t);
extern template hipError_t launch_merge<PA_DTYPE_BF16>(const MergeParams &, int, hipStream_t);
extern template hipError_t launch_merge<PA_DTYPE_F16>(const MergeParams &, int, hipStream_t);

}  // namespace pa_detail

#endif  // PA_INTERNAL_H
