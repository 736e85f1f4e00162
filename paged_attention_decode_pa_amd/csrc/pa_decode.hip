// pa_decode.hip -- the C ABI of the paged-attention decode library: argument
// validation, the partition heuristic, library-owned buffers and the choice of
// kernel.  What is computed is declared in include/pa_decode.h; the kernels
// are in pa_kernels.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "pa_decode.h"
#include "pa_internal.h"
#include "pa_breakdown.h"
#include "pa_timeline.h"

namespace {

using namespace pa_detail;

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kMinTilesPerPartitionLog2 = 3;  // 8 tiles, 128 tokens
constexpr int kMinTilesPerPartition = 1 << kMinTilesPerPartitionLog2;
// When the (sequence, kv head) units alone cover the device, a sequence of at
// most kLongUnsplitTiles tiles (2048 tokens) stays whole -- a uniform batch
// then needs no merge -- and a longer one splits into partitions of 64 tiles
// (1024 tokens), at most kMaxLongSplit: a long sequence in a batch of short
// ones otherwise sets the pace on its own.
constexpr int kLongUnsplitTiles = 128;
constexpr int kLongPartitionTilesLog2 = 6;  // 64 tiles
constexpr int kMaxLongSplit = 16;
// A sequence of at most this many tiles is read by one workgroup in two rounds
// of loads (4 waves x 2 tiles); splitting it saves at most one round trip,
// less than the split's store-ticket-reload chain costs, so the heuristic
// leaves it whole.
constexpr int kUnsplitMaxTiles = 16;
constexpr int kMaxPartitions = 4096;
// A table of at most this many tiles (512 tokens) that the heuristic would
// split in two runs as a single pass with V split instead (when allowed).
constexpr int kShortTableTiles = 32;

#ifndef PA_SPLIT_V
#define PA_SPLIT_V 1
#endif
// Whether the launcher may split V's head dim over two workgroups (the
// kSingleSplitV and kFusedSplitV modes) where it would not have to.  The
// library is built with 1; the ablation library libpa_decode_no_vsplit.so is
// built with 0 to measure what the split costs and saves, all else identical
// (the shapes built only with V split, v_split_only, split it in both).
bool use_split_v(int d) { return PA_SPLIT_V != 0 && split_v_built(d); }

size_t round256(size_t bytes) { return (bytes + 255) & ~(size_t)255; }

#ifndef PA_TIMELINE
#define PA_TIMELINE 0
#endif
// The timeline build's stamp buffer (pa_timeline_enable); null otherwise.
unsigned long long *g_timeline = nullptr;
unsigned g_timeline_cap = 0;

#ifndef PA_BREAKDOWN
#define PA_BREAKDOWN 0
#endif
// The breakdown build's stopping point (pa_breakdown_stop_after); 0 otherwise.
std::atomic<int> g_stop_after{0};

// Workspace layout: [B][H][P] float2 (max, sum) | [B][H][P][d] float partial
// sums, the second region starting on a 256-byte boundary.
struct Layout {
    size_t ml, acc, total;
};

Layout workspace_layout(int B, int H, int P, int d) {
    Layout l;
    l.ml = 0;
    l.acc = round256((size_t)B * H * P * sizeof(float2));
    l.total = l.acc + (size_t)B * H * P * d * sizeof(float);
    return l;
}

bool supported_head_dim(int d) { return d == 64 || d == 128 || d == 256; }
bool known_dtype(int dtype) {
    return dtype == PA_DTYPE_F32 || dtype == PA_DTYPE_BF16 || dtype == PA_DTYPE_F16;
}
int elem_bytes(int dtype) { return dtype == PA_DTYPE_F32 ? 4 : 2; }

bool aligned(const void *ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const char *x = static_cast<const char *>(a), *y = static_cast<const char *>(b);
    return x < y + nb && y < x + na;
}

struct Validated {
    int G;
    int esize;
};

int validate(void *out, const void *q, const void *k_cache, const void *v_cache,
             const int32_t *block_tables, const int32_t *context_lens, int B, int H, int Hkv,
             int d, int block_size, int max_blocks, float scale, int dtype, bool need_out,
             Validated *v) {
    if (B < 0 || H <= 0 || Hkv <= 0 || d <= 0 || block_size <= 0 || max_blocks <= 0)
        return PA_ERR_SHAPE;
    if (H % Hkv != 0) return PA_ERR_SHAPE;
    if (!known_dtype(dtype)) return PA_ERR_DTYPE;
    if (!std::isfinite(scale)) return PA_ERR_VALUE;
    if (!supported_head_dim(d) || block_size < kTile || block_size > kMaxBlockSize ||
        (block_size & (block_size - 1)) != 0)
        return PA_ERR_UNSUPPORTED;
    const int G = H / Hkv;
    if (!shape_built(dtype, d, G)) return PA_ERR_UNSUPPORTED;
    if ((long long)max_blocks * block_size > (1LL << 30)) return PA_ERR_UNSUPPORTED;
    // (sequence, head) pairs are counted in 32 bits (tickets, merge groups)
    if ((long long)B * H > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;
    v->G = G;
    v->esize = elem_bytes(dtype);
    // a tile's rows of one kv head are addressed with 32-bit buffer offsets
    if ((long long)kTile * Hkv * d * v->esize > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;
    if (B == 0) return PA_OK;
    if (!q || !k_cache || !v_cache || !block_tables || !context_lens || (need_out && !out))
        return PA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        (need_out && !aligned(out, 16)) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
        return PA_ERR_ALIGN;
    if (need_out) {
        const size_t qbytes = (size_t)B * H * d * v->esize;
        if (overlaps(out, qbytes, q, qbytes) || out == k_cache || out == v_cache)
            return PA_ERR_ALIAS;
    }
    return PA_OK;
}

// Whether a caller workspace of `bytes` bytes overlaps out (if given) or q,
// each B * H * d elements.
bool workspace_overlaps(const void *ws, size_t bytes, const void *out, const void *q, int B,
                        int H, int d, int esize) {
    const size_t qbytes = (size_t)B * H * d * esize;
    return (out && overlaps(ws, bytes, out, qbytes)) || overlaps(ws, bytes, q, qbytes);
}

std::mutex g_mutex;
std::map<int, int> g_cus;  // device -> CU count

// Library-owned buffers per (device, stream): the partials, and the arrival
// tickets of the fused split.  The tickets live in a buffer of their own,
// zeroed when it is (re)allocated; every fused call leaves the tickets it used
// at zero and nothing else writes there, so they are zero between calls.
struct LibBuffers {
    void *partials = nullptr;
    size_t partial_bytes = 0;
    int *tickets = nullptr;
    size_t num_tickets = 0;
};
std::map<std::pair<int, hipStream_t>, LibBuffers> g_buffers;

int current_device(int *dev) {
    if (hipGetDevice(dev) != hipSuccess) return PA_ERR_DEVICE;
    return PA_OK;
}

int device_cus(int dev) {
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        auto it = g_cus.find(dev);
        if (it != g_cus.end()) return it->second;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return PA_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_mutex);
    g_cus[dev] = cus;
    return cus;
}

// The caller holds g_mutex, and keeps holding it until the work using the
// buffers is enqueued: a concurrent call on the same stream that grows them
// then frees them only after that work (it synchronises the stream first).
int library_buffers(int dev, hipStream_t stream, size_t partial_bytes, size_t num_tickets,
                    void **partials, int **tickets) {
    LibBuffers &lb = g_buffers[{dev, stream}];
    if (lb.partial_bytes < partial_bytes || lb.num_tickets < num_tickets) {
        // no allocation, synchronisation or memset may land in a graph capture
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return PA_ERR_HIP;
        if (cs != hipStreamCaptureStatusNone) return PA_ERR_WORKSPACE;
        // the previous buffers may still be in use by work on this stream
        if ((lb.partials || lb.tickets) && hipStreamSynchronize(stream) != hipSuccess)
            return PA_ERR_HIP;
    }
    if (lb.partial_bytes < partial_bytes) {
        if (lb.partials && hipFree(lb.partials) != hipSuccess) return PA_ERR_HIP;
        lb.partials = nullptr;
        lb.partial_bytes = 0;
        if (hipMalloc(&lb.partials, partial_bytes) != hipSuccess) return PA_ERR_HIP;
        lb.partial_bytes = partial_bytes;
    }
    if (lb.num_tickets < num_tickets) {
        if (lb.tickets && hipFree(lb.tickets) != hipSuccess) return PA_ERR_HIP;
        lb.tickets = nullptr;
        lb.num_tickets = 0;
        if (hipMalloc(&lb.tickets, num_tickets * sizeof(int)) != hipSuccess) return PA_ERR_HIP;
        // zeroed on the stream the kernels run on, so it is ordered before them
        // even when that stream does not synchronise with the null stream
        if (hipMemsetAsync(lb.tickets, 0, num_tickets * sizeof(int), stream) != hipSuccess)
            return PA_ERR_HIP;
        lb.num_tickets = num_tickets;
    }
    *partials = lb.partials;
    *tickets = lb.tickets;
    return PA_OK;
}

// The decode kernel over all B sequences, in launches of at most kMaxGridY.
int run_main(Params p, int dtype, int d, int G, int mode, hipStream_t stream) {
    for (int b0 = 0; b0 < p.B; b0 += kMaxGridY) {
        const int nseq = p.B - b0 < kMaxGridY ? p.B - b0 : kMaxGridY;
        p.b0 = b0;
        hipError_t e;
        switch (dtype) {
            case PA_DTYPE_BF16:
                e = launch_decode<PA_DTYPE_BF16>(p, d, G, mode, nseq, stream);
                break;
            case PA_DTYPE_F16:
                e = launch_decode<PA_DTYPE_F16>(p, d, G, mode, nseq, stream);
                break;
            default:
                e = launch_decode<PA_DTYPE_F32>(p, d, G, mode, nseq, stream);
                break;
        }
        if (e != hipSuccess) return PA_ERR_HIP;
    }
    return PA_OK;
}

int run_merge(void *out, void *ws, int B, int H, int P, int d, int dtype, hipStream_t stream) {
    const Layout l = workspace_layout(B, H, P, d);
    MergeParams mp;
    mp.part_ml = reinterpret_cast<const float2 *>(static_cast<char *>(ws) + l.ml);
    mp.part_acc = reinterpret_cast<const float *>(static_cast<char *>(ws) + l.acc);
    mp.out = out;
    mp.B = B;
    mp.H = H;
    mp.P = P;
    mp.d = d;
    const long long groups = (long long)B * H;
    if (groups > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;
    hipError_t e;
    switch (dtype) {
        case PA_DTYPE_BF16: e = launch_merge<PA_DTYPE_BF16>(mp, (int)groups, stream); break;
        case PA_DTYPE_F16: e = launch_merge<PA_DTYPE_F16>(mp, (int)groups, stream); break;
        default: e = launch_merge<PA_DTYPE_F32>(mp, (int)groups, stream); break;
    }
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int log2_int(int x) {
    int l = 0;
    while ((1 << l) < x) ++l;
    return l;
}

// Tiles of 16 tokens in a table row of max_blocks blocks of block_size tokens.
int table_tiles(int max_blocks, int block_size) { return max_blocks * (block_size / kTile); }

Params make_params(const void *q, const void *k_cache, const void *v_cache,
                   const int32_t *block_tables, const int32_t *context_lens, int B, int H,
                   int Hkv, int d, int max_blocks, int block_size, float scale, int esize,
                   long long pool, int P) {
    Params p;
    p.q = static_cast<const char *>(q);
    p.k = static_cast<const char *>(k_cache);
    p.v = static_cast<const char *>(v_cache);
    p.table = block_tables;
    p.lens = context_lens;
    p.out = nullptr;
    p.part_ml = nullptr;
    p.part_acc = nullptr;
    p.counters = nullptr;
    p.tok_bytes = Hkv * d * esize;
    p.blk_bytes = (long long)block_size * p.tok_bytes;
    // ids are int32: a guard at or beyond 2^31 only has to skip negative ids
    p.pool_limit = pool > 0 && pool < 0x7FFFFFFF ? (unsigned)pool : 0x7FFFFFFFu;
    p.B = B;
    p.b0 = 0;
    p.H = H;
    p.Hkv = Hkv;
    p.max_blocks = max_blocks;
    p.P = P;
    p.tiles_log2 = log2_int(block_size / kTile);
    p.part_tiles_log2 = 0;  // every partition up to min(n, P) busy
    p.solo_tiles = 0;
    p.merge_ways = 1;
    p.cus = 0;
    p.timeline = g_timeline;
    p.timeline_cap = g_timeline_cap;
    p.stop_after = g_stop_after.load(std::memory_order_relaxed);
    p.max_tiles = table_tiles(max_blocks, block_size);
    p.qk_scale = scale * kLog2e;
    return p;
}

void attach_workspace(Params &p, void *ws, int d) {
    const Layout l = workspace_layout(p.B, p.H, p.P, d);
    char *base = static_cast<char *>(ws);
    p.part_ml = reinterpret_cast<float2 *>(base + l.ml);
    p.part_acc = reinterpret_cast<float *>(base + l.acc);
}

// P limited to [1, tiles]: with at most one partition per tile, a full table
// row leaves no partition empty.
int clamp_partitions(int tiles, int P) {
    if (P > tiles) P = tiles;
    return P < 1 ? 1 : P;
}

// What pa_decode_ex launches: the partition count, the kernel mode and the
// per-sequence split rule.
struct Plan {
    int P;
    int mode;
    int part_tiles_log2;  // (see Params)
    int solo_tiles;
};

int choose_partitions(int B, int Hkv, int max_blocks, int block_size, int num_cus);

Plan make_plan(int B, int Hkv, int d, int max_blocks, int block_size, int cus,
               int num_partitions, bool caller_workspace, bool split_only) {
    Plan plan{1, kSingle, 0, 0};  // forced counts: every partition up to min(n, P) busy
    const long long units = (long long)B * Hkv;
    const bool covered = units >= cus;
    const bool uniform = num_partitions == PA_PARTITIONS_UNIFORM;
    if (uniform) num_partitions = 0;
    if (num_partitions == 0) {
        plan.P = choose_partitions(B, Hkv, max_blocks, block_size, cus);
        // A shape built only with V split runs two workgroups per partition:
        // half the partitions keep them within the compute units (its kernels
        // run one workgroup per CU at a time).
        if (split_only && !covered && plan.P > 1) plan.P /= 2;
        // Two partitions of a short table lose to the single pass with V's
        // head dim split over the same two workgroups per unit, which needs
        // no merge (measured at 96-128 units: at 512 tokens the single pass is
        // 7-8 % faster, at 1024 tokens 4-9 % slower).
        if (plan.P == 2 && use_split_v(d) &&
            table_tiles(max_blocks, block_size) <= kShortTableTiles && 2 * units <= cus)
            plan.P = 1;
        // Told that every sequence has the same length, a batch whose units
        // already cover the device runs as a single pass: with no long tail
        // to cut, the split's partials and merges only cost (measured 6-10 %
        // on uniform batches of 32-128 x 4096-8192 tokens).
        if (uniform && covered) plan.P = 1;
        // a sequence uses the partitions its length fills: at least 8 tiles
        // each (none of 16 tiles or fewer splits), or, when the units alone
        // cover the device, 64 tiles each (none of 128 tiles or fewer splits)
        plan.part_tiles_log2 = covered ? kLongPartitionTilesLog2 : kMinTilesPerPartitionLog2;
        plan.solo_tiles = covered ? kLongUnsplitTiles : kUnsplitMaxTiles;
    } else {
        plan.P = clamp_partitions(table_tiles(max_blocks, block_size),
                                  num_partitions < kMaxPartitions ? num_partitions
                                                                  : kMaxPartitions);
    }
    if (split_only) {
        plan.mode = plan.P == 1 ? kSingleSplitV : (caller_workspace ? kPartialsSplitV : kFusedSplitV);
    } else if (plan.P == 1) {
        // A single pass whose units fill at most half of the compute units
        // runs as two workgroups per unit, each with half of V's head dim.
        plan.mode = use_split_v(d) && 2 * units <= cus ? kSingleSplitV : kSingle;
    } else if (caller_workspace) {
        plan.mode = kPartials;
    } else if (num_partitions == 0 && covered) {
        plan.mode = kFusedLate;  // most partitions of such a launch are empty
    } else if (use_split_v(d) && 4 * units * plan.P <= cus) {
        // a split whose workgroups fill at most a quarter of the compute
        // units also splits V's head dim over two workgroups per partition
        // (measured: 32 -> 64 workgroups gains ~5 %; 128 -> 256 loses 10-18 %,
        // the doubled K reads then costing more than the halved V saves)
        plan.mode = kFusedSplitV;
    } else {
        plan.mode = kFused;
    }
    return plan;
}

// Workgroups that share each fused merge.  Only when a unit's partials are at
// least kSharedMergeBytes and every workgroup of the launch can be resident at
// once (at most one per compute unit), since the waiting mergers then wait
// only for running workgroups; else the last arrival merges alone.  A waiting
// merger learns that the last partition is in about a microsecond after the
// last arrival does, so sharing pays only when reading the whole unit's
// partials through one CU takes longer than that (measured: -0.3 us with 64
// KiB per unit, +0.4 to +0.7 us with 16 KiB or less).  Then the partials are
// cut into slices of about kMergeBytesPerWay each (a power of two of them, at
// most kMergeWays): one CU reads them at a rate set by its loads in flight,
// so smaller slices finish sooner (measured against 4 fixed ways: 8 ways -0.1
// to -0.2 us at 64-94 KiB per unit, -0.8 us at 512 KiB).
constexpr long long kSharedMergeBytes = 48 << 10;
#ifndef PA_MERGE_BYTES_PER_WAY
#define PA_MERGE_BYTES_PER_WAY (8 << 10)
#endif
constexpr long long kMergeBytesPerWay = PA_MERGE_BYTES_PER_WAY;
int merge_ways(int mode, int B, int Hkv, int G, int d, int P, int cus) {
    if (mode != kFused && mode != kFusedSplitV) return 1;
    const long long bytes = (long long)P * G * d * 4;
    if (bytes < kSharedMergeBytes) return 1;
    const long long per_launch =
        (long long)(B < kMaxGridY ? B : kMaxGridY) * Hkv * P * v_slices(mode);
    if (per_launch > cus) return 1;
    int ways = 2;
    while (ways < kMergeWays && bytes > ways * kMergeBytesPerWay) ways *= 2;
    return ways;
}

int choose_partitions(int B, int Hkv, int max_blocks, int block_size, int num_cus) {
    if (B <= 0 || Hkv <= 0 || max_blocks <= 0 || block_size < kTile || num_cus <= 0) return 1;
    const long long units = (long long)B * Hkv;
    const long long tiles = (long long)max_blocks * block_size / kTile;
    if (tiles > 0x7FFFFFFF) return 1;
    if (units >= num_cus) {
        if (tiles <= kLongUnsplitTiles) return 1;
        const long long P = (tiles + (1LL << kLongPartitionTilesLog2) - 1) >> kLongPartitionTilesLog2;
        return P < kMaxLongSplit ? (int)P : kMaxLongSplit;
    }
    if (tiles <= kUnsplitMaxTiles) return 1;
    // at most one workgroup per compute unit: a few more would put two on some
    // units, each taking twice as long as the rest (measured: 96 units, P = 3
    // is 10-35 % slower than P = 2)
    long long P = num_cus / units;
    const long long cap = tiles / kMinTilesPerPartition;
    if (P > cap) P = cap;
    if (P > kMaxPartitions) P = kMaxPartitions;
    return clamp_partitions((int)tiles, (int)P);
}

// ---- the allocation-free entry point's scratch -----------------------------
// pa_decode_noalloc keeps the fused split's tickets and partials in this
// file-scope device array instead of library-owned allocations: each device
// the library runs on holds one copy for the life of the process.  In host
// code `scratch` names a host-side stand-in, never the device memory: the
// device address is taken once per device with hipGetSymbolAddress and kept
// in g_scratch_ptr, and only that address reaches kernels.  Layout: a fixed
// region of kScratchTickets tickets from offset 0 (a call uses the first
// B * Hkv), then the partials (the workspace layout of the split path) from
// kScratchPartials on.  The ticket region is never used for anything else,
// so the zeros the set-up writes and every call leaves behind hold whatever
// shapes the calls have.
constexpr size_t kScratchBytes = 64u << 20;
constexpr size_t kScratchTickets = 1u << 14;  // (sequence, kv head) units
constexpr size_t kScratchPartials = kScratchTickets * kTicketStride * sizeof(int);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::map<int, char *> g_scratch_ptr;  // device -> address of its `scratch`

__global__ void clear_words(unsigned *p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// The device address of this device's `scratch`, set up on first use: the
// address is taken with the device current, and the ticket region is zeroed
// by a fill kernel enqueued on `stream` (ordered before the call's kernels; a
// kernel, not a memset, so that a capture may hold it).  The caller holds
// g_mutex.
int scratch_for(int dev, hipStream_t stream, char **out) {
    auto it = g_scratch_ptr.find(dev);
    if (it != g_scratch_ptr.end()) {
        *out = it->second;
        return PA_OK;
    }
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return PA_ERR_HIP;
    const int n = (int)(kScratchTickets * kTicketStride);
    hipLaunchKernelGGL(clear_words, dim3((n + 255) / 256), dim3(256), 0, stream,
                       static_cast<unsigned *>(ptr), n);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<char *>(ptr);
    *out = static_cast<char *>(ptr);
    return PA_OK;
}

}  // namespace

extern "C" {

int pa_choose_partitions(int B, int Hkv, int max_blocks, int block_size, int num_cus) {
    return choose_partitions(B, Hkv, max_blocks, block_size, num_cus);
}

size_t pa_workspace_bytes(int B, int H, int d, int num_partitions) {
    if (B <= 0 || H <= 0 || d <= 0 || num_partitions <= 1) return 0;
    return workspace_layout(B, H, num_partitions, d).total;
}

int pa_device_num_cus(int device) { return device_cus(device); }

const char *pa_strerror(int code) {
    switch (code) {
        case PA_OK: return "ok";
        case PA_ERR_NULL: return "a required pointer is NULL";
        case PA_ERR_SHAPE: return "negative or inconsistent sizes";
        case PA_ERR_UNSUPPORTED:
            return "shape not supported (needs d in {64,128,256}, block_size a power of 2 in "
                   "16..256, H/Hkv in {1,2,4,8,16}, and the size limits of pa_decode.h)";
        case PA_ERR_DTYPE: return "unknown dtype";
        case PA_ERR_ALIGN: return "pointer alignment (16 bytes for tensors, 4 for int32 arrays)";
        case PA_ERR_WORKSPACE:
            return "workspace missing or too small, or the library would allocate one while the "
                   "stream is being captured, or pa_decode_noalloc needs more than its 64 MiB "
                   "scratch";
        case PA_ERR_HIP: return "HIP runtime call or kernel launch failed";
        case PA_ERR_DEVICE: return "no usable HIP device";
        case PA_ERR_ALIAS: return "out or a caller workspace overlaps q or another buffer";
        case PA_ERR_VALUE: return "scale not finite or a negative count";
        default: return "unknown error code";
    }
}

int pa_decode_ex(void *out, const void *q, const void *k_cache, const void *v_cache,
                 const int32_t *block_tables, const int32_t *context_lens, int B, int H, int Hkv,
                 int d, int block_size, int max_blocks, float scale, int dtype, void *stream,
                 int num_partitions, long long num_pool_blocks, void *workspace,
                 size_t workspace_bytes) {
    Validated v;
    int rc = validate(out, q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv, d,
                      block_size, max_blocks, scale, dtype, true, &v);
    if (rc != PA_OK) return rc;
    if (num_partitions < PA_PARTITIONS_UNIFORM || num_pool_blocks < 0) return PA_ERR_VALUE;
    if (workspace && !aligned(workspace, 16)) return PA_ERR_ALIGN;
    if (B == 0) return PA_OK;
    // the merge reads the partials while it writes out, and the split reads q
    // while it writes the partials
    if (workspace && workspace_bytes > 0 &&
        workspace_overlaps(workspace, workspace_bytes, out, q, B, H, d, v.esize))
        return PA_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = 0;
    if ((rc = current_device(&dev)) != PA_OK) return rc;
    const int cus = device_cus(dev);
    if (cus < 0) return cus;
    const Plan plan = make_plan(B, Hkv, d, max_blocks, block_size, cus, num_partitions,
                                workspace != nullptr, v_split_only(dtype, d, v.G));
    const int P = plan.P;
    Params p = make_params(q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv, d,
                           max_blocks, block_size, scale, v.esize, num_pool_blocks, P);
    p.part_tiles_log2 = plan.part_tiles_log2;
    p.solo_tiles = plan.solo_tiles;
    p.out = out;
    if (P == 1) return run_main(p, dtype, d, v.G, plan.mode, s);
    const size_t need = workspace_layout(B, H, P, d).total;
    if (workspace) {
        // caller workspace: split kernel, then the merge kernel (no tickets)
        if (workspace_bytes < need) return PA_ERR_WORKSPACE;
        attach_workspace(p, workspace, d);
        if ((rc = run_main(p, dtype, d, v.G, plan.mode, s)) != PA_OK) return rc;
        return run_merge(out, workspace, B, H, P, d, dtype, s);
    }
    void *ws = nullptr;
    int *tickets = nullptr;
    std::lock_guard<std::mutex> lock(g_mutex);
    if ((rc = library_buffers(dev, s, need, (size_t)B * Hkv * kTicketStride, &ws, &tickets)) !=
        PA_OK)
        return rc;
    attach_workspace(p, ws, d);
    p.counters = tickets;
    p.merge_ways = merge_ways(plan.mode, B, Hkv, v.G, d, P, cus);
    p.cus = cus;
    return run_main(p, dtype, d, v.G, plan.mode, s);
}

int pa_plan(int B, int H, int Hkv, int d, int dtype, int max_blocks, int block_size,
            int num_cus, int num_partitions, int *partitions, int *v_slices_out) {
    if (!partitions || !v_slices_out) return PA_ERR_NULL;
    if (B < 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || max_blocks <= 0 || num_cus <= 0)
        return PA_ERR_SHAPE;
    if (!known_dtype(dtype)) return PA_ERR_DTYPE;
    if (num_partitions < PA_PARTITIONS_UNIFORM) return PA_ERR_VALUE;
    if (!supported_head_dim(d) || block_size < kTile || block_size > kMaxBlockSize ||
        (block_size & (block_size - 1)) != 0 || !shape_built(dtype, d, H / Hkv))
        return PA_ERR_UNSUPPORTED;
    const Plan plan = make_plan(B, Hkv, d, max_blocks, block_size, num_cus, num_partitions, false,
                                v_split_only(dtype, d, H / Hkv));
    *partitions = plan.P;
    *v_slices_out = v_slices(plan.mode);
    return PA_OK;
}

int pa_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
              const int32_t *block_tables, const int32_t *context_lens, int B, int H, int Hkv,
              int d, int block_size, int max_blocks, float scale, int dtype, void *stream) {
    return pa_decode_ex(out, q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv, d,
                        block_size, max_blocks, scale, dtype, stream, 0, 0, nullptr, 0);
}

int pa_decode_noalloc(void *out, const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens, int B, int H,
                      int Hkv, int d, int block_size, int max_blocks, float scale, int dtype,
                      void *stream) {
    Validated v;
    int rc = validate(out, q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv, d,
                      block_size, max_blocks, scale, dtype, true, &v);
    if (rc != PA_OK) return rc;
    if (B == 0) return PA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = 0;
    if ((rc = current_device(&dev)) != PA_OK) return rc;
    const int cus = device_cus(dev);
    if (cus < 0) return cus;
    const Plan plan = make_plan(B, Hkv, d, max_blocks, block_size, cus, 0, false,
                                v_split_only(dtype, d, v.G));
    const int P = plan.P;
    Params p = make_params(q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv, d,
                           max_blocks, block_size, scale, v.esize, 0, P);
    p.part_tiles_log2 = plan.part_tiles_log2;
    p.solo_tiles = plan.solo_tiles;
    p.out = out;
    if (P == 1) return run_main(p, dtype, d, v.G, plan.mode, s);
    const size_t units = (size_t)B * Hkv;
    if (units > kScratchTickets ||
        workspace_layout(B, H, P, d).total > kScratchBytes - kScratchPartials)
        return PA_ERR_WORKSPACE;
    std::lock_guard<std::mutex> lock(g_mutex);
    char *base = nullptr;
    if ((rc = scratch_for(dev, s, &base)) != PA_OK) return rc;
    p.counters = reinterpret_cast<int *>(base);
    attach_workspace(p, base + kScratchPartials, d);
    p.merge_ways = merge_ways(plan.mode, B, Hkv, v.G, d, P, cus);
    p.cus = cus;
    return run_main(p, dtype, d, v.G, plan.mode, s);
}

int pa_decode_partials(const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *block_tables, const int32_t *context_lens, int B, int H,
                       int Hkv, int d, int block_size, int max_blocks, float scale, int dtype,
                       int num_partitions, long long num_pool_blocks, void *workspace,
                       size_t workspace_bytes, void *stream) {
    Validated v;
    int rc = validate(nullptr, q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv, d,
                      block_size, max_blocks, scale, dtype, false, &v);
    if (rc != PA_OK) return rc;
    if (num_partitions < 1 || num_pool_blocks < 0) return PA_ERR_VALUE;
    if (num_partitions > kMaxPartitions) return PA_ERR_UNSUPPORTED;
    if (B == 0) return PA_OK;
    if (!workspace) return PA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return PA_ERR_ALIGN;
    const int P = num_partitions;
    if (workspace_bytes < workspace_layout(B, H, P, d).total) return PA_ERR_WORKSPACE;
    if (workspace_overlaps(workspace, workspace_bytes, nullptr, q, B, H, d, v.esize))
        return PA_ERR_ALIAS;
    Params p = make_params(q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv, d,
                           max_blocks, block_size, scale, v.esize, num_pool_blocks, P);
    attach_workspace(p, workspace, d);
    return run_main(p, dtype, d, v.G, v_split_only(dtype, d, v.G) ? kPartialsSplitV : kPartials,
                    static_cast<hipStream_t>(stream));
}

int pa_merge_partials(void *out, const void *workspace, size_t workspace_bytes, int B, int H,
                      int d, int num_partitions, int dtype, void *stream) {
    if (B < 0 || H <= 0 || d <= 0) return PA_ERR_SHAPE;
    if (!known_dtype(dtype)) return PA_ERR_DTYPE;
    if (!supported_head_dim(d)) return PA_ERR_UNSUPPORTED;
    if (num_partitions < 1) return PA_ERR_VALUE;
    if (num_partitions > kMaxPartitions) return PA_ERR_UNSUPPORTED;
    if (B == 0) return PA_OK;
    if (!out) return PA_ERR_NULL;
    if (!workspace) return PA_ERR_WORKSPACE;
    if (!aligned(out, 16) || !aligned(workspace, 16)) return PA_ERR_ALIGN;
    const int P = num_partitions;
    const size_t need = workspace_layout(B, H, P, d).total;
    if (workspace_bytes < need) return PA_ERR_WORKSPACE;
    const size_t esize = elem_bytes(dtype);
    if (overlaps(out, (size_t)B * H * d * esize, workspace, need)) return PA_ERR_ALIAS;
    return run_merge(out, const_cast<void *>(workspace), B, H, P, d, dtype,
                     static_cast<hipStream_t>(stream));
}

#if PA_BREAKDOWN
int pa_breakdown_stop_after(int stage) {
    if (stage < 0 || stage > 3) return PA_ERR_VALUE;
    g_stop_after.store(stage, std::memory_order_relaxed);
    return PA_OK;
}
#endif

#if PA_TIMELINE
int pa_timeline_enable(int workgroups) {
    if (workgroups <= 0) return PA_ERR_VALUE;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_timeline && (hipDeviceSynchronize() != hipSuccess || hipFree(g_timeline) != hipSuccess))
        return PA_ERR_HIP;
    g_timeline = nullptr;
    g_timeline_cap = 0;
    const size_t bytes = (size_t)workgroups * kTimelineSlots * sizeof(unsigned long long);
    void *ptr = nullptr;
    if (hipMalloc(&ptr, bytes) != hipSuccess) return PA_ERR_HIP;
    if (hipMemset(ptr, 0, bytes) != hipSuccess) return PA_ERR_HIP;
    g_timeline = static_cast<unsigned long long *>(ptr);
    g_timeline_cap = (unsigned)workgroups;
    return PA_OK;
}

int pa_timeline_copy(unsigned long long *host, int workgroups) {
    if (!host) return PA_ERR_NULL;
    if (workgroups <= 0 || (unsigned)workgroups > g_timeline_cap) return PA_ERR_VALUE;
    const size_t bytes = (size_t)workgroups * kTimelineSlots * sizeof(unsigned long long);
    return hipMemcpy(host, g_timeline, bytes, hipMemcpyDeviceToHost) == hipSuccess ? PA_OK
                                                                                   : PA_ERR_HIP;
}
#endif

void pa_release(void) {
    std::lock_guard<std::mutex> lock(g_mutex);
    int prev = -1;
    const bool have_prev = hipGetDevice(&prev) == hipSuccess;
    for (auto &kv : g_buffers) {
        if (hipSetDevice(kv.first.first) != hipSuccess) continue;
        (void)hipDeviceSynchronize();
        if (kv.second.partials) (void)hipFree(kv.second.partials);
        if (kv.second.tickets) (void)hipFree(kv.second.tickets);
    }
    g_buffers.clear();
    if (have_prev) (void)hipSetDevice(prev);
}

}  // extern "C"
