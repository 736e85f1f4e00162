/*
 * pa_decode.h -- C ABI of the paged-attention decode library (HIP, gfx950).
 *
 * The operation (one decode step).  For each sequence b < B and query head
 * h < H, the single query vector q[b][h] attends over the context_lens[b]
 * cached key/value rows of its sequence:
 *
 *   kvh      = h / (H / Hkv)                          grouped-query mapping
 *   token t  -> blk = block_tables[b][t / block_size], slot = t % block_size
 *   K_t      = k_cache[blk][slot][kvh][:],  V_t = v_cache[blk][slot][kvh][:]
 *   out[b][h] = sum_t softmax_t(scale * q[b][h] . K_t) * V_t
 *
 * Sources: "Decoding Benchmark" docs page (MinivLLM), sections "What paged
 * attention decode does" (shapes of q, the paged pool and the lookup pattern)
 * and "Block table lookup mechanics" (table shape; -1 = slot never allocated);
 * benchmark_decoding.py, the Triton (new) kernel (grouped-query mapping
 * h // (num_heads // num_kv_heads), masking of tokens past the context and of
 * -1 entries, fp32 accumulation, output in the query's dtype) and
 * reference_output (the definition as gather + softmax); the
 * flash-decoding-bench design note, implementations section (Flash-Decoding:
 * split the context into chunks processed in parallel, each keeping local
 * max / sum / weighted values, merged by a reduction afterwards).
 *
 * Layouts (all row-major, contiguous, device memory):
 *   q, out          [B][H][d]                       dtype
 *   k_cache,v_cache [num_pool_blocks][block_size][Hkv][d]   dtype
 *   block_tables    [B][max_blocks]                 int32
 *   context_lens    [B]                             int32
 * dtype (PA_DTYPE_*) applies to q, k_cache, v_cache and out alike.  Scores,
 * softmax statistics and accumulation are fp32; bf16 and fp16 outputs are
 * rounded to nearest even.  fp16 is the element type of the benchmark
 * script's inputs (benchmark_decoding.py, setup_test_data).
 *
 * Conventions:
 *   - Supported shapes: d in {64, 128, 256} (the benchmark script's head_dim
 *     argument; 128 in every configuration of the docs page); block_size a
 *     power of two from 16 to 256; H % Hkv == 0 with G = H / Hkv in
 *     {1, 2, 4, 8, 16}; B * H < 2^31; max_blocks * block_size <= 2^30;
 *     16 token rows of one kv head (16 * Hkv * d * element size bytes)
 *     below 2^31.  Others return PA_ERR_UNSUPPORTED.  With d = 256 and
 *     G = 16 (bf16, fp16), or G >= 8 (fp32), the fp32 accumulators of a
 *     whole head row for every head of the group would not fit the register
 *     file, so those shapes always run with V's head dim split over two
 *     workgroups (see pa_decode), and with half the heuristic's partitions
 *     while the units are fewer than the compute units.
 *     Sequences are processed in tiles of 16 tokens; a row of the table
 *     covers T = max_blocks * block_size / 16 tiles.
 *   - All calls only enqueue work on `stream` (a hipStream_t, NULL = the null
 *     stream); nothing synchronises with the host.  The return code reports
 *     errors the host can see: argument validation (checked before any HIP
 *     call) and launch failures.  Faults inside a kernel surface later, from
 *     the HIP runtime, and leave the HIP context unusable.
 *   - q, k_cache, v_cache, out and workspace must be 16-byte aligned;
 *     block_tables and context_lens 4-byte aligned.  out must not overlap q,
 *     k_cache or v_cache, and a caller workspace must not overlap out or q
 *     (PA_ERR_ALIAS; the library sees no cache sizes, so it checks the
 *     caches only against out's start).
 *   - The caller owns every buffer.  The library keeps no pointer past the
 *     call, except the workspace it allocates itself (see pa_decode).
 *   - B == 0 is a no-op that returns PA_OK.
 *   - Device-side preconditions the host cannot check without a copy:
 *     context_lens[b] is clamped to [0, max_blocks * block_size]; a negative
 *     table entry inside the context (-1) removes that block's tokens from
 *     the softmax; every other entry used must be a valid pool block.  A
 *     sequence with no live token gets an all-zero output row.
 *   - Range: scores and sums are fp32, so inputs must keep them finite there.
 *     |scale * q . K| finite in fp32 and |V| < 2^90 suffice, since softmax
 *     weights up to 2^8 are summed over at most 2^30 tokens.
 */
#ifndef PA_DECODE_H
#define PA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_DTYPE_F32 = 0, PA_DTYPE_BF16 = 1, PA_DTYPE_F16 = 2 } pa_dtype_t;

enum {
    PA_OK = 0,
    PA_ERR_NULL = -1,        /* a required pointer is NULL                        */
    PA_ERR_SHAPE = -2,       /* negative or inconsistent sizes (e.g. H % Hkv != 0) */
    PA_ERR_UNSUPPORTED = -3, /* valid but not built: d, block_size or H/Hkv       */
    PA_ERR_DTYPE = -4,       /* dtype is not a pa_dtype_t value                   */
    PA_ERR_ALIGN = -5,       /* a pointer breaks the alignment rule               */
    PA_ERR_WORKSPACE = -6,   /* workspace missing or too small, or the library   */
                             /* would have to allocate one during graph capture */
    PA_ERR_HIP = -7,         /* a HIP runtime call or a launch failed             */
    PA_ERR_DEVICE = -8,      /* no current HIP device                             */
    PA_ERR_ALIAS = -9,       /* out, or a workspace, overlaps an input            */
    PA_ERR_VALUE = -10       /* scale not finite, or a negative count             */
};

/*
 * Partitions.  With P partitions, sequence b's n_b = ceil(context_lens[b] / 16)
 * tiles of 16 tokens go to its first busy_b partitions: the tiles are dealt in
 * runs of 2 consecutive tiles to the 4 * busy_b lanes (4 per partition) in
 * turn, partition p owning lanes 4p .. 4p + 3.  So the split follows each
 * sequence's own length -- a batch of short contexts in a wide table still
 * keeps its partitions busy -- and the merge is a sum over the partitions'
 * tokens, which need not be contiguous.  busy_b = min(n_b, P) when the count
 * is given (pa_decode_ex with num_partitions > 0, pa_decode_partials); with
 * the heuristic count (pa_decode) a sequence uses only the partitions its
 * length fills, busy_b = min(P, ceil(n_b / T)), T = 8 tiles while the B * Hkv
 * (sequence, kv head) units are fewer than the device's compute units (and
 * busy_b = 1 for n_b <= 16: one workgroup reads 16 tiles in two rounds of
 * loads, faster than a split and its merge) and T = 64 otherwise, with
 * busy_b = 1 for n_b <= 128, so that in a batch that already covers the device
 * only sequences longer than 2048 tokens split.
 * Partitions p >= busy_b are empty.
 *
 * One decode step (the signature the docs page's kernel launch wraps:
 * output, query, k_cache, v_cache, block_tables, context_lens plus the scalar
 * shape parameters).  Picks the number of context partitions P with
 * pa_choose_partitions for the current device, except that P = 2 on a table
 * of at most 32 tiles becomes P = 1 when the single pass then splits V (see
 * below): the same two workgroups per unit, without a merge.  P == 1 runs one kernel that
 * writes out directly; when the B * Hkv (sequence, kv head) units fill at most
 * half of the device's compute units (and d >= 128), it runs two workgroups
 * per unit, each reading all of K and one half of every V row and writing
 * that half of the output.  P > 1 runs the split kernel in its fused form: every
 * workgroup of a non-empty partition writes its (max, sum, weighted values) to
 * a library-owned workspace and takes an atomic ticket; the last workgroup of
 * each (sequence, kv head) merges those partials and writes out (shared with
 * the arrivals before it, each taking one slice of the head dim of about
 * 8 KiB of partials, 2 to 16 slices in all, when the unit's partials are at
 * least 48 KiB and the launch's workgroups fit the device at once, at most
 * one per compute unit).  When the
 * B * Hkv * P workgroups fill at most a quarter of the compute units (and
 * d >= 128), each partition is again served by two workgroups, one per half
 * of V's head dim, and the ticket counts both.  The shapes that always split V
 * (see Supported shapes) do so whatever the launch's size: as the single pass,
 * the fused split, and the split kernel of a caller workspace.  A sequence
 * with at most one non-empty partition is written directly by partition 0
 * (zeros for an empty sequence); empty partitions do nothing.
 *
 * Sharing the device.  The arrivals that share a merge wait on the GPU for
 * the rest of their (sequence, kv head) to arrive, holding their workgroup
 * slot meanwhile.  The library shares merges only when the launch's
 * workgroups fit the device at once, and it keeps each launch's waiters
 * below half of the workgroups the device holds at once (sharing among fewer
 * arrivals where needed), so one such launch, or two running concurrently on
 * different streams, always leave a slot for the workgroups they wait for.
 * Kernels of other streams or processes only delay the wait, since they end.
 * Three or more fused launches running at once could in principle fill every
 * slot with waiters: a waiter gives up after 2^22 polls of its ticket
 * (seconds) and writes NaN over its slice of the output rather than a wrong
 * value.
 *
 * Library-owned buffers.  The partials buffer and the ticket buffer are
 * allocated on first need per (device, stream) and grown when larger ones are
 * needed; growing synchronises `stream` once.  Tickets are zeroed on `stream`
 * when allocated, and every call leaves them zero.  Calls on one stream are
 * ordered by the stream.  Calls from several host threads are safe: the
 * lookup, any growth and the launch happen under one lock.  pa_release frees
 * the buffers.
 *
 * Graph capture.  A call that would allocate or grow the buffers while
 * `stream` is being captured returns PA_ERR_WORKSPACE, so make one call of
 * the same or a larger shape on that stream first.  A captured call keeps the
 * addresses of its stream's buffers.  So (a) replay such a graph only where
 * it cannot overlap other work that uses them (any call on that stream, or
 * another replay), and (b) capture again after a larger call on that stream
 * or pa_release, either of which may free them.  A caller workspace
 * (pa_decode_ex) avoids both.
 *
 * max_blocks is the width of block_tables (its row stride).
 * Returns PA_OK or a negative PA_ERR_* code.
 */
int pa_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
              const int32_t *block_tables, const int32_t *context_lens, int B, int H, int Hkv,
              int d, int block_size, int max_blocks, float scale, int dtype, void *stream);

/* num_partitions value of pa_decode_ex and pa_plan: the heuristic, told that
 * every sequence of the batch has the same context length. */
#define PA_PARTITIONS_UNIFORM (-1)

/*
 * pa_decode with the choices exposed.
 *   num_partitions   0 = heuristic (as pa_decode), 1 = single pass, n > 1 =
 *                    P = min(n, W, 4096) partitions, W = max_blocks *
 *                    block_size / 16 the tiles of a table row, split as
 *                    above.  PA_PARTITIONS_UNIFORM = the heuristic for a
 *                    batch whose context_lens are all equal (the caller's
 *                    promise; the lengths are in device memory): when the
 *                    B * Hkv units already fill the device it runs the single
 *                    pass instead of splitting the sequences longer than 2048
 *                    tokens, which only pays off when a few long sequences
 *                    would otherwise set the pace; below that it is the
 *                    heuristic.  Results are correct whatever the lengths.
 *   num_pool_blocks  0 = unknown; > 0 = table entries >= num_pool_blocks are
 *                    treated like -1 instead of being read (a guard against
 *                    out-of-range ids).
 *   workspace        NULL = library-owned, fused split as in pa_decode.  Else
 *                    a device buffer of workspace_bytes >=
 *                    pa_workspace_bytes(B, H, d, P) for the partition
 *                    count P actually used (else PA_ERR_WORKSPACE); then the
 *                    split kernel and a separate merge kernel run (no tickets,
 *                    so the buffer needs no initialisation).  Unused when
 *                    P == 1.
 */
int pa_decode_ex(void *out, const void *q, const void *k_cache, const void *v_cache,
                 const int32_t *block_tables, const int32_t *context_lens, int B, int H, int Hkv,
                 int d, int block_size, int max_blocks, float scale, int dtype, void *stream,
                 int num_partitions, long long num_pool_blocks, void *workspace,
                 size_t workspace_bytes);

/*
 * pa_decode without any allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, same launch (heuristic partition count)
 * and same results as pa_decode; the fused split's tickets and partials live
 * in a fixed device array of 64 MiB inside the library (one per device, held
 * until the process ends) instead of library-owned allocations, so the call
 * never allocates, frees or synchronises.  The first call on a device takes
 * that device's array address and enqueues a small kernel on `stream` that
 * clears the tickets; every call leaves them clear.  Limit: the array holds
 * 16384 tickets (2 MiB, one 128-byte line each) and 62 MiB of partials, so a
 * split with B * Hkv > 16384 or pa_workspace_bytes(B, H, d, P) > 62 MiB
 * returns PA_ERR_WORKSPACE before launching anything (the single pass needs
 * none).
 * All calls on one device share the array: calls that may overlap in time on
 * one device (on different streams, or graph replays beside other calls) race
 * on it and must be ordered by the caller.  Returns PA_OK or a negative
 * PA_ERR_* code, as pa_decode.
 */
int pa_decode_noalloc(void *out, const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, const int32_t *context_lens, int B, int H,
                      int Hkv, int d, int block_size, int max_blocks, float scale, int dtype,
                      void *stream);

/*
 * The two halves of the split path, for callers that schedule them apart or
 * time them separately (Flash-Decoding's per-chunk pass and its merge).
 * pa_decode_partials runs only the split kernel: for every (b, h) and
 * partition p < P it writes a reference max m, the normaliser
 * l = sum_t 2^(s_t - m) and the unnormalised weighted sum O = sum_t
 * 2^(s_t - m) V_t over the partition's tokens t, with scores in log2 units
 * (s_t = scale * log2(e) * q.K_t), into `workspace`; the partition's result is
 * O / l.  m is within 8 of the largest score: max_t s_t - 8 <= m <= max_t s_t
 * (up to fp32 rounding).  Layout: [B][H][P] float pairs (max, sum),
 * then, from the next 256-byte boundary, [B][H][P][d] float sums.  An empty
 * partition stores
 * (-1e30, 0, zeros).  pa_merge_partials combines them into out.
 * Partitions are split as above; every partition, empty ones included,
 * writes its slot.  num_partitions must be >= 1 (else PA_ERR_VALUE) and at
 * most 4096 (else PA_ERR_UNSUPPORTED), and is used as given (P =
 * num_partitions).
 */
int pa_decode_partials(const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *block_tables, const int32_t *context_lens, int B, int H,
                       int Hkv, int d, int block_size, int max_blocks, float scale, int dtype,
                       int num_partitions, long long num_pool_blocks, void *workspace,
                       size_t workspace_bytes, void *stream);
int pa_merge_partials(void *out, const void *workspace, size_t workspace_bytes, int B, int H,
                      int d, int num_partitions, int dtype, void *stream);

/* Workspace bytes the split path needs for P partitions (0 when P <= 1). */
size_t pa_workspace_bytes(int B, int H, int d, int num_partitions);

/*
 * The launch heuristic (pure; no HIP call).  The flash-decoding-bench design
 * note, implementations section, picks the chunk size of its split from the
 * KV length, trading loop overhead against parallelism; here the partition
 * count follows the table width and how many (sequence, kv head) units the
 * device's compute units can take.  Work units are the B * Hkv
 * (sequence, kv-head) pairs; each is one workgroup in a single pass.  When
 * they are fewer than num_cus it splits the W = max_blocks * block_size / 16
 * tiles of a table row into floor(num_cus / units) partitions, so that the
 * workgroups never outnumber the compute units, keeping at least 8 tiles
 * (128 tokens) per partition of a full row; a row of at most 16 tiles (256
 * tokens) does not split.  When they already cover the device it
 * returns 1 for W <= 128, else ceil(W / 64), at most 16: room for the
 * sequences longer than 2048 tokens to split into partitions of 1024 tokens
 * (see Partitions).  Returns
 * >= 1 (1 for non-positive inputs or block_size below 16).
 */
int pa_choose_partitions(int B, int Hkv, int max_blocks, int block_size, int num_cus);

/*
 * The launch pa_decode_ex makes for these sizes on a device of num_cus compute
 * units when no caller workspace is given (pure; no HIP call), i.e. the
 * length-based choice of the split (flash-decoding-bench design note,
 * implementations section) as pa_decode applies it: *partitions =
 * the context partition count P it uses (num_partitions as in pa_decode_ex:
 * 0 = heuristic, PA_PARTITIONS_UNIFORM, n > 0 = forced), *v_slices = 2 when
 * each unit (P == 1) or
 * each partition (P > 1) is served by two workgroups, one per half of V's
 * head dim, else 1.  H and dtype matter only for the shapes that always split
 * V (see Supported shapes).  Returns PA_OK, PA_ERR_NULL, PA_ERR_SHAPE (B < 0,
 * H, Hkv, max_blocks or num_cus <= 0, or H % Hkv != 0), PA_ERR_DTYPE,
 * PA_ERR_VALUE (num_partitions < -1) or PA_ERR_UNSUPPORTED (d, block_size or
 * H / Hkv not supported).
 */
int pa_plan(int B, int H, int Hkv, int d, int dtype, int max_blocks, int block_size,
            int num_cus, int num_partitions, int *partitions, int *v_slices);

/* Compute units of HIP device `device` (cached), or a negative PA_ERR_*. */
int pa_device_num_cus(int device);

/* Static text for a return code. */
const char *pa_strerror(int code);

/* Frees every library-owned buffer (synchronises the devices that own one). */
void pa_release(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_DECODE_H */
