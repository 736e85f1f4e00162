// pa_read_probe.hip -- measuring sticks for the decode kernel's bandwidth.  A
// plain streaming read of a buffer with the decode kernel's load shape
// (workgroups of 4 waves, 16-byte non-temporal raw buffer loads, 16 KB in
// flight per wave), and the decode kernel's own gather of the K and V rows
// through the block table: both do nothing else -- no scores, no softmax, no
// merge -- so their times for the bytes of one decode step bound what the
// kernel can reach with that shape.  Beside them, a one-thread kernel that
// writes the device clock, which the benchmark captures around its timed
// steps.  Built into its own library, libpa_read_probe.so; the decode library
// does not contain or call any of them.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_read_probe.h"

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kChunk = kWave * 16;  // bytes one load instruction of a wave covers

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// The xor of `acc` over the workgroup (valid in thread 0): a butterfly over
// each wave, then the 4 waves' words through LDS.
__device__ __forceinline__ unsigned fold_workgroup(unsigned acc, int wave, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) acc ^= __shfl_xor(acc, o);
    __shared__ unsigned folded[kWaves];
    if (lane == 0) folded[wave] = acc;
    __syncthreads();
    return folded[0] ^ folded[1] ^ folded[2] ^ folded[3];
}

// Workgroup g reads bytes [g * slice, min((g + 1) * slice, bytes)); wave w
// takes runs of DEPTH consecutive 1 KB chunks, run r of the workgroup going
// to wave r % kWaves, all DEPTH loads of a run in flight before any is used.
// The descriptor covers exactly the slice, so the loads of a run past its end
// return zeros without a memory access.  Every lane folds what it read into
// one word and the workgroup writes a single word, so the loads stay live.
template <int DEPTH>
__global__ __launch_bounds__(kWaves * kWave) void read_kernel(const char *src, long long bytes,
                                                              long long slice, unsigned *sink) {
    const long long begin = (long long)blockIdx.x * slice;
    long long len = bytes - begin;
    if (len > slice) len = slice;
    if (len < 0) len = 0;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(src + begin), 0, (int)len, 0x00020000);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    unsigned acc = 0;
    const long long run_bytes = (long long)DEPTH * kChunk;
    for (long long off = wave * run_bytes; off < len; off += kWaves * run_bytes) {
        u32x4 x[DEPTH];
#pragma unroll
        for (int j = 0; j < DEPTH; ++j)
            x[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 r, (unsigned)(off + j * kChunk + 16 * lane), 0, 2));
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) acc ^= x[j][0] ^ x[j][1] ^ x[j][2] ^ x[j][3];
    }
    const unsigned a = fold_workgroup(acc, wave, lane);
    if (threadIdx.x == 0) sink[blockIdx.x] = a;
}

// The decode kernel's gather without its arithmetic: grid (kv head, sequence,
// partition) of 4 waves, the sequence's 16-token tiles dealt in runs of two to
// the P * 4 (partition, wave) lanes in turn, two tiles in flight per wave, the
// table entry of each tile read as a scalar, and per tile one buffer
// descriptor over its live rows of this kv head for K and one for V (rows
// past the context and -1 blocks read as zeros without a memory access).
// Each load instruction of a wave covers whole rows (ROWB / 16 lanes per
// row), 16 bytes per lane, non-temporal.  With VS = 2, as in the decode
// kernel's V-split modes, two workgroups serve each partition (grid z = 2
// partition + slice): both read all of K, each one half of every V row.  The
// words read are folded with xor, and each workgroup writes the xor of all of
// them to sink, so the xor of the whole sink is the xor of every live K row
// read VS times and every live V row once, whatever the deal.
template <int ROWB, int VS>
__global__ __launch_bounds__(kWaves * kWave) void gather_kernel(
    const char *k, const char *v, const int *table, const int *lens, int max_blocks, int P,
    int tok_bytes, long long blk_bytes, int tiles_log2, unsigned *sink) {
    constexpr int kDepth = 2;                    // tiles in flight per wave
    constexpr int kLoads = ROWB / 64;            // 16-byte K loads per lane per 16-row tile
    constexpr int kLanesPerRow = ROWB / 16;
    constexpr int kVLoads = kLoads / VS;         // the same for this slice of V
    constexpr int kVLanesPerRow = kLanesPerRow / VS;
    const int kvh = blockIdx.x, b = blockIdx.y;
    const int part = VS > 1 ? (int)(blockIdx.z >> 1) : (int)blockIdx.z;
    const int vslice = VS > 1 ? (int)(blockIdx.z & 1) : 0;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int *trow = table + (long long)b * max_blocks;
    auto table_at = [&](int j) -> int {
        const int e = j >> tiles_log2;
        return trow[e < max_blocks ? e : max_blocks - 1];
    };
    // the length and the first group's table entries leave together, as in
    // the decode kernel (a lane's first tiles do not depend on the length)
    const int first = kDepth * (part * kWaves + wave);
    int ctx = lens[b];
    int nid[kDepth];
#pragma unroll
    for (int s = 0; s < kDepth; ++s) nid[s] = table_at(first + s);
    const int cap = max_blocks << (tiles_log2 + 4);
    ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
    const int ntiles = (ctx + 15) / 16;
    const int stride = P * kWaves * kDepth;
    const char *kb = k + (long long)kvh * ROWB;
    const char *vb = v + (long long)kvh * ROWB + vslice * (ROWB / VS);
    unsigned off[kLoads], voff[kVLoads];
#pragma unroll
    for (int m = 0; m < kLoads; ++m) {
        const int c = m * kWave + lane;
        off[m] = (c / kLanesPerRow) * tok_bytes + 16 * (c % kLanesPerRow);
    }
#pragma unroll
    for (int m = 0; m < kVLoads; ++m) {
        const int c = m * kWave + lane;
        voff[m] = (c / kVLanesPerRow) * tok_bytes + 16 * (c % kVLanesPerRow);
    }
    u32x4 kr[kDepth][kLoads], vr[kDepth][kVLoads];
    auto issue = [&](int s, int j, int id) {
        int nl = ctx - 16 * j;
        nl = nl < 16 ? nl : 16;
        if (j >= ntiles || id < 0) nl = 0;
        const long long o = nl > 0 ? (long long)id * blk_bytes +
                                         (long long)(j & ((1 << tiles_log2) - 1)) * 16 * tok_bytes
                                   : 0;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(kb + o), 0, nl * tok_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(vb + o), 0, nl * tok_bytes, 0x00020000);
#pragma unroll
        for (int m = 0; m < kLoads; ++m)
            kr[s][m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off[m], 0, 2));
#pragma unroll
        for (int m = 0; m < kVLoads; ++m)
            vr[s][m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff[m], 0, 2));
    };
    unsigned acc = 0;
    auto fold = [&](int s) {
#pragma unroll
        for (int m = 0; m < kLoads; ++m) acc ^= kr[s][m][0] ^ kr[s][m][1] ^ kr[s][m][2] ^ kr[s][m][3];
#pragma unroll
        for (int m = 0; m < kVLoads; ++m) acc ^= vr[s][m][0] ^ vr[s][m][1] ^ vr[s][m][2] ^ vr[s][m][3];
    };
#pragma unroll
    for (int s = 0; s < kDepth; ++s) issue(s, first + s, nid[s]);
    for (int g = 1; first + stride * g < ntiles; ++g) {
        const int nbase = first + stride * g;
#pragma unroll
        for (int s = 0; s < kDepth; ++s) nid[s] = table_at(nbase + s);
#pragma unroll
        for (int s = 0; s < kDepth; ++s) {
            fold(s);
            issue(s, nbase + s, nid[s]);
        }
    }
#pragma unroll
    for (int s = 0; s < kDepth; ++s) fold(s);
    const unsigned a = fold_workgroup(acc, wave, lane);
    if (threadIdx.x == 0)
        sink[((long long)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x] = a;
}

// One thread writes the device's constant-rate clock (s_memrealtime, 100 MHz)
// to dst[0].
__global__ void stamp_kernel(unsigned long long *dst) {
    if (threadIdx.x == 0) dst[0] = __builtin_amdgcn_s_memrealtime();
}

}  // namespace

extern "C" int pa_probe_stamp(unsigned long long *dst, void *stream) {
    if (!dst) return -1;
    hipLaunchKernelGGL(stamp_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), dst);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

extern "C" int pa_probe_gather(const void *k_cache, const void *v_cache,
                               const int32_t *block_tables, const int32_t *context_lens, int B,
                               int Hkv, int row_bytes, int block_size, int max_blocks,
                               int partitions, int v_slices, unsigned *sink, void *stream) {
    if (!k_cache || !v_cache || !block_tables || !context_lens || !sink) return -1;
    if (B < 0 || Hkv <= 0 || max_blocks <= 0 || partitions <= 0 || v_slices <= 0) return -2;
    if ((row_bytes != 128 && row_bytes != 256 && row_bytes != 512) || v_slices > 2 ||
        block_size < 16 || block_size > 256 || (block_size & (block_size - 1)) != 0 ||
        partitions > 4096 || B > 65535 || Hkv > 65535 ||
        (long long)max_blocks * block_size > (1LL << 30) ||
        16LL * Hkv * row_bytes > 0x7FFFFFFFLL)
        return -3;
    if (B == 0) return 0;
    int tiles_log2 = 0;
    while ((16 << tiles_log2) < block_size) ++tiles_log2;
    const int tok = Hkv * row_bytes;
    const long long blk = (long long)block_size * tok;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const char *k = static_cast<const char *>(k_cache);
    const char *v = static_cast<const char *>(v_cache);
    const dim3 grid(Hkv, B, partitions * v_slices), block(kWaves * kWave);
#define PA_PROBE_GATHER(R, S)                                                                   \
    hipLaunchKernelGGL((gather_kernel<R, S>), grid, block, 0, s, k, v, block_tables,            \
                       context_lens, max_blocks, partitions, tok, blk, tiles_log2, sink)
    if (v_slices == 1) {
        switch (row_bytes) {
            case 128: PA_PROBE_GATHER(128, 1); break;
            case 256: PA_PROBE_GATHER(256, 1); break;
            default: PA_PROBE_GATHER(512, 1); break;
        }
    } else {
        switch (row_bytes) {
            case 128: PA_PROBE_GATHER(128, 2); break;
            case 256: PA_PROBE_GATHER(256, 2); break;
            default: PA_PROBE_GATHER(512, 2); break;
        }
    }
#undef PA_PROBE_GATHER
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

extern "C" int pa_probe_read(const void *src, long long bytes, int workgroups, int depth,
                             unsigned *sink, void *stream) {
    if (!src || !sink) return -1;
    if (bytes < 0 || workgroups <= 0) return -2;
    // a slice is addressed with 32-bit buffer offsets
    const long long slice = ((bytes + workgroups - 1) / workgroups + kChunk - 1) / kChunk * kChunk;
    if (slice > 0x7FFFFFFFLL - 64LL * kChunk) return -3;
    if (bytes == 0) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const char *p = static_cast<const char *>(src);
    switch (depth) {
        case 8: hipLaunchKernelGGL(read_kernel<8>, dim3(workgroups), dim3(kWaves * kWave), 0, s, p, bytes, slice, sink); break;
        case 16: hipLaunchKernelGGL(read_kernel<16>, dim3(workgroups), dim3(kWaves * kWave), 0, s, p, bytes, slice, sink); break;
        case 32: hipLaunchKernelGGL(read_kernel<32>, dim3(workgroups), dim3(kWaves * kWave), 0, s, p, bytes, slice, sink); break;
        default: return -3;
    }
    return hipGetLastError() == hipSuccess ? 0 : -7;
}
