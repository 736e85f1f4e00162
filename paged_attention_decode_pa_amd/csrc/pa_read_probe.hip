// pa_read_probe.hip -- a plain streaming read, the measuring stick for the
// decode kernel's bandwidth.  It reads a buffer once with the decode kernel's
// load shape (workgroups of 4 waves, 16-byte non-temporal raw buffer loads,
// 16 KB in flight per wave) and does nothing else: no table, no scores, no
// merge.  Its time for the bytes one decode step reads is the time no kernel
// with that load shape can beat on this part.  Beside it, a one-thread kernel
// that writes the device clock, which the benchmark captures around its timed
// steps.  Built into its own library, libpa_read_probe.so; the decode library
// does not contain or call either.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_read_probe.h"

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kChunk = kWave * 16;  // bytes one load instruction of a wave covers

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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
    __shared__ unsigned folded[kWaves * kWave];
    folded[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned a = 0;
        for (int i = 0; i < kWaves * kWave; ++i) a ^= folded[i];
        sink[blockIdx.x] = a;
    }
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
