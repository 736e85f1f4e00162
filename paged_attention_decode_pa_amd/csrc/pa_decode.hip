// pa_decode.hip -- paged-attention decode step for gfx950 (MI355X), C ABI.
//
// What is computed is declared in include/pa_decode.h.  This file holds the
// three kernels and the host launcher behind that ABI.
//
// Design (one work unit = one (sequence b, kv head kvh) pair, optionally one
// partition of its context):
//
// * One workgroup per (kvh, b[, partition]) serves all G = H / Hkv query heads
//   of the group, so each K/V row is read from HBM once per kv head, not once
//   per query head.
// * A wave consumes one 16-token physical block per step.  The block id is
//   wave-uniform (read from a per-wave register copy of the table slice with
//   readlane), so each K/V load is an SGPR base plus a per-lane 32-bit offset
//   that never changes: 16-byte loads, 64 contiguous bytes per token for K and
//   the full 256-byte row per token for V.
// * Scores: the 16 tokens x G heads x 128 product is a small dense
//   contraction, run on the matrix cores: rows = the block's 16 tokens,
//   columns = the G query heads repeated to 16, reduction = head_dim.  Each
//   lane's 16-byte K load is exactly its MFMA A operand, so no cross-lane
//   reduction is needed for q.K.  After the MFMAs lane (row g = lane/16,
//   column c = lane%16) holds the scores of tokens 4g..4g+3 for head c % G.
// * Online softmax per (row g, head): running max m and normaliser l in log2
//   units (scale * log2 e is folded into one multiply), so each lane updates
//   its own statistics from its 4 scores with no cross-lane max per block.
// * V accumulate on the vector ALUs in fp32: lane (g, c) holds 8 elements of
//   the V rows of tokens 4g..4g+3 and accumulates them for all G heads; the
//   weights of the other heads come from neighbouring lanes by DPP broadcast.
// * Epilogue: rows, then waves, are merged with the rescale-and-sum rule
//   (M = max m, L = sum l * 2^(m - M), O = sum acc * 2^(m - M)); a single
//   pass writes O / L, the split kernel writes (M, L, O) per partition and a
//   merge kernel applies the same rule across partitions.
//
// Masking: tokens past context_len inside the last block get score -inf and a
// zero V (select, so NaN in unused slots never leaks); blocks whose table entry
// is negative (or >= num_pool_blocks when that is given) are skipped whole.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "pa_decode.h"

namespace {

constexpr int kWave = 64;
constexpr int kBlockTokens = 16;  // tokens per physical block (block_size)
constexpr int kHeadDim = 128;     // d
constexpr float kLog2e = 1.44269504088896340736f;
// Start value of a running max: finite, so 2^(m - m') never sees inf - inf.
constexpr float kMaxInit = -1.0e30f;

constexpr int kWavesPerGroup = 4;  // waves per workgroup
constexpr int kDepth = 2;          // blocks whose loads are in flight per wave

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct Params {
    const char *q;
    const char *k;
    const char *v;
    const int32_t *table;
    const int32_t *lens;
    void *out;          // single pass: [B][H][d] dtype
    float2 *part_ml;    // split: [B][H][P] (max, sum)
    float *part_acc;    // split: [B][H][P][d]
    long long blk_bytes;  // bytes per physical block: block_size * Hkv * d * esize
    long long pool;       // > 0: ids >= pool are skipped
    int tok_bytes;        // bytes between tokens of a block: Hkv * d * esize
    int B, H, Hkv, max_blocks, P, bpp;
    float qk_scale;       // scale * log2(e)
};

// Per-dtype load geometry: 16-byte loads per lane per block for K and V.
template <int DT> struct Geometry;
template <> struct Geometry<PA_DTYPE_BF16> {
    static constexpr int kEs = 2, kKLoads = 4, kVLoads = 4;
};
template <> struct Geometry<PA_DTYPE_F32> {
    static constexpr int kEs = 4, kKLoads = 8, kVLoads = 8;
};

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Value of x held by the lane of this lane's group of G lanes that serves head H_.
template <int G, int H_>
__device__ __forceinline__ float group_bcast(float x) {
    if constexpr (G == 1) {
        return x;
    } else if constexpr (G == 2) {
        constexpr int ctrl = H_ | (H_ << 2) | ((2 + H_) << 4) | ((2 + H_) << 6);
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xF, 0xF, false));
    } else if constexpr (G == 4) {
        constexpr int ctrl = H_ * 0x55;  // quad_perm [H_, H_, H_, H_]
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xF, 0xF, false));
    } else {
        // ds_swizzle bit-mask mode: lane' = (lane & and_mask) | or_mask within 32 lanes
        constexpr int and_mask = G == 8 ? 0x18 : 0x10;
        constexpr int pattern = and_mask | (H_ << 5);
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), pattern));
    }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16 bytes of V row -> 8 fp32 (bf16) or the low 4 of them (f32 uses two loads).
__device__ __forceinline__ void unpack_bf16(const u32x4 &w, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

template <int DT, int G>
struct WaveState {
    float m;           // running max (log2 units) of this lane's (row, head)
    float l;           // running normaliser
    float acc[G][8];   // unnormalised sum of p * V for every head of the group
};

// One block's scores, softmax update and V accumulation.  rem = live tokens in
// this block (only looked at when TAIL).
template <int DT, int G, bool TAIL>
__device__ __forceinline__ void consume_block(WaveState<DT, G> &st, const u32x4 *kr,
                                              const u32x4 *vr, const u32x4 *qr, float qk_scale,
                                              int g, int rem) {
    using Geo = Geometry<DT>;
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
    if constexpr (DT == PA_DTYPE_BF16) {
#pragma unroll
        for (int m = 0; m < Geo::kKLoads; ++m)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[m]),
                                                         __builtin_bit_cast(bf16x8, qr[m]), c,
                                                         0, 0, 0);
    } else {
#pragma unroll
        for (int m = 0; m < Geo::kKLoads; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kr[m][j]),
                                                          __uint_as_float(qr[m][j]), c, 0, 0, 0);
    }
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        s[r] = c[r] * qk_scale;
        if constexpr (TAIL) s[r] = (4 * g + r < rem) ? s[r] : -INFINITY;
    }
    const float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    const float mn = fmaxf(st.m, bm);
    const float alpha = fast_exp2(st.m - mn);
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(s[r] - mn);
    st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    st.m = mn;

    static_for<G>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        const float a = group_bcast<G, h>(alpha);
#pragma unroll
        for (int e = 0; e < 8; ++e) st.acc[h][e] *= a;
    });
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float vf[8];
        if constexpr (DT == PA_DTYPE_BF16) {
            unpack_bf16(vr[r], vf);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                vf[j] = __uint_as_float(vr[2 * r][j]);
                vf[4 + j] = __uint_as_float(vr[2 * r + 1][j]);
            }
        }
        if constexpr (TAIL) {
            const bool live = 4 * g + r < rem;
#pragma unroll
            for (int e = 0; e < 8; ++e) vf[e] = live ? vf[e] : 0.f;
        }
        static_for<G>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            const float ph = group_bcast<G, h>(p[r]);
#pragma unroll
            for (int e = 0; e < 8; ++e) st.acc[h][e] = fmaf(ph, vf[e], st.acc[h][e]);
        });
    }
}

// Head-dim element held in accumulator slot e by the lane in column c16.
template <int DT>
__device__ __forceinline__ int acc_elem(int c16, int e) {
    if constexpr (DT == PA_DTYPE_BF16) return 8 * c16 + e;
    else return 64 * (e / 4) + 4 * c16 + (e % 4);
}

__device__ __forceinline__ void store_out(void *out, long long idx, float x, int dt) {
    if (dt == PA_DTYPE_BF16) static_cast<__bf16 *>(out)[idx] = static_cast<__bf16>(x);
    else static_cast<float *>(out)[idx] = x;
}

template <int DT, int G, int NW, int D>
__global__ __launch_bounds__(NW * kWave) void pa_decode_kernel(Params p) {
    using Geo = Geometry<DT>;
    constexpr int KL = Geo::kKLoads, VL = Geo::kVLoads, VPT = VL / 4;

    const int wg = blockIdx.x;
    const int kvh = wg % p.Hkv;
    const int b = (wg / p.Hkv) % p.B;
    const int part = wg / (p.Hkv * p.B);
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int c16 = lane & 15;  // MFMA column / token of the block for K
    const int g = lane >> 4;    // MFMA row group: tokens 4g..4g+3 for V

    int ctx = p.lens[b];
    ctx = ctx < 0 ? 0 : (ctx > p.max_blocks * kBlockTokens ? p.max_blocks * kBlockTokens : ctx);
    const int nblk = (ctx + kBlockTokens - 1) / kBlockTokens;
    const int lo = part * p.bpp;
    const int hi = min(lo + p.bpp, nblk);

    // B operand: the query of head kvh*G + c16%G, chunk (4m + g) of 16 bytes.
    const char *qrow = p.q + ((long long)b * p.H + kvh * G + (c16 % G)) * (kHeadDim * Geo::kEs);
    u32x4 qr[KL];
#pragma unroll
    for (int m = 0; m < KL; ++m) qr[m] = *reinterpret_cast<const u32x4 *>(qrow + 64 * m + 16 * g);

    const int head_off = kvh * kHeadDim * Geo::kEs;
    const int koff = c16 * p.tok_bytes + head_off + 16 * g;
    int voff[VL];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int s = 0; s < VPT; ++s)
            voff[r * VPT + s] = (4 * g + r) * p.tok_bytes + head_off + 16 * c16 + 256 * s;

    WaveState<DT, G> st;
    st.m = kMaxInit;
    st.l = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) st.acc[h][e] = 0.f;

    const int first = lo + wave;  // this wave's blocks: first, first + NW, ...
    const int nw = hi > first ? (hi - first + NW - 1) / NW : 0;
    const int32_t *trow = p.table + (long long)b * p.max_blocks;

    for (int c0 = 0; c0 < nw; c0 += kWave) {
        const int cnt = min(kWave, nw - c0);
        const int tbl = lane < cnt ? trow[first + NW * (c0 + lane)] : -1;

        u32x4 kr[D][KL], vr[D][VL];
        auto live_block = [&](int blk) { return blk >= 0 && (p.pool <= 0 || blk < p.pool); };
        auto issue = [&](u32x4 *kd, u32x4 *vd, int i) {
            const int blk = __builtin_amdgcn_readlane(tbl, i);
            if (!live_block(blk)) return;
            const char *kb = p.k + (long long)blk * p.blk_bytes;
            const char *vb = p.v + (long long)blk * p.blk_bytes;
#pragma unroll
            for (int m = 0; m < KL; ++m) kd[m] = *reinterpret_cast<const u32x4 *>(kb + koff + 64 * m);
#pragma unroll
            for (int n = 0; n < VL; ++n) vd[n] = *reinterpret_cast<const u32x4 *>(vb + voff[n]);
        };

#pragma unroll
        for (int s = 0; s < D; ++s)
            if (s < cnt) issue(kr[s], vr[s], s);

        for (int i0 = 0; i0 < cnt; i0 += D) {
#pragma unroll
            for (int s = 0; s < D; ++s) {
                const int i = i0 + s;
                if (i < cnt) {
                    const int blk = __builtin_amdgcn_readlane(tbl, i);
                    if (live_block(blk)) {
                        const int rem = ctx - (first + NW * (c0 + i)) * kBlockTokens;
                        if (rem < kBlockTokens)
                            consume_block<DT, G, true>(st, kr[s], vr[s], qr, p.qk_scale, g, rem);
                        else
                            consume_block<DT, G, false>(st, kr[s], vr[s], qr, p.qk_scale, g, rem);
                    }
                    if (i + D < cnt) issue(kr[s], vr[s], i + D);
                }
            }
        }
    }

    // ---- merge the 4 row groups of the wave: lanes 16g + c16 share c16 ------
    // The (m, l) of row g and head h sit in the lanes of row g whose column is
    // h modulo G; fetch them for every head of the group.
    float mh[G], lh[G];
    static_for<G>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        mh[h] = group_bcast<G, h>(st.m);
        lh[h] = group_bcast<G, h>(st.l);
    });
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float M = fmaxf(mh[h], __shfl_xor(mh[h], 16));
        M = fmaxf(M, __shfl_xor(M, 32));
        const float f = fast_exp2(mh[h] - M);
        float L = lh[h] * f;
        L += __shfl_xor(L, 16);
        L += __shfl_xor(L, 32);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float a = st.acc[h][e] * f;
            a += __shfl_xor(a, 16);
            a += __shfl_xor(a, 32);
            st.acc[h][e] = a;
        }
        mh[h] = M;
        lh[h] = L;
    }

    // ---- merge the waves through LDS ----------------------------------------
    __shared__ float2 sm_ml[NW][G];
    __shared__ float sm_acc[NW][G][kHeadDim];
    if (lane < 16) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) sm_acc[wave][h][acc_elem<DT>(c16, e)] = st.acc[h][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) sm_ml[wave][h] = make_float2(mh[h], lh[h]);
    }
    __syncthreads();

    for (int idx = threadIdx.x; idx < G * kHeadDim; idx += NW * kWave) {
        const int h = idx / kHeadDim, e = idx % kHeadDim;
        float M = kMaxInit;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_ml[w][h].x);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = fast_exp2(sm_ml[w][h].x - M);
            L = fmaf(sm_ml[w][h].y, f, L);
            O = fmaf(sm_acc[w][h][e], f, O);
        }
        const long long bh = (long long)b * p.H + kvh * G + h;
        if (p.part_acc == nullptr) {
            store_out(p.out, bh * kHeadDim + e, L > 0.f ? O / L : 0.f, DT);
        } else {
            p.part_acc[(bh * p.P + part) * kHeadDim + e] = O;
            if (e == 0) p.part_ml[bh * p.P + part] = make_float2(M, L);
        }
    }
}

struct MergeParams {
    const float2 *part_ml;
    const float *part_acc;
    void *out;
    int B, H, P;
};

// One wave per (b, h): rescale every partition to the global max and sum.
template <int DT>
__global__ __launch_bounds__(kWave) void pa_merge_kernel(MergeParams mp) {
    extern __shared__ float sm_w[];  // P weights
    const long long bh = blockIdx.x;
    const int lane = threadIdx.x;
    const float2 *ml = mp.part_ml + bh * mp.P;
    float M = kMaxInit;
    for (int q = lane; q < mp.P; q += kWave) M = fmaxf(M, ml[q].x);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float L = 0.f;
    for (int q = lane; q < mp.P; q += kWave) {
        const float2 x = ml[q];
        const float f = fast_exp2(x.x - M);
        sm_w[q] = f;
        L = fmaf(x.y, f, L);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
    __syncthreads();
    const float *acc = mp.part_acc + bh * mp.P * kHeadDim + 2 * lane;
    float o0 = 0.f, o1 = 0.f;
    int q = 0;
    for (; q + 4 <= mp.P; q += 4) {
        float2 a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const float2 *>(acc + (q + j) * kHeadDim);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            o0 = fmaf(a[j].x, sm_w[q + j], o0);
            o1 = fmaf(a[j].y, sm_w[q + j], o1);
        }
    }
    for (; q < mp.P; ++q) {
        const float2 a = *reinterpret_cast<const float2 *>(acc + q * kHeadDim);
        o0 = fmaf(a.x, sm_w[q], o0);
        o1 = fmaf(a.y, sm_w[q], o1);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    store_out(mp.out, bh * kHeadDim + 2 * lane, o0 * inv, DT);
    store_out(mp.out, bh * kHeadDim + 2 * lane + 1, o1 * inv, DT);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

constexpr int kMinBlocksPerPartition = 8;
constexpr int kMaxPartitions = 4096;

size_t ml_region_bytes(int B, int H, int P) {
    size_t bytes = (size_t)B * H * P * sizeof(float2);
    return (bytes + 255) & ~(size_t)255;
}

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
    if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_ERR_DTYPE;
    if (!std::isfinite(scale)) return PA_ERR_VALUE;
    if (d != kHeadDim || block_size != kBlockTokens) return PA_ERR_UNSUPPORTED;
    const int G = H / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return PA_ERR_UNSUPPORTED;
    if ((long long)max_blocks * block_size > (1LL << 30)) return PA_ERR_UNSUPPORTED;
    v->G = G;
    v->esize = dtype == PA_DTYPE_BF16 ? 2 : 4;
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

std::mutex g_mutex;
std::map<int, int> g_cus;                                  // device -> CU count
std::map<std::pair<int, hipStream_t>, std::pair<void *, size_t>> g_workspace;

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

int library_workspace(int dev, hipStream_t stream, size_t bytes, void **ptr) {
    std::lock_guard<std::mutex> lock(g_mutex);
    auto &slot = g_workspace[{dev, stream}];
    if (slot.second < bytes) {
        if (slot.first) {
            // the previous buffer may still be in use by work on this stream
            if (hipStreamSynchronize(stream) != hipSuccess) return PA_ERR_HIP;
            if (hipFree(slot.first) != hipSuccess) return PA_ERR_HIP;
            slot = {nullptr, 0};
        }
        void *p = nullptr;
        if (hipMalloc(&p, bytes) != hipSuccess) return PA_ERR_HIP;
        slot = {p, bytes};
    }
    *ptr = slot.first;
    return PA_OK;
}

template <int DT, int G>
hipError_t launch_main(const Params &p, int groups, hipStream_t stream) {
    hipLaunchKernelGGL((pa_decode_kernel<DT, G, kWavesPerGroup, kDepth>), dim3(groups),
                       dim3(kWavesPerGroup * kWave), 0, stream, p);
    return hipGetLastError();
}

template <int DT>
hipError_t dispatch_g(const Params &p, int G, int groups, hipStream_t stream) {
    switch (G) {
        case 1: return launch_main<DT, 1>(p, groups, stream);
        case 2: return launch_main<DT, 2>(p, groups, stream);
        case 4: return launch_main<DT, 4>(p, groups, stream);
        case 8: return launch_main<DT, 8>(p, groups, stream);
        default: return launch_main<DT, 16>(p, groups, stream);
    }
}

int run_main(const Params &p, int dtype, int G, hipStream_t stream) {
    const long long groups = (long long)p.Hkv * p.B * p.P;
    if (groups > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;
    const hipError_t e = dtype == PA_DTYPE_BF16
                             ? dispatch_g<PA_DTYPE_BF16>(p, G, (int)groups, stream)
                             : dispatch_g<PA_DTYPE_F32>(p, G, (int)groups, stream);
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int run_merge(void *out, const void *ws, int B, int H, int P, int dtype, hipStream_t stream) {
    MergeParams mp;
    mp.part_ml = static_cast<const float2 *>(ws);
    mp.part_acc = reinterpret_cast<const float *>(static_cast<const char *>(ws) +
                                                  ml_region_bytes(B, H, P));
    mp.out = out;
    mp.B = B;
    mp.H = H;
    mp.P = P;
    const long long groups = (long long)B * H;
    if (groups > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;
    const size_t lds = (size_t)P * sizeof(float);
    if (dtype == PA_DTYPE_BF16)
        hipLaunchKernelGGL(pa_merge_kernel<PA_DTYPE_BF16>, dim3((int)groups), dim3(kWave), lds,
                           stream, mp);
    else
        hipLaunchKernelGGL(pa_merge_kernel<PA_DTYPE_F32>, dim3((int)groups), dim3(kWave), lds,
                           stream, mp);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

Params make_params(const void *q, const void *k_cache, const void *v_cache,
                   const int32_t *block_tables, const int32_t *context_lens, int B, int H,
                   int Hkv, int max_blocks, float scale, int esize, long long pool, int P) {
    Params p;
    p.q = static_cast<const char *>(q);
    p.k = static_cast<const char *>(k_cache);
    p.v = static_cast<const char *>(v_cache);
    p.table = block_tables;
    p.lens = context_lens;
    p.out = nullptr;
    p.part_ml = nullptr;
    p.part_acc = nullptr;
    p.tok_bytes = Hkv * kHeadDim * esize;
    p.blk_bytes = (long long)kBlockTokens * p.tok_bytes;
    p.pool = pool;
    p.B = B;
    p.H = H;
    p.Hkv = Hkv;
    p.max_blocks = max_blocks;
    p.P = P;
    p.bpp = (max_blocks + P - 1) / P;
    p.qk_scale = scale * kLog2e;
    return p;
}

int even_partitions(int max_blocks, int P) {
    if (P < 1) P = 1;
    if (P > max_blocks) P = max_blocks;
    const int bpp = (max_blocks + P - 1) / P;
    return (max_blocks + bpp - 1) / bpp;
}

}  // namespace

extern "C" {

int pa_choose_partitions(int B, int Hkv, int max_blocks, int block_size, int num_cus) {
    if (B <= 0 || Hkv <= 0 || max_blocks <= 0 || block_size <= 0 || num_cus <= 0) return 1;
    const long long units = (long long)B * Hkv;
    if (units >= num_cus) return 1;
    long long P = (num_cus + units - 1) / units;
    const long long cap = max_blocks / kMinBlocksPerPartition;
    if (P > cap) P = cap;
    if (P > kMaxPartitions) P = kMaxPartitions;
    if (P < 1) P = 1;
    return even_partitions(max_blocks, (int)P);
}

size_t pa_workspace_bytes(int B, int H, int d, int num_partitions) {
    if (B <= 0 || H <= 0 || d <= 0 || num_partitions <= 1) return 0;
    return ml_region_bytes(B, H, num_partitions) +
           (size_t)B * H * num_partitions * d * sizeof(float);
}

int pa_device_num_cus(int device) { return device_cus(device); }

const char *pa_strerror(int code) {
    switch (code) {
        case PA_OK: return "ok";
        case PA_ERR_NULL: return "a required pointer is NULL";
        case PA_ERR_SHAPE: return "negative or inconsistent sizes";
        case PA_ERR_UNSUPPORTED: return "shape not supported (needs d=128, block_size=16, H/Hkv in {1,2,4,8,16})";
        case PA_ERR_DTYPE: return "unknown dtype";
        case PA_ERR_ALIGN: return "pointer alignment (16 bytes for tensors, 4 for int32 arrays)";
        case PA_ERR_WORKSPACE: return "workspace missing or too small";
        case PA_ERR_HIP: return "HIP runtime call or kernel launch failed";
        case PA_ERR_DEVICE: return "no usable HIP device";
        case PA_ERR_ALIAS: return "out overlaps an input";
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
    if (num_partitions < 0 || num_pool_blocks < 0) return PA_ERR_VALUE;
    if (workspace && !aligned(workspace, 16)) return PA_ERR_ALIGN;
    if (B == 0) return PA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = 0;
    if ((rc = current_device(&dev)) != PA_OK) return rc;
    int P;
    if (num_partitions == 0) {
        const int cus = device_cus(dev);
        if (cus < 0) return cus;
        P = pa_choose_partitions(B, Hkv, max_blocks, block_size, cus);
    } else {
        P = even_partitions(max_blocks, num_partitions);
    }
    if (P > kMaxPartitions) return PA_ERR_UNSUPPORTED;
    Params p = make_params(q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv,
                           max_blocks, scale, v.esize, num_pool_blocks, P);
    if (P == 1) {
        p.out = out;
        return run_main(p, dtype, v.G, s);
    }
    const size_t need = pa_workspace_bytes(B, H, d, P);
    void *ws = workspace;
    if (ws) {
        if (workspace_bytes < need) return PA_ERR_WORKSPACE;
    } else if ((rc = library_workspace(dev, s, need, &ws)) != PA_OK) {
        return rc;
    }
    p.part_ml = static_cast<float2 *>(ws);
    p.part_acc = reinterpret_cast<float *>(static_cast<char *>(ws) + ml_region_bytes(B, H, P));
    if ((rc = run_main(p, dtype, v.G, s)) != PA_OK) return rc;
    return run_merge(out, ws, B, H, P, dtype, s);
}

int pa_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
              const int32_t *block_tables, const int32_t *context_lens, int B, int H, int Hkv,
              int d, int block_size, int max_blocks, float scale, int dtype, void *stream) {
    return pa_decode_ex(out, q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv, d,
                        block_size, max_blocks, scale, dtype, stream, 0, 0, nullptr, 0);
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
    const size_t need = ml_region_bytes(B, H, P) + (size_t)B * H * P * d * sizeof(float);
    if (workspace_bytes < need) return PA_ERR_WORKSPACE;
    Params p = make_params(q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv,
                           max_blocks, scale, v.esize, num_pool_blocks, P);
    p.part_ml = static_cast<float2 *>(workspace);
    p.part_acc =
        reinterpret_cast<float *>(static_cast<char *>(workspace) + ml_region_bytes(B, H, P));
    return run_main(p, dtype, v.G, static_cast<hipStream_t>(stream));
}

int pa_merge_partials(void *out, const void *workspace, size_t workspace_bytes, int B, int H,
                      int d, int num_partitions, int dtype, void *stream) {
    if (B < 0 || H <= 0 || d <= 0) return PA_ERR_SHAPE;
    if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16) return PA_ERR_DTYPE;
    if (d != kHeadDim) return PA_ERR_UNSUPPORTED;
    if (num_partitions < 1) return PA_ERR_VALUE;
    if (num_partitions > kMaxPartitions) return PA_ERR_UNSUPPORTED;
    if (B == 0) return PA_OK;
    if (!out) return PA_ERR_NULL;
    if (!workspace) return PA_ERR_WORKSPACE;
    if (!aligned(out, 16) || !aligned(workspace, 16)) return PA_ERR_ALIGN;
    const int P = num_partitions;
    const size_t need = ml_region_bytes(B, H, P) + (size_t)B * H * P * d * sizeof(float);
    if (workspace_bytes < need) return PA_ERR_WORKSPACE;
    const size_t esize = dtype == PA_DTYPE_BF16 ? 2 : 4;
    if (overlaps(out, (size_t)B * H * d * esize, workspace, need)) return PA_ERR_ALIAS;
    return run_merge(out, workspace, B, H, P, dtype, static_cast<hipStream_t>(stream));
}

void pa_release(void) {
    std::lock_guard<std::mutex> lock(g_mutex);
    int prev = -1;
    const bool have_prev = hipGetDevice(&prev) == hipSuccess;
    for (auto &kv : g_workspace) {
        if (!kv.second.first) continue;
        if (hipSetDevice(kv.first.first) == hipSuccess) {
            (void)hipDeviceSynchronize();
            (void)hipFree(kv.second.first);
        }
    }
    g_workspace.clear();
    if (have_prev) (void)hipSetDevice(prev);
}

}  // extern "C"
