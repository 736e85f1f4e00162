// pa_decode.hip -- paged-attention decode step for gfx950 (MI355X), C ABI.
//
// What is computed is declared in include/pa_decode.h.  This file holds the
// kernels and the host launcher behind that ABI.
//
// Design (one work unit = one (sequence b, kv head kvh) pair, optionally one
// partition of its context):
//
// * One workgroup per (kvh, b[, partition]) serves all G = H / Hkv query heads
//   of the group, so each K/V row is read from HBM once per kv head, not once
//   per query head.
// * A wave consumes one 16-token physical block per step.  Block ids are read
//   with scalar loads one group of blocks ahead, so they are wave-uniform and
//   each block gets a raw buffer descriptor (SGPRs) over exactly its live
//   rows of head kvh; the per-lane offsets never change.  Slots past the
//   context and -1 blocks fall outside the descriptor's range and read as
//   zeros without a memory access, so the streaming loop has no branches.
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
// * Epilogue: the 4 row groups of a wave are merged with permlane swaps, the
//   waves through LDS, always with the rescale-and-sum rule
//   (M = max m, L = sum l * 2^(m - M), O = sum acc * 2^(m - M)).  A single
//   pass writes O / L.  With partitions, each workgroup writes (M, L, O) to
//   the workspace; then either a separate merge kernel combines them, or (fused
//   mode) the last workgroup of each (b, kvh) to finish -- found with an atomic
//   ticket -- combines them with the same rule and writes out.
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
// The kernels walk a sequence in tiles of 16 tokens, the row count of one MFMA
// tile.  A physical block of block_size tokens (a power of two from 16 to 256)
// holds block_size / 16 tiles; each tile lies inside one block.
constexpr int kTile = 16;
constexpr int kMaxBlockSize = 256;
constexpr int kHeadDim = 128;     // d
constexpr float kLog2e = 1.44269504088896340736f;
// Start value of a running max: finite, so 2^(m - m') never sees inf - inf.
constexpr float kMaxInit = -1.0e30f;

#ifndef PA_WAVES_PER_GROUP
#define PA_WAVES_PER_GROUP 4
#endif
#ifndef PA_PIPELINE_DEPTH
#define PA_PIPELINE_DEPTH 2
#endif
constexpr int kWavesPerGroup = PA_WAVES_PER_GROUP;  // waves per workgroup
constexpr int kDepth = PA_PIPELINE_DEPTH;           // blocks in flight per wave
// Word 3 of a raw (untyped, stride 0) buffer descriptor on GFX9-family parts.
constexpr int kRsrcWord3 = 0x00020000;

// What a workgroup does with its merged (M, L, O).
enum Mode { kSingle = 0, kPartials = 1, kFused = 2 };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct Params {
    const char *q;
    const char *k;
    const char *v;
    const int32_t *table;
    const int32_t *lens;
    void *out;          // [B][H][d] dtype (single pass, fused merge)
    float2 *part_ml;    // [B][H][P] (max, sum)
    float *part_acc;    // [B][H][P][d]
    int *counters;      // [B][Hkv] arrival tickets (fused mode), zero between calls
    long long blk_bytes;  // bytes per physical block: block_size * Hkv * d * esize
    long long pool;       // > 0: ids >= pool are skipped
    int tok_bytes;        // bytes between tokens of a block: Hkv * d * esize
    int B, H, Hkv, max_blocks, P;
    int tiles_log2;       // log2(block_size / 16): tiles per physical block
    int max_tiles;        // max_blocks * block_size / 16
    int bpp;              // tiles per partition
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

// x combined over the 4 rows of 16 lanes (lanes l, l^16, l^32, l^48), result in
// every lane: a swap of the two 32-lane halves, then of neighbouring rows.
template <typename Op>
__device__ __forceinline__ float across_rows(float x, Op op) {
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float y = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const unsigned w = __float_as_uint(y);
    const auto c = __builtin_amdgcn_permlane16_swap(w, w, false, false);
    return op(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
    return across_rows(x, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ float rows_max(float x) {
    return across_rows(x, [](float a, float b) { return fmaxf(a, b); });
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16 bytes of a bf16 V row -> 8 fp32.
__device__ __forceinline__ void unpack_bf16(const u32x4 &w, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

template <int G>
struct WaveState {
    float m;           // running max (log2 units) of this lane's (row, head)
    float l;           // running normaliser
    float acc[G][8];   // unnormalised sum of p * V for every head of the group
};

// One block's scores, softmax update and V accumulation.  nlive = tokens of the
// block that take part (0..16); K/V slots at or past nlive were read as zeros
// (they lie outside the block's buffer range), so only their scores need
// masking.
template <int DT, int G>
__device__ __forceinline__ void consume_block(WaveState<G> &st, const u32x4 *kr, const u32x4 *vr,
                                              const u32x4 *qr, float qk_scale, int g, int nlive) {
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
    for (int r = 0; r < 4; ++r) s[r] = (4 * g + r < nlive) ? c[r] * qk_scale : -INFINITY;
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

template <int DT>
__device__ __forceinline__ void store_pair(void *out, long long idx, float x0, float x1) {
    if constexpr (DT == PA_DTYPE_BF16) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        bf16x2 v = {static_cast<__bf16>(x0), static_cast<__bf16>(x1)};
        *reinterpret_cast<bf16x2 *>(static_cast<__bf16 *>(out) + idx) = v;
    } else {
        *reinterpret_cast<float2 *>(static_cast<float *>(out) + idx) = make_float2(x0, x1);
    }
}

// Raw buffer descriptor over [base, base + nbytes): loads at offsets >= nbytes
// return zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const char *base, int nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), 0, nbytes, kRsrcWord3);
}

#ifndef PA_KV_CACHE_POLICY
#define PA_KV_CACHE_POLICY 2
#endif
// Cache-policy bits of the K/V stream loads (the buffer instruction's aux field):
// 2 = non-temporal, so the single-use stream does not evict the table, the
// query, the partials or the kernel code from the caches.
constexpr int kKvPolicy = PA_KV_CACHE_POLICY;

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kKvPolicy));
}

// Float pair access at agent scope.  The split kernel's fused merge exchanges
// partials between workgroups that may run on different XCDs (each with its own
// L2): these stores write through to the device-coherent level and these loads
// read from it, so no L2 writeback or invalidate is needed.
__device__ __forceinline__ void store_pair_coherent(float *p, float x0, float x1) {
    __hip_atomic_store(reinterpret_cast<unsigned long long *>(p),
                       __builtin_bit_cast(unsigned long long, make_float2(x0, x1)),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_pair_coherent(const float *p) {
    return __builtin_bit_cast(
        float2, __hip_atomic_load(reinterpret_cast<const unsigned long long *>(p),
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

template <bool COHERENT>
__device__ __forceinline__ float2 load_pair(const float *p) {
    if constexpr (COHERENT) return load_pair_coherent(p);
    else return *reinterpret_cast<const float2 *>(p);
}

// Combine the P partitions of (b, h) for head-dim elements e, e + 1 with the
// rescale-and-sum rule, running over the partitions in order.  ml points at
// the (max, sum) pairs of (b, h), acc at element e of its first partition.
// Returns the normalised pair (zeros when no partition saw a live token).
// All loads of a chunk of CHUNK partitions leave before the first is used.
// Reads past P are clamped to the last partition and replaced by an empty
// partition (max -1e30, sum 0, zeros), which leaves the running state as it is.
template <int CHUNK, bool COHERENT>
__device__ __forceinline__ float2 merge_chunked(const float2 *ml, const float *acc, int P) {
    float M = kMaxInit, L = 0.f, o0 = 0.f, o1 = 0.f;
    for (int q0 = 0; q0 < P; q0 += CHUNK) {
        float2 s[CHUNK], a[CHUNK];
#pragma unroll
        for (int j = 0; j < CHUNK; ++j) {
            const int q = q0 + j < P ? q0 + j : P - 1;
            s[j] = load_pair<COHERENT>(reinterpret_cast<const float *>(ml + q));
            a[j] = load_pair<COHERENT>(acc + (long long)q * kHeadDim);
        }
#pragma unroll
        for (int j = 0; j < CHUNK; ++j) {
            const bool live = q0 + j < P;
            s[j] = live ? s[j] : make_float2(kMaxInit, 0.f);
            a[j] = live ? a[j] : make_float2(0.f, 0.f);
            const float mn = fmaxf(M, s[j].x);
            const float fo = fast_exp2(M - mn), fp = fast_exp2(s[j].x - mn);
            L = L * fo + s[j].y * fp;
            o0 = o0 * fo + a[j].x * fp;
            o1 = o1 * fo + a[j].y * fp;
            M = mn;
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    return make_float2(o0 * inv, o1 * inv);
}

// The chunk is the smallest of 4, 8, 16, 32 that holds P (32 beyond that), so
// few partitions do not pay for loads of padding.
template <bool COHERENT>
__device__ __forceinline__ float2 merge_partitions(const float2 *ml, const float *acc, int P) {
    if (P <= 4) return merge_chunked<4, COHERENT>(ml, acc, P);
    if (P <= 8) return merge_chunked<8, COHERENT>(ml, acc, P);
    if (P <= 16) return merge_chunked<16, COHERENT>(ml, acc, P);
    return merge_chunked<32, COHERENT>(ml, acc, P);
}

template <int DT, int G, int NW, int D, int MODE>
__global__ __launch_bounds__(NW * kWave) void pa_decode_kernel(Params p) {
    using Geo = Geometry<DT>;
    constexpr int KL = Geo::kKLoads, VL = Geo::kVLoads, VPT = VL / 4;

    const int wg = blockIdx.x;
    const int kvh = wg % p.Hkv;
    const int b = (wg / p.Hkv) % p.B;
    const int part = wg / (p.Hkv * p.B);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform per wave
    const int lane = threadIdx.x % kWave;
    const int c16 = lane & 15;  // MFMA column / token of the block for K
    const int g = lane >> 4;    // MFMA row group: tokens 4g..4g+3 for V

    const int lo = part * p.bpp;
    const int first = lo + wave;  // this wave's tiles: first, first + NW, ...
    const int32_t *trow = p.table + (long long)b * p.max_blocks;
    // Table entry of the block holding the wave's i-th tile, the read clamped
    // into the row so it always stays in bounds (entries past the context are
    // read, never used).
    auto tile_of = [&](int i) -> int { return first + NW * i; };
    auto table_at = [&](int i) -> int {
        const int e = tile_of(i) >> p.tiles_log2;
        return trow[e < p.max_blocks ? e : p.max_blocks - 1];
    };

    // Independent loads first: the context length, the first group's table
    // entries and the query all leave before any of them is waited for.
    int ctx = p.lens[b];
    int raw0[D];
#pragma unroll
    for (int s = 0; s < D; ++s) raw0[s] = table_at(s);
    // B operand: the query of head kvh*G + c16%G, chunk (4m + g) of 16 bytes.
    const char *qrow = p.q + ((long long)b * p.H + kvh * G + (c16 % G)) * (kHeadDim * Geo::kEs);
    u32x4 qr[KL];
#pragma unroll
    for (int m = 0; m < KL; ++m) qr[m] = *reinterpret_cast<const u32x4 *>(qrow + 64 * m + 16 * g);

    ctx = ctx < 0 ? 0 : (ctx > p.max_tiles * kTile ? p.max_tiles * kTile : ctx);
    const int ntiles = (ctx + kTile - 1) / kTile;
    const int hi = min(lo + p.bpp, ntiles);
    const int nw = hi > first ? (hi - first + NW - 1) / NW : 0;

    // Per-lane byte offsets inside one block's rows of head kvh; never change.
    const unsigned koff = c16 * p.tok_bytes + 16 * g;
    unsigned voff[VL];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int s = 0; s < VPT; ++s)
            voff[r * VPT + s] = (4 * g + r) * p.tok_bytes + 16 * c16 + 256 * s;
    const char *kbase = p.k + kvh * kHeadDim * Geo::kEs;
    const char *vbase = p.v + kvh * kHeadDim * Geo::kEs;

    WaveState<G> st;
    st.m = kMaxInit;
    st.l = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) st.acc[h][e] = 0.f;

    // Live tokens of the wave's i-th tile given its block's table entry: 0 past
    // the wave's range and for -1 (or out-of-pool) entries.
    auto live_tokens = [&](int i, int id) -> int {
        const int j = tile_of(i);
        if (j >= hi || id < 0 || (p.pool > 0 && id >= p.pool)) return 0;
        const int rem = ctx - j * kTile;
        return rem < kTile ? rem : kTile;
    };
    // Loads of the wave's i-th tile: its rows start at the block's base plus
    // the tile's place inside the block.
    auto issue = [&](u32x4 *kd, u32x4 *vd, int i, int id, int nlive) {
        const int in_block = tile_of(i) & ((1 << p.tiles_log2) - 1);
        const long long off =
            nlive > 0 ? (long long)id * p.blk_bytes + (long long)in_block * kTile * p.tok_bytes : 0;
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kbase + off, nlive * p.tok_bytes);
        const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vbase + off, nlive * p.tok_bytes);
#pragma unroll
        for (int m = 0; m < KL; ++m) kd[m] = load16(rk, koff + 64 * m);
#pragma unroll
        for (int n = 0; n < VL; ++n) vd[n] = load16(rv, voff[n]);
    };

    if (nw > 0) {
        // D blocks in flight: slot s of group k holds the wave's block kD + s.
        u32x4 kr[D][KL], vr[D][VL];
        int nl[D];
#pragma unroll
        for (int s = 0; s < D; ++s) {
            nl[s] = live_tokens(s, raw0[s]);
            issue(kr[s], vr[s], s, raw0[s], nl[s]);
        }
        const int ngroups = (nw + D - 1) / D;
        for (int k = 0; k < ngroups; ++k) {
            int nid[D];
#pragma unroll
            for (int s = 0; s < D; ++s) nid[s] = table_at((k + 1) * D + s);
#pragma unroll
            for (int s = 0; s < D; ++s) {
                consume_block<DT, G>(st, kr[s], vr[s], qr, p.qk_scale, g, nl[s]);
                nl[s] = live_tokens((k + 1) * D + s, nid[s]);
                issue(kr[s], vr[s], (k + 1) * D + s, nid[s], nl[s]);
            }
        }
    }

    // ---- merge the 4 row groups of the wave -----------------------------------
    // The (m, l) of row g and head h sit in the lanes of row g whose column is
    // h modulo G; after the merge every row holds the same totals.
    float mh[G], lh[G];
    static_for<G>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        mh[h] = group_bcast<G, h>(st.m);
        lh[h] = group_bcast<G, h>(st.l);
    });
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float M = rows_max(mh[h]);
        const float f = fast_exp2(mh[h] - M);
        lh[h] = rows_sum(lh[h] * f);
#pragma unroll
        for (int e = 0; e < 8; ++e) st.acc[h][e] = rows_sum(st.acc[h][e] * f);
        mh[h] = M;
    }

    // ---- merge the waves through LDS ------------------------------------------
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

    // Thread t handles head h = idx / 64 and elements 2 (idx % 64) + {0, 1}.
    for (int idx = threadIdx.x; idx < G * (kHeadDim / 2); idx += NW * kWave) {
        const int h = idx / (kHeadDim / 2), e = 2 * (idx % (kHeadDim / 2));
        float M = kMaxInit;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_ml[w][h].x);
        float L = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = fast_exp2(sm_ml[w][h].x - M);
            L = fmaf(sm_ml[w][h].y, f, L);
            o0 = fmaf(sm_acc[w][h][e], f, o0);
            o1 = fmaf(sm_acc[w][h][e + 1], f, o1);
        }
        const long long bh = (long long)b * p.H + kvh * G + h;
        if constexpr (MODE == kSingle) {
            const float inv = L > 0.f ? 1.f / L : 0.f;
            store_pair<DT>(p.out, bh * kHeadDim + e, o0 * inv, o1 * inv);
        } else if constexpr (MODE == kPartials) {
            *reinterpret_cast<float2 *>(p.part_acc + (bh * p.P + part) * kHeadDim + e) =
                make_float2(o0, o1);
            if (e == 0) p.part_ml[bh * p.P + part] = make_float2(M, L);
        } else {
            store_pair_coherent(p.part_acc + (bh * p.P + part) * kHeadDim + e, o0, o1);
            if (e == 0)
                store_pair_coherent(reinterpret_cast<float *>(p.part_ml + bh * p.P + part), M, L);
        }
    }

    if constexpr (MODE == kFused) {
        // Publish this partition (its coherent stores complete before the
        // barrier), take a ticket; the last of the P workgroups of (b, kvh)
        // merges all partitions and resets the ticket for the next call.
        __shared__ int sm_last;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) {
            const int prev = __hip_atomic_fetch_add(p.counters + b * p.Hkv + kvh, 1,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sm_last = prev == p.P - 1;
        }
        __syncthreads();
        if (sm_last) {
            for (int idx = threadIdx.x; idx < G * (kHeadDim / 2); idx += NW * kWave) {
                const int h = idx / (kHeadDim / 2), e = 2 * (idx % (kHeadDim / 2));
                const long long bh = (long long)b * p.H + kvh * G + h;
                const float2 o = merge_partitions<true>(p.part_ml + bh * p.P,
                                                        p.part_acc + bh * p.P * kHeadDim + e, p.P);
                store_pair<DT>(p.out, bh * kHeadDim + e, o.x, o.y);
            }
            if (threadIdx.x == 0)
                __hip_atomic_store(p.counters + b * p.Hkv + kvh, 0, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

struct MergeParams {
    const float2 *part_ml;
    const float *part_acc;
    void *out;
    int B, H, P;
};

// One wave per (b, h); lane l produces elements 2l, 2l + 1.
template <int DT>
__global__ __launch_bounds__(kWave) void pa_merge_kernel(MergeParams mp) {
    const long long bh = blockIdx.x;
    const int e = 2 * threadIdx.x;
    const float2 o = merge_partitions<false>(mp.part_ml + bh * mp.P,
                                             mp.part_acc + bh * mp.P * kHeadDim + e, mp.P);
    store_pair<DT>(mp.out, bh * kHeadDim + e, o.x, o.y);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

constexpr int kMinTilesPerPartition = 8;  // 128 tokens
constexpr int kMaxPartitions = 4096;

size_t round256(size_t bytes) { return (bytes + 255) & ~(size_t)255; }

// Workspace layout: [B][H][P] float2 (max, sum) | [B][H][P][d] float partial
// sums, the second region starting on a 256-byte boundary.
struct Layout {
    size_t ml, acc, total;
};

Layout workspace_layout(int B, int H, int P) {
    Layout l;
    l.ml = 0;
    l.acc = round256((size_t)B * H * P * sizeof(float2));
    l.total = l.acc + (size_t)B * H * P * kHeadDim * sizeof(float);
    return l;
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
    if (d != kHeadDim || block_size < kTile || block_size > kMaxBlockSize ||
        (block_size & (block_size - 1)) != 0)
        return PA_ERR_UNSUPPORTED;
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

int library_buffers(int dev, hipStream_t stream, size_t partial_bytes, size_t num_tickets,
                    void **partials, int **tickets) {
    std::lock_guard<std::mutex> lock(g_mutex);
    LibBuffers &lb = g_buffers[{dev, stream}];
    if (lb.partial_bytes < partial_bytes || lb.num_tickets < num_tickets) {
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
        if (hipMemset(lb.tickets, 0, num_tickets * sizeof(int)) != hipSuccess) return PA_ERR_HIP;
        lb.num_tickets = num_tickets;
    }
    *partials = lb.partials;
    *tickets = lb.tickets;
    return PA_OK;
}

template <int DT, int G, int MODE>
hipError_t launch_main(const Params &p, int groups, hipStream_t stream) {
    hipLaunchKernelGGL((pa_decode_kernel<DT, G, kWavesPerGroup, kDepth, MODE>), dim3(groups),
                       dim3(kWavesPerGroup * kWave), 0, stream, p);
    return hipGetLastError();
}

template <int DT, int MODE>
hipError_t dispatch_g(const Params &p, int G, int groups, hipStream_t stream) {
    switch (G) {
        case 1: return launch_main<DT, 1, MODE>(p, groups, stream);
        case 2: return launch_main<DT, 2, MODE>(p, groups, stream);
        case 4: return launch_main<DT, 4, MODE>(p, groups, stream);
        case 8: return launch_main<DT, 8, MODE>(p, groups, stream);
        default: return launch_main<DT, 16, MODE>(p, groups, stream);
    }
}

template <int DT>
hipError_t dispatch_mode(const Params &p, int G, int mode, int groups, hipStream_t stream) {
    switch (mode) {
        case kSingle: return dispatch_g<DT, kSingle>(p, G, groups, stream);
        case kPartials: return dispatch_g<DT, kPartials>(p, G, groups, stream);
        default: return dispatch_g<DT, kFused>(p, G, groups, stream);
    }
}

int run_main(const Params &p, int dtype, int G, int mode, hipStream_t stream) {
    const long long groups = (long long)p.Hkv * p.B * p.P;
    if (groups > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;
    const hipError_t e = dtype == PA_DTYPE_BF16
                             ? dispatch_mode<PA_DTYPE_BF16>(p, G, mode, (int)groups, stream)
                             : dispatch_mode<PA_DTYPE_F32>(p, G, mode, (int)groups, stream);
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int run_merge(void *out, void *ws, int B, int H, int P, int dtype, hipStream_t stream) {
    const Layout l = workspace_layout(B, H, P);
    MergeParams mp;
    mp.part_ml = reinterpret_cast<const float2 *>(static_cast<char *>(ws) + l.ml);
    mp.part_acc = reinterpret_cast<const float *>(static_cast<char *>(ws) + l.acc);
    mp.out = out;
    mp.B = B;
    mp.H = H;
    mp.P = P;
    const long long groups = (long long)B * H;
    if (groups > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;
    if (dtype == PA_DTYPE_BF16)
        hipLaunchKernelGGL(pa_merge_kernel<PA_DTYPE_BF16>, dim3((int)groups), dim3(kWave), 0,
                           stream, mp);
    else
        hipLaunchKernelGGL(pa_merge_kernel<PA_DTYPE_F32>, dim3((int)groups), dim3(kWave), 0,
                           stream, mp);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
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
                   int Hkv, int max_blocks, int block_size, float scale, int esize,
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
    p.tok_bytes = Hkv * kHeadDim * esize;
    p.blk_bytes = (long long)block_size * p.tok_bytes;
    p.pool = pool;
    p.B = B;
    p.H = H;
    p.Hkv = Hkv;
    p.max_blocks = max_blocks;
    p.P = P;
    p.tiles_log2 = log2_int(block_size / kTile);
    p.max_tiles = table_tiles(max_blocks, block_size);
    p.bpp = (p.max_tiles + P - 1) / P;
    p.qk_scale = scale * kLog2e;
    return p;
}

void attach_workspace(Params &p, void *ws) {
    const Layout l = workspace_layout(p.B, p.H, p.P);
    char *base = static_cast<char *>(ws);
    p.part_ml = reinterpret_cast<float2 *>(base + l.ml);
    p.part_acc = reinterpret_cast<float *>(base + l.acc);
}

// P reduced so that no partition of a row of `tiles` tiles is empty.
int even_partitions(int tiles, int P) {
    if (P < 1) P = 1;
    if (P > tiles) P = tiles;
    const int per = (tiles + P - 1) / P;
    return (tiles + per - 1) / per;
}

}  // namespace

extern "C" {

int pa_choose_partitions(int B, int Hkv, int max_blocks, int block_size, int num_cus) {
    if (B <= 0 || Hkv <= 0 || max_blocks <= 0 || block_size < kTile || num_cus <= 0) return 1;
    const long long units = (long long)B * Hkv;
    if (units >= num_cus) return 1;
    const long long tiles = (long long)max_blocks * block_size / kTile;
    if (tiles > 0x7FFFFFFF) return 1;
    long long P = (num_cus + units - 1) / units;
    const long long cap = tiles / kMinTilesPerPartition;
    if (P > cap) P = cap;
    if (P > kMaxPartitions) P = kMaxPartitions;
    if (P < 1) P = 1;
    return even_partitions((int)tiles, (int)P);
}

size_t pa_workspace_bytes(int B, int H, int d, int num_partitions) {
    if (B <= 0 || H <= 0 || d <= 0 || num_partitions <= 1) return 0;
    return workspace_layout(B, H, num_partitions).total;
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
        P = even_partitions(table_tiles(max_blocks, block_size), num_partitions);
    }
    if (P > kMaxPartitions) return PA_ERR_UNSUPPORTED;
    Params p = make_params(q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv,
                           max_blocks, block_size, scale, v.esize, num_pool_blocks, P);
    p.out = out;
    if (P == 1) return run_main(p, dtype, v.G, kSingle, s);
    const size_t need = workspace_layout(B, H, P).total;
    if (workspace) {
        // caller workspace: split kernel, then the merge kernel (no tickets)
        if (workspace_bytes < need) return PA_ERR_WORKSPACE;
        attach_workspace(p, workspace);
        if ((rc = run_main(p, dtype, v.G, kPartials, s)) != PA_OK) return rc;
        return run_merge(out, workspace, B, H, P, dtype, s);
    }
    void *ws = nullptr;
    int *tickets = nullptr;
    if ((rc = library_buffers(dev, s, need, (size_t)B * Hkv, &ws, &tickets)) != PA_OK) return rc;
    attach_workspace(p, ws);
    p.counters = tickets;
    return run_main(p, dtype, v.G, kFused, s);
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
    if (workspace_bytes < workspace_layout(B, H, P).total) return PA_ERR_WORKSPACE;
    Params p = make_params(q, k_cache, v_cache, block_tables, context_lens, B, H, Hkv,
                           max_blocks, block_size, scale, v.esize, num_pool_blocks, P);
    attach_workspace(p, workspace);
    return run_main(p, dtype, v.G, kPartials, static_cast<hipStream_t>(stream));
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
    const size_t need = workspace_layout(B, H, P).total;
    if (workspace_bytes < need) return PA_ERR_WORKSPACE;
    const size_t esize = dtype == PA_DTYPE_BF16 ? 2 : 4;
    if (overlaps(out, (size_t)B * H * d * esize, workspace, need)) return PA_ERR_ALIAS;
    return run_merge(out, const_cast<void *>(workspace), B, H, P, dtype,
                     static_cast<hipStream_t>(stream));
}

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
