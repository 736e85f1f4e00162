// pa_kernels.h -- the decode and merge kernels for gfx950, as templates over
// the element type DT, head dim D and group size G, and the launchers that
// pick an instance.  Each pa_kernels_<dtype>.hip instantiates the launchers
// for one element type, so the three compile in parallel.
//
// Design (one work unit = one (sequence b, kv head kvh) pair, optionally one
// partition of its context):
//
// * One workgroup per (kvh, b[, partition]) serves all G = H / Hkv query heads
//   of the group, so each K/V row is read from HBM once per kv head, not once
//   per query head.  (A launch too small to fill the device gives each unit or
//   partition two workgroups, one per half of V's head dim; both read K, the
//   second mostly from the XCD's L2.)
// * A wave consumes 16-token tiles, two in flight at a time (one group); a
//   sequence's tiles are dealt in runs of 2 to the 4 * busy (partition, wave)
//   lanes in turn, busy being the partitions its length fills.  Block
//   ids are read with scalar loads one group of tiles ahead, so they are
//   wave-uniform and each tile gets a raw buffer descriptor (SGPRs) over
//   exactly its live rows of head kvh; the per-lane offsets never change.
//   Slots past the context and -1 blocks fall outside the descriptor's range
//   and read as zeros without a memory access, so the streaming loop has no
//   branches.
// * Scores: the 16 tokens x G heads x D product is a small dense contraction,
//   run on the matrix cores.  Each lane's 16-byte K load is its MFMA A
//   operand.  In the column layout the rows are the tile's 16 tokens, the
//   columns the G query heads repeated to 16, and the reduction the head dim,
//   so no cross-lane reduction is needed; lane (row g = lane/16, column
//   c = lane%16) ends with the scores of tokens 4g..4g+3 for head c % G.  In
//   the row layout (16-bit elements, D = 64 or 128, see k_rows_layout) each
//   MFMA takes whole rows of a few tokens, so K loads cover whole cache
//   lines; DPP adds sum the row parts, and for D = 128 lane (g, c) ends with
//   tokens g, g+4, g+8, g+12.
// * Online softmax per (row g, head): running max m and normaliser l in log2
//   units (scale * log2 e is folded into one multiply), so each lane updates
//   its own statistics from its 4 scores with no cross-lane max per tile.  The
//   max is a reference that moves only when a score exceeds it by more than 8
//   (log2 units, a wave-wide vote), so most tiles skip the rescale of the
//   state; when it moves it takes the head's max over the 4 rows, so it is
//   the same in every row.
// * V accumulate on the vector ALUs in fp32: lane (g, c) holds D / 16 elements
//   of the V rows of its 4 tokens and accumulates them for all G heads; the
//   weights of the other heads come from neighbouring lanes by DPP broadcast.
// * Epilogue: the 4 row groups of a wave are merged with permlane swaps (the
//   accumulators reduce-scattered, a quarter to each row), the waves through
//   LDS, always with the rescale-and-sum rule
//   (M = max m, L = sum l * 2^(m - M), O = sum acc * 2^(m - M)).  A single
//   pass writes O / L (in kSingleSplitV two workgroups per unit each do so for
//   one half of the head dim of V; kFusedSplitV and kPartialsSplitV split V
//   the same way in the fused split and the split kernel).  With partitions,
//   each workgroup writes (M, L, O) to the workspace; then either a separate
//   merge kernel combines them, or (fused mode) the last workgroups of each
//   (b, kvh) to finish -- found with an atomic ticket -- combine them with the
//   same rule and write out, each one slice of the head dim.
//
// Build-time settings (macros).  libpa_decode.so is built with the defaults;
// the other values exist only to measure the alternatives the defaults were
// chosen over: PA_WAVES_PER_GROUP (4), PA_PIPELINE_DEPTH (2 tiles in flight
// per wave), PA_K_ROWS (1 = the row K layout where k_rows_layout picks it,
// 0 = the column layout everywhere), PA_KV_CACHE_POLICY (2 = non-temporal
// K/V loads), PA_QK_VALU (0; 1 = the vector-ALU q.K of the ablation
// library libpa_decode_valu_qk.so, which is built and tested),
// PA_ORDERED_TICKET (0; 1 = the fused merge ordered by release / acquire, the
// ablation library libpa_decode_ordered.so, also built and tested), and two
// measuring aids that change no arithmetic: PA_TIMELINE (per-workgroup time
// stamps, libpa_decode_timeline.so) and PA_BREAKDOWN (a fused split stopped
// after its stream, its combine or its stores, libpa_decode_breakdown.so).
#ifndef PA_KERNELS_H
#define PA_KERNELS_H

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <utility>

#include "pa_internal.h"

namespace pa_detail {

constexpr float kLog2e = 1.44269504088896340736f;
// Start value of a running max: finite, so 2^(m - m') never sees inf - inf.
constexpr float kMaxInit = -1.0e30f;
// How far (log2 units) a score may exceed the running reference max before
// the state is rescaled: weights stay <= 2^8, so the fp32 sums cannot overflow
// (at most 2^8 per token, 2^30 tokens) and keep their relative precision.
constexpr float kRescaleSlack = 8.0f;

#ifndef PA_PIPELINE_DEPTH
#define PA_PIPELINE_DEPTH 2
#endif
constexpr int kDepth = PA_PIPELINE_DEPTH;           // tiles in flight per wave
// Word 3 of a raw (untyped, stride 0) buffer descriptor on GFX9-family parts.
constexpr int kRsrcWord3 = 0x00020000;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int DT> struct ElemBytes;
template <> struct ElemBytes<PA_DTYPE_F32> { static constexpr int value = 4; };
template <> struct ElemBytes<PA_DTYPE_BF16> { static constexpr int value = 2; };
template <> struct ElemBytes<PA_DTYPE_F16> { static constexpr int value = 2; };

// Load geometry of one 16-token tile for element type DT and head dim D.
// Lane (g = lane / 16, c16 = lane % 16), column layout (k_rows_layout below
// for the other):
//  * K: token c16's 16-byte chunks 4m + g, m < kKLoads -- exactly the MFMA A
//    operand of reduction step m (the query's B operand uses the same chunks);
//  * V: kVElems = D / 16 elements of each of tokens 4g..4g+3, read as kVLoads
//    loads of kVWidth bytes; load s of token r starts at byte
//    16 * kVWidth * s + kVWidth * c16 of the row, so the 16 lanes of a row
//    read each 16 * kVWidth-byte stretch of the row together.
template <int DT, int D>
struct Geometry {
    static constexpr int kEs = ElemBytes<DT>::value;
    static constexpr int kRowBytes = D * kEs;
    static constexpr int kKLoads = kRowBytes / 64;
    static constexpr int kVElems = D / 16;
    static constexpr int kVWidth = kVElems * kEs < 16 ? kVElems * kEs : 16;
    static constexpr int kVLoads = kVElems * kEs / kVWidth;
    static constexpr int kVWords = kVElems * kEs / 4;   // 32-bit words per token
    static constexpr int kElemsPerLoad = kVWidth / kEs;
    static_assert(kKLoads >= 1 && kRowBytes % 64 == 0, "head dim too small for the K layout");
    static_assert(kVWidth == 8 || kVWidth == 16, "V loads are 8 or 16 bytes");
};

#ifndef PA_K_ROWS
#define PA_K_ROWS 1
#endif
// Which K layout a kernel reads.  The column layout above hands each MFMA
// step 64 bytes of each of the tile's 16 rows, so every K load instruction
// touches 16 half cache lines.  The row layout instead cuts each row into
// Q = D * 2 / 64 parts of 64 bytes (16-bit elements) and gives MFMA step j
// the whole rows of T = 16 / Q tokens: A row Q t + a is part a of token
// T j + t, B column T b + hh is part b of the query of head hh % G.  A K load
// then covers whole cache lines like a V load, and the parts' partial dot
// products are summed across lanes afterwards.  A lane's useful products
// must fall in its own row of 16 lanes: 16-bit elements with D = 128 (Q = 4)
// or D = 64 (Q = 2).  When G exceeds the T heads one set of columns holds,
// each step runs G / T MFMAs, one per set of T heads (row_query_sets), and
// the extra MFMAs and selects cost more than the whole-line loads save except
// for D = 128, G = 8 in the bandwidth-bound modes (a single pass, or a batch
// covering the device): measured ~10 % faster there, ~0.5 us slower in a
// split of one long sequence, and slower for G = 16.
template <int DT, int D, int G, int MODE>
constexpr bool k_rows_layout() {
    if (!PA_K_ROWS || DT == PA_DTYPE_F32) return false;
    if (D == 64) return G <= 8;
    if (D == 128)
        return G <= 4 ||
               (G == 8 && (MODE == kSingle || MODE == kSingleSplitV || MODE == kFusedLate));
    return false;
}
// Query operand sets of the row layout: T = 16 / Q heads per set.
template <int D, int G>
constexpr int row_query_sets() {
    return G * (D / 32) <= 16 ? 1 : G * (D / 32) / 16;
}

// Token of slot r (0..3) of the lanes in MFMA row group g: the scores and V
// rows a lane holds for one tile.
template <int D, bool ROWS>
__device__ __forceinline__ int slot_token(int g, int r) {
    if constexpr (!ROWS) return 4 * g + r;
    else if constexpr (D == 128) return 4 * r + g;
    else return 8 * (r >> 1) + 2 * g + (r & 1);
}

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

// Word i of a row chunk -> its elements as fp32 (two for 16-bit types).
template <int DT>
__device__ __forceinline__ void unpack_word(unsigned w, float *f) {
    if constexpr (DT == PA_DTYPE_BF16) {
        f[0] = __uint_as_float(w << 16);
        f[1] = __uint_as_float(w & 0xFFFF0000u);
    } else if constexpr (DT == PA_DTYPE_F16) {
        const f16x2 h = __builtin_bit_cast(f16x2, w);
        f[0] = static_cast<float>(h[0]);
        f[1] = static_cast<float>(h[1]);
    } else {
        f[0] = __uint_as_float(w);
    }
}

template <int G, int VE>
struct WaveState {
    float m;            // running max (log2 units) of this lane's (row, head)
    float l;            // running normaliser
    float acc[G][VE];   // unnormalised sum of p * V for every head of the group
};

// One tile's scores (q.K for its 16 tokens and the G heads, on the matrix
// cores; softmax update and V accumulation follow in update_tile).  nlive =
// tokens of the tile that take part (0..16); K/V slots at or past nlive were
// read as zeros (they lie outside the tile's buffer range), so only their
// scores need masking.
template <int DT, int D>
__device__ __forceinline__ f32x4 tile_scores(const u32x4 *kr, const u32x4 *qr) {
    using Geo = Geometry<DT, D>;
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
    if constexpr (DT == PA_DTYPE_BF16) {
#pragma unroll
        for (int m = 0; m < Geo::kKLoads; ++m)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[m]),
                                                         __builtin_bit_cast(bf16x8, qr[m]), c,
                                                         0, 0, 0);
    } else if constexpr (DT == PA_DTYPE_F16) {
#pragma unroll
        for (int m = 0; m < Geo::kKLoads; ++m)
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, kr[m]),
                                                        __builtin_bit_cast(f16x8, qr[m]), c,
                                                        0, 0, 0);
    } else {
#pragma unroll
        for (int m = 0; m < Geo::kKLoads; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kr[m][j]),
                                                          __uint_as_float(qr[m][j]), c, 0, 0, 0);
    }
    return c;
}

// x plus its value in the lane N places along this lane's row of 16 (DPP
// row_ror:N, N = 4 or 8).
template <int N>
__device__ __forceinline__ float add_row_ror(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xF,
                                                          0xF, false));
}

template <int DT>
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    if constexpr (DT == PA_DTYPE_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), zero, 0, 0,
                                                       0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), zero, 0, 0, 0);
}

// Row-layout scores (k_rows_layout), slot r for token slot_token<D, true>(g, r),
// head c16 % G; `part` = c16 / T, the query part of this lane's column.  Step
// j's MFMA leaves in lane (g, c16), register i, the product of row 4g + i
// (part (4g + i) % Q of a token) with query part `part`; the registers whose
// parts match are that part's partial dot products, and the sum over the Q
// parts -- lanes T apart in the row of 16, reached by DPP rotations -- is the
// score.  Each sum adds the same pairs in every lane, so all Q lanes hold the
// same bits.
//  * D = 128 (Q = 4, T = 4): register `part` holds token 4j + g.
//  * D = 64 (Q = 2, T = 8): registers `part` and `part` + 2 hold tokens
//    8j + 2g and 8j + 2g + 1.
// With NS query sets (qr[set], heads set * T + c16 % T) every step runs NS
// MFMAs and the lane keeps the score of set `set` = its head's.
template <int DT, int D, int NS>
__device__ __forceinline__ f32x4 tile_scores_rows(const u32x4 *kr, const u32x4 *qr, int part,
                                                  int set) {
    f32x4 s;
    if constexpr (D == 128) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float y = 0.f;
#pragma unroll
            for (int n = 0; n < NS; ++n) {
                const f32x4 c = mfma_16x16x32<DT>(kr[j], qr[n]);
                const float x =
                    (part & 2) ? ((part & 1) ? c[3] : c[2]) : ((part & 1) ? c[1] : c[0]);
                const float z = add_row_ror<4>(add_row_ror<8>(x));
                y = NS == 1 || set == n ? z : y;
            }
            s[j] = y;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float y0 = 0.f, y1 = 0.f;
#pragma unroll
            for (int n = 0; n < NS; ++n) {
                const f32x4 c = mfma_16x16x32<DT>(kr[j], qr[n]);
                const float z0 = add_row_ror<8>(part ? c[1] : c[0]);
                const float z1 = add_row_ror<8>(part ? c[3] : c[2]);
                y0 = NS == 1 || set == n ? z0 : y0;
                y1 = NS == 1 || set == n ? z1 : y1;
            }
            s[2 * j] = y0;
            s[2 * j + 1] = y1;
        }
    }
    return s;
}

#ifndef PA_QK_VALU
#define PA_QK_VALU 0
#endif
// Build option for measuring the matrix cores' worth (0 in the library):
// with PA_QK_VALU=1 the row layout's q.K for 16-bit elements, D = 128 and
// G = 4 runs on the vector ALUs instead (tile_scores_rows_valu), everything
// else unchanged.
template <int DT, int D, int G, bool ROWS>
constexpr bool valu_scores() {
    return PA_QK_VALU && ROWS && DT != PA_DTYPE_F32 && D == 128 && G == 4;
}

// acc + the dot product of 8 16-bit elements (4 packed words) of k and q.
// (Each word is copied to a scalar before the bit cast: this compiler casts a
// vector element operand as if it were element 0.)
template <int DT>
__device__ __forceinline__ float dot8(u32x4 k, u32x4 q, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned kw = k[i], qw = q[i];
        if constexpr (DT == PA_DTYPE_BF16)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw),
                                                  __builtin_bit_cast(bf16x2, qw), acc, false);
        else
            acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, kw),
                                         __builtin_bit_cast(f16x2, qw), acc, false);
    }
    return acc;
}

// Row-layout scores (D = 128, G = 4) on the vector ALUs, in the layout
// tile_scores_rows returns: slot j of lane (g, c16) is the score of token
// 4j + g for head c16 % 4.  Load j gives lane (g, c16) elements
// [32 a + 8 g, + 8) of token 4j + t, a = c16 % 4, t = c16 / 4, and qh[h]
// holds the same elements of head h's query.  Each lane forms its 4 partial
// dot products (one per head); two rounds of half swaps (as in the epilogue)
// reduce-scatter them over the 4 row groups so that row g keeps head g, two
// DPP adds sum the 4 parts of the quad, and the lane fetches the score of
// token 4j + g for its head from row c16 % 4, quad g.
template <int DT>
__device__ __forceinline__ f32x4 tile_scores_rows_valu(const u32x4 *kr, const u32x4 *qh, int g,
                                                       int c16) {
    const int src = 4 * (16 * (c16 & 3) + 4 * g);  // byte address of the source lane
    f32x4 s;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float P[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) P[h] = dot8<DT>(kr[j], qh[h], 0.f);
        const auto r0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(P[0]),
                                                         __float_as_uint(P[2]), false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(P[1]),
                                                         __float_as_uint(P[3]), false, false);
        const float a0 = __uint_as_float(r0[0]) + __uint_as_float(r0[1]);
        const float a1 = __uint_as_float(r1[0]) + __uint_as_float(r1[1]);
        const auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a0), __float_as_uint(a1),
                                                         false, false);
        float x = __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF,
                                                        false));  // quad_perm [1,0,3,2]
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF,
                                                        false));  // quad_perm [2,3,0,1]
        s[j] = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(x)));
    }
    return s;
}

// The softmax update and V accumulation of one tile given its raw scores c
// (tile_scores or tile_scores_rows): slot r holds token slot_token<D, ROWS>(g,
// r), whose V row (or the DV-element slice of it this workgroup serves) vw[r]
// is.
template <int DT, int D, int G, bool ROWS, int DV = D>
__device__ __forceinline__ void update_tile(WaveState<G, DV / 16> &st, f32x4 c,
                                            const unsigned (*vw)[Geometry<DT, DV>::kVWords],
                                            float qk_scale, int g, int nlive) {
    using Geo = Geometry<DT, DV>;  // of the V slice (DV = D, or D / 2 when V is split)
    constexpr int VE = Geo::kVElems;
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        s[r] = (slot_token<D, ROWS>(g, r) < nlive) ? c[r] * qk_scale : -INFINITY;
    const float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    // The reference max m only moves (and l, acc are rescaled by 2^(m - m'))
    // when some lane of the wave sees a score more than kRescaleSlack above
    // its m; otherwise weights 2^(s - m) up to 2^kRescaleSlack are summed as
    // they are.  The result is the same -- every state (m, l, acc) stands for
    // acc / l whatever its m -- and the wave skips the rescale, and its wait
    // for this tile's max, on almost every tile.
    if (__builtin_amdgcn_ballot_w64(bm > st.m + kRescaleSlack) != 0) {
        // the new reference is the head's max over all 4 rows, so it stays the
        // same in every row and the epilogue merges the rows without rescaling
        const float mn = fmaxf(st.m, rows_max(bm));
        const float alpha = fast_exp2(st.m - mn);
        st.l *= alpha;
        st.m = mn;
        static_for<G>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            const float a = group_bcast<G, h>(alpha);
#pragma unroll
            for (int e = 0; e < VE; ++e) st.acc[h][e] *= a;
        });
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = fast_exp2(s[r] - st.m);
    st.l += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float vf[VE];
        constexpr int per_word = 4 / Geo::kEs;
#pragma unroll
        for (int i = 0; i < Geo::kVWords; ++i) unpack_word<DT>(vw[r][i], vf + per_word * i);
        static_for<G>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            const float ph = group_bcast<G, h>(p[r]);
#pragma unroll
            for (int e = 0; e < VE; ++e) st.acc[h][e] = fmaf(ph, vf[e], st.acc[h][e]);
        });
    }
}

// Head-dim element held in accumulator slot e by the lane in column c16.
template <int DT, int D>
__device__ __forceinline__ int acc_elem(int c16, int e) {
    constexpr int epl = Geometry<DT, D>::kElemsPerLoad;
    return (e / epl) * 16 * epl + epl * c16 + e % epl;
}

template <int DT>
__device__ __forceinline__ void store_pair(void *out, long long idx, float x0, float x1) {
    if constexpr (DT == PA_DTYPE_BF16) {
        const bf16x2 v = {static_cast<__bf16>(x0), static_cast<__bf16>(x1)};
        *reinterpret_cast<bf16x2 *>(static_cast<__bf16 *>(out) + idx) = v;
    } else if constexpr (DT == PA_DTYPE_F16) {
        const f16x2 v = {static_cast<_Float16>(x0), static_cast<_Float16>(x1)};
        *reinterpret_cast<f16x2 *>(static_cast<_Float16 *>(out) + idx) = v;
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

// BYTES (8 or 16) bytes at `off` into dst[0 .. BYTES / 4).
template <int BYTES>
__device__ __forceinline__ void load_words(__amdgpu_buffer_rsrc_t r, unsigned off, unsigned *dst) {
    if constexpr (BYTES == 16) {
        const u32x4 x = load16(r, off);
        dst[0] = x[0]; dst[1] = x[1]; dst[2] = x[2]; dst[3] = x[3];
    } else {
        const u32x2 x = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kKvPolicy));
        dst[0] = x[0]; dst[1] = x[1];
    }
}

// Float pair store at agent scope.  The split kernel's fused merge exchanges
// partials between workgroups that may run on different XCDs (each with its own
// L2): these stores write through to the device-coherent level and the merge
// reads from it (kCoherent loads), so no L2 writeback or invalidate is needed.
__device__ __forceinline__ void store_pair_coherent(float *p, float x0, float x1) {
    __hip_atomic_store(reinterpret_cast<unsigned long long *>(p),
                       __builtin_bit_cast(unsigned long long, make_float2(x0, x1)),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Combine the P partitions of (b, h) for head-dim elements e, e + 1 with the
// rescale-and-sum rule, running over the partitions in order.  ml points at
// the (max, sum) pairs of (b, h), acc at element e of its first partition;
// partitions are d floats apart.  Returns the normalised pair (zeros when no
// partition saw a live token).  All loads of a chunk of CHUNK partitions leave
// before the first is used.  Reads past P are clamped to the last partition
// and replaced by an empty partition (max -1e30, sum 0, zeros), which leaves
// the running state as it is.
template <int CHUNK>
__device__ __forceinline__ float2 merge_chunked(const float2 *ml, const float *acc, int P, int d) {
    float M = kMaxInit, L = 0.f, o0 = 0.f, o1 = 0.f;
    for (int q0 = 0; q0 < P; q0 += CHUNK) {
        float2 s[CHUNK], a[CHUNK];
#pragma unroll
        for (int j = 0; j < CHUNK; ++j) {
            const int q = q0 + j < P ? q0 + j : P - 1;
            s[j] = ml[q];
            a[j] = *reinterpret_cast<const float2 *>(acc + (long long)q * d);
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
__device__ __forceinline__ float2 merge_partitions(const float2 *ml, const float *acc, int P,
                                                   int d) {
    if (P <= 4) return merge_chunked<4>(ml, acc, P, d);
    if (P <= 8) return merge_chunked<8>(ml, acc, P, d);
    if (P <= 16) return merge_chunked<16>(ml, acc, P, d);
    return merge_chunked<32>(ml, acc, P, d);
}

#ifndef PA_TIMELINE
#define PA_TIMELINE 0
#endif
// Whether the kernel writes per-workgroup time stamps (s_memrealtime, 100 MHz)
// to p.timeline: 0 in the library, 1 in the timeline library
// libpa_decode_timeline.so (layout in include/pa_timeline.h).
constexpr bool kTimeline = PA_TIMELINE != 0;
__device__ __forceinline__ unsigned long long stamp_now() {
    return __builtin_amdgcn_s_memrealtime();
}

#ifndef PA_BREAKDOWN
#define PA_BREAKDOWN 0
#endif
// Whether a fused split may stop early for timing (p.stop_after): 0 in the
// library, 1 in the breakdown library libpa_decode_breakdown.so, whose early
// stops write no output (include/pa_breakdown.h).
constexpr bool kBreakdown = PA_BREAKDOWN != 0;

#ifndef PA_ORDERED_TICKET
#define PA_ORDERED_TICKET 0
#endif
// Whether the fused merge's ticket carries release / acquire ordering (see
// the kernel's epilogue): 0 in the library, 1 in the ablation library
// libpa_decode_ordered.so.
constexpr bool kOrderedTicket = PA_ORDERED_TICKET != 0;

// Cache-policy bits (sc1) that make a buffer access agent-coherent: loads
// read past this XCD's L2, which may hold stale copies of lines other XCDs
// have rewritten since.
constexpr int kCoherent = 16;

// The fused merge of the `busy` partitions of (b, kvh), or of one of WAYS
// slices of its head dim (columns [slice * D / WAYS, (slice + 1) * D / WAYS)),
// by one workgroup.  Each (head, 4-element quad) of the slice is shared by S
// threads; thread `split` folds partitions split, split + S, ... (all of a
// chunk's loads in flight at once), then the S partial states are folded
// together with an xor butterfly, all with the rescale-and-sum rule.  S is
// chosen so that the items fill the workgroup, which keeps each thread's
// loads few enough to leave in one round trip; CH (the chunk) is the smallest
// power of two up to 16 that holds a thread's share, so few partitions load
// no padding.  Every element's fold order is fixed, so the output bits do not
// depend on which workgroups merge.  If `poisoned`, the slice is written as
// NaN instead (a merger that stopped waiting).
template <int DT, int D, int G, int NW, int WAYS = 1>
constexpr int merge_split() {
    constexpr int kThreads = NW * kWave, kItems = G * D / (4 * WAYS);
    // (at most a wave: with few items the waves past kItems * S have none)
    return kItems >= kThreads ? 1 : (kThreads / kItems > kWave ? kWave : kThreads / kItems);
}

template <int DT, int D, int G, int NW, int CH, int WAYS>
__device__ __forceinline__ void merge_group_chunked(const Params &p, int b, int kvh, int busy,
                                                    int slice, bool poisoned) {
    constexpr int kThreads = NW * kWave;
    constexpr int kQuads = D / (4 * WAYS);
    constexpr int kItems = G * kQuads;
    constexpr int S = merge_split<DT, D, G, NW, WAYS>();
    static_assert(S <= kWave, "the butterfly stays inside a wave");
    static_assert(kItems >= 1, "a slice holds at least one quad of the head dim");
    static_assert(kItems % kThreads == 0 || (kItems * S) % kWave == 0,
                  "every thread of a wave with items takes part in the butterfly");
    const long long bh0 = (long long)b * p.H + kvh * G;
    const __amdgpu_buffer_rsrc_t rml =
        buffer_rsrc(reinterpret_cast<const char *>(p.part_ml + bh0 * p.P), G * p.P * 8);
    const __amdgpu_buffer_rsrc_t racc =
        buffer_rsrc(reinterpret_cast<const char *>(p.part_acc + bh0 * p.P * D), G * p.P * D * 4);
    for (int t = threadIdx.x; t < kItems * S; t += kThreads) {
        const int item = t / S, split = t % S;
        const int h = item / kQuads, quad = slice * kQuads + item % kQuads;
        float M = kMaxInit, L = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
        for (int q0 = split; q0 < busy; q0 += S * CH) {
            float2 sm[CH];
            f32x4 ac[CH];
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int q = q0 + S * j < busy ? q0 + S * j : q0;  // clamped into range
                sm[j] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(
                                                       rml, (h * p.P + q) * 8, 0, kCoherent));
                ac[j] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               racc, ((h * p.P + q) * D + 4 * quad) * 4, 0, kCoherent));
            }
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const bool live = q0 + S * j < busy;
                const float mj = live ? sm[j].x : kMaxInit;
                const float mn = fmaxf(M, mj);
                const float fo = fast_exp2(M - mn);
                const float fp = live ? fast_exp2(mj - mn) : 0.f;
                L = L * fo + sm[j].y * fp;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = o[e] * fo + ac[j][e] * fp;
                M = mn;
            }
        }
#pragma unroll
        for (int off = 1; off < S; off <<= 1) {
            const float M2 = __shfl_xor(M, off), L2 = __shfl_xor(L, off);
            const float mn = fmaxf(M, M2);
            const float f1 = fast_exp2(M - mn), f2 = fast_exp2(M2 - mn);
            L = L * f1 + L2 * f2;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = o[e] * f1 + __shfl_xor(o[e], off) * f2;
            M = mn;
        }
        if (split == 0) {
            const float inv = poisoned ? __builtin_nanf("") : (L > 0.f ? 1.f / L : 0.f);
            const long long at = (bh0 + h) * D + 4 * quad;
            store_pair<DT>(p.out, at, o[0] * inv, o[1] * inv);
            store_pair<DT>(p.out, at + 2, o[2] * inv, o[3] * inv);
        }
    }
}

template <int DT, int D, int G, int NW, int WAYS>
__device__ __forceinline__ void merge_group_ways(const Params &p, int b, int kvh, int busy,
                                                 int slice, bool poisoned) {
    constexpr int S = merge_split<DT, D, G, NW, WAYS>();
    const int share = (busy + S - 1) / S;  // partitions per thread
    if constexpr (WAYS >= 4) {
        // (a wide merge's threads share few partitions each: chunks of up to 4,
        // looped over for more, keep the code the kernel carries small -- each
        // XCD fetches its own copy of it every launch)
        if (share <= 1) merge_group_chunked<DT, D, G, NW, 1, WAYS>(p, b, kvh, busy, slice, poisoned);
        else if (share <= 2) merge_group_chunked<DT, D, G, NW, 2, WAYS>(p, b, kvh, busy, slice, poisoned);
        else merge_group_chunked<DT, D, G, NW, 4, WAYS>(p, b, kvh, busy, slice, poisoned);
        return;
    }
    if (share <= 1) merge_group_chunked<DT, D, G, NW, 1, WAYS>(p, b, kvh, busy, slice, poisoned);
    else if (share <= 2) merge_group_chunked<DT, D, G, NW, 2, WAYS>(p, b, kvh, busy, slice, poisoned);
    else if (share <= 4) merge_group_chunked<DT, D, G, NW, 4, WAYS>(p, b, kvh, busy, slice, poisoned);
    else if (share <= 8) merge_group_chunked<DT, D, G, NW, 8, WAYS>(p, b, kvh, busy, slice, poisoned);
    else merge_group_chunked<DT, D, G, NW, 16, WAYS>(p, b, kvh, busy, slice, poisoned);
}

template <int DT, int D, int G, int NW>
__device__ __forceinline__ void merge_group(const Params &p, int b, int kvh, int busy, int ways,
                                            int slice, bool poisoned) {
    if (ways == 16) merge_group_ways<DT, D, G, NW, 16>(p, b, kvh, busy, slice, poisoned);
    else if (ways == 8) merge_group_ways<DT, D, G, NW, 8>(p, b, kvh, busy, slice, poisoned);
    else if (ways == 4) merge_group_ways<DT, D, G, NW, 4>(p, b, kvh, busy, slice, poisoned);
    else if (ways == 2) merge_group_ways<DT, D, G, NW, 2>(p, b, kvh, busy, slice, poisoned);
    else merge_group_ways<DT, D, G, NW, 1>(p, b, kvh, busy, 0, poisoned);
}

template <int DT, int D, int G, int NW, int DEPTH, int MODE>
__global__ __launch_bounds__(NW * kWave) void pa_decode_kernel(Params p) {
    using Geo = Geometry<DT, D>;
    // V slices per row (the V-split modes: this workgroup serves elements
    // [vslice * DV, (vslice + 1) * DV) of V, of the output and of the partials)
    constexpr int VS = v_slices(MODE);
    constexpr int DV = D / VS;
    static_assert(VS == 1 || split_v_built(D), "V split needs a head dim of 128 or more");
    using GeoV = Geometry<DT, DV>;
    constexpr int KL = Geo::kKLoads, VE = GeoV::kVElems, VW = GeoV::kVWords;
    constexpr int VLD = GeoV::kVLoads, VWIDTH = GeoV::kVWidth;
    constexpr bool kSinglePass = MODE == kSingle || MODE == kSingleSplitV;
    constexpr bool kFusedMerge = MODE == kFused || MODE == kFusedLate || MODE == kFusedSplitV;
    constexpr bool kRows = k_rows_layout<DT, D, G, MODE>();
    constexpr int kRowsQ = KL, kRowsT = 16 / KL;  // row layout: parts per row, tokens per step
    constexpr int kSets = row_query_sets<D, G>();   // row layout: query sets of kRowsT heads
    constexpr bool kValu = valu_scores<DT, D, G, kRows>();
    constexpr int QL = kValu ? G : (kRows ? kSets : KL);  // query registers (16 bytes each)

    // Grid (Hkv, sequences of this launch, P), or z = 2 part + vslice in the
    // V-split modes: kv head fastest in dispatch order.
    const int kvh = blockIdx.x;
    const int b = p.b0 + blockIdx.y;
    const int part = VS > 1 ? (int)(blockIdx.z >> 1) : (int)blockIdx.z;
    const int vslice = VS > 1 ? (int)(blockIdx.z & 1) : 0;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform per wave
    const int lane = threadIdx.x % kWave;
    const int c16 = lane & 15;  // MFMA column / token of the tile for K
    const int g = lane >> 4;    // MFMA row group (its tokens: 4g..4g+3, or g + 4r)
    unsigned long long *tl = nullptr;  // this workgroup's stamps (timeline build)
    if constexpr (kTimeline) {
        const unsigned lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
        if (p.timeline && lin < p.timeline_cap) tl = p.timeline + (size_t)kTimelineSlots * lin;
        if (tl && threadIdx.x == 0) {
            tl[0] = stamp_now();
            for (int i = 1; i < kTimelineSlots; ++i) tl[i] = 0;
            tl[10] = __builtin_amdgcn_s_getreg(20 | (3 << 11));   // HW_REG_XCC_ID [3:0]
            tl[11] = __builtin_amdgcn_s_getreg(4 | (31 << 11));   // HW_REG_HW_ID
        }
    }

    // Tiles are dealt in runs of DEPTH consecutive tiles (one group) to the
    // busy * NW (partition, wave) lanes in turn: lane L = part * NW + wave
    // takes runs L, L + busy * NW, ...  `busy`, the partitions a sequence
    // uses, follows its length -- ceil(n / 2^part_tiles_log2) of them, at most
    // P, or one if n <= solo_tiles -- but a lane's first run does not depend
    // on it, so its first table entries are fetched before the length has
    // arrived.
    const int first = DEPTH * (part * NW + wave);  // first tile of the lane's first run
    const int32_t *trow = p.table + (long long)b * p.max_blocks;
    // Table entry of the block holding tile j, the read clamped into the row so
    // it always stays in bounds (entries past the context are read, never used).
    auto table_at = [&](int j) -> int {
        const int e = j >> p.tiles_log2;
        return trow[e < p.max_blocks ? e : p.max_blocks - 1];
    };

    // Tiles of a context length (clamped to the table row), and the
    // partitions a sequence of nt tiles asks for (capped at P below).
    auto tiles_of = [&](int len) -> int {
        const int c = len < 0 ? 0 : (len > p.max_tiles * kTile ? p.max_tiles * kTile : len);
        return (int)(((unsigned)c + kTile - 1) / kTile);
    };
    auto partitions_for = [&](int nt) -> int {
        return nt > p.solo_tiles ? (nt + (1 << p.part_tiles_log2) - 1) >> p.part_tiles_log2
                                 : (nt > 0 ? 1 : 0);
    };

    // Independent loads first: the context length, the first group's table
    // entries and the query all leave before any of them is waited for.
    int ctx = p.lens[b];
    if constexpr (MODE == kFusedLate) {
        // With the units covering the device most partitions past the first
        // are empty: those leave on the length alone, before any table load.
        if (part > 0 && part >= partitions_for(tiles_of(ctx))) return;
    }
    int raw0[DEPTH];
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) raw0[s] = table_at(first + s);
    // B operand: the query of head kvh*G + c16%G, chunk (4m + g) of 16 bytes.
    // Loaded here, with the length and table entries, except in kFusedLate
    // (after the empty partitions have left; loads complete in order, so a
    // query issued behind the first tiles delays their update a little).
    const char *qrow = p.q + ((long long)b * p.H + kvh * G + (c16 % G)) * Geo::kRowBytes;
    // (row layout: chunk g of part c16 / T of the row of head
    // (set * T + c16 % T) % G, T = 16 / Q tokens per MFMA step)
    const char *qgroup = p.q + ((long long)b * p.H + kvh * G) * Geo::kRowBytes;
    u32x4 qr[QL];
    auto load_query = [&]() {
#pragma unroll
        for (int m = 0; m < QL; ++m)
            qr[m] = *reinterpret_cast<const u32x4 *>(
                kValu   ? qgroup + m * Geo::kRowBytes + 64 * (c16 % kRowsQ) + 16 * g
                : kRows ? qgroup + ((m * kRowsT + c16 % kRowsT) % G) * Geo::kRowBytes +
                              64 * (c16 / kRowsT) + 16 * g
                        : qrow + 64 * m + 16 * g);
    };
    if constexpr (MODE != kFusedLate) load_query();

    const int ntiles = tiles_of(ctx);
    ctx = ctx < 0 ? 0 : (ctx > p.max_tiles * kTile ? p.max_tiles * kTile : ctx);
    // Partitions holding tiles (the first `busy`); the fused merge waits for
    // exactly these.
    const int want = partitions_for(ntiles);
    const int busy = want < p.P ? want : p.P;
    const bool idle = part >= busy;             // owns no tile
    const int stride = busy * NW * DEPTH;       // tiles between a lane's runs
    // One busy partition (or none) writes the output itself, as a single pass;
    // in the fused mode a partition without tiles adds nothing to the merge
    // and writes nothing (partition 0 of an empty sequence writes zeros).
    const bool direct = kSinglePass || (kFusedMerge && busy <= 1);
    const bool silent = kFusedMerge && part >= max(busy, 1);

    // Per-lane byte offsets inside one tile's rows of head kvh; never change.
    // Column layout: K chunk 4m + g of token c16.  Row layout: K part
    // c16 % Q (chunk g of it) of token T m + c16 / Q.  V rows of the slots'
    // tokens (slot_token).
    unsigned koff[kRows ? KL : 1];
    if constexpr (kRows) {
#pragma unroll
        for (int m = 0; m < KL; ++m)
            koff[m] = (kRowsT * m + c16 / kRowsQ) * p.tok_bytes + 64 * (c16 % kRowsQ) + 16 * g;
    } else {
        koff[0] = c16 * p.tok_bytes + 16 * g;
    }
    unsigned voff[4][VLD];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int s = 0; s < VLD; ++s)
            voff[r][s] = slot_token<D, kRows>(g, r) * p.tok_bytes + VWIDTH * c16 +
                         16 * VWIDTH * s;
    const char *kbase = p.k + kvh * Geo::kRowBytes;
    const char *vbase = p.v + kvh * Geo::kRowBytes + vslice * GeoV::kRowBytes;

    WaveState<G, VE> st;
    st.m = kMaxInit;
    st.l = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < VE; ++e) st.acc[h][e] = 0.f;

    // Live tokens of tile j given its block's table entry: 0 past the context,
    // for -1 (or out-of-pool) entries and in an idle partition.  (Negative ids
    // compare above any pool limit as unsigned.)
    auto live_tokens = [&](int j, int id) -> int {
        const int rem = ctx - j * kTile;
        const int n = rem < kTile ? rem : kTile;
        return (!idle && j < ntiles && (unsigned)id < p.pool_limit) ? n : 0;
    };
    // Loads of tile j: its rows start at the block's base plus the tile's place
    // inside the block.
    auto issue = [&](u32x4 *kd, unsigned (*vd)[VW], int j, int id, int nlive) {
        const int in_block = j & ((1 << p.tiles_log2) - 1);
        const long long off =
            nlive > 0 ? (long long)id * p.blk_bytes + (long long)in_block * kTile * p.tok_bytes : 0;
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kbase + off, nlive * p.tok_bytes);
        const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vbase + off, nlive * p.tok_bytes);
#pragma unroll
        for (int m = 0; m < KL; ++m) kd[m] = load16(rk, kRows ? koff[m] : koff[0] + 64 * m);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int s = 0; s < VLD; ++s)
                load_words<VWIDTH>(rv, voff[r][s], vd[r] + s * (VWIDTH / 4));
    };

    // DEPTH tiles in flight: slot s of group k holds tile first + stride * k + s.
    // The first group is issued even by a lane with no tile: its descriptors
    // are empty, so the loads return zeros without a memory access.  Issuing
    // it before any exit keeps the table loads' uses unconditional, so the
    // compiler issues them together with the context-length load.
    u32x4 kr[DEPTH][KL];
    unsigned vr[DEPTH][4][VW];
    int nl[DEPTH];
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) {
        nl[s] = live_tokens(first + s, raw0[s]);
        issue(kr[s], vr[s], first + s, raw0[s], nl[s]);
    }
    if constexpr (kFusedMerge) {
        if (silent) return;  // nothing in flight touches memory
    }
    if constexpr (MODE == kFusedLate) load_query();
    // Group k is updated while group k + 1 streams in.  The last group is
    // peeled off the loop: issuing loads after it (empty, but still a trip
    // through the load pipeline that the epilogue's use of their registers
    // would wait for) measured 0.05-0.2 us slower on workloads 1-5, and a
    // branch around that issue inside the loop slower still.
    auto update_slot = [&](int s) {
        if constexpr (kValu)
            update_tile<DT, D, G, true, DV>(st, tile_scores_rows_valu<DT>(kr[s], qr, g, c16),
                                        vr[s], p.qk_scale, g, nl[s]);
        else if constexpr (kRows)
            update_tile<DT, D, G, true, DV>(st,
                                        tile_scores_rows<DT, D, kSets>(
                                            kr[s], qr, c16 / kRowsT, (c16 % G) / kRowsT),
                                        vr[s], p.qk_scale, g, nl[s]);
        else
            update_tile<DT, D, G, false, DV>(st, tile_scores<DT, D>(kr[s], qr), vr[s],
                                         p.qk_scale, g, nl[s]);
    };
    int k = 0;
    while (!idle && first + stride * (k + 1) < ntiles) {  // group k + 1 holds a live tile
        const int nbase = first + stride * (k + 1);  // the next group's first tile
        int nid[DEPTH];
#pragma unroll
        for (int s = 0; s < DEPTH; ++s) nid[s] = table_at(nbase + s);
        // (each tile's scores right before its update: computing the group's
        // scores first makes the first update wait for the later tiles' K
        // rows as well, since loads complete in order, and measures slower)
#pragma unroll
        for (int s = 0; s < DEPTH; ++s) {
            update_slot(s);
            nl[s] = live_tokens(nbase + s, nid[s]);
            // (a slot of the group past the context is issued too, with an
            // empty range: a branch here measures slower than the loads it
            // would save)
            issue(kr[s], vr[s], nbase + s, nid[s], nl[s]);
        }
        ++k;
    }
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) update_slot(s);  // the last group
    if constexpr (kBreakdown && kFusedMerge) {
        if (p.stop_after == 1) {
            // stop after the stream: the state is kept live (every load and
            // update is needed for it) and nothing is written
            float x = st.l + st.m;
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < VE; ++e) x += st.acc[h][e];
            asm volatile("; stream state %0" ::"v"(x));
            return;
        }
    }
    if constexpr (kTimeline) {
        if (tl && lane == 0 && wave < 4) tl[1 + wave] = stamp_now();
    }

    // ---- merge the 4 row groups of the wave -----------------------------------
    // The (m, l) of row g and head h sit in the lanes of row g whose column is
    // h modulo G.  A head's reference max is the same in the 4 rows
    // (update_tile), so the normalisers are summed over the rows in every lane
    // and the N = G * VE accumulators of a lane are reduce-scattered as they
    // are: row g ends with the totals of values [g N/4, (g + 1) N/4), value i
    // standing for head i / VE, slot i % VE.
    float mh[G], lh[G];
    static_for<G>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        mh[h] = group_bcast<G, h>(st.m);
        lh[h] = rows_sum(group_bcast<G, h>(st.l));
    });
    constexpr int N = G * VE, N2 = N / 2, N4 = N / 4;
    // A swap of (x, y) hands the upper 32 lanes' x to the lower lanes' y and
    // the lower lanes' y to the upper lanes' x (likewise odd and even rows for
    // the 16-lane swap).  So after swap(a, z) the lower lanes hold (own a,
    // upper a) and the upper lanes (lower z, own z): the sum of the pair is
    // the lower half's total of a and the upper half's of z, with no select.
    float half[N2];
#pragma unroll
    for (int j = 0; j < N2; ++j) {
        const float a = st.acc[j / VE][j % VE];
        const float z = st.acc[(N2 + j) / VE][(N2 + j) % VE];
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(z),
                                                        false, false);
        half[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    float quarter[N4];
#pragma unroll
    for (int j = 0; j < N4; ++j) {
        const auto r = __builtin_amdgcn_permlane16_swap(
            __float_as_uint(half[j]), __float_as_uint(half[N4 + j]), false, false);
        quarter[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }

    if constexpr (kTimeline) {
        if (tl && threadIdx.x == 0) tl[13] = stamp_now();  // wave 0's rows merged
    }

    // ---- merge the waves through LDS ------------------------------------------
    __shared__ float2 sm_ml[NW][G];
    __shared__ float sm_acc[NW][G][DV];
#pragma unroll
    for (int j = 0; j < N4; ++j) {
        const int i = g * N4 + j;
        sm_acc[wave][i / VE][acc_elem<DT, DV>(c16, i % VE)] = quarter[j];
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) sm_ml[wave][h] = make_float2(mh[h], lh[h]);
    }
    __syncthreads();
    if constexpr (kTimeline) {
        if (tl && threadIdx.x == 0) tl[14] = stamp_now();  // every wave in LDS
    }

    // Thread t handles head h = idx / (DV / 2) and elements 2 (idx % (DV / 2)) + {0, 1}
    // of this workgroup's slice.
    for (int idx = threadIdx.x; idx < G * (DV / 2); idx += NW * kWave) {
        const int h = idx / (DV / 2), e = 2 * (idx % (DV / 2));
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
        if (silent) {
            // nothing to write
        } else if (direct) {
            const float inv = L > 0.f ? 1.f / L : 0.f;
            store_pair<DT>(p.out, bh * D + vslice * DV + e, o0 * inv, o1 * inv);
        } else if constexpr (MODE == kPartials || MODE == kPartialsSplitV) {
            // (with V split, each slice stores its half; slice 0 the (max, sum))
            *reinterpret_cast<float2 *>(p.part_acc + (bh * p.P + part) * D + vslice * DV + e) =
                make_float2(o0, o1);
            if (e == 0 && vslice == 0) p.part_ml[bh * p.P + part] = make_float2(M, L);
        } else {
            if constexpr (kBreakdown) {
                if (p.stop_after == 2) {  // combined, kept live, not stored
                    asm volatile("; combined %0 %1 %2 %3" ::"v"(o0), "v"(o1), "v"(M), "v"(L));
                    continue;
                }
            }
            // (with V split, each slice stores its half; slice 0 the (max, sum))
            store_pair_coherent(p.part_acc + (bh * p.P + part) * D + vslice * DV + e, o0, o1);
            if (e == 0 && vslice == 0)
                store_pair_coherent(reinterpret_cast<float *>(p.part_ml + bh * p.P + part), M, L);
        }
    }

    if constexpr (kTimeline) {
        if (tl && threadIdx.x == 0) {
            tl[6] = stamp_now();  // thread 0's share of the output or record issued
            tl[12] = silent ? 3 : (direct ? 1 : 2);
        }
    }
    if constexpr (kFusedMerge) {
        if (direct || silent) return;
        if constexpr (kBreakdown) {
            // stage 2: nothing stored; stage 3: the partial sums stored, no ticket
            if (p.stop_after == 2 || p.stop_after == 3) return;
        }
        // Publish this partition and take a ticket.  The ticket of (b, kvh)
        // is 64 bits, an arrival count (low half) and a generation (high
        // half).  Of the n = VS * busy workgroups, the last to arrive (count
        // n - 1) resets the count and moves the generation on with one
        // atomic add, and merges; with K > 1 (K the largest power of two up
        // to p.merge_ways that n fills) the K - 1 before it (counts n - K ..
        // n - 2) merge too, each its own slice of the head dim, once they see
        // the generation move on (a bounded wait on the ticket's line).
        // p.merge_ways > 1 only when every workgroup of the launch can be
        // resident at once, so the ones they wait for are running.
        //
        // Ordering (PA_ORDERED_TICKET = 0, the library): the partial sums are
        // agent-scope atomic stores, which on this part write through to the
        // device-coherent level (past every XCD's L2); the waitcnt returns only
        // once each of this wave's stores is acknowledged there, and the
        // barrier holds thread 0 until all four waves have passed theirs.  The
        // ticket is an agent-scope atomic, performed at that same level and
        // issued after the barrier, so when a workgroup's ticket reads n - 1
        // the stores behind every earlier ticket are already there, and so
        // they are when a waiting merger reads the moved-on generation, which
        // the last arrival writes after its own ticket.  Mergers issue their
        // loads after that, with the coherent cache policy (kCoherent), which
        // reads past a stale L2 copy.  This rests on the cache policy of the
        // stores and loads and on where atomics are performed, not on the HIP
        // memory model: in the model the relaxed ticket orders nothing.
        //
        // PA_ORDERED_TICKET = 1 (the ablation library libpa_decode_ordered.so)
        // orders the same exchange within the memory model: thread 0's ticket
        // is an agent-scope release read-modify-write, so every thread's
        // stores, sequenced before the barrier that synchronises the
        // workgroup with thread 0, happen before it.  The tickets of (b, kvh)
        // and the last arrival's reset form a release sequence of every one
        // of them, so a merger's agent-scope acquire fence -- after its own
        // ticket read n - 1, or after it read the moved-on generation --
        // makes every other workgroup's stores happen before it, and through
        // the second barrier before every thread's merge loads.  On gfx950
        // the release is an L2 writeback in every publishing workgroup,
        // which queues: measured +1.2 us on one 16384-token sequence (256
        // workgroups) and +47 % on a batch of 32 x 8192 tokens (2048).
        __shared__ int sm_role, sm_ways, sm_poisoned;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if constexpr (kTimeline) {
            if (tl && threadIdx.x == 0) tl[15] = stamp_now();  // stores acknowledged
        }
        if (threadIdx.x == 0) {
            auto *ticket = reinterpret_cast<unsigned long long *>(
                p.counters + (long long)kTicketStride * (b * p.Hkv + kvh));
            const int n = VS * busy;
            // the largest power of two up to p.merge_ways that n workgroups fill
            int ways = 1;
            while (2 * ways <= p.merge_ways && 2 * ways <= n) ways *= 2;
            const unsigned long long old = __hip_atomic_fetch_add(
                ticket, 1ull, kOrderedTicket ? __ATOMIC_RELEASE : __ATOMIC_RELAXED,
                __HIP_MEMORY_SCOPE_AGENT);
            const int count = (int)(unsigned)(old & 0xFFFFFFFFull);
            const unsigned gen = (unsigned)(old >> 32);
            int role = -1, poisoned = 0;
            if (count == n - 1) {
                if (kOrderedTicket) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                __hip_atomic_fetch_add(ticket, (1ull << 32) - (unsigned long long)n,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                role = ways - 1;
            } else if (count >= n - ways) {
                int rounds = 0;
                while ((unsigned)(__hip_atomic_load(ticket, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT) >> 32) == gen) {
                    if (++rounds >= kMaxPollRounds) {
                        poisoned = 1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                if (kOrderedTicket) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                role = count - (n - ways);
            }
            sm_role = role;
            sm_ways = ways;
            sm_poisoned = poisoned;
            if constexpr (kTimeline) {
                if (tl) {
                    tl[7] = stamp_now();
                    tl[8] = (unsigned long long)(role + 1) | ((unsigned long long)count << 8) |
                            ((unsigned long long)ways << 40);
                }
            }
        }
        __syncthreads();
        if (sm_role >= 0)
            merge_group<DT, D, G, NW>(p, b, kvh, busy, sm_ways, sm_role, sm_poisoned != 0);
        if constexpr (kTimeline) {
            if (sm_role >= 0) {
                __syncthreads();
                if (tl && threadIdx.x == 0) tl[9] = stamp_now();
            }
        }
    }
}


// One wave per (b, h); lane l produces elements 2l + 128 j, 2l + 1 + 128 j.
template <int DT>
__global__ __launch_bounds__(kWave) void pa_merge_kernel(MergeParams mp) {
    const long long bh = blockIdx.x;
    for (int e = 2 * threadIdx.x; e < mp.d; e += 2 * kWave) {
        const float2 o = merge_partitions(mp.part_ml + bh * mp.P,
                                                 mp.part_acc + bh * mp.P * mp.d + e, mp.P, mp.d);
        store_pair<DT>(mp.out, bh * mp.d + e, o.x, o.y);
    }
}

template <int DT, int D, int G, int MODE>
hipError_t launch_instance(const Params &p, int nseq, hipStream_t stream) {
    if constexpr (mode_built(DT, D, G, MODE)) {
        Params q = p;
        if (q.merge_ways > 1) {
            // The arrivals that wait to share a merge hold their compute unit
            // while they wait.  Keep each launch's waiters (at most K - 1 per
            // (sequence, kv head) unit) below half of the workgroups the
            // device holds at once, so that even two such launches running
            // together leave a slot for a workgroup they wait for.
            // (queried once per instance; a failed query is not kept, and
            // that call merges with the last arrival alone)
            static std::atomic<int> cached{-1};
            int resident = cached.load(std::memory_order_relaxed);
            if (resident < 0) {
                int n = 0;
                if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                        &n,
                        reinterpret_cast<const void *>(
                            &pa_decode_kernel<DT, D, G, kWavesPerGroup, kDepth, MODE>),
                        kWavesPerGroup * kWave, 0) == hipSuccess) {
                    cached.store(n, std::memory_order_relaxed);
                    resident = n;
                } else {
                    resident = 0;
                }
            }
            const long long units = (long long)nseq * q.Hkv;
            while (q.merge_ways > 1 &&
                   2 * units * (q.merge_ways - 1) >= (long long)q.cus * resident)
                q.merge_ways /= 2;
        }
        hipLaunchKernelGGL((pa_decode_kernel<DT, D, G, kWavesPerGroup, kDepth, MODE>),
                           dim3(q.Hkv, nseq, v_slices(MODE) * q.P),
                           dim3(kWavesPerGroup * kWave), 0, stream, q);
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;
    }
}

template <int DT, int D, int MODE>
hipError_t dispatch_g(const Params &p, int G, int nseq, hipStream_t stream) {
    switch (G) {
        case 1: return launch_instance<DT, D, 1, MODE>(p, nseq, stream);
        case 2: return launch_instance<DT, D, 2, MODE>(p, nseq, stream);
        case 4: return launch_instance<DT, D, 4, MODE>(p, nseq, stream);
        case 8: return launch_instance<DT, D, 8, MODE>(p, nseq, stream);
        case 16: return launch_instance<DT, D, 16, MODE>(p, nseq, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int DT, int D>
hipError_t dispatch_mode(const Params &p, int G, int mode, int nseq, hipStream_t stream) {
    switch (mode) {
        case kSingle: return dispatch_g<DT, D, kSingle>(p, G, nseq, stream);
        case kSingleSplitV:
            if constexpr (split_v_built(D)) return dispatch_g<DT, D, kSingleSplitV>(p, G, nseq, stream);
            else return hipErrorInvalidValue;
        case kFusedSplitV:
            if constexpr (split_v_built(D)) return dispatch_g<DT, D, kFusedSplitV>(p, G, nseq, stream);
            else return hipErrorInvalidValue;
        case kPartials: return dispatch_g<DT, D, kPartials>(p, G, nseq, stream);
        case kPartialsSplitV:
            if constexpr (split_v_built(D)) return dispatch_g<DT, D, kPartialsSplitV>(p, G, nseq, stream);
            else return hipErrorInvalidValue;
        case kFused: return dispatch_g<DT, D, kFused>(p, G, nseq, stream);
        default: return dispatch_g<DT, D, kFusedLate>(p, G, nseq, stream);
    }
}

template <int DT>
hipError_t launch_decode(const Params &p, int d, int G, int mode, int nseq,
                         hipStream_t stream) {
    switch (d) {
        case 64: return dispatch_mode<DT, 64>(p, G, mode, nseq, stream);
        case 128: return dispatch_mode<DT, 128>(p, G, mode, nseq, stream);
        case 256: return dispatch_mode<DT, 256>(p, G, mode, nseq, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int DT>
hipError_t launch_merge(const MergeParams &mp, int groups, hipStream_t stream) {
    hipLaunchKernelGGL(pa_merge_kernel<DT>, dim3(groups), dim3(kWave), 0, stream, mp);
    return hipGetLastError();
}

}  // namespace pa_detail

#endif  // PA_KERNELS_H
