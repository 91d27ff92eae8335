// tk_topk.hip -- deterministic top-k expert gating for MI355X (gfx950),
// behind tk_topk_gate in include/tk.h.
//
// The operation is the Gating module of "TileLang + TileKernels：DeepSeek 的 GPU
// 内核开发新范式" ("1. Gating": each token's top-k experts from
// [num_tokens, num_experts] scores, equal scores going to the smaller index)
// with the group step of "【DeepSeek】TileKernels从入门到精通" ch.3
// "导诊台的“工号制度”" (groups ranked by the sum of their two best scores,
// equal sums going to the smaller group index; then pick the best, label it,
// pick the next).
//
// gfx950 design (the pages use a 32-lane warp per token).  Up to 256 experts
// and k <= 32 (topk_pair_kernel): one 64-lane wave serves two tokens, lanes
// 0-31 the first and 32-63 the second, lane l holding experts
// (l & 31)*C .. +C-1 of its token (C = ceil(experts/32) <= 8).  Otherwise
// (topk_kernel): one wave per token, lane l holding experts l*C .. l*C+C-1
// (C = ceil(experts/64) <= 8).  Either way a group of experts is a block of
// consecutive lanes and lane order is index order.  When a token's kept
// groups fit 16 lanes of the two-token layout (at most 8 groups, k <= 16;
// 256 experts in 8 groups keeping 4, for one), the groups are ranked first,
// the kept lanes move into one 16-lane row per token and steps 1 and 3 run
// on four tokens per wave: topk_row_kernel for a multiple of 32 experts from
// 64 to 256 in 2, 4 or 8 groups (one token per 16-lane row from the start,
// 4 to 16 experts per lane, group ranks by row broadcasts), topk_quad_kernel
// for the other such shapes (two passes of the two-token layout).  Without
// groups and k <= 16, one token per 16-lane row goes straight to steps 1 and
// 3: topk_row1_kernel up to 128 experts (one list per lane), topk_row2_kernel
// from 129 to 256 (two lists per lane, a round taking the larger head),
// topk_rowl_kernel from 257 to 512 (three or four lists per lane).
//   1. Each lane sorts its C candidates once, best first, by the key (score
//      in an order-preserving uint32 map, -0 == +0; then smaller index).
//   2. Groups: each lane's two best, merged over the group's lanes (DPP
//      quad_perm / half-row and row mirrors, lane shuffles past 16 lanes);
//      a NaN group sum (+inf and -inf) counts as -inf.  Group ranks: with at
//      most 8 groups, lane 8h + h' compares group h' with group h and one
//      ballot per token holds every pair (group h's rank = set bits in byte
//      h); with more, wave-uniform reads of every group sum.  Lanes of
//      dropped groups empty their lists.
//   3. k rounds of a tournament between the lanes' list heads: a DPP max of
//      the head keys (quad_perm, row_half_mirror, row_mirror, then row
//      broadcasts; v_readlane of the lane that ends with the maximum), the
//      first lane whose head equals it (ballot + s_ff1: the smallest index
//      among equal scores), the winner's expert index from its packed slot
//      list (one v_readlane and scalar arithmetic), and the winner pops its
//      head (its keys shift, its slot list shifts by 3 bits); lane `round`
//      keeps the pick's index.  In the two-token layout every one of these
//      wave-wide instructions serves both tokens.
//      Output lane j then re-reads pick j's own score, and the
//      normalising sum adds those k values in pick order after the rounds.
//      In the four-token kernels a pick's weight is its key's value instead
//      (one read again only for a zero key, whose sign the key does not keep).
// The one- and two-token kernels use no LDS beyond the two lane shuffles of
// the group rank.  topk_row_kernel takes each group's two best on the scores
// themselves (v_med3_f32) and maps to keys only the kept lanes, after the
// move.  Scores are taken to be non-NaN: a NaN score may be ranked
// differently by different kernels.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "tk.h"

namespace {

constexpr int kWave = 64;
constexpr int kThreads = 256;
constexpr int kMaxExperts = 512;

__device__ __forceinline__ uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float ffrom(uint32_t u) { return __builtin_bit_cast(float, u); }

// Order-preserving map of a (non-NaN) float to uint32; -0 and +0 map alike.
// Every non-NaN value maps above 0, which therefore marks "no candidate".
__device__ __forceinline__ uint32_t ordered(float f)
{
    const uint32_t b = fbits(f + 0.0f); // -0 + +0 = +0
    // negative: all bits flipped; otherwise only the sign bit set
    return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}

// The value of a key (a zero comes back as +0).
__device__ __forceinline__ float unordered(uint32_t h)
{
    return ffrom((h & 0x80000000u) ? (h & 0x7FFFFFFFu) : ~h);
}

// "a beats b": larger score, or equal score and smaller index
__device__ __forceinline__ bool beats(float sa, uint32_t a, float sb, uint32_t b)
{
    return sa > sb || (sa == sb && a < b);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v)
{
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false));
}

// maximum over all 64 lanes (every lane active), as a wave-uniform value
__device__ __forceinline__ uint32_t wave_umax(uint32_t v)
{
    v = dpp_umax<0xB1>(v);  // quad_perm [1,0,3,2]
    v = dpp_umax<0x4E>(v);  // quad_perm [2,3,0,1]
    v = dpp_umax<0x141>(v); // row_half_mirror
    v = dpp_umax<0x140>(v); // row_mirror: every lane holds its 16-lane row's max
    // row_bcast:15 into rows 1 and 3, then row_bcast:31 into rows 2 and 3:
    // lane 63 ends with the wave's max
    // (rows left out read 0, the identity of the unsigned max)
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
    return __builtin_amdgcn_readlane(v, 63);
}

// (a1, a2) <- the two largest keys of (a1, a2) and (b1, b2), each pair ordered
__device__ __forceinline__ void merge_top2_from(uint32_t& a1, uint32_t& a2, uint32_t b1, uint32_t b2)
{
    const uint32_t hi = max(a1, b1);
    a2 = max(min(a1, b1), max(a2, b2));
    a1 = hi;
}

template <int CTRL>
__device__ __forceinline__ void merge_top2(uint32_t& a1, uint32_t& a2)
{
    const uint32_t b1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a1, CTRL, 0xF, 0xF, false);
    const uint32_t b2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a2, CTRL, 0xF, 0xF, false);
    merge_top2_from(a1, a2, b1, b2);
}

// +inf or -inf in a scalar register whose value the compiler does not see:
// a median against it stays one v_med3_f32 (against a known infinity the
// compiler turns it into an IEEE max or min, which first quiets each loaded
// operand with an instruction of its own)
__device__ __forceinline__ float opaque_inf(bool negative)
{
    uint32_t b;
    if (negative)
        asm volatile("s_mov_b32 %0, 0xff800000" : "=s"(b));
    else
        asm volatile("s_mov_b32 %0, 0x7f800000" : "=s"(b));
    return ffrom(b);
}

// max / min of two non-NaN floats, as a median against an infinity
__device__ __forceinline__ float fmax2(float a, float b, float pinf) { return __builtin_amdgcn_fmed3f(a, b, pinf); }
__device__ __forceinline__ float fmin2(float a, float b, float ninf) { return __builtin_amdgcn_fmed3f(a, b, ninf); }

// (a1, a2) <- the two largest of (a1, a2) and the pair CTRL brings from
// another lane, each pair ordered: the second is the median of the two
// firsts and the larger second
template <int CTRL>
__device__ __forceinline__ void merge_top2f(float& a1, float& a2, float pinf)
{
    const float b1 = ffrom((uint32_t)__builtin_amdgcn_update_dpp(0, (int)fbits(a1), CTRL, 0xF, 0xF, false));
    const float b2 = ffrom((uint32_t)__builtin_amdgcn_update_dpp(0, (int)fbits(a2), CTRL, 0xF, 0xF, false));
    a2 = __builtin_amdgcn_fmed3f(a1, b1, fmax2(a2, b2, pinf));
    a1 = fmax2(a1, b1, pinf);
}

template <int C>
__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores, uint32_t tokens,
                                                        uint32_t experts, uint32_t k, uint32_t n_group,
                                                        uint32_t topk_group, uint32_t gl_log2, int normalise,
                                                        int32_t* __restrict__ idx_out, float* __restrict__ w_out)
{
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t t = __builtin_amdgcn_readfirstlane(blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave);
    if (t >= tokens)
        return;
    const float* s_row = scores + (size_t)t * experts;

    // ---- 1. this lane's candidates, sorted best first
    // every load is issued (a slot past the last expert re-reads the last
    // one and is then emptied), so all C are in flight together
    uint32_t key[C], idx[C];
    float v[C];
#pragma unroll
    for (int j = 0; j < C; ++j)
        v[j] = s_row[min(lane * C + j, experts - 1u)];
#pragma unroll
    for (int j = 0; j < C; ++j) {
        const uint32_t e = lane * C + j;
        key[j] = e < experts ? ordered(v[j]) : 0u;
        idx[j] = (uint32_t)j; // slot within the lane
    }
#pragma unroll
    for (int i = 1; i < C; ++i) {
#pragma unroll
        for (int j = i; j > 0; --j) {
            // insertion by strict comparison is stable and the indices start
            // ascending, so equal keys stay smallest index first
            const bool swap = key[j] > key[j - 1];
            const uint32_t k0 = key[j - 1], i0 = idx[j - 1];
            key[j - 1] = swap ? key[j] : k0;
            idx[j - 1] = swap ? idx[j] : i0;
            key[j] = swap ? k0 : key[j];
            idx[j] = swap ? i0 : idx[j];
        }
    }

    // ---- 2. group selection
    if (n_group > 1) {
        // the group's two best keys (a lane's two best are its list head; 0 =
        // none), merged as order-preserving integers and turned back into
        // values for the sum (the sign of a zero does not matter to the sums'
        // comparisons).  Merge over the group's 2^gl_log2 lanes: DPP within
        // 16-lane rows (after each step a block of lanes holds one merged
        // pair, so the mirror partner always brings the other block's), lane
        // shuffles above.
        uint32_t a1 = key[0], a2 = C > 1 ? key[C > 1 ? 1 : 0] : 0u;
        if (gl_log2 >= 1)
            merge_top2<0xB1>(a1, a2); // quad_perm [1,0,3,2]
        if (gl_log2 >= 2)
            merge_top2<0x4E>(a1, a2); // quad_perm [2,3,0,1]
        if (gl_log2 >= 3)
            merge_top2<0x141>(a1, a2); // row_half_mirror
        if (gl_log2 >= 4)
            merge_top2<0x140>(a1, a2); // row_mirror
        for (uint32_t m = 16; m < (1u << gl_log2); m <<= 1)
            merge_top2_from(a1, a2, (uint32_t)__shfl_xor((int)a1, (int)m), (uint32_t)__shfl_xor((int)a2, (int)m));
        float gsum = (a1 ? unordered(a1) : -INFINITY) + (a2 ? unordered(a2) : -INFINITY);
        if (gsum != gsum) // +inf + -inf: a NaN group score ranks as -inf (groups stay totally ordered)
            gsum = -INFINITY;
        const uint32_t my_g = lane >> gl_log2;
        uint32_t rank = 0;
        if (n_group <= 8) {
            // all pairs at once: lane 8h + h' compares group h' against group
            // h, and group h's rank is the count of set bits in byte h of the
            // ballot
            const uint32_t h = lane >> 3, h2 = lane & 7u;
            // ds_bpermute addresses lanes in bytes; rows and columns past the
            // last group read the last group and are masked out below
            const float g_h = ffrom((uint32_t)__builtin_amdgcn_ds_bpermute(
                (int)((min(h, n_group - 1u) << gl_log2) << 2), (int)fbits(gsum)));
            const float g_h2 = ffrom((uint32_t)__builtin_amdgcn_ds_bpermute(
                (int)((min(h2, n_group - 1u) << gl_log2) << 2), (int)fbits(gsum)));
            // beats(g_h2, h2, g_h, h) without short-circuit branches
            const uint32_t b = (uint32_t)(max(h, h2) < n_group) &
                               ((uint32_t)(g_h2 > g_h) | ((uint32_t)(g_h2 == g_h) & (uint32_t)(h2 < h)));
            const uint64_t m = __builtin_amdgcn_ballot_w64(b != 0u);
            rank = (uint32_t)__builtin_popcountll((m >> (8u * my_g)) & 0xFFull);
        } else {
            for (uint32_t hh = 0; hh < n_group; ++hh) {
                const float gh = ffrom(__builtin_amdgcn_readlane(fbits(gsum), hh << gl_log2));
                rank += beats(gh, hh, gsum, my_g) ? 1u : 0u;
            }
        }
        if (rank >= topk_group) {
#pragma unroll
            for (int j = 0; j < C; ++j)
                key[j] = 0u;
        }
    }

    // ---- 3. k rounds between the list heads; pick it goes to lane it.  The
    // lane's sorted slots are packed 3 bits each (C <= 8), head lowest, so a
    // pop is one shift and the winner's expert index comes from one readlane.
    uint32_t slots = 0;
#pragma unroll
    for (int j = 0; j < C; ++j)
        slots |= idx[j] << (3 * j);
    int32_t my_idx = 0;
    for (uint32_t it = 0; it < k; ++it) {
        const uint32_t best = wave_umax(key[0]);
        const uint64_t hit = __builtin_amdgcn_ballot_w64(key[0] == best);
        const uint32_t owner = (uint32_t)__builtin_ctzll(hit); // lowest lane = smallest index
        const uint32_t e = owner * C + (__builtin_amdgcn_readlane(slots, owner) & 7u);
        if (lane == owner) {
#pragma unroll
            for (int j = 0; j + 1 < C; ++j)
                key[j] = key[j + 1];
            key[C - 1] = 0u;
            slots >>= 3;
        }
        my_idx = lane == it ? (int32_t)e : my_idx;
    }
    // each pick's own value (keeps -0), summed in pick order for the normalisation
    const float my_w = lane < k ? s_row[my_idx] : 0.0f;
    float sum = 0.0f;
    if (normalise) {
        for (uint32_t it = 0; it < k; ++it)
            sum += ffrom(__builtin_amdgcn_readlane(fbits(my_w), it));
    }
    if (lane < k) {
        idx_out[(size_t)t * k + lane] = my_idx;
        w_out[(size_t)t * k + lane] = (normalise && sum != 0.0f) ? my_w / sum : my_w;
    }
}

// Two tokens per wave, for up to 256 experts and k <= 32: lanes 0-31 serve
// token 2w and lanes 32-63 token 2w+1, lane l holding experts
// (l & 31)*C .. +C-1 of its token (C = ceil(experts/32)).  The steps are those
// of topk_kernel, each wave-wide instruction of a round now serving both
// tokens; the price is a longer per-lane sort (8 keys at 256 experts).

// maximum over each 16-lane row, then row 0's into row 1 and row 2's into
// row 3: lane 31 ends with the low half's maximum, lane 63 with the high half's
__device__ __forceinline__ uint32_t half_umax_at_ends(uint32_t v)
{
    v = dpp_umax<0xB1>(v);  // quad_perm [1,0,3,2]
    v = dpp_umax<0x4E>(v);  // quad_perm [2,3,0,1]
    v = dpp_umax<0x141>(v); // row_half_mirror
    v = dpp_umax<0x140>(v); // row_mirror
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false)); // row_bcast:15
}

// A lane's C candidates sorted best first by (key, smaller slot); idx[j] is
// 7 - slot of entry j, so that as a low word beside the key it breaks ties
// toward the smaller index.
template <int C>
__device__ __forceinline__ void sort_lane(uint32_t (&key)[C], uint32_t (&idx)[C])
{
    if constexpr (C == 8) {
        // 19-comparator network on (key, 7 - slot): every pair of entries is
        // strictly ordered, so the network's lack of stability does not matter
        uint64_t x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            x[j] = ((uint64_t)key[j] << 32) | (uint32_t)(7 - j);
        constexpr int net[19][2] = {{0, 2}, {1, 3}, {4, 6}, {5, 7}, {0, 4}, {1, 5}, {2, 6}, {3, 7}, {0, 1}, {2, 3},
                                    {4, 5}, {6, 7}, {2, 4}, {3, 5}, {1, 4}, {3, 6}, {1, 2}, {3, 4}, {5, 6}};
#pragma unroll
        for (int c = 0; c < 19; ++c) {
            // one 64-bit compare drives both selects (the round trip through
            // a lane mask keeps them from being rebuilt as a max and a min)
            const uint64_t a = x[net[c][0]], b = x[net[c][1]];
            const bool swap = __builtin_amdgcn_inverse_ballot_w64(__builtin_amdgcn_ballot_w64(b > a));
            x[net[c][0]] = swap ? b : a;
            x[net[c][1]] = swap ? a : b;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            key[j] = (uint32_t)(x[j] >> 32);
            idx[j] = (uint32_t)x[j];
        }
    } else {
#pragma unroll
        for (int j = 0; j < C; ++j)
            idx[j] = (uint32_t)(7 - j);
        // stable insertion by strict comparison (slots start in index order)
#pragma unroll
        for (int i = 1; i < C; ++i) {
#pragma unroll
            for (int j = i; j > 0; --j) {
                const bool swap = key[j] > key[j - 1];
                const uint32_t k0 = key[j - 1], i0 = idx[j - 1];
                key[j - 1] = swap ? key[j] : k0;
                idx[j - 1] = swap ? idx[j] : i0;
                key[j] = swap ? k0 : key[j];
                idx[j] = swap ? i0 : idx[j];
            }
        }
    }
}

// A lane's 8 raw scores (float bits, none NaN) sorted best first by (score,
// smaller slot), as sort_lane<8> sorts their keys, on 64-bit doubles: the
// high word is the score's own bits (-0 made +0), the low word the tie-break,
// 7 - slot for a non-negative score and slot for a negative one (a double's
// order runs backwards with its sign).  No NaN score makes a NaN or infinite
// double (that needs the top three mantissa bits set under an all-ones
// exponent), fp64 denormals are kept, and every word of a lane differs, so the
// 19 comparators are a max and a min each (v_max_f64 / v_min_f64, written out
// so that the compiler adds no canonicalising operation): 38 instructions
// instead of a 64-bit compare and four selects per comparator.  Returns the
// order-preserving keys and idx[j] = 7 - slot of entry j, as sort_lane does.
__device__ __forceinline__ double dmax(double a, double b)
{
    double r;
    asm("v_max_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ double dmin(double a, double b)
{
    double r;
    asm("v_min_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ void sort_lane_raw8(uint32_t (&key)[8], uint32_t (&idx)[8])
{
    double x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t h = fbits(ffrom(key[j]) + 0.0f); // -0 + +0 = +0
        const uint32_t l = (uint32_t)(7 - j) ^ ((uint32_t)((int32_t)h >> 31) & 7u);
        x[j] = __builtin_bit_cast(double, ((uint64_t)h << 32) | l);
    }
    constexpr int net[19][2] = {{0, 2}, {1, 3}, {4, 6}, {5, 7}, {0, 4}, {1, 5}, {2, 6}, {3, 7}, {0, 1}, {2, 3},
                                {4, 5}, {6, 7}, {2, 4}, {3, 5}, {1, 4}, {3, 6}, {1, 2}, {3, 4}, {5, 6}};
#pragma unroll
    for (int c = 0; c < 19; ++c) {
        const double a = x[net[c][0]], b = x[net[c][1]];
        x[net[c][0]] = dmax(a, b);
        x[net[c][1]] = dmin(a, b);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint64_t u = __builtin_bit_cast(uint64_t, x[j]);
        const uint32_t h = (uint32_t)(u >> 32);
        const uint32_t s = (uint32_t)((int32_t)h >> 31);
        key[j] = h ^ (s | 0x80000000u);
        idx[j] = (uint32_t)u ^ (s & 7u);
    }
}

// The rank of this lane's group among its token's groups in the two-token
// layout (a group is 2^gl_log2 <= 32 lanes inside its half), from the lane's
// two best keys a1 >= a2 (0 = none); 0 is the best group.
__device__ __forceinline__ uint32_t pair_group_rank(uint32_t a1, uint32_t a2, uint32_t lane, uint32_t gl_log2,
                                                    uint32_t n_group)
{
    const bool hi = lane >= 32u;
    const uint32_t hl = lane & 31u;
    if (gl_log2 >= 1)
        merge_top2<0xB1>(a1, a2);
    if (gl_log2 >= 2)
        merge_top2<0x4E>(a1, a2);
    if (gl_log2 >= 3)
        merge_top2<0x141>(a1, a2);
    if (gl_log2 >= 4)
        merge_top2<0x140>(a1, a2);
    if (gl_log2 >= 5)
        merge_top2_from(a1, a2, (uint32_t)__shfl_xor((int)a1, 16), (uint32_t)__shfl_xor((int)a2, 16));
    float gsum = (a1 ? unordered(a1) : -INFINITY) + (a2 ? unordered(a2) : -INFINITY);
    if (gsum != gsum) // +inf + -inf: a NaN group score ranks as -inf
        gsum = -INFINITY;
    const uint32_t my_g = hl >> gl_log2;
    uint32_t rank = 0;
    if (n_group <= 8) {
        // one ballot per token: lane 8h + h' compares that token's group
        // h' against its group h; group h's rank is the count of set bits
        // in byte h
        const uint32_t h = lane >> 3, h2 = lane & 7u;
        const uint32_t in = (uint32_t)(max(h, h2) < n_group);
        const uint32_t lt = (uint32_t)(h2 < h);
        uint64_t m[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const uint32_t base = 32u * p;
            const float g_h = ffrom((uint32_t)__builtin_amdgcn_ds_bpermute(
                (int)((base + (min(h, n_group - 1u) << gl_log2)) << 2), (int)fbits(gsum)));
            const float g_h2 = ffrom((uint32_t)__builtin_amdgcn_ds_bpermute(
                (int)((base + (min(h2, n_group - 1u) << gl_log2)) << 2), (int)fbits(gsum)));
            const uint32_t b = in & ((uint32_t)(g_h2 > g_h) | ((uint32_t)(g_h2 == g_h) & lt));
            m[p] = __builtin_amdgcn_ballot_w64(b != 0u);
        }
        rank = (uint32_t)__builtin_popcountll(((hi ? m[1] : m[0]) >> (8u * my_g)) & 0xFFull);
    } else {
        for (uint32_t hh = 0; hh < n_group; ++hh) {
            const float g0 = ffrom(__builtin_amdgcn_readlane(fbits(gsum), hh << gl_log2));
            const float g1 = ffrom(__builtin_amdgcn_readlane(fbits(gsum), 32u + (hh << gl_log2)));
            rank += beats(hi ? g1 : g0, hh, gsum, my_g) ? 1u : 0u;
        }
    }
    return rank;
}

template <int C, bool FULL, bool K8>
__global__ __launch_bounds__(kThreads) void topk_pair_kernel(const float* __restrict__ scores, uint32_t tokens,
                                                             uint32_t experts, uint32_t k, uint32_t n_group,
                                                             uint32_t topk_group, uint32_t gl_log2, int normalise,
                                                             int32_t* __restrict__ idx_out, float* __restrict__ w_out)
{
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t t0 = 2u * __builtin_amdgcn_readfirstlane(blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave);
    if (t0 >= tokens)
        return;
    const bool hi = lane >= 32u;
    const uint32_t hl = lane & 31u;
    const uint32_t t = t0 + (hi ? 1u : 0u);
    // a wave past an odd last token repeats that token in its high half and stores nothing from it
    const float* s_row = scores + (size_t)min(t, tokens - 1u) * experts;

    // ---- 1. this lane's candidates, sorted best first.  The slot of entry j
    // is kept as 7 - j, so that as a low word beside the key it breaks ties
    // toward the smaller index.
    // (FULL: experts == 32*C, every slot holds an expert)
    uint32_t key[C], idx[C];
    float v[C];
#pragma unroll
    for (int j = 0; j < C; ++j)
        v[j] = FULL ? s_row[hl * C + j] : s_row[min(hl * C + j, experts - 1u)];
#pragma unroll
    for (int j = 0; j < C; ++j)
        key[j] = (FULL || hl * C + j < experts) ? ordered(v[j]) : 0u;
    sort_lane<C>(key, idx);

    // ---- 2. group selection, per half (a group is 2^gl_log2 <= 32 lanes)
    if (n_group > 1) {
        const uint32_t rank = pair_group_rank(key[0], C > 1 ? key[C > 1 ? 1 : 0] : 0u, lane, gl_log2, n_group);
        if (rank >= topk_group) {
#pragma unroll
            for (int j = 0; j < C; ++j)
                key[j] = 0u;
        }
    }

    // ---- 3. k rounds, both tokens at once; pick it goes to lane it of its half
    uint32_t slots = 0;
#pragma unroll
    for (int j = 0; j < C; ++j)
        slots |= idx[j] << (3 * j);
    int32_t my_idx = 0;
    // Lane masks are built as scalars and turned into per-lane conditions by
    // inverse ballots, so the round's lane selections cost no vector compares.
    // Rounds are taken in pairs (the loop cannot be unrolled by the compiler
    // across its cross-lane operations): the pop then compiles to masked moves
    // in place rather than selects plus a register rotation per round.
    // depth: the picks left including this one (a lane popped now can be
    // popped at most depth - 1 more times, so only its first depth - 1
    // entries are read again)
    auto round = [&](uint32_t it, uint32_t depth) {
        const uint32_t m = half_umax_at_ends(key[0]);
        const uint32_t b0 = __builtin_amdgcn_readlane(m, 31), b1 = __builtin_amdgcn_readlane(m, 63);
        const uint32_t h0 = (uint32_t)__builtin_amdgcn_ballot_w64(key[0] == b0);
        const uint32_t h1 = (uint32_t)(__builtin_amdgcn_ballot_w64(key[0] == b1) >> 32);
        // each half's maximum is held by one of its lanes, so neither h0 nor h1 is 0
        const uint32_t o0 = (uint32_t)__builtin_ctz(h0), o1 = (uint32_t)__builtin_ctz(h1);
        const uint32_t e0 = o0 * C + 7u - (__builtin_amdgcn_readlane(slots, o0) & 7u);
        const uint32_t e1 = o1 * C + 7u - (__builtin_amdgcn_readlane(slots, 32u + o1) & 7u);
        if (__builtin_amdgcn_inverse_ballot_w64((uint64_t)(h0 & (0u - h0)) | ((uint64_t)(h1 & (0u - h1)) << 32))) {
#pragma unroll
            for (int j = 0; j + 1 < C; ++j)
                if (j + 1u < depth)
                    key[j] = key[j + 1];
            if (depth > (uint32_t)C)
                key[C - 1] = 0u;
            slots >>= 3;
        }
        my_idx = __builtin_amdgcn_inverse_ballot_w64(1ull << it) ? (int32_t)e0 : my_idx;
        my_idx = __builtin_amdgcn_inverse_ballot_w64(1ull << (32u + it)) ? (int32_t)e1 : my_idx;
    };
    if constexpr (K8) {
        // k == 8, straight-line rounds: each pop shifts only what later rounds read
#pragma unroll
        for (uint32_t it = 0; it < 8; ++it)
            round(it, 8u - it);
    } else {
        uint32_t it = 0;
        for (; it + 1 < k; it += 2) {
            round(it, 64u);
            round(it + 1, 64u);
        }
        if (it < k)
            round(it, 64u);
    }
    const float my_w = hl < k ? s_row[min((uint32_t)my_idx, experts - 1u)] : 0.0f;
    float sum0 = 0.0f, sum1 = 0.0f;
    if (normalise) {
        if (k <= 16) {
            // running sum in pick order inside each half's first 16-lane row:
            // after step m lane i holds ((w[i-m+1] + ...) + w[i]) added oldest
            // first (row_shr:1 reads 0 into a row's first lane), so lane k-1
            // of each half ends with 0 + w[0] + w[1] + ... + w[k-1] in that order
            float run = 0.0f;
            for (uint32_t it = 0; it < k; ++it)
                run = ffrom((uint32_t)__builtin_amdgcn_update_dpp(0, (int)fbits(run), 0x111, 0xF, 0xF, true)) + my_w;
            sum0 = ffrom(__builtin_amdgcn_readlane(fbits(run), k - 1u));
            sum1 = ffrom(__builtin_amdgcn_readlane(fbits(run), 31u + k));
        } else {
            for (uint32_t it = 0; it < k; ++it) {
                sum0 += ffrom(__builtin_amdgcn_readlane(fbits(my_w), it));
                sum1 += ffrom(__builtin_amdgcn_readlane(fbits(my_w), 32u + it));
            }
        }
    }
    const float sum = hi ? sum1 : sum0;
    if (hl < k && t < tokens) {
        idx_out[(size_t)t * k + hl] = my_idx;
        w_out[(size_t)t * k + hl] = (normalise && sum != 0.0f) ? my_w / sum : my_w;
    }
}

// The part of the four-tokens-per-wave kernels after the kept lanes have been
// written to LDS: row r = lane / 16 holds token t0 + r, its `filled_lanes`
// first lanes a kept lane's C keys each (index order along the row; RAW: the
// scores themselves, mapped to keys here) and s_src the expert index of each
// lane's first key.  Each lane sorts its keys, the k rounds run on the rows (a
// DPP maximum inside each 16-lane row, so one round serves four tokens; a
// round's winners write their pick and its key into s_pick at the round's
// position), and output lane q of row r stores pick q, its weight the key's
// value.
template <int C, bool K8, bool RAW8 = false>
__device__ __forceinline__ void rows_select(uint32_t (&key)[C], uint32_t base, bool filled,
                                            const float* __restrict__ scores, uint32_t tokens, uint32_t experts,
                                            uint32_t k, int normalise, int32_t* __restrict__ idx_out,
                                            float* __restrict__ w_out, uint32_t t0, uint32_t lane, uint2* s_pick);

template <bool K8>
__device__ __forceinline__ void rows_store(const float* __restrict__ scores, uint32_t tokens, uint32_t experts,
                                           uint32_t k, int normalise, int32_t* __restrict__ idx_out,
                                           float* __restrict__ w_out, uint32_t t0, uint32_t lane,
                                           const uint2* s_pick);

template <int C, bool K8, bool RAW>
__device__ __forceinline__ void quad_rows_finish(const float* __restrict__ scores, uint32_t tokens, uint32_t experts,
                                                 uint32_t k, uint32_t filled_lanes, int normalise,
                                                 int32_t* __restrict__ idx_out, float* __restrict__ w_out,
                                                 uint32_t t0, uint32_t lane, const uint4 (*s_keys)[kWave],
                                                 const uint32_t* s_src, uint2* s_pick)
{
    constexpr int kWords = C > 4 ? 2 : 1;
    const uint32_t q = lane & 15u;
    const bool filled = q < filled_lanes;
    uint32_t key[C];
    {
        uint32_t w8[4 * kWords];
#pragma unroll
        for (int w = 0; w < kWords; ++w) {
            const uint4 x = s_keys[w][lane];
            w8[4 * w] = x.x;
            w8[4 * w + 1] = x.y;
            w8[4 * w + 2] = x.z;
            w8[4 * w + 3] = x.w;
        }
#pragma unroll
        for (int j = 0; j < C; ++j) // eight raw scores go to rows_select as they are (sort_lane_raw8)
            key[j] = (RAW && C != 8) ? ordered(ffrom(w8[j])) : w8[j];
    }
    // the expert index of this lane's first slot (read by every lane: an
    // empty lane never wins, since k is at most the candidates)
    rows_select<C, K8, RAW && C == 8>(key, s_src[lane], filled, scores, tokens, experts, k, normalise, idx_out,
                                      w_out, t0, lane, s_pick);
}

// The steps of the four-tokens-per-wave kernels from the sort on: row r =
// lane / 16 holds token t0 + r, lane q of a row C keys of that token (lane
// order in the row is index order, `base` the expert index of the lane's first
// key; a lane that is not `filled` holds no candidate).  Each lane sorts its
// keys, the k rounds run on the rows (a DPP maximum inside each 16-lane row,
// so one round serves four tokens; a round's winners write their pick and its
// key into s_pick at the round's position), and output lane q of row r stores
// pick q, its weight the key's value.
// RAW8: C = 8 and key[] holds the raw scores (float bits), which
// sort_lane_raw8 sorts and turns into keys.
template <int C, bool K8, bool RAW8>
__device__ __forceinline__ void rows_select(uint32_t (&key)[C], uint32_t base, bool filled,
                                            const float* __restrict__ scores, uint32_t tokens, uint32_t experts,
                                            uint32_t k, int normalise, int32_t* __restrict__ idx_out,
                                            float* __restrict__ w_out, uint32_t t0, uint32_t lane, uint2* s_pick)
{
    const uint32_t q = lane & 15u;
    const uint32_t row = lane >> 4;
    uint32_t idx[C];
    if constexpr (RAW8) {
        static_assert(C == 8, "eight raw scores");
        sort_lane_raw8(key, idx);
    } else {
        sort_lane<C>(key, idx);
    }
    // a lane past the row's filled ones sorts whatever it was given; an empty
    // head keeps it from ever winning, so its other keys are never read
    key[0] = filled ? key[0] : 0u;
    // slot lists, head lowest, 3 bits each: the slots themselves (7 - idx)
    uint32_t slots = 0;
#pragma unroll
    for (int j = 0; j < C; ++j)
        slots |= idx[j] << (3 * j);
    slots ^= 0xFFFFFFu;

    // ---- k rounds, four tokens at once
    uint2* pick_row = &s_pick[row << 4];
    auto round = [&](uint32_t it, uint32_t depth) {
        uint32_t m = key[0];
        m = dpp_umax<0xB1>(m);  // quad_perm [1,0,3,2]
        m = dpp_umax<0x4E>(m);  // quad_perm [2,3,0,1]
        m = dpp_umax<0x141>(m); // row_half_mirror
        m = dpp_umax<0x140>(m); // row_mirror: every lane holds its row's maximum
        const uint64_t hit = __builtin_amdgcn_ballot_w64(key[0] == m);
        // the lowest set bit of each row's 16 bits (every row has one: its
        // maximum is some lane's head, so no borrow crosses a row)
        const uint64_t win = hit & ~(hit - 0x0001000100010001ull);
        if (__builtin_amdgcn_inverse_ballot_w64(win)) {
            pick_row[it] = make_uint2(C == 8 ? (base | (slots & 7u)) : (base + (slots & 7u)), key[0]);
#pragma unroll
            for (int j = 0; j + 1 < C; ++j)
                if (j + 1u < depth)
                    key[j] = key[j + 1];
            if (depth > (uint32_t)C)
                key[C - 1] = 0u;
            slots >>= 3;
        }
    };
    if constexpr (K8) {
#pragma unroll
        for (uint32_t it = 0; it < 8; ++it)
            round(it, 8u - it);
    } else {
        uint32_t it = 0;
        for (; it + 1 < k; it += 2) {
            round(it, 64u);
            round(it + 1, 64u);
        }
        if (it < k)
            round(it, 64u);
    }
    rows_store<K8>(scores, tokens, experts, k, normalise, idx_out, w_out, t0, lane, s_pick);
}

// After the rounds of a four-tokens-per-wave kernel (s_pick[r * 16 + q] holds
// row r's pick q and its key): output lane q of row r stores pick q of token
// t0 + r, its weight the key's value, normalised by the running sum in pick
// order.
template <bool K8>
__device__ __forceinline__ void rows_store(const float* __restrict__ scores, uint32_t tokens, uint32_t experts,
                                           uint32_t k, int normalise, int32_t* __restrict__ idx_out,
                                           float* __restrict__ w_out, uint32_t t0, uint32_t lane,
                                           const uint2* s_pick)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint32_t q = lane & 15u;
    const uint32_t row = lane >> 4;
    const uint32_t t = t0 + row;
    const float* s_row = scores + (size_t)min(t, tokens - 1u) * experts;
    const uint2 pk = s_pick[lane];
    const int32_t my_idx = q < k ? (int32_t)pk.x : 0;
    const uint32_t my_key = pk.y;
    // the pick's score is its key's value; a zero key stands for either sign
    // of zero, so only then is the score read again
    float my_w = q < k ? unordered(my_key) : 0.0f;
    if (q < k && my_key == 0x80000000u)
        my_w = s_row[min((uint32_t)my_idx, experts - 1u)];
    float sum = 0.0f;
    if (normalise) {
        // running sum in pick order inside each row (row_shr:1 reads 0 into a
        // row's first lane): lane k-1 ends with 0 + w[0] + ... + w[k-1]
        float run = 0.0f;
        auto add_step = [&]() {
            run = ffrom((uint32_t)__builtin_amdgcn_update_dpp(0, (int)fbits(run), 0x111, 0xF, 0xF, true)) + my_w;
        };
        if constexpr (K8) {
#pragma unroll
            for (int it = 0; it < 8; ++it)
                add_step();
        } else {
            for (uint32_t it = 0; it < k; ++it)
                add_step();
        }
        sum = ffrom((uint32_t)__builtin_amdgcn_ds_bpermute((int)(((row << 4) + k - 1u) << 2), (int)fbits(run)));
    }
    if (q < k && t < tokens) {
        idx_out[(size_t)t * k + q] = my_idx;
        w_out[(size_t)t * k + q] = (normalise && sum != 0.0f) ? my_w / sum : my_w;
    }
}

// Four tokens per wave, for shapes of the two-token layout whose kept groups
// fill at most 16 lanes of a token (topk_group * 2^gl_log2 <= 16; with 256
// experts: 8 groups keep up to 4, 4 keep up to 2, 2 keep 1) and k <= 16.
// Groups are ranked first, from each lane's two best keys; then the lanes of
// the kept groups move through LDS, in group order, into one 16-lane row per
// token, so that lane order in a row is still index order.  The sort and the
// k rounds then run on those rows: a round's maximum is a DPP maximum inside
// each 16-lane row (every lane of the row ends with it, so no lane reads),
// and one round serves four tokens instead of two.  A round's winners write
// their expert index into LDS at the round's position; output lane j of a
// row reads pick j from there.
template <int C, bool FULL, bool K8>
__global__ __launch_bounds__(kThreads) void topk_quad_kernel(const float* __restrict__ scores, uint32_t tokens,
                                                             uint32_t experts, uint32_t k, uint32_t n_group,
                                                             uint32_t topk_group, uint32_t gl_log2, int normalise,
                                                             int32_t* __restrict__ idx_out, float* __restrict__ w_out)
{
    constexpr int kWaves = kThreads / kWave;
    constexpr int kWords = C > 4 ? 2 : 1; // 16-byte words of a lane's candidate keys
    __shared__ uint4 s_keys[kWaves][kWords][kWave];
    __shared__ uint32_t s_src[kWaves][kWave];
    __shared__ uint2 s_pick[kWaves][kWave]; // [row * 16 + round]: (expert, key)
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t wv = threadIdx.x / kWave;
    const uint32_t t0 = 4u * __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + wv);
    if (t0 >= tokens)
        return;
    const bool hi = lane >= 32u;
    const uint32_t hl = lane & 31u;
    const uint32_t gmask = (1u << gl_log2) - 1u;

    // ---- 1. the two-token layout twice: tokens t0 + 2p (lanes 0-31) and
    // t0 + 2p + 1 (lanes 32-63); a wave past the last token repeats it and
    // stores nothing from it.  Both passes' loads are issued first.
    float v[2][C];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const float* s_row = scores + (size_t)min(t0 + 2u * p + (hi ? 1u : 0u), tokens - 1u) * experts;
#pragma unroll
        for (int j = 0; j < C; ++j)
            v[p][j] = FULL ? s_row[hl * C + j] : s_row[min(hl * C + j, experts - 1u)];
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        uint32_t key[C + (C % 4 ? 4 - C % 4 : 0)];
#pragma unroll
        for (int j = 0; j < C; ++j)
            key[j] = (FULL || hl * C + j < experts) ? ordered(v[p][j]) : 0u;
#pragma unroll
        for (int j = C; j < (int)(sizeof(key) / sizeof(key[0])); ++j)
            key[j] = 0u;
        // the lane's two best keys, unsorted
        uint32_t a1 = key[0], a2 = 0u;
        if constexpr (C > 1) {
            a1 = max(key[0], key[1]);
            a2 = min(key[0], key[1]);
#pragma unroll
            for (int j = 2; j < C; ++j) {
                a2 = max(a2, min(a1, key[j]));
                a1 = max(a1, key[j]);
            }
        }
        const uint32_t rank = pair_group_rank(a1, a2, lane, gl_log2, n_group);
        const bool kept = (hl >> gl_log2) < n_group && rank < topk_group;
        // kept groups below this lane's own: the last lanes of kept groups below it in its half
        const uint64_t last = __builtin_amdgcn_ballot_w64(kept && (hl & gmask) == gmask);
        const uint32_t below = hi ? __builtin_amdgcn_mbcnt_hi((uint32_t)(last >> 32), 0u)
                                  : __builtin_amdgcn_mbcnt_lo((uint32_t)last, 0u);
        if (kept) {
            const uint32_t d = 16u * (2u * p + (hi ? 1u : 0u)) + ((below << gl_log2) | (hl & gmask));
#pragma unroll
            for (int w = 0; w < kWords; ++w)
                s_keys[wv][w][d] = make_uint4(key[4 * w], key[4 * w + 1], key[4 * w + 2], key[4 * w + 3]);
            s_src[wv][d] = hl * C;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    quad_rows_finish<C, K8, false>(scores, tokens, experts, k, topk_group << gl_log2, normalise, idx_out, w_out, t0, lane,
                            s_keys[wv], s_src[wv], s_pick[wv]);
}

// Four tokens per wave without groups, up to 128 experts and k <= 16: lane q
// of row r holds experts q*C .. +C-1 of token 4w + r (C = ceil(experts / 16);
// without FULL, slots past the last expert are empty), each lane's keys go
// straight to the sort, and the rows go on as in topk_quad_kernel.
template <int C, bool K8, bool FULL>
__global__ __launch_bounds__(kThreads) void topk_row1_kernel(const float* __restrict__ scores, uint32_t tokens,
                                                             uint32_t experts, uint32_t k, int normalise,
                                                             int32_t* __restrict__ idx_out, float* __restrict__ w_out)
{
    constexpr int kWaves = kThreads / kWave;
    __shared__ uint2 s_pick[kWaves][kWave]; // [row * 16 + round]: (expert, key)
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t wv = threadIdx.x / kWave;
    const uint32_t t0 = 4u * __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + wv);
    if (t0 >= tokens)
        return;
    const uint32_t q = lane & 15u;
    // a wave past the last token repeats it in its other rows and stores nothing from them
    const float* s_row = scores + (size_t)min(t0 + (lane >> 4), tokens - 1u) * experts;
    float v[C];
#pragma unroll
    for (int j = 0; j < C; ++j)
        v[j] = FULL ? s_row[q * C + j] : s_row[min(q * C + j, experts - 1u)];
    // eight scores of a full row go to rows_select raw (sort_lane_raw8)
    constexpr bool kRaw8 = C == 8 && FULL;
    uint32_t key[C];
#pragma unroll
    for (int j = 0; j < C; ++j)
        key[j] = kRaw8 ? fbits(v[j]) : (FULL || q * C + j < experts) ? ordered(v[j]) : 0u;
    rows_select<C, K8, kRaw8>(key, q * C, true, scores, tokens, experts, k, normalise, idx_out, w_out, t0, lane,
                              s_pick[wv]);
}

// Four tokens per wave without groups, 129 to 256 experts and k <= 16: lane q
// of row r holds experts q*2C .. +2C-1 of token 4w + r (C = ceil(experts / 32);
// without FULL, slots past the last expert are empty) as two lists of C, each
// sorted on its own.  A round's row maximum is taken over the lanes' larger
// heads; a winning lane pops the list that holds it (the first list on equal
// keys: its experts have the smaller indices).
template <int C, bool K8, bool FULL>
__global__ __launch_bounds__(kThreads) void topk_row2_kernel(const float* __restrict__ scores, uint32_t tokens,
                                                             uint32_t experts, uint32_t k, int normalise,
                                                             int32_t* __restrict__ idx_out, float* __restrict__ w_out)
{
    constexpr int kWaves = kThreads / kWave;
    __shared__ uint2 s_pick[kWaves][kWave]; // [row * 16 + round]: (expert, key)
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t wv = threadIdx.x / kWave;
    const uint32_t t0 = 4u * __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + wv);
    if (t0 >= tokens)
        return;
    const uint32_t q = lane & 15u;
    const uint32_t row = lane >> 4;
    // a wave past the last token repeats it in its other rows and stores nothing from them
    const float* s_row = scores + (size_t)min(t0 + row, tokens - 1u) * experts;
    float v[2 * C];
#pragma unroll
    for (int j = 0; j < 2 * C; ++j)
        v[j] = FULL ? s_row[q * (2 * C) + j] : s_row[min(q * (2 * C) + j, experts - 1u)];
    uint32_t ka[C], kb[C], ia[C], ib[C];
    if constexpr (C == 8 && FULL) { // full lists of eight: sorted from the raw scores
#pragma unroll
        for (int j = 0; j < C; ++j) {
            ka[j] = fbits(v[j]);
            kb[j] = fbits(v[C + j]);
        }
        sort_lane_raw8(ka, ia);
        sort_lane_raw8(kb, ib);
    } else {
#pragma unroll
        for (int j = 0; j < C; ++j) {
            ka[j] = (FULL || q * (2 * C) + j < experts) ? ordered(v[j]) : 0u;
            kb[j] = (FULL || q * (2 * C) + C + j < experts) ? ordered(v[C + j]) : 0u;
        }
        sort_lane<C>(ka, ia);
        sort_lane<C>(kb, ib);
    }
    // slot lists, head lowest, 3 bits each
    uint32_t sa = 0, sb = 0;
#pragma unroll
    for (int j = 0; j < C; ++j) {
        sa |= ia[j] << (3 * j);
        sb |= ib[j] << (3 * j);
    }
    sa ^= 0xFFFFFFu;
    sb ^= 0xFFFFFFu;
    const uint32_t base = q * (2 * C);

    uint2* pick_row = &s_pick[wv][row << 4];
    // a pop as selects on the lane's condition (as branches on the list the
    // compiler would address the lists through memory)
    auto pop = [&](uint32_t (&key)[C], uint32_t& slots, uint32_t depth, bool p) {
#pragma unroll
        for (int j = 0; j + 1 < C; ++j)
            if (j + 1u < depth)
                key[j] = p ? key[j + 1] : key[j];
        if (depth > (uint32_t)C)
            key[C - 1] = p ? 0u : key[C - 1];
        slots = p ? slots >> 3 : slots;
    };
    auto round = [&](uint32_t it, uint32_t depth) {
        const uint32_t h = max(ka[0], kb[0]);
        uint32_t m = h;
        m = dpp_umax<0xB1>(m);  // quad_perm [1,0,3,2]
        m = dpp_umax<0x4E>(m);  // quad_perm [2,3,0,1]
        m = dpp_umax<0x141>(m); // row_half_mirror
        m = dpp_umax<0x140>(m); // row_mirror: every lane holds its row's maximum
        const uint64_t hit = __builtin_amdgcn_ballot_w64(h == m);
        // the lowest set bit of each row's 16 bits (every row has one)
        const uint64_t win = hit & ~(hit - 0x0001000100010001ull);
        const bool w = __builtin_amdgcn_inverse_ballot_w64(win);
        const bool from_a = ka[0] >= kb[0];
        const uint2 pick = make_uint2(from_a ? base + (sa & 7u) : base + C + (sb & 7u), h);
        pop(ka, sa, depth, w && from_a);
        pop(kb, sb, depth, w && !from_a);
        if (w)
            pick_row[it] = pick;
    };
    if constexpr (K8) {
#pragma unroll
        for (uint32_t it = 0; it < 8; ++it)
            round(it, 8u - it);
    } else {
        uint32_t it = 0;
        for (; it + 1 < k; it += 2) {
            round(it, 64u);
            round(it + 1, 64u);
        }
        if (it < k)
            round(it, 64u);
    }
    rows_store<K8>(scores, tokens, experts, k, normalise, idx_out, w_out, t0, lane, s_pick[wv]);
}

// Four tokens per wave without groups, 257 to 512 experts and k <= 16: the
// layout of topk_row2_kernel with L = 3 or 4 lists of C per lane (lane q of
// row r holds experts q*L*C .. +L*C-1; without FULL, slots past the last
// expert are empty).  A round's row maximum is taken over each lane's largest
// head; a winning lane pops the first list that holds it.
template <int C, int L, bool K8, bool FULL>
__global__ __launch_bounds__(kThreads) void topk_rowl_kernel(const float* __restrict__ scores, uint32_t tokens,
                                                             uint32_t experts, uint32_t k, int normalise,
                                                             int32_t* __restrict__ idx_out, float* __restrict__ w_out)
{
    constexpr int kWaves = kThreads / kWave;
    constexpr int kLane = L * C; // experts per lane
    __shared__ uint2 s_pick[kWaves][kWave]; // [row * 16 + round]: (expert, key)
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t wv = threadIdx.x / kWave;
    const uint32_t t0 = 4u * __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + wv);
    if (t0 >= tokens)
        return;
    const uint32_t q = lane & 15u;
    const uint32_t row = lane >> 4;
    // a wave past the last token repeats it in its other rows and stores nothing from them
    const float* s_row = scores + (size_t)min(t0 + row, tokens - 1u) * experts;
    const uint32_t base = q * kLane;
    float v[kLane];
#pragma unroll
    for (int j = 0; j < kLane; ++j)
        v[j] = FULL ? s_row[base + j] : s_row[min(base + j, experts - 1u)];
    uint32_t key[L][C], sl[L];
#pragma unroll
    for (int l = 0; l < L; ++l) {
        uint32_t id[C];
        // (sort_lane_raw8 here: 512 experts 4% slower)
#pragma unroll
        for (int j = 0; j < C; ++j)
            key[l][j] = (FULL || base + l * C + j < experts) ? ordered(v[l * C + j]) : 0u;
        sort_lane<C>(key[l], id);
        // slot list, head lowest, 3 bits each
        sl[l] = 0;
#pragma unroll
        for (int j = 0; j < C; ++j)
            sl[l] |= id[j] << (3 * j);
        sl[l] ^= 0xFFFFFFu;
    }

    uint2* pick_row = &s_pick[wv][row << 4];
    // a pop as selects on the lane's condition (as branches on the list the
    // compiler would address the lists through memory)
    auto pop = [&](uint32_t (&kl)[C], uint32_t& slots, uint32_t depth, bool p) {
#pragma unroll
        for (int j = 0; j + 1 < C; ++j)
            if (j + 1u < depth)
                kl[j] = p ? kl[j + 1] : kl[j];
        if (depth > (uint32_t)C)
            kl[C - 1] = p ? 0u : kl[C - 1];
        slots = p ? slots >> 3 : slots;
    };
    auto round = [&](uint32_t it, uint32_t depth) {
        uint32_t h = key[0][0];
#pragma unroll
        for (int l = 1; l < L; ++l)
            h = max(h, key[l][0]);
        uint32_t m = h;
        m = dpp_umax<0xB1>(m);  // quad_perm [1,0,3,2]
        m = dpp_umax<0x4E>(m);  // quad_perm [2,3,0,1]
        m = dpp_umax<0x141>(m); // row_half_mirror
        m = dpp_umax<0x140>(m); // row_mirror: every lane holds its row's maximum
        const uint64_t hit = __builtin_amdgcn_ballot_w64(h == m);
        // the lowest set bit of each row's 16 bits (every row has one)
        const uint64_t win = hit & ~(hit - 0x0001000100010001ull);
        const bool w = __builtin_amdgcn_inverse_ballot_w64(win);
        // the first list whose head is the lane's head (equal keys: the
        // earlier list's experts have the smaller indices)
        bool taken = false;
        uint32_t pick = 0;
        bool p[L];
#pragma unroll
        for (int l = 0; l < L; ++l) {
            const bool is_l = !taken && key[l][0] == h;
            pick = is_l ? base + l * C + (sl[l] & 7u) : pick;
            taken = taken || is_l;
            p[l] = w && is_l;
        }
#pragma unroll
        for (int l = 0; l < L; ++l)
            pop(key[l], sl[l], depth, p[l]);
        if (w)
            pick_row[it] = make_uint2(pick, h);
    };
    if constexpr (K8) {
#pragma unroll
        for (uint32_t it = 0; it < 8; ++it)
            round(it, 8u - it);
    } else {
        uint32_t it = 0;
        for (; it + 1 < k; it += 2) {
            round(it, 64u);
            round(it + 1, 64u);
        }
        if (it < k)
            round(it, 64u);
    }
    rows_store<K8>(scores, tokens, experts, k, normalise, idx_out, w_out, t0, lane, s_pick[wv]);
}

// Group ranks within 16-lane rows (one token per row, 16 >> GL groups of
// 2^GL lanes): group H's sum, as an order-preserving key, reaches every lane
// of the row by row_newbcast from the group's first lane, and a lane counts
// the groups that beat its own ("a beats b": larger sum, or equal sums and the
// smaller group index): a group below its own by a key at least its own
// (above gkey_less = gkey - 1), one above it by a larger key.
template <int GL, int H = 0>
__device__ __forceinline__ void row_group_rank(uint32_t gkey, uint32_t gkey_less, uint32_t& rank)
{
    if constexpr ((H << GL) < 16) {
        const uint32_t gh = (uint32_t)__builtin_amdgcn_mov_dpp((int)gkey, 0x150 + (H << GL), 0xF, 0xF, false);
        // the lanes of groups above H, whose equal sums lose to group H (a
        // constant lane mask), count group H when its key is at least theirs
        constexpr uint64_t kAbove = (uint64_t)(0xFFFFu & ~((1u << ((H + 1) << GL)) - 1u)) * 0x0001000100010001ull;
        const uint32_t thr = __builtin_amdgcn_inverse_ballot_w64(kAbove) ? gkey_less : gkey;
        rank += gh > thr ? 1u : 0u;
        row_group_rank<GL, H + 1>(gkey, gkey_less, rank);
    }
}

// Four tokens per wave in one pass, for 16 * C16 experts (C16 even, 4 to 16
// experts per lane, 16 lanes per token) in 2, 4 or 8 groups (16 >> GL groups
// of 2^GL lanes) whose kept groups fill at most 8 lanes, and k <= 16: lane q of
// row r holds experts q*C16 .. +C16-1 of token 4w + r.  Each row ranks its
// groups with row broadcasts (no LDS), and a kept lane writes the two halves
// of its keys to two lanes of its own row, in group order, so that lane
// order in the row is still index order; then the rows go on as in
// topk_quad_kernel.
template <int C16, bool K8, int GL>
__global__ __launch_bounds__(kThreads) void topk_row_kernel(const float* __restrict__ scores, uint32_t tokens,
                                                            uint32_t k, uint32_t topk_group, int normalise,
                                                            int32_t* __restrict__ idx_out, float* __restrict__ w_out)
{
    constexpr uint32_t kExperts = 16 * C16;
    constexpr int C = C16 / 2; // keys per row lane after the move
    constexpr int kWaves = kThreads / kWave;
    constexpr int kWords = C > 4 ? 2 : 1;
    constexpr uint32_t kGMask = (1u << GL) - 1u;
    static_assert(C16 % 2 == 0 && C16 >= 4 && C16 <= 16, "an even count of 4 to 16 experts per lane");
    __shared__ uint4 s_keys[kWaves][kWords][kWave];
    __shared__ uint32_t s_src[kWaves][kWave];
    __shared__ uint2 s_pick[kWaves][kWave]; // [row * 16 + round]: (expert, key)
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t wv = threadIdx.x / kWave;
    const uint32_t t0 = 4u * __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + wv);
    if (t0 >= tokens)
        return;
    const uint32_t q = lane & 15u;
    const uint32_t row = lane >> 4;
    // a wave past the last token repeats it in its other rows and stores nothing from them
    const float* s_row = scores + (size_t)min(t0 + row, tokens - 1u) * kExperts;
    float x[C16];
#pragma unroll
    for (int j = 0; j < C16; ++j)
        x[j] = s_row[q * C16 + j];
    // the lane's two best scores, then the group's over its 2^GL lanes (as
    // values: the sign of a zero does not change a sum's comparisons)
    const float pinf = opaque_inf(false);
    float a1 = fmax2(x[0], x[1], pinf), a2 = fmin2(x[0], x[1], opaque_inf(true));
#pragma unroll
    for (int j = 2; j < C16; ++j) {
        a2 = __builtin_amdgcn_fmed3f(a1, a2, x[j]);
        a1 = fmax2(a1, x[j], pinf);
    }
    if constexpr (GL >= 1)
        merge_top2f<0xB1>(a1, a2, pinf); // quad_perm [1,0,3,2]
    if constexpr (GL >= 2)
        merge_top2f<0x4E>(a1, a2, pinf); // quad_perm [2,3,0,1]
    if constexpr (GL >= 3)
        merge_top2f<0x141>(a1, a2, pinf); // row_half_mirror
    float gsum = a1 + a2;
    if (gsum != gsum) // +inf + -inf: a NaN group score ranks as -inf
        gsum = -INFINITY;
    uint32_t rank = 0;
    // the sums as keys (above 0, -0 == +0), so that one unsigned compare per
    // group decides it
    const uint32_t gkey = ordered(gsum);
    uint32_t gkey_less = gkey - 1u; // opaque to the compiler, so each group's threshold stays one select
    asm volatile("" : "+v"(gkey_less));
    row_group_rank<GL>(gkey, gkey_less, rank);
    const bool kept = rank < topk_group;
    // kept groups below this lane's own in its row: the last lanes of kept
    // groups below it, counted over the wave and less those of the rows above
    const uint64_t last = __builtin_amdgcn_ballot_w64(kept && (q & kGMask) == kGMask);
    const uint32_t below_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(last >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)last, 0u));
    const uint32_t above = row == 0 ? 0u
                           : (uint32_t)__builtin_popcountll(last & (row == 1 ? 0xFFFFull : row == 2 ? 0xFFFFFFFFull
                                                                                                      : 0xFFFFFFFFFFFFull));
    const uint32_t below = below_wave - above;
    if (kept) {
        const uint32_t d = (row << 4) + 2u * ((below << GL) | (q & kGMask));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int w = 0; w < kWords; ++w) {
                // the half's C scores, then zeros up to the words' 4 * kWords slots
                auto at = [&](int i) { return i < C ? fbits(x[h * C + i]) : 0u; };
                s_keys[wv][w][d + h] = make_uint4(at(4 * w), at(4 * w + 1), at(4 * w + 2), at(4 * w + 3));
            }
            s_src[wv][d + h] = q * C16 + h * C;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    quad_rows_finish<C, K8, true>(scores, tokens, kExperts, k, 2u * (topk_group << GL), normalise, idx_out, w_out, t0, lane,
                            s_keys[wv], s_src[wv], s_pick[wv]);
}

bool overlaps(const void* a, size_t an, const void* b, size_t bn)
{
    if (!a || !b || an == 0 || bn == 0)
        return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

} // namespace

extern "C" tk_status tk_topk_gate(const float* scores, int64_t tokens, int64_t experts, int64_t k, int64_t n_group,
                                  int64_t topk_group, int normalise, int32_t* topk_idx, float* topk_weight,
                                  void* stream)
{
    if (tokens < 0 || tokens >= (int64_t)INT_MAX || experts <= 0 || k <= 0 || n_group <= 0 || topk_group <= 0)
        return TK_ERR_INVALID_ARG;
    if (experts % n_group != 0 || topk_group > n_group)
        return TK_ERR_INVALID_ARG;
    const int64_t per = experts / n_group;
    if ((n_group > 1 && per < 2) || k > topk_group * per)
        return TK_ERR_INVALID_ARG;
    if (tokens > 0 && (!scores || !topk_idx || !topk_weight))
        return TK_ERR_INVALID_ARG;
    if (((uintptr_t)scores & 3) || ((uintptr_t)topk_idx & 3) || ((uintptr_t)topk_weight & 3))
        return TK_ERR_INVALID_ARG;
    const size_t s_bytes = (size_t)tokens * (size_t)experts * 4u, o_bytes = (size_t)tokens * (size_t)k * 4u;
    if (tokens > 0 && (overlaps(topk_idx, o_bytes, scores, s_bytes) || overlaps(topk_weight, o_bytes, scores, s_bytes) ||
                       overlaps(topk_idx, o_bytes, topk_weight, o_bytes)))
        return TK_ERR_INVALID_ARG;
    if (experts > kMaxExperts || k > kWave)
        return TK_ERR_UNSUPPORTED;
    // Experts per lane for a layout of `lanes` lanes per token: the smallest C
    // from ceil(experts / lanes) up to 8 whose groups are blocks of 2^j whole
    // lanes (per % C == 0 and per / C a power of two); 0 when there is none.
    // A C above the minimum leaves the lanes past experts / C empty.
    auto experts_per_lane = [&](int64_t lanes, uint32_t& gl) -> uint32_t {
        for (int64_t c = (experts + lanes - 1) / lanes; c <= 8; ++c) {
            if (n_group == 1) {
                gl = 0;
                return (uint32_t)c;
            }
            const int64_t l = per / c;
            if (per % c == 0 && (l & (l - 1)) == 0) {
                gl = (uint32_t)__builtin_ctzll((unsigned long long)l);
                return (uint32_t)c;
            }
        }
        return 0;
    };
    // the two-tokens-per-wave layout (up to 256 experts, k <= 32) first, then one token per wave
    uint32_t gl2 = 0, gl_log2 = 0;
    const uint32_t C2 = (experts <= 8 * (kWave / 2) && k <= kWave / 2) ? experts_per_lane(kWave / 2, gl2) : 0u;
    const uint32_t C = C2 ? 0u : experts_per_lane(kWave, gl_log2);
    if (!C2 && !C)
        return TK_ERR_UNSUPPORTED;
    if (tokens == 0)
        return TK_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // no groups, up to 128 experts, k <= 16: one token per 16-lane row
    if (n_group == 1 && experts <= 128 && k <= 16) {
        const uint32_t tpb = 4 * (kThreads / kWave);
        const uint32_t rblocks = (uint32_t)((tokens + tpb - 1) / tpb);
#define TK_TOPK1_LAUNCH(CC, K8, FULL)                                                                         \
    hipLaunchKernelGGL((topk_row1_kernel<CC, K8, FULL>), dim3(rblocks), dim3(kThreads), 0, s, scores,         \
                       (uint32_t)tokens, (uint32_t)experts, (uint32_t)k, normalise, topk_idx, topk_weight)
#define TK_TOPK1(CC)                                                                                          \
    case CC:                                                                                                  \
        if (experts == 16 * (CC)) {                                                                           \
            if (k == 8) TK_TOPK1_LAUNCH(CC, true, true); else TK_TOPK1_LAUNCH(CC, false, true);               \
        } else {                                                                                              \
            if (k == 8) TK_TOPK1_LAUNCH(CC, true, false); else TK_TOPK1_LAUNCH(CC, false, false);             \
        }                                                                                                     \
        break;
        switch ((experts + 15) / 16) {
            TK_TOPK1(1)
            TK_TOPK1(2)
            TK_TOPK1(3)
            TK_TOPK1(4)
            TK_TOPK1(5)
            TK_TOPK1(6)
            TK_TOPK1(7)
            TK_TOPK1(8)
        }
#undef TK_TOPK1
#undef TK_TOPK1_LAUNCH
        return hipGetLastError() == hipSuccess ? TK_OK : TK_ERR_HIP;
    }
    // no groups, 129 to 256 experts, k <= 16: one token per 16-lane row, two lists per lane
    if (n_group == 1 && experts > 128 && experts <= 256 && k <= 16) {
        const uint32_t tpb = 4 * (kThreads / kWave);
        const uint32_t rblocks = (uint32_t)((tokens + tpb - 1) / tpb);
#define TK_TOPK2L_LAUNCH(CC, K8, FULL)                                                                        \
    hipLaunchKernelGGL((topk_row2_kernel<CC, K8, FULL>), dim3(rblocks), dim3(kThreads), 0, s, scores,         \
                       (uint32_t)tokens, (uint32_t)experts, (uint32_t)k, normalise, topk_idx, topk_weight)
#define TK_TOPK2L(CC)                                                                                         \
    case CC:                                                                                                  \
        if (experts == 32 * (CC)) {                                                                           \
            if (k == 8) TK_TOPK2L_LAUNCH(CC, true, true); else TK_TOPK2L_LAUNCH(CC, false, true);             \
        } else {                                                                                              \
            if (k == 8) TK_TOPK2L_LAUNCH(CC, true, false); else TK_TOPK2L_LAUNCH(CC, false, false);           \
        }                                                                                                     \
        break;
        switch ((experts + 31) / 32) {
            TK_TOPK2L(5)
            TK_TOPK2L(6)
            TK_TOPK2L(7)
            TK_TOPK2L(8)
        }
#undef TK_TOPK2L
#undef TK_TOPK2L_LAUNCH
        return hipGetLastError() == hipSuccess ? TK_OK : TK_ERR_HIP;
    }
    // no groups, 257 to 512 experts, k <= 16: one token per 16-lane row, L = 3 or 4 lists per lane
    if (n_group == 1 && experts > 256 && k <= 16) {
        const uint32_t tpb = 4 * (kThreads / kWave);
        const uint32_t rblocks = (uint32_t)((tokens + tpb - 1) / tpb);
        const uint32_t L = (uint32_t)((experts + 127) / 128), Cl = (uint32_t)((experts + 16 * L - 1) / (16 * L));
        const bool full = experts == (int64_t)(16 * L * Cl);
#define TK_TOPKL_LAUNCH(CC, LL, K8, FULL)                                                                     \
    hipLaunchKernelGGL((topk_rowl_kernel<CC, LL, K8, FULL>), dim3(rblocks), dim3(kThreads), 0, s, scores,     \
                       (uint32_t)tokens, (uint32_t)experts, (uint32_t)k, normalise, topk_idx, topk_weight)
#define TK_TOPKL(CC, LL)                                                                                      \
    if (Cl == (CC) && L == (LL)) {                                                                            \
        if (full) {                                                                                           \
            if (k == 8) TK_TOPKL_LAUNCH(CC, LL, true, true); else TK_TOPKL_LAUNCH(CC, LL, false, true);       \
        } else {                                                                                              \
            if (k == 8) TK_TOPKL_LAUNCH(CC, LL, true, false); else TK_TOPKL_LAUNCH(CC, LL, false, false);     \
        }                                                                                                     \
        return hipGetLastError() == hipSuccess ? TK_OK : TK_ERR_HIP;                                          \
    }
        TK_TOPKL(6, 3)
        TK_TOPKL(7, 3)
        TK_TOPKL(8, 3)
        TK_TOPKL(7, 4)
        TK_TOPKL(8, 4)
#undef TK_TOPKL
#undef TK_TOPKL_LAUNCH
    }
    // one token per 16-lane row in one pass: 16 * C16 experts (C16 even, 4 to
    // 16 per lane) in 2, 4 or 8 groups of 2^GL lanes, kept groups within 8 lanes
    if (experts % 32 == 0 && experts >= 64 && experts <= 256 && (n_group == 2 || n_group == 4 || n_group == 8) &&
        k <= 16) {
        const uint32_t GLr = (uint32_t)__builtin_ctzll((unsigned long long)(16 / n_group));
        if (2 * (topk_group << GLr) <= 16) {
            const uint32_t tpb = 4 * (kThreads / kWave);
            const uint32_t rblocks = (uint32_t)((tokens + tpb - 1) / tpb);
#define TK_TOPKR_LAUNCH(C16, K8, GL)                                                                          \
    hipLaunchKernelGGL((topk_row_kernel<C16, K8, GL>), dim3(rblocks), dim3(kThreads), 0, s, scores,           \
                       (uint32_t)tokens, (uint32_t)k, (uint32_t)topk_group, normalise, topk_idx, topk_weight)
#define TK_TOPKR(C16)                                                                                         \
    case C16:                                                                                                 \
        if (GLr == 1) {                                                                                       \
            if (k == 8) TK_TOPKR_LAUNCH(C16, true, 1); else TK_TOPKR_LAUNCH(C16, false, 1);                   \
        } else if (GLr == 2) {                                                                                \
            if (k == 8) TK_TOPKR_LAUNCH(C16, true, 2); else TK_TOPKR_LAUNCH(C16, false, 2);                   \
        } else {                                                                                              \
            if (k == 8) TK_TOPKR_LAUNCH(C16, true, 3); else TK_TOPKR_LAUNCH(C16, false, 3);                   \
        }                                                                                                     \
        break;
            switch (experts / 16) {
                TK_TOPKR(4)
                TK_TOPKR(6)
                TK_TOPKR(8)
                TK_TOPKR(10)
                TK_TOPKR(12)
                TK_TOPKR(14)
                TK_TOPKR(16)
            }
#undef TK_TOPKR
#undef TK_TOPKR_LAUNCH
            return hipGetLastError() == hipSuccess ? TK_OK : TK_ERR_HIP;
        }
    }
    if (C2) {
        // four tokens per wave when each token's kept groups fit one 16-lane row
        const bool quad = n_group >= 2 && n_group <= 8 && (topk_group << gl2) <= 16 && k <= 16;
        const uint32_t tpb = (quad ? 4 : 2) * (kThreads / kWave);
        const uint32_t pblocks = (uint32_t)((tokens + tpb - 1) / tpb);
#define TK_TOPK2_LAUNCH(CC, FULL, K8)                                                                         \
    if (quad)                                                                                                 \
        hipLaunchKernelGGL((topk_quad_kernel<CC, FULL, K8>), dim3(pblocks), dim3(kThreads), 0, s, scores,     \
                           (uint32_t)tokens, (uint32_t)experts, (uint32_t)k, (uint32_t)n_group,               \
                           (uint32_t)topk_group, gl2, normalise, topk_idx, topk_weight);                      \
    else                                                                                                      \
        hipLaunchKernelGGL((topk_pair_kernel<CC, FULL, K8>), dim3(pblocks), dim3(kThreads), 0, s, scores,     \
                           (uint32_t)tokens, (uint32_t)experts, (uint32_t)k, (uint32_t)n_group,               \
                           (uint32_t)topk_group, gl2, normalise, topk_idx, topk_weight)
#define TK_TOPK2(CC)                                                                                          \
    if (experts == 32 * (CC)) {                                                                               \
        if (k == 8)                                                                                           \
            TK_TOPK2_LAUNCH(CC, true, true);                                                                  \
        else                                                                                                  \
            TK_TOPK2_LAUNCH(CC, true, false);                                                                 \
    } else {                                                                                                  \
        if (k == 8)                                                                                           \
            TK_TOPK2_LAUNCH(CC, false, true);                                                                 \
        else                                                                                                  \
            TK_TOPK2_LAUNCH(CC, false, false);                                                                \
    }
        switch (C2) {
        case 1: TK_TOPK2(1); break;
        case 2: TK_TOPK2(2); break;
        case 3: TK_TOPK2(3); break;
        case 4: TK_TOPK2(4); break;
        case 5: TK_TOPK2(5); break;
        case 6: TK_TOPK2(6); break;
        case 7: TK_TOPK2(7); break;
        default: TK_TOPK2(8); break;
        }
#undef TK_TOPK2
#undef TK_TOPK2_LAUNCH
        return hipGetLastError() == hipSuccess ? TK_OK : TK_ERR_HIP;
    }
    const uint32_t blocks = (uint32_t)((tokens + kThreads / kWave - 1) / (kThreads / kWave));
#define TK_TOPK(CC)                                                                                           \
    hipLaunchKernelGGL(topk_kernel<CC>, dim3(blocks), dim3(kThreads), 0, s, scores, (uint32_t)tokens,         \
                       (uint32_t)experts, (uint32_t)k, (uint32_t)n_group, (uint32_t)topk_group, gl_log2, normalise, \
                       topk_idx, topk_weight)
    switch (C) {
    case 1: TK_TOPK(1); break;
    case 2: TK_TOPK(2); break;
    case 3: TK_TOPK(3); break;
    case 4: TK_TOPK(4); break;
    case 5: TK_TOPK(5); break;
    case 6: TK_TOPK(6); break;
    case 7: TK_TOPK(7); break;
    default: TK_TOPK(8); break;
    }
#undef TK_TOPK
    return hipGetLastError() == hipSuccess ? TK_OK : TK_ERR_HIP;
}
