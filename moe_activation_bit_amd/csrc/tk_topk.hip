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
// gfx950 design: one 64-lane wave per token (the pages use a 32-lane warp);
// lane l holds experts l*C .. l*C+C-1 (C = ceil(experts/64) <= 4), so a group
// of experts is a block of consecutive lanes.  Group top-2 sums come from an
// xor-butterfly over the group's lanes; group ranks from wave-uniform reads of
// every group's sum.  Each of the k picks is a wave-wide max of a 64-bit key
// (order-preserving score bits above the complemented expert index), so the
// larger score wins and equal scores go to the smaller index; -0 and +0
// compare equal.  The winner's own score is read back from its lane.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "tk.h"

namespace {

constexpr int kWave = 64;
constexpr int kThreads = 256;
constexpr int kMaxExperts = 256;

__device__ __forceinline__ uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float ffrom(uint32_t u) { return __builtin_bit_cast(float, u); }

// Order-preserving map of a (non-NaN) float to uint32; -0 and +0 map alike.
__device__ __forceinline__ uint32_t ordered(float f)
{
    const uint32_t b = fbits(f + 0.0f); // -0 + +0 = +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// "a beats b": larger score, or equal score and smaller index
__device__ __forceinline__ bool beats(float sa, uint32_t a, float sb, uint32_t b)
{
    return sa > sb || (sa == sb && a < b);
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

    float s[C];
    bool allowed[C];
#pragma unroll
    for (int j = 0; j < C; ++j) {
        const uint32_t e = lane * C + j;
        allowed[j] = e < experts;
        s[j] = allowed[j] ? s_row[e] : 0.0f;
    }

    if (n_group > 1) {
        // the two best values of this lane's experts, then of the group's lanes
        float a1 = -INFINITY, a2 = -INFINITY;
#pragma unroll
        for (int j = 0; j < C; ++j) {
            if (allowed[j]) {
                const float v = s[j];
                if (v > a1) {
                    a2 = a1;
                    a1 = v;
                } else if (v > a2) {
                    a2 = v;
                }
            }
        }
        for (uint32_t m = 1; m < (1u << gl_log2); m <<= 1) {
            const float b1 = __shfl_xor(a1, (int)m), b2 = __shfl_xor(a2, (int)m);
            const float hi = fmaxf(a1, b1);
            a2 = fmaxf(fminf(a1, b1), fmaxf(a2, b2));
            a1 = hi;
        }
        const float gsum = a1 + a2;
        const uint32_t my_g = lane >> gl_log2;
        uint32_t rank = 0;
        for (uint32_t h = 0; h < n_group; ++h) {
            const float gh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(fbits(gsum), h << gl_log2));
            rank += beats(gh, h, gsum, my_g) ? 1u : 0u;
        }
        const bool keep = rank < topk_group;
#pragma unroll
        for (int j = 0; j < C; ++j)
            allowed[j] = allowed[j] && keep;
    }

    bool taken[C];
#pragma unroll
    for (int j = 0; j < C; ++j)
        taken[j] = false;
    int32_t my_idx = 0;
    float my_w = 0.0f, sum = 0.0f;
    for (uint32_t it = 0; it < k; ++it) {
        uint32_t hi = 0, lo = 0; // best key of this lane
#pragma unroll
        for (int j = 0; j < C; ++j) {
            if (allowed[j] && !taken[j]) {
                const uint32_t h = ordered(s[j]), l = 0xFFFFFFFFu - (lane * C + j);
                if (h > hi || (h == hi && l > lo)) {
                    hi = h;
                    lo = l;
                }
            }
        }
        for (int m = 1; m < kWave; m <<= 1) {
            const uint32_t oh = (uint32_t)__shfl_xor((int)hi, m), ol = (uint32_t)__shfl_xor((int)lo, m);
            if (oh > hi || (oh == hi && ol > lo)) {
                hi = oh;
                lo = ol;
            }
        }
        const uint32_t e = __builtin_amdgcn_readfirstlane(0xFFFFFFFFu - lo);
        const uint32_t owner = e / C, slot = e - owner * C;
        uint32_t mine = 0;
#pragma unroll
        for (int j = 0; j < C; ++j)
            if ((uint32_t)j == slot)
                mine = fbits(s[j]);
        const float score = ffrom(__builtin_amdgcn_readlane(mine, owner)); // the winner's own value (keeps -0)
        if (lane == owner) {
#pragma unroll
            for (int j = 0; j < C; ++j)
                if ((uint32_t)j == slot)
                    taken[j] = true;
        }
        if (lane == it) {
            my_idx = (int32_t)e;
            my_w = score;
        }
        sum += score; // best first, as the weights are normalised
    }
    if (lane < k) {
        idx_out[(size_t)t * k + lane] = my_idx;
        w_out[(size_t)t * k + lane] = (normalise && sum != 0.0f) ? my_w / sum : my_w;
    }
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
    const uint32_t C = (uint32_t)((experts + kWave - 1) / kWave);
    uint32_t gl_log2 = 0;
    if (n_group > 1) {
        // a group must be a block of 2^j whole lanes
        if (per % C != 0)
            return TK_ERR_UNSUPPORTED;
        const uint32_t lanes = (uint32_t)(per / C);
        if ((lanes & (lanes - 1)) != 0)
            return TK_ERR_UNSUPPORTED;
        gl_log2 = (uint32_t)__builtin_ctz(lanes);
    }
    if (tokens == 0)
        return TK_OK;
    const uint32_t blocks = (uint32_t)((tokens + kThreads / kWave - 1) / (kThreads / kWave));
    hipStream_t s = static_cast<hipStream_t>(stream);
#define TK_TOPK(CC)                                                                                           \
    hipLaunchKernelGGL(topk_kernel<CC>, dim3(blocks), dim3(kThreads), 0, s, scores, (uint32_t)tokens,         \
                       (uint32_t)experts, (uint32_t)k, (uint32_t)n_group, (uint32_t)topk_group, gl_log2, normalise, \
                       topk_idx, topk_weight)
    switch (C) {
    case 1: TK_TOPK(1); break;
    case 2: TK_TOPK(2); break;
    case 3: TK_TOPK(3); break;
    default: TK_TOPK(4); break;
    }
#undef TK_TOPK
    return hipGetLastError() == hipSuccess ? TK_OK : TK_ERR_HIP;
}
