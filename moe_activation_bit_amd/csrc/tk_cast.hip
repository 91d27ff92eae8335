// tk_cast.hip -- the stand-alone per-token / per-block cast of bf16 or fp32
// rows to FP8 E4M3 or FP4 E2M1 codes with fp32 or UE8M0 scales, behind the
// C ABI in include/tk.h (tk_cast_fp8, tk_cast_fp4).
//
// It is the "per_token_cast" of "【DeepSeek】TileKernels从入门到精通" ch.1
// ("透视底层", "闭环": a dtype/shape-specialised cast kernel with T.dynamic row
// count and an abs-max reduction) and the "cast" of the unfused reference in
// ch.5 "越过性能红线" (swiglu_forward, then cast).  The abs-max -> scale ->
// cast tail is the fused kernel's (tk_quant.h), so a value quantises to the
// same code on either path.
//
// gfx950 layout: as in the fused kernel a wave owns units of 512-column steps;
// lane l holds the 8 columns of slot 64*step + l (16 bytes of bf16, or 32
// bytes of fp32 as two 16-byte loads).  No table is needed, so the grid is
// non-persistent: one unit per wave, which streams fastest on MI355X.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "tk.h"
#include "tk_quant.h"

namespace {

using namespace tk_detail;

constexpr uint32_t kMaxCastBlocks = 1u << 20; // 2^28 threads: far more than the chip holds
constexpr uint32_t kMaxCastXwBlocks = 2048;    // multi-wave groups: 8 workgroups per CU

__device__ __forceinline__ float bf16_lo(uint32_t w) { return as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return as_float(w & 0xFFFF0000u); }

// Load unit u (SPU steps of one row, 16 or 32 bytes per lane per step),
// widen it to fp32 and take the lane-local abs-max of every step.
template <bool F32IN, int SPU, bool ROWRED, bool PARTIAL>
__device__ __forceinline__ void cast_load_unit(const Params& p, uint32_t u, uint32_t lane, uint32_t& row,
                                               uint32_t& unit_in_row, uint32_t& step0, uint32_t& nst,
                                               float (&y)[SPU][8], uint32_t (&mbits)[SPU])
{
    constexpr uint32_t kSlotBytes = F32IN ? 32u : 16u;
    row = u / p.upr;
    unit_in_row = u - row * p.upr;
    step0 = unit_in_row * p.spu;
    nst = ROWRED ? min(p.spu, p.steps_row - step0) : (uint32_t)SPU;
    const char* xr = reinterpret_cast<const char*>(p.x) + (size_t)row * (p.slots * kSlotBytes);
    const uint32_t lane_off = (step0 * kWaveSize + lane) * kSlotBytes;

    uint4 raw[SPU][F32IN ? 2 : 1];
#pragma unroll
    for (int s = 0; s < SPU; ++s) {
        if (!ROWRED || s < (int)nst) {
            uint32_t off = lane_off + (uint32_t)s * (kWaveSize * kSlotBytes);
            if (PARTIAL) // lanes past the row end re-read its last slot
                off = min(off, (p.slots - 1u) * kSlotBytes);
            raw[s][0] = load16(reinterpret_cast<const uint4*>(xr + off));
            if constexpr (F32IN)
                raw[s][F32IN ? 1 : 0] = load16(reinterpret_cast<const uint4*>(xr + off + 16u));
        }
    }

#pragma unroll
    for (int s = 0; s < SPU; ++s) {
        if (!ROWRED || s < (int)nst) {
            if constexpr (F32IN) {
                const uint4 a = raw[s][0], b = raw[s][F32IN ? 1 : 0];
                const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    y[s][j] = as_float(w[j]);
            } else {
                const uint32_t w[4] = {raw[s][0].x, raw[s][0].y, raw[s][0].z, raw[s][0].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    y[s][2 * k] = bf16_lo(w[k]);
                    y[s][2 * k + 1] = bf16_hi(w[k]);
                }
            }
            float m = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; j += 2)
                m = fmaxf(m, fmaxf(fabsf(y[s][j]), fabsf(y[s][j + 1])));
            if (PARTIAL && (step0 + s) * kWaveSize + lane >= p.slots)
                m = 0.0f;
            mbits[s] = as_uint(m);
        }
    }
}

template <int FMT, int SFMT, bool F32IN, int SPU, bool ROWRED, bool PARTIAL>
__global__ __launch_bounds__(kThreads) void cast_kernel(Params p)
{
    const uint32_t lane = threadIdx.x & (kWaveSize - 1);
    const uint32_t waves_per_block = kThreads / kWaveSize;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(blockIdx.x * waves_per_block + (threadIdx.x / kWaveSize));
    const uint32_t nwaves = gridDim.x * waves_per_block;

    for (uint32_t u = wave; u < p.units; u += nwaves) {
        uint32_t row, unit_in_row, step0, nst;
        float y[SPU][8];
        uint32_t mbits[SPU];
        cast_load_unit<F32IN, SPU, ROWRED, PARTIAL>(p, u, lane, row, unit_in_row, step0, nst, y, mbits);
        quantize_unit<FMT, SFMT, SPU, ROWRED, PARTIAL>(p, lane, row, unit_in_row, step0, nst, y, mbits);
    }
}

// Row-reduced groups longer than one wave holds: W waves of a workgroup share
// one group (each ceil(k/W) of its k steps), their abs-maxes meet in LDS, and
// every wave quantises its own steps; the group's first wave stores the scale.
// A workgroup takes passes of 4/W groups, grid-strided over a capped grid (the
// maxes double-buffered, one barrier per pass; every wave runs the same
// passes, so all of them reach it).
template <int FMT, int SFMT, bool F32IN, int SPU, bool PARTIAL, int W>
__global__ __launch_bounds__(kThreads) void cast_xw_kernel(Params p)
{
    constexpr uint32_t kWaves = kThreads / kWaveSize;
    constexpr uint32_t kGroupsPerPass = kWaves / W;
    static_assert(kWaves % W == 0, "waves per group must divide the workgroup");
    __shared__ uint32_t part_max[2][kWaves];
    const uint32_t lane = threadIdx.x & (kWaveSize - 1);
    const uint32_t wib = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
    const uint32_t slot_in_pass = wib / W, part = wib % W;
    const uint32_t groups = p.units / W;
    const uint32_t passes = (groups + kGroupsPerPass - 1) / kGroupsPerPass;
    uint32_t parity = 0;
    for (uint32_t it = blockIdx.x; it < passes; it += gridDim.x, parity ^= 1u) {
        const uint32_t g = it * kGroupsPerPass + slot_in_pass;
        const bool valid = g < groups; // wave-uniform
        uint32_t row = 0, unit_in_row = 0, step0 = 0, nst = 0, mb = 0;
        float y[SPU][8];
        uint32_t mbits[SPU];
        if (valid) {
            cast_load_unit<F32IN, SPU, true, PARTIAL>(p, g * W + part, lane, row, unit_in_row, step0, nst, y,
                                                       mbits);
            mb = wave_umax(lane_max<SPU>(mbits, nst));
        }
        if (lane == 0)
            part_max[parity][wib] = mb;
        __syncthreads();
        uint32_t gm = 0;
#pragma unroll
        for (int j = 0; j < W; ++j)
            gm = max(gm, part_max[parity][slot_in_pass * W + j]);
        if (valid)
            quantize_rowred<FMT, SFMT, SPU, PARTIAL>(p, lane, row, unit_in_row / W, step0, nst, y, gm,
                                                     part == 0 && lane == 0);
    }
}

// A span of `nslots` lane slots of row `row` from slot `slot0` on, widened to
// fp32: lane l of step s holds slot slot0 + 64*s + l; lanes past the span
// re-read its last slot and give abs-max bits 0.  Loads run up to four steps
// ahead of the widening.  Used by the segmented and two-pass kernels, whose
// spans start at any slot.  NT: non-temporal loads (data read once); a
// two-pass group's first read leaves NT off so that its second read finds
// the data in the caches.
template <bool F32IN, int SPU, bool NT = true>
__device__ __forceinline__ void cast_span_load(const Params& p, uint32_t lane, uint32_t row, uint32_t slot0,
                                               uint32_t nslots, float (&y)[SPU][8], uint32_t (&mbits)[SPU])
{
    constexpr uint32_t kSlotBytes = F32IN ? 32u : 16u;
    constexpr int D = SPU < 4 ? SPU : 4;
    constexpr int P = F32IN ? 2 : 1;
    const char* xr = reinterpret_cast<const char*>(p.x) + (size_t)row * (p.slots * kSlotBytes);
    const uint32_t last = slot0 + nslots - 1u;
    auto off = [&](int s) { return min(slot0 + (uint32_t)s * kWaveSize + lane, last) * kSlotBytes; };
    auto ld = [](const char* a) { return NT ? load16(reinterpret_cast<const uint4*>(a)) : *reinterpret_cast<const uint4*>(a); };
    uint4 q[D][P];
#pragma unroll
    for (int s = 0; s < D; ++s)
#pragma unroll
        for (int h = 0; h < P; ++h)
            q[s][h] = ld(xr + off(s) + 16u * h);
#pragma unroll
    for (int s = 0; s < SPU; ++s) {
        uint4 cur[P];
#pragma unroll
        for (int h = 0; h < P; ++h)
            cur[h] = q[s % D][h];
        if (s + D < SPU) {
#pragma unroll
            for (int h = 0; h < P; ++h)
                q[s % D][h] = ld(xr + off(s + D) + 16u * h);
        }
        if constexpr (F32IN) {
            const uint32_t w[8] = {cur[0].x, cur[0].y, cur[0].z, cur[0].w,
                                   cur[P - 1].x, cur[P - 1].y, cur[P - 1].z, cur[P - 1].w};
#pragma unroll
            for (int j = 0; j < 8; ++j)
                y[s][j] = as_float(w[j]);
        } else {
            const uint32_t w[4] = {cur[0].x, cur[0].y, cur[0].z, cur[0].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                y[s][2 * k] = bf16_lo(w[k]);
                y[s][2 * k + 1] = bf16_hi(w[k]);
            }
        }
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; j += 2)
            m = fmaxf(m, fmaxf(fabsf(y[s][j]), fabsf(y[s][j + 1])));
        mbits[s] = (uint32_t)s * kWaveSize + lane < nslots ? as_uint(m) : 0u;
    }
}

// Groups whose width is not a power of two of lane slots up to 64 and not a
// multiple of 64, up to 8192 columns: each unit is a run of whole groups of
// one row that one wave holds in SPU steps, reduced in the wave's own LDS
// buffer (quantize_seg).  One unit per wave, like cast_kernel.
template <int FMT, int SFMT, bool F32IN, int SPU>
__global__ __launch_bounds__(kThreads) void cast_seg_kernel(Params p)
{
    constexpr int kWaves = kThreads / kWaveSize;
    __shared__ uint32_t seg_buf[kWaves][SegLds<SPU>::kSlots];
    __shared__ float seg_inv[kWaves][SegLds<SPU>::kGroups];
    const uint32_t lane = threadIdx.x & (kWaveSize - 1);
    const uint32_t wib = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + wib);
    const uint32_t nwaves = gridDim.x * kWaves;
    for (uint32_t u = wave; u < p.units; u += nwaves) {
        const uint32_t row = u / p.upr;
        const uint32_t g0 = (u - row * p.upr) * p.gpu;
        const uint32_t ngr = min(p.gpu, p.groups_row - g0);
        const uint32_t slot0 = g0 * p.gslots;
        float y[SPU][8];
        uint32_t mbits[SPU];
        cast_span_load<F32IN, SPU>(p, lane, row, slot0, ngr * p.gslots, y, mbits);
        quantize_seg<FMT, SFMT, SPU>(p, lane, row, g0, ngr, slot0, y, mbits, seg_buf[wib], seg_inv[wib]);
    }
}

// Groups no other kernel covers (wider than 8192 columns and not split evenly
// over 2 or 4 waves, or wider than 32768 columns): one wave per group, which
// reads the group twice, kTwoPassSteps steps at a time -- first for its
// abs-max, then for the codes with the group's scale.
template <int FMT, int SFMT, bool F32IN>
__global__ __launch_bounds__(kThreads) void cast_2p_kernel(Params p)
{
    constexpr int S = kTwoPassSteps;
    constexpr uint32_t kChunk = S * kWaveSize;
    constexpr int kWaves = kThreads / kWaveSize;
    const uint32_t lane = threadIdx.x & (kWaveSize - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x / kWaveSize));
    const uint32_t nwaves = gridDim.x * kWaves;
    const uint32_t gs = p.gslots;
    for (uint32_t u = wave; u < p.units; u += nwaves) {
        const uint32_t row = u / p.upr;
        const uint32_t k = u - row * p.upr;
        const uint32_t slot0 = k * gs;
        uint32_t mb = 0;
        for (uint32_t c = 0; c < gs; c += kChunk) {
            float y[S][8];
            uint32_t mbits[S];
            cast_span_load<F32IN, S, false>(p, lane, row, slot0 + c, min(kChunk, gs - c), y, mbits);
            mb = max(mb, lane_max<S>(mbits, S));
        }
        mb = wave_umax(mb);
        float s32 = 0.0f;
        uint32_t s8 = 0;
        const float inv = group_scale<FMT, SFMT>(mb, s32, s8);
        if (lane == 0)
            store_scale<SFMT>(p, row, k, s32, s8);
        uint8_t* row_codes = p.codes + (size_t)row * (FMT == 8 ? p.slots * 8u : p.slots * 4u);
        for (uint32_t c = 0; c < gs; c += kChunk) {
            float y[S][8];
            uint32_t mbits[S];
            cast_span_load<F32IN, S>(p, lane, row, slot0 + c, min(kChunk, gs - c), y, mbits);
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const uint32_t rel = c + (uint32_t)s * kWaveSize + lane;
                if (rel < gs)
                    quantize_store<FMT>(row_codes, slot0 + rel, y[s], inv);
            }
        }
    }
}

template <int FMT, int SFMT, bool F32IN>
bool launch_cast_seg(const UnitPlan& plan, const Params& p, int blocks, hipStream_t s)
{
    if (plan.twopass) {
        hipLaunchKernelGGL((cast_2p_kernel<FMT, SFMT, F32IN>),
                           dim3(blocks < (int)kMaxCastXwBlocks ? blocks : (int)kMaxCastXwBlocks), dim3(kThreads), 0, s,
                           p);
        return true;
    }
    switch (plan.spu_max) {
#define TK_CAST_SEG(N)                                                                                          \
    case N:                                                                                                     \
        hipLaunchKernelGGL((cast_seg_kernel<FMT, SFMT, F32IN, N>), dim3(blocks), dim3(kThreads), 0, s, p);      \
        return true;
        TK_CAST_SEG(1)
        TK_CAST_SEG(2)
        TK_CAST_SEG(4)
        TK_CAST_SEG(8)
        TK_CAST_SEG(12)
        TK_CAST_SEG(16)
#undef TK_CAST_SEG
    default: return false;
    }
}

template <int FMT, int SFMT, bool F32IN, bool ROWRED, bool PARTIAL>
bool launch_cast(int spu_max, const Params& p, int blocks, hipStream_t s)
{
#define TK_CAST_CASE(N)                                                                                 \
    case N:                                                                                             \
        hipLaunchKernelGGL((cast_kernel<FMT, SFMT, F32IN, N, ROWRED, PARTIAL>), dim3(blocks), dim3(kThreads), \
                           0, s, p);                                                                    \
        return true;
    switch (spu_max) {
        TK_CAST_CASE(1)
        TK_CAST_CASE(2)
        TK_CAST_CASE(4)
    case 8:
        if constexpr (ROWRED) {
            hipLaunchKernelGGL((cast_kernel<FMT, SFMT, F32IN, 8, ROWRED, PARTIAL>), dim3(blocks), dim3(kThreads), 0,
                               s, p);
            return true;
        }
        return false;
    case 12:
        if constexpr (ROWRED) {
            hipLaunchKernelGGL((cast_kernel<FMT, SFMT, F32IN, 12, ROWRED, PARTIAL>), dim3(blocks), dim3(kThreads),
                               0, s, p);
            return true;
        }
        return false;
    case 16:
        if constexpr (ROWRED) {
            hipLaunchKernelGGL((cast_kernel<FMT, SFMT, F32IN, 16, ROWRED, PARTIAL>), dim3(blocks), dim3(kThreads),
                               0, s, p);
            return true;
        }
        return false;
    default:
        return false;
    }
#undef TK_CAST_CASE
}

template <int FMT, int SFMT, bool F32IN>
bool dispatch_cast2(const UnitPlan& plan, const Params& p, int blocks, hipStream_t s)
{
    const int spu = (int)plan.spu_max;
    if (plan.rowred)
        return plan.partial ? launch_cast<FMT, SFMT, F32IN, true, true>(spu, p, blocks, s)
                            : launch_cast<FMT, SFMT, F32IN, true, false>(spu, p, blocks, s);
    return plan.partial ? launch_cast<FMT, SFMT, F32IN, false, true>(spu, p, blocks, s)
                        : launch_cast<FMT, SFMT, F32IN, false, false>(spu, p, blocks, s);
}

template <int FMT, int SFMT, bool F32IN>
bool launch_cast_xw(const UnitPlan& plan, const Params& p, hipStream_t s)
{
    // one pass per workgroup up to 2048 workgroups (8 per CU), passes beyond
    uint32_t blocks = (p.units + (kThreads / kWaveSize) - 1) / (kThreads / kWaveSize);
    if (blocks > kMaxCastXwBlocks)
        blocks = kMaxCastXwBlocks;
#define TK_CAST_XW(SP, PA, WW)                                                                           \
    if (plan.spu_max == SP && plan.partial == PA && plan.xwaves == WW) {                                  \
        hipLaunchKernelGGL((cast_xw_kernel<FMT, SFMT, F32IN, SP, PA, WW>), dim3(blocks), dim3(kThreads), 0, s, p); \
        return true;                                                                                      \
    }
    // a wave's share, ceil(k / W), is 9..16 steps
    TK_CAST_XW(12u, false, 2u)
    TK_CAST_XW(12u, false, 4u)
    TK_CAST_XW(12u, true, 2u)
    TK_CAST_XW(12u, true, 4u)
    TK_CAST_XW(16u, false, 2u)
    TK_CAST_XW(16u, false, 4u)
    TK_CAST_XW(16u, true, 2u)
    TK_CAST_XW(16u, true, 4u)
#undef TK_CAST_XW
    return false;
}

template <int FMT>
bool dispatch_cast(int sfmt, bool f32in, const UnitPlan& plan, const Params& p, int blocks, hipStream_t s)
{
    if (plan.seg || plan.twopass) {
        if (sfmt == TK_SCALE_FP32)
            return f32in ? launch_cast_seg<FMT, TK_SCALE_FP32, true>(plan, p, blocks, s)
                         : launch_cast_seg<FMT, TK_SCALE_FP32, false>(plan, p, blocks, s);
        return f32in ? launch_cast_seg<FMT, TK_SCALE_UE8M0, true>(plan, p, blocks, s)
                     : launch_cast_seg<FMT, TK_SCALE_UE8M0, false>(plan, p, blocks, s);
    }
    if (plan.xwaves > 1) {
        if (sfmt == TK_SCALE_FP32)
            return f32in ? launch_cast_xw<FMT, TK_SCALE_FP32, true>(plan, p, s)
                         : launch_cast_xw<FMT, TK_SCALE_FP32, false>(plan, p, s);
        return f32in ? launch_cast_xw<FMT, TK_SCALE_UE8M0, true>(plan, p, s)
                     : launch_cast_xw<FMT, TK_SCALE_UE8M0, false>(plan, p, s);
    }
    if (sfmt == TK_SCALE_FP32)
        return f32in ? dispatch_cast2<FMT, TK_SCALE_FP32, true>(plan, p, blocks, s)
                     : dispatch_cast2<FMT, TK_SCALE_FP32, false>(plan, p, blocks, s);
    return f32in ? dispatch_cast2<FMT, TK_SCALE_UE8M0, true>(plan, p, blocks, s)
                 : dispatch_cast2<FMT, TK_SCALE_UE8M0, false>(plan, p, blocks, s);
}

tk_status cast(int fmt, const void* x, int in_dtype, int64_t n, int64_t hidden, int64_t group_size, int scale_fmt,
               void* codes, void* scales, void* stream)
{
    // ---- validation: no HIP call before every argument is checked ----
    if (n < 0 || n >= (int64_t)INT_MAX)
        return TK_ERR_INVALID_ARG;
    if (hidden <= 0 || hidden % kSlotCols != 0 || hidden > (int64_t)INT_MAX / 8)
        return TK_ERR_INVALID_ARG;
    if (group_size < 0 || (group_size != 0 && (group_size % kSlotCols != 0 || hidden % group_size != 0)))
        return TK_ERR_INVALID_ARG;
    if (in_dtype != TK_DTYPE_BF16 && in_dtype != TK_DTYPE_FP32)
        return TK_ERR_INVALID_ARG;
    const int64_t groups_row = hidden / (group_size ? group_size : hidden);
    ScaleSpec sp;
    if (!scale_spec(scale_fmt, n, groups_row, sp))
        return TK_ERR_INVALID_ARG;
    if (n > 0 && (!x || !codes || !scales))
        return TK_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(codes, fmt == 8 ? 8 : 4) || !aligned(scales, sp.align))
        return TK_ERR_INVALID_ARG;
    const size_t x_bytes = (size_t)n * (size_t)hidden * (in_dtype == TK_DTYPE_FP32 ? 4u : 2u);
    const size_t c_bytes = (size_t)n * (size_t)(fmt == 8 ? hidden : hidden / 2);
    const size_t s_bytes = sp.bytes;
    if (n > 0 && (overlaps(codes, c_bytes, x, x_bytes) || overlaps(scales, s_bytes, x, x_bytes) ||
                  overlaps(codes, c_bytes, scales, s_bytes)))
        return TK_ERR_INVALID_ARG;

    Params p{};
    UnitPlan plan;
    {
        const tk_status rc = plan_units(n, hidden, group_size, n >= 1024 ? 4u : (n >= 256 ? 2u : 1u), p, plan);
        if (rc != TK_OK)
            return rc;
    }
    if (n == 0)
        return TK_OK;
    p.x = static_cast<const uint4*>(x);
    p.codes = static_cast<uint8_t*>(codes);
    p.scales = scales;
    p.scale_layout = sp.layout;
    p.scale_ld = sp.ld;

    const uint32_t waves_per_block = kThreads / kWaveSize;
    // one unit per wave; a grid past kMaxCastBlocks loops (a launch holds at
    // most 2^32 work-items)
    const uint32_t want = (p.units + waves_per_block - 1) / waves_per_block;
    const int blocks = (int)(want < kMaxCastBlocks ? want : kMaxCastBlocks);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool f32in = in_dtype == TK_DTYPE_FP32;
    const bool ok = fmt == 8 ? dispatch_cast<8>(sp.kind, f32in, plan, p, blocks, s)
                             : dispatch_cast<4>(sp.kind, f32in, plan, p, blocks, s);
    if (!ok)
        return TK_ERR_UNSUPPORTED;
    return hipGetLastError() == hipSuccess ? TK_OK : TK_ERR_HIP;
}

} // namespace

extern "C" {

tk_status tk_cast_fp8(const void* x, tk_dtype in_dtype, int64_t n, int64_t hidden, int64_t group_size,
                      tk_scale_fmt scale_fmt, void* codes, void* scales, void* stream)
{
    return cast(8, x, (int)in_dtype, n, hidden, group_size, (int)scale_fmt, codes, scales, stream);
}

tk_status tk_cast_fp4(const void* x, tk_dtype in_dtype, int64_t n, int64_t hidden, int64_t group_size,
                      tk_scale_fmt scale_fmt, void* codes, void* scales, void* stream)
{
    return cast(4, x, (int)in_dtype, n, hidden, group_size, (int)scale_fmt, codes, scales, stream);
}

} // extern "C"
