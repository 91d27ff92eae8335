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
