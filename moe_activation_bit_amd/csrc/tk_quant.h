// tk_quant.h -- device and host pieces shared by the fused SwiGLU + cast
// kernels (tk_swiglu_cast.hip) and the stand-alone cast (tk_cast.hip): the
// launch parameters, the wave/group abs-max reductions, the scale of a group
// and the quantise-and-store tail.  The operation they implement is the
// abs-max -> scale factor -> FP8/FP4 step of "【DeepSeek】TileKernels从入门到精通"
// ch.2 "算子融合的“三重境界”" (step 3) with the formats of "TileLang +
// TileKernels：DeepSeek 的 GPU 内核开发新范式" "3. Quantization".
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cstdint>

#include "tk.h"

namespace tk_detail {

constexpr int kWaveSize = 64;
constexpr int kSlotCols = 8;                     // columns per lane per step (16 B of bf16)
constexpr int kMaxStepsPerUnit = 16;             // steps one wave holds: 8192 columns
constexpr int kMaxWavesPerGroup = 4;             // a row-reduced group split over up to 4 waves: 32768 columns

__device__ __forceinline__ float as_float(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_uint(float f) { return __builtin_bit_cast(uint32_t, f); }

struct Params {
    const uint4* x;         // [n][2*slots] 16-byte lane slots (gate slots, then up slots)
    const float* w;         // [n] or null
    uint8_t* codes;         // fp8: [n][hidden]; fp4: [n][hidden/2]
    void* scales;           // [n][groups_row], fp32 or uint8
    unsigned long long* count;
    uint32_t slots;         // hidden / 8
    uint32_t steps_row;     // ceil(slots / 64)
    uint32_t upr;           // units per row
    uint32_t spu;           // steps per unit (<= SPU)
    uint32_t units;         // n * upr
    uint32_t gl_log2;       // per-block: lanes per group = 1 << gl_log2
    uint32_t groups_row;    // scales per row
    float clamp;            // L (clamp variants)
    uint32_t scale_layout;  // kScaleRowMajor, kScaleColMajor or kScalePacked
    uint32_t scale_ld;      // column-major / packed: elements between consecutive groups' columns
    uint32_t gslots;        // segmented and two-pass units: lane slots (8 columns) per group
    uint32_t gpu;           // segmented units: groups per unit
    uint32_t gmagic;        // segmented units: ceil(2^32 / gslots), so that q / gslots = mulhi(q, gmagic)
    uint32_t xcd_order;     // fused grid-stride kernels: 1 = XCD-contiguous block order (grid a multiple of 8)
};

// Scale layouts (the value kind -- fp32 or UE8M0 byte -- is the SFMT template):
//   row-major [n][groups];  column-major [groups][ld] (ld >= n, 16-byte
//   aligned columns);  packed [ceil(groups/4)][ld] 32-bit words holding the
//   UE8M0 bytes of groups 4j..4j+3 of one row, lowest group in the low byte.
constexpr uint32_t kScaleRowMajor = 0;
constexpr uint32_t kScaleColMajor = 1;
constexpr uint32_t kScalePacked = 2;

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

// Abs-max reductions run on the bit patterns of non-negative floats, whose
// unsigned order is their numeric order; umax with identity 0 folds into a
// single v_max_u32_dpp per butterfly step.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v)
{
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false));
}

// max over the 2^gl_log2 consecutive lanes of each group (all lanes active)
__device__ __forceinline__ uint32_t group_umax(uint32_t v, uint32_t gl_log2)
{
    if (gl_log2 >= 1) v = dpp_umax<0xB1>(v);  // quad_perm [1,0,3,2]: lane ^ 1
    if (gl_log2 >= 2) v = dpp_umax<0x4E>(v);  // quad_perm [2,3,0,1]: lane ^ 2
    if (gl_log2 >= 3) v = dpp_umax<0x141>(v); // row_half_mirror: quads of 8 lanes
    if (gl_log2 >= 4) v = dpp_umax<0x140>(v); // row_mirror: halves of 16 lanes
    if (gl_log2 >= 5) v = max(v, (uint32_t)__shfl_xor((int)v, 16));
    if (gl_log2 >= 6) v = max(v, (uint32_t)__shfl_xor((int)v, 32));
    return v;
}

// The same for the N steps of a unit at once: one uniform branch per level
// serves all N steps, whose lane exchanges then overlap.  Used for groups of
// 32 or 64 lanes, whose ds_bpermute levels each wait for LDS (E2M1, 256
// columns, fp32 scales: 56.5 -> 52.3 us at 32768 x 2048); for groups of up to
// 16 lanes (DPP only) the step-by-step order above measured 1% faster.
template <int N>
__device__ __forceinline__ void group_umax_steps(uint32_t (&v)[N], uint32_t gl_log2)
{
#define TK_LEVEL(COND, EXPR)                 \
    if (COND) {                              \
        _Pragma("unroll") for (int s = 0; s < N; ++s) v[s] = EXPR; \
    }
    TK_LEVEL(gl_log2 >= 1, dpp_umax<0xB1>(v[s]))  // quad_perm [1,0,3,2]: lane ^ 1
    TK_LEVEL(gl_log2 >= 2, dpp_umax<0x4E>(v[s]))  // quad_perm [2,3,0,1]: lane ^ 2
    TK_LEVEL(gl_log2 >= 3, dpp_umax<0x141>(v[s])) // row_half_mirror: quads of 8 lanes
    TK_LEVEL(gl_log2 >= 4, dpp_umax<0x140>(v[s])) // row_mirror: halves of 16 lanes
    TK_LEVEL(gl_log2 >= 5, max(v[s], (uint32_t)__shfl_xor((int)v[s], 16)))
    TK_LEVEL(gl_log2 >= 6, max(v[s], (uint32_t)__shfl_xor((int)v[s], 32)))
#undef TK_LEVEL
}

__device__ __forceinline__ uint32_t wave_umax(uint32_t v)
{
    v = dpp_umax<0xB1>(v);
    v = dpp_umax<0x4E>(v);
    v = dpp_umax<0x141>(v);
    v = dpp_umax<0x140>(v);
    const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return max(max(a, b), max(c, d));
}

template <int FMT>
struct FmtTraits;
template <>
struct FmtTraits<8> {
    static constexpr float kMax = 448.0f;         // 1.75 * 2^8
    static constexpr int kExpBias = 127 + 8;      // biased exponent of 448
    static constexpr uint32_t kMant = 0x600000u;  // mantissa field of 1.75
};
template <>
struct FmtTraits<4> {
    static constexpr float kMax = 6.0f;           // 1.5 * 2^2
    static constexpr int kExpBias = 127 + 2;
    static constexpr uint32_t kMant = 0x400000u;  // mantissa field of 1.5
};

// Scale of one group from the bit pattern of its abs-max.  Returns the
// multiplier applied before the cast (2^-k for UE8M0) and writes the stored
// scale representation.
template <int FMT, int SFMT>
__device__ __forceinline__ float group_scale(uint32_t amax_bits, float& scale_f32, uint32_t& scale_u8)
{
    using T = FmtTraits<FMT>;
    if constexpr (SFMT == TK_SCALE_FP32) {
        const float amax = as_float(amax_bits);
        scale_f32 = amax / T::kMax;                   // IEEE division, round to nearest even
        return fminf(T::kMax / amax, FLT_MAX);        // amax == 0 -> +inf -> FLT_MAX
    } else {
        // smallest k with fmt_max * 2^k >= amax: compare amax = 1.M * 2^(E-127)
        // with fmt_max = 1.F * 2^P; k = E - 127 - P + (M > F), at least -127.
        int k = (int)(amax_bits >> 23) - T::kExpBias + ((amax_bits & 0x7FFFFFu) > T::kMant ? 1 : 0);
        k = max(k, -127);
        scale_u8 = (uint32_t)(k + 127);
        return as_float((uint32_t)(127 - k) << 23);   // 2^-k, exact
    }
}

// q = RN(y * inv), cast, and one non-temporal store of the lane's 8 codes.
template <int FMT>
__device__ __forceinline__ void quantize_store(uint8_t* row_codes, uint32_t slot, const float* y, float inv)
{
    float q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        q[j] = y[j] * inv;
    if constexpr (FMT == 8) {
        uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], lo, true);
        uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], hi, true);
        const v2u v = {lo, hi};
        __builtin_nontemporal_store(v, reinterpret_cast<v2u*>(row_codes) + slot);
    } else {
        uint32_t v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q[0], q[1], 1.0f, 0);
        v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, q[2], q[3], 1.0f, 1);
        v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, q[4], q[5], 1.0f, 2);
        v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, q[6], q[7], 1.0f, 3);
        __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(row_codes) + slot);
    }
}

// Store the scale of group k of row `row` in the requested layout.
template <int SFMT>
__device__ __forceinline__ void store_scale(const Params& p, uint32_t row, uint32_t k, float s32, uint32_t s8)
{
    size_t idx;
    if (p.scale_layout == kScaleRowMajor)
        idx = (size_t)row * p.groups_row + k;
    else if (p.scale_layout == kScaleColMajor)
        idx = (size_t)k * p.scale_ld + row;
    else // packed: byte (k & 3) of word (k >> 2, row)
        idx = ((size_t)(k >> 2) * p.scale_ld + row) * 4u + (k & 3u);
    if constexpr (SFMT == TK_SCALE_FP32)
        static_cast<float*>(p.scales)[idx] = s32;
    else
        static_cast<uint8_t*>(p.scales)[idx] = (uint8_t)s8;
}

constexpr int kThreads = 256;

// Streaming 16-byte load, marked non-temporal: the input is read exactly once.
__device__ __forceinline__ uint4 load16(const uint4* p)
{
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Lane-local abs-max (bit pattern) over the first nst steps of a unit.
template <int SPU>
__device__ __forceinline__ uint32_t lane_max(const uint32_t (&mbits)[SPU], uint32_t nst)
{
    uint32_t mb = 0;
#pragma unroll
    for (int s = 0; s < SPU; ++s)
        if (s < (int)nst)
            mb = max(mb, mbits[s]);
    return mb;
}

// Quantise the lane's steps step0 .. step0+nst-1 of one row-reduced group
// (per-token, or a 512k-column group) whose abs-max bit pattern is mb; the lane
// given store_scale_here writes the group's scale.
template <int FMT, int SFMT, int SPU, bool PARTIAL>
__device__ __forceinline__ void quantize_rowred(const Params& p, uint32_t lane, uint32_t row, uint32_t group,
                                                uint32_t step0, uint32_t nst, const float (&y)[SPU][8], uint32_t mb,
                                                bool store_scale_here)
{
    uint8_t* row_codes = p.codes + (size_t)row * (FMT == 8 ? p.slots * 8u : p.slots * 4u);
    float s32 = 0.0f;
    uint32_t s8 = 0;
    const float inv = group_scale<FMT, SFMT>(mb, s32, s8);
#pragma unroll
    for (int s = 0; s < SPU; ++s) {
        if (s < (int)nst) {
            const uint32_t slot = (step0 + s) * kWaveSize + lane;
            if (!PARTIAL || slot < p.slots)
                quantize_store<FMT>(row_codes, slot, y[s], inv);
        }
    }
    if (store_scale_here)
        store_scale<SFMT>(p, row, group, s32, s8);
}

// The data of one unit held in registers between its load and its use.

// The quantisation tail of one unit: y[s][j] are the unit's fp32 values (step
// s, element j of the lane's 8-column slot), mbits[s] the lane-local abs-max of
// step s as a bit pattern (0 for lanes past the row end).  Writes codes and
// scales.  Per-block mode (ROWRED false): groups are 2^gl_log2 lanes of one
// step; row mode: the whole unit is one group (per-token, or a 512k-column
// group).
// WIDE: per-block groups of 32 or 64 lanes (p.gl_log2 >= 5), compiled apart
// so that the other kernels keep their code as it is.
template <int FMT, int SFMT, int SPU, bool ROWRED, bool PARTIAL, bool WIDE = false>
__device__ __forceinline__ void quantize_unit(const Params& p, uint32_t lane, uint32_t row, uint32_t unit_in_row,
                                              uint32_t step0, uint32_t nst, const float (&y)[SPU][8],
                                              const uint32_t (&mbits)[SPU])
{
    uint8_t* row_codes = p.codes + (size_t)row * (FMT == 8 ? p.slots * 8u : p.slots * 4u);
    if constexpr (ROWRED) {
        const uint32_t mb = wave_umax(lane_max<SPU>(mbits, nst));
        quantize_rowred<FMT, SFMT, SPU, PARTIAL>(p, lane, row, unit_in_row, step0, nst, y, mb, lane == 0);
    } else {
        auto finish = [&](int s, uint32_t mb) { // scale, codes and the group's scale of step s
            float s32 = 0.0f;
            uint32_t s8 = 0;
            const float inv = group_scale<FMT, SFMT>(mb, s32, s8);
            const uint32_t slot = (step0 + s) * kWaveSize + lane;
            if (!PARTIAL || slot < p.slots) {
                quantize_store<FMT>(row_codes, slot, y[s], inv);
                if ((lane & ((1u << p.gl_log2) - 1u)) == 0)
                    store_scale<SFMT>(p, row, slot >> p.gl_log2, s32, s8);
            }
        };
        if constexpr (WIDE) {
            uint32_t gmax[SPU];
#pragma unroll
            for (int s = 0; s < SPU; ++s)
                gmax[s] = mbits[s];
            group_umax_steps<SPU>(gmax, p.gl_log2);
#pragma unroll
            for (int s = 0; s < SPU; ++s)
                finish(s, gmax[s]);
        } else {
#pragma unroll
            for (int s = 0; s < SPU; ++s)
                finish(s, group_umax(mbits[s], p.gl_log2));
        }
    }
}

// Segmented units: groups whose width is not a power of two of lane slots up
// to 64 and not a multiple of 64 (24, 40, 48, 96, 896 columns, ...).  A unit
// is a run of ngr whole groups of one row starting at lane slot slot0; lane l
// of step s holds slot slot0 + 64*s + l, so a group's slots straddle lanes and
// steps at any offset.  The lanes' per-slot abs-max bits go to `buf` (the
// wave's own SPU*64 words of LDS); lanes then reduce the groups from there --
// L = 64/ngr lanes per group (a power of two, 1 when ngr > 64), each over a
// contiguous chunk of its group's slots, then a butterfly over the L lanes --
// and the group's first lane stores the scale and leaves the multiplier in
// `invs`; finally every lane reads its slot's multiplier back (the group of a
// slot by a multiply-high with p.gmagic) and quantises.  All lanes of the wave
// must call this; `mbits` is 0 for lanes past the unit's last slot.
template <int FMT, int SFMT, int SPU>
__device__ __forceinline__ void quantize_seg(const Params& p, uint32_t lane, uint32_t row, uint32_t g0, uint32_t ngr,
                                             uint32_t slot0, const float (&y)[SPU][8], const uint32_t (&mbits)[SPU],
                                             uint32_t* buf, float* invs)
{
    const uint32_t gs = p.gslots;
    const uint32_t nslots = ngr * gs;
#pragma unroll
    for (int s = 0; s < SPU; ++s)
        buf[s * kWaveSize + lane] = mbits[s];
    __builtin_amdgcn_wave_barrier();
    // lanes per group, as a power of two: floor(log2(64 / ngr)), 0 when ngr > 64 (wave-uniform)
    const uint32_t l_log2 = ngr > (uint32_t)kWaveSize ? 0u : 31u - (uint32_t)__builtin_clz((uint32_t)kWaveSize / ngr);
    const uint32_t lpg = 1u << l_log2;
    const uint32_t chunk = (gs + lpg - 1u) >> l_log2; // slots per lane
    for (uint32_t base = 0; base < ngr; base += (uint32_t)kWaveSize >> l_log2) {
        const uint32_t k = base + (lane >> l_log2);
        const uint32_t sub = lane & (lpg - 1u);
        uint32_t m = 0;
        if (k < ngr) {
            const uint32_t b = k * gs + sub * chunk;
            const uint32_t e = min(b + chunk, (k + 1u) * gs);
            for (uint32_t i = b; i < e; ++i)
                m = max(m, buf[i]);
        }
        m = group_umax(m, l_log2);
        if (k < ngr && sub == 0) {
            float s32 = 0.0f;
            uint32_t s8 = 0;
            invs[k] = group_scale<FMT, SFMT>(m, s32, s8);
            store_scale<SFMT>(p, row, g0 + k, s32, s8);
        }
    }
    __builtin_amdgcn_wave_barrier();
    uint8_t* row_codes = p.codes + (size_t)row * (FMT == 8 ? p.slots * 8u : p.slots * 4u);
#pragma unroll
    for (int s = 0; s < SPU; ++s) {
        const uint32_t rel = (uint32_t)s * kWaveSize + lane;
        if (rel < nslots)
            quantize_store<FMT>(row_codes, slot0 + rel, y[s], invs[__umulhi(rel, p.gmagic)]);
    }
}

// The steps one wave holds for a segmented unit of up to SPU*64 slots, and the
// size of the per-wave multiplier array (groups are at least 3 slots wide).
template <int SPU>
struct SegLds {
    static constexpr int kSlots = SPU * kWaveSize;
    static constexpr int kGroups = kSlots / 3 + 1;
};

// ---------------------------------------------------------------------------
// Host helpers
// ---------------------------------------------------------------------------
inline bool overlaps(const void* a, size_t an, const void* b, size_t bn)
{
    if (!a || !b || an == 0 || bn == 0)
        return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// The compile-time step count a row-reduced unit of k <= 16 steps runs in: the
// smallest of 1, 2, 4, 8, 12, 16 that holds it (steps past k are not computed).
inline uint32_t template_steps(uint32_t k)
{
    if (k <= 2)
        return k;
    return k <= 4 ? 4u : k <= 8 ? 8u : k <= 12 ? 12u : 16u;
}

// A tk_scale_fmt value split into the value kind (TK_SCALE_FP32 or
// TK_SCALE_UE8M0), the layout and its leading dimension, and the bytes the
// scale tensor spans.  Returns false for an unknown format.
struct ScaleSpec {
    int kind = TK_SCALE_FP32;
    uint32_t layout = kScaleRowMajor;
    uint32_t ld = 0;
    size_t bytes = 0;
    uintptr_t align = 1;
};

inline bool scale_spec(int scale_fmt, int64_t n, int64_t groups, ScaleSpec& sp)
{
    const auto round_up = [](int64_t v, int64_t m) { return (v + m - 1) / m * m; };
    switch (scale_fmt) {
    case TK_SCALE_FP32:
        sp = {TK_SCALE_FP32, kScaleRowMajor, 0, (size_t)(n * groups) * 4u, 4};
        return true;
    case TK_SCALE_UE8M0:
        sp = {TK_SCALE_UE8M0, kScaleRowMajor, 0, (size_t)(n * groups), 1};
        return true;
    case TK_SCALE_FP32_COLMAJOR: {
        const int64_t ld = round_up(n, 4);
        sp = {TK_SCALE_FP32, kScaleColMajor, (uint32_t)ld, (size_t)(groups * ld) * 4u, 16};
        return true;
    }
    case TK_SCALE_UE8M0_COLMAJOR: {
        const int64_t ld = round_up(n, 16);
        sp = {TK_SCALE_UE8M0, kScaleColMajor, (uint32_t)ld, (size_t)(groups * ld), 16};
        return true;
    }
    case TK_SCALE_UE8M0_PACKED: {
        const int64_t ld = round_up(n, 4);
        sp = {TK_SCALE_UE8M0, kScalePacked, (uint32_t)ld, (size_t)((groups + 3) / 4 * ld) * 4u, 16};
        return true;
    }
    default:
        return false;
    }
}

// How a [n, hidden] row set is cut into units for a group size G (0 = the
// whole row).  A row-reduced group longer than kMaxStepsPerUnit steps becomes
// plan.xwaves consecutive units (one per wave of a workgroup).  Fills p.spu, p.upr, p.gl_log2, p.slots, p.steps_row, p.units,
// p.groups_row.  Returns TK_ERR_UNSUPPORTED for groups the kernels do not
// cover.  spu_pref: preferred steps per unit for per-block groups (a power of
// two up to 4; reduced until it divides the row's steps).
struct UnitPlan {
    bool rowred = false;
    bool partial = false;
    bool seg = false;     // segmented units (quantize_seg)
    bool twopass = false; // one wave per group, read twice: abs-max, then codes
    uint32_t spu_max = 1; // the kernel's compile-time steps per unit (per wave for split groups)
    uint32_t xwaves = 1;  // row-reduced groups: waves of one workgroup per group (1, 2 or 4)
};

// Segmented units hold whole groups of up to kMaxSegSlots lane slots (8192
// columns, 16 steps of one wave); wider groups that the row-reduced kernels
// do not cover take the two-pass kernels.
constexpr uint32_t kMaxSegSlots = (uint32_t)(kMaxStepsPerUnit * kWaveSize);
constexpr uint32_t kTwoPassSteps = 4; // steps per pass chunk of a two-pass group

// A row-reduced group of k steps: one wave up to kMaxStepsPerUnit steps, else
// split over 2 or 4 waves of one workgroup, each holding ceil(k / waves)
// steps.  Several such groups in one row need k % waves == 0, so that every
// part starts at a multiple of its step count.
inline bool rowred_split(uint32_t k, uint32_t groups_row, uint32_t& waves, uint32_t& spw)
{
    if (k <= (uint32_t)kMaxStepsPerUnit) {
        waves = 1;
        spw = k;
        return true;
    }
    if (k > (uint32_t)(kMaxStepsPerUnit * kMaxWavesPerGroup))
        return false;
    waves = k <= 2u * kMaxStepsPerUnit ? 2u : 4u;
    spw = (k + waves - 1) / waves;
    return groups_row == 1 || k % waves == 0;
}

// One wave per group, the group read twice (abs-max, then codes), kTwoPassSteps
// steps at a time: for groups no other plan covers.
inline void plan_twopass(uint32_t gslots, uint32_t groups, Params& p, UnitPlan& plan)
{
    plan.twopass = true;
    plan.spu_max = kTwoPassSteps;
    p.gslots = gslots;
    p.spu = kTwoPassSteps;
    p.upr = groups;
}

inline tk_status plan_units(int64_t n, int64_t hidden, int64_t group_size, uint32_t spu_pref, Params& p,
                            UnitPlan& plan)
{
    const int64_t G = group_size ? group_size : hidden;
    const uint32_t slots = (uint32_t)(hidden / kSlotCols);
    const uint32_t steps_row = (slots + kWaveSize - 1) / kWaveSize;
    const uint32_t gslots = (uint32_t)(G / kSlotCols);
    const uint32_t groups = (uint32_t)(hidden / G);
    if (G == hidden) {
        uint32_t waves = 1, spw = 1;
        if (rowred_split(steps_row, 1, waves, spw)) {
            plan.rowred = true;
            plan.xwaves = waves;
            p.spu = spw;
            p.upr = waves;
            plan.spu_max = template_steps(spw);
        } else {
            plan_twopass(gslots, 1, p, plan);
        }
    } else if ((gslots & (gslots - 1)) == 0 && gslots <= (uint32_t)kWaveSize) {
        plan.rowred = false;
        p.gl_log2 = (uint32_t)__builtin_ctz(gslots);
        uint32_t spu = spu_pref;
        while (steps_row % spu)
            spu >>= 1;
        plan.spu_max = spu;
        p.spu = spu;
        p.upr = steps_row / spu;
    } else if (gslots % kWaveSize == 0) {
        const uint32_t k = gslots / kWaveSize;
        uint32_t waves = 1, spw = 1;
        if (rowred_split(k, groups, waves, spw)) {
            plan.rowred = true;
            plan.xwaves = waves;
            p.spu = spw;
            p.upr = groups * waves;
            plan.spu_max = template_steps(spw);
        } else {
            plan_twopass(gslots, groups, p, plan);
        }
    } else if (gslots <= kMaxSegSlots) {
        // the smallest step count of 1, 2, 4, 8, 12, 16 that holds one group
        // and is at least spu_pref; as many whole groups per unit as fit
        uint32_t spu = 1;
        while (spu < (uint32_t)kMaxStepsPerUnit && (spu * kWaveSize < gslots || spu < spu_pref))
            spu = spu == 8 ? 12u : spu == 12 ? 16u : spu << 1;
        plan.seg = true;
        plan.spu_max = spu;
        p.spu = spu;
        p.gslots = gslots;
        p.gpu = min(spu * (uint32_t)kWaveSize / gslots, groups);
        p.upr = (groups + p.gpu - 1) / p.gpu;
        p.gmagic = (uint32_t)(((1ull << 32) + gslots - 1) / gslots);
    } else {
        plan_twopass(gslots, groups, p, plan);
    }
    if ((uint64_t)n * p.upr >= (uint64_t)INT_MAX)
        return TK_ERR_UNSUPPORTED;
    p.slots = slots;
    p.steps_row = steps_row;
    p.units = (uint32_t)(n * p.upr);
    p.groups_row = groups;
    plan.partial = (slots % kWaveSize) != 0;
    return TK_OK;
}

} // namespace tk_detail
