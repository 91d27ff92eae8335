// tk_swiglu_cast.hip -- fused SwiGLU + MoE top-k weight + FP8/FP4 cast for
// MI355X (gfx950, CDNA4), behind the C ABI declared in include/tk.h.
//
// The operation is DeepSeek TileKernels' swiglu_forward_and_per_token_cast as
// described in "【DeepSeek】TileKernels从入门到精通" (zhichai.net/topic/
// 177618752) ch.2 (packed gate|up row; sigmoid(x_L)*x_L*x_R*topk_weight;
// abs-max -> scale -> cast; clamp with an atomic counter; persistent grid),
// with the formats of "TileLang + TileKernels：DeepSeek 的 GPU 内核开发新范式"
// (zhichai.net/topic/177618740) "3. Quantization" (E4M3 / E2M1, per-token or
// per-block, UE8M0 scales).
//
// gfx950 design (no code from the pages' TileLang/CUDA kernel):
//  - A wavefront of 64 lanes owns one "unit": SPU "steps" of one row, where a
//    step is 512 columns: lane l reads 16 bytes (8 bf16) of the gate half and
//    16 bytes of the up half at column 8*(64*step + l).  Loads are 128-bit,
//    fully coalesced (1 KiB per wave instruction) and non-temporal; the row
//    base is wave-uniform (scalar registers), lanes add a 32-bit offset.
//  - sigma(g) comes from a 32 KiB table in LDS indexed by the bf16 bits of g
//    (the gate is bf16, so sigma has only 65536 possible inputs; outside the
//    4096 tabulated magnitudes it is constant in fp32).  The table holds the
//    correctly rounded fp32 sigma and is computed on the GPU once per device.
//  - Group abs-max: lane-local max over 8 values, then DPP butterflies on the
//    bit patterns (v_max_u32_dpp) inside the 2^j lanes of a group
//    (quad_perm, row_half_mirror, row_mirror), or a whole-wave reduction for
//    per-token / 512k-column groups.
//  - Casts use the gfx950 converters: v_cvt_pk_fp8_f32 (OCP E4M3, round to
//    nearest even) and v_cvt_scalef32_pk_fp4_f32 with scale 1 (E2M1, round to
//    nearest even, saturating).  Quantised values never exceed fmt_max by
//    more than one fp32 ulp, so the E4M3 converter's lack of saturation above
//    464 is never reached.  Codes leave with non-temporal stores.
//  - A persistent grid of two 256-thread workgroups per CU for large launches
//    and four for small ones (measured best on MI355X); every wave strides
//    over units, so the LDS table is filled once per workgroup.
//  - Row-reduced units of 8 to 16 steps (per-token rows beyond 2048 columns,
//    512k-column groups) stream their loads four steps ahead of the
//    arithmetic; groups of more than 16 steps are split over 2 or 4 waves of
//    a workgroup, which meet in LDS for the group's abs-max.
//  - The clamp counter is reduced per wave with ballots and added to the
//    int64 counter with one vector atomic per wave.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "tk.h"
#include "tk_quant.h"

namespace {

using namespace tk_detail;

// Sigmoid table: magnitudes m of bf16 bit patterns in [kLutFirst, kLutFirst+kLutSize),
// one (sigma(+g), sigma(-g)) pair per magnitude.  Below 2^-25 sigma rounds to
// 0.5 and at 127.5 and beyond it rounds to 1 (positive) or 0 (negative) in fp32,
// so clamping the magnitude into the table range is exact.
constexpr uint32_t kLutFirst = 0x3300u; // bf16 2^-25
constexpr uint32_t kLutLast = 0x42FFu;  // bf16 127.5
constexpr int kLutSize = 4096;
static_assert(kLutLast - kLutFirst + 1 == kLutSize, "table span");

__device__ float2 g_sigma_lut[kLutSize];
// The same sigmoids in 16 KiB, for small launches (where filling and reading
// the table is a fifth of the launch): per magnitude sigma(-|g|), which lies in
// (0, 0.5] so its two top bits are 0, and in those two bits 1 + the difference
// in ulps between sigma(+|g|) and RN(1 - sigma(-|g|)).  That difference is -1,
// 0 or +1 for every tabulated magnitude, so sigma(+|g|) is recovered exactly
// from one subtraction and one integer add.
__device__ uint32_t g_sigma_lut16[kLutSize];

// ---------------------------------------------------------------------------
// Correctly rounded fp32 sigmoid for table set-up and for the clamp limit.
// |g| < 2^-12: Taylor series 1/2 + g/4 - g^3/48 + g^5/480 (next term below
//   2^-96), summed as a double-double with Knuth's TwoSum; the double-double
//   is rounded to fp32 once, the low word deciding exact fp64 midpoints.
// otherwise: 1/(1+exp(-g)) in fp64.  Its error (a few fp64 ulps) is far below
//   the distance of any bf16 gate's sigmoid from an fp32 rounding midpoint
//   (at least 5.8e-5 fp32 ulps for |g| >= 2^-12); for other fp32 inputs it is
//   correct unless sigma lies within ~2^-50 of a midpoint.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e)
{
    s = a + b;
    const double bb = s - a;
    e = (a - (s - bb)) + (b - bb);
}

__device__ float round_dd_to_float(double hi, double lo)
{
    const float f = (float)hi;
    const double df = (double)f;
    if (df == hi || lo == 0.0)
        return f;
    const float f2 = nextafterf(f, hi > df ? INFINITY : -INFINITY);
    const double mid = 0.5 * (df + (double)f2); // exact
    if (mid != hi)
        return f; // hi is not a tie, so hi + lo rounds like hi
    // hi sits exactly on the midpoint between f and f2: lo decides.
    return ((lo > 0.0) == (hi > df)) ? f2 : f;
}

__device__ float sigmoid_rn(float gf)
{
    const double g = (double)gf;
    if (fabs(g) < 0x1p-12) {
        if (fabs(g) < 0x1p-40)
            return 0.5f; // |g/4| is far below half an ulp of 0.5
        double s, e;
        two_sum(0.5, 0.25 * g, s, e);
        const double g2 = g * g;
        const double c = g * g2 * (-1.0 / 48.0 + g2 * (1.0 / 480.0));
        double hi, lo;
        two_sum(s, e + c, hi, lo);
        return round_dd_to_float(hi, lo);
    }
    return (float)(1.0 / (1.0 + exp(-g)));
}

__global__ void sigma_lut_init_kernel()
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= kLutSize)
        return;
    const float g = as_float((kLutFirst + (uint32_t)i) << 16);
    const float sp = sigmoid_rn(g), sn = sigmoid_rn(-g);
    g_sigma_lut[i] = make_float2(sp, sn);
    const int corr = (int)(as_uint(sp) - as_uint(1.0f - sn));
    g_sigma_lut16[i] = as_uint(sn) | ((uint32_t)(corr + 1) << 30);
}

// ---------------------------------------------------------------------------
// Kernel
// ---------------------------------------------------------------------------
typedef float2 LutT;
// The whole table into LDS by a workgroup of kThreads threads: every thread's
// loads go out together, then the stores, then one barrier.
__device__ __forceinline__ void load_lut_to_lds(float2* lut)
{
    constexpr int kPer = kLutSize / 2 / kThreads; // 16-byte pieces per thread
    static_assert(kPer * kThreads * 2 == kLutSize, "table split");
    const uint4* src = reinterpret_cast<const uint4*>(g_sigma_lut);
    uint4* dst = reinterpret_cast<uint4*>(lut);
    uint4 v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        v[i] = src[i * kThreads + threadIdx.x];
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        dst[i * kThreads + threadIdx.x] = v[i];
    __syncthreads();
}
// sigma(g) for a gate whose bf16 bits sit in bits [POS, POS+16) of `word`;
// gbits is the fp32 bit pattern of the same gate (its sign selects the entry).
template <int POS>
__device__ __forceinline__ float lut_sigma(const float2* lut, uint32_t word, uint32_t gbits)
{
    const uint32_t m = __builtin_amdgcn_ubfe(word, POS, 15);                 // |g| as bf16 bits
    const uint32_t c = min(max(m, kLutFirst), kLutLast) - kLutFirst;         // v_med3_u32
    const float2 pr = lut[c];
    return ((int32_t)gbits < 0) ? pr.y : pr.x;
}

// The 16 KiB form of the same lookup (g_sigma_lut16's layout).
template <int POS>
__device__ __forceinline__ float lut16_sigma(const uint32_t* lut, uint32_t word, uint32_t gbits)
{
    const uint32_t m = __builtin_amdgcn_ubfe(word, POS, 15);
    const uint32_t c = min(max(m, kLutFirst), kLutLast) - kLutFirst;
    const uint32_t e = lut[c];
    const float sn = as_float(e & 0x3FFFFFFFu);
    const float sp = as_float(as_uint(1.0f - sn) + (e >> 30) - 1u);
    return ((int32_t)gbits < 0) ? sn : sp;
}

constexpr int kLutLdsBytes = kLutSize * 8;
constexpr int kLut16LdsBytes = kLutSize * 4;

// Clamp counters: a wave's count of gates above the limit.  WaveCount keeps
// the wave's total in scalar registers (a ballot and popcount per element);
// LaneCount keeps one count per lane (a VALU add per element) and sums the
// lanes once at the end.  Row-reduced units use WaveCount; per-block units use
// LaneCount, because there the compiler holds every element's compare mask in
// scalar registers until the step's group reductions are done and spills them
// to VGPR lanes (the per-block clamp launch of 32768 x 2048 took 65 us without
// the counter's atomics against 57 us unclamped; with LaneCount, 59.5 us).
struct WaveCount {
    unsigned long long n = 0;
    __device__ __forceinline__ void add(bool hit) { n += __builtin_popcountll(__ballot(hit)); }
    __device__ __forceinline__ unsigned long long total() const { return n; }
};
struct LaneCount {
    // a lane counts at most 32 gates per unit and ceil(units / waves) units,
    // with units < 2^31 and 8 waves per CU: below 2^32 on any device of more
    // than two CUs
    uint32_t n = 0;
    __device__ __forceinline__ void add(bool hit) { n += hit ? 1u : 0u; }
    // every lane of the wave must call this
    __device__ __forceinline__ unsigned long long total() const
    {
        unsigned long long t = n;
#pragma unroll
        for (int m = kWaveSize / 2; m >= 1; m >>= 1)
            t += __shfl_xor(t, m);
        return t;
    }
};

// The workgroup's clamp count into the caller's int64 counter: each wave adds
// its total to `wg` in LDS and one global atomic goes out per workgroup.
// Adding from every wave put 2048 atomics on one address at the end of a
// persistent launch, where they serialise: 11-16 us at the end of a
// 32768-row launch.  Every thread of the workgroup calls this; `wg` was
// zeroed by thread 0 before an earlier barrier.
template <class CNT>
__device__ __forceinline__ void flush_clamp_count(unsigned long long* count, unsigned long long* wg, const CNT& c,
                                                  uint32_t lane)
{
    const unsigned long long t = c.total();
    if (lane == 0 && t)
        atomicAdd(wg, t);
    __syncthreads();
    if (threadIdx.x == 0 && count && *wg)
        atomicAdd(count, *wg);
}

// One element: gate and up are the bf16 halves at bit POS of `gword` / `uword`.
// a = RN(g * sigma(g)) (or the clamped gate's activation), b = RN(a * u),
// y = RN(b * w); three fp32 products, never fused.  `counts` is false on lanes
// past the end of the row, whose gates must not enter the clamp count.
template <int POS, bool CLAMP, class CNT, bool T16 = false>
__device__ __forceinline__ float swiglu_elem(const LutT* lut, uint32_t gword, uint32_t uword, float w,
                                             float limit, float a_limit, CNT& clamped, bool counts = true)
{
    const uint32_t gbits = POS ? (gword & 0xFFFF0000u) : (gword << 16);
    float u = as_float(POS ? (uword & 0xFFFF0000u) : (uword << 16));
    const float g = as_float(gbits);
    float a = g * (T16 ? lut16_sigma<POS>(reinterpret_cast<const uint32_t*>(lut), gword, gbits)
                       : lut_sigma<POS>(lut, gword, gbits));
    if constexpr (CLAMP) {
        clamped.add(g > limit && counts);
        // The clamped gate's activation, RN(min(g, L) * sigma(min(g, L))), is
        // min(a, a_limit) with a_limit = RN(L * sigma(L)): L > 0, and
        // RN(g * sigma(g)) does not decrease with g > 0 and is <= -0 for g <= -0,
        // so a >= a_limit when g > L and a <= a_limit when g <= L.  The min is
        // taken on the bit patterns as signed integers, which order every
        // negative value (-0 included) below a_limit >= +0: a gate of -0 keeps
        // its -0 even when a_limit rounds to +0 (the smallest L).
        a = __builtin_bit_cast(float, min(__builtin_bit_cast(int32_t, a), __builtin_bit_cast(int32_t, a_limit)));
        u = __builtin_amdgcn_fmed3f(u, -limit, limit);
    }
    const float b = a * u;
    return b * w;
}

template <int SPU>
struct Unit {
    uint4 g[SPU], u[SPU];
    uint32_t row, unit_in_row, step0, nst;
    float w;
};

// NOBRANCH: a row-reduced unit shorter than SPU steps re-reads its last step
// for the rest instead of skipping them, so that no branch surrounds the loads
// (a branch would make a later wait for loads issued before these count the
// worst case of both paths).
template <int SPU, bool ROWRED, bool PARTIAL, bool NOBRANCH = false>
__device__ __forceinline__ void load_unit(const Params& p, uint32_t u, uint32_t lane, Unit<SPU>& d)
{
    d.row = u / p.upr;
    d.unit_in_row = u - d.row * p.upr;
    d.step0 = d.unit_in_row * p.spu;
    d.nst = ROWRED ? min(p.spu, p.steps_row - d.step0) : (uint32_t)SPU;
    // uniform row bases (scalar registers) + a 32-bit per-lane byte offset
    const char* xg = reinterpret_cast<const char*>(p.x) + (size_t)d.row * (p.slots * 32u);
    const char* xu = xg + p.slots * 16u;
    const uint32_t lane_off = (d.step0 * kWaveSize + lane) * 16u;
#pragma unroll
    for (int s = 0; s < SPU; ++s) {
        if (NOBRANCH || !ROWRED || s < (int)d.nst) {
            const uint32_t st = (ROWRED && NOBRANCH) ? min((uint32_t)s, d.nst - 1u) : (uint32_t)s;
            uint32_t off = lane_off + st * (kWaveSize * 16u);
            if (PARTIAL) // lanes past the row end re-read its last slot
                off = min(off, (p.slots - 1u) * 16u);
            d.g[s] = load16(reinterpret_cast<const uint4*>(xg + off));
            d.u[s] = load16(reinterpret_cast<const uint4*>(xu + off));
        }
    }
    d.w = p.w ? p.w[d.row] : 1.0f;
}

// One 8-column step of a loaded unit: ys = w * silu(gate) * up for the lane's
// columns; returns the lane's abs-max bits (0 for a lane past the row end).
template <bool CLAMP, bool PARTIAL, class CNT, bool T16 = false>
__device__ __forceinline__ uint32_t compute_step(const LutT* lut, uint4 g, uint4 u, float w, bool valid, float limit,
                                                 float a_limit, CNT& clamped, float (&ys)[8])
{
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
    const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        ys[2 * k] = swiglu_elem<0, CLAMP, CNT, T16>(lut, gw[k], uw[k], w, limit, a_limit, clamped, valid);
        ys[2 * k + 1] = swiglu_elem<16, CLAMP, CNT, T16>(lut, gw[k], uw[k], w, limit, a_limit, clamped, valid);
        m = fmaxf(m, fmaxf(fabsf(ys[2 * k]), fabsf(ys[2 * k + 1])));
    }
    if (PARTIAL && !valid)
        m = 0.0f;
    return as_uint(m);
}

// Row-reduced units of kStreamMinSteps steps or more: the loads run kStreamDepth
// steps ahead of the arithmetic instead of all being issued up front, so a
// wave computes while its next steps are in flight and holds the raw data of
// only kStreamDepth steps (the unit's y stays in registers for the quantise
// pass).  Fills y and mbits of steps 0 .. nst-1 of unit u.
constexpr int kStreamMinSteps = 8;
constexpr int kStreamDepth = 4;

template <bool CLAMP, int SPU, bool PARTIAL, class CNT>
__device__ __forceinline__ void stream_unit(const Params& p, const LutT* lut, uint32_t lane, uint32_t u, float limit,
                                            float a_limit, CNT& clamped, uint32_t& row,
                                            uint32_t& unit_in_row, uint32_t& step0, uint32_t& nst, float (&y)[SPU][8],
                                            uint32_t (&mbits)[SPU])
{
    constexpr int D = kStreamDepth;
    row = u / p.upr;
    unit_in_row = u - row * p.upr;
    step0 = unit_in_row * p.spu;
    nst = min(p.spu, p.steps_row - step0);
    const char* xg = reinterpret_cast<const char*>(p.x) + (size_t)row * (p.slots * 32u);
    const char* xu = xg + p.slots * 16u;
    const uint32_t lane_off = (step0 * kWaveSize + lane) * 16u;
    const float w = p.w ? p.w[row] : 1.0f;
    // Every load is issued unconditionally so that no load sits under a
    // branch: the wait before each step then counts only the loads still
    // ahead of it.  A step past the unit's end reads the first KiB of the
    // sigmoid table in global memory (hot in cache: every workgroup reads it),
    // except in the variants where that address would push the kernel past
    // 256 VGPRs (one workgroup per CU instead of two): the clamp variants and
    // 16-step units of ragged rows re-read the unit's last step instead.
    constexpr bool kSpareRead = !CLAMP && !(PARTIAL && SPU > 12);
    const uint32_t last = nst - 1u;
    const uint32_t row_end = (p.slots - 1u) * 16u;
    auto step_off = [&](int s) {
        uint32_t off = lane_off + min((uint32_t)s, last) * (kWaveSize * 16u);
        if (PARTIAL) // lanes past the row end re-read its last slot
            off = min(off, row_end);
        return off;
    };
    const char* spare = reinterpret_cast<const char*>(g_sigma_lut) + lane * 16u;
    auto addr = [&](const char* half, int s) {
        if constexpr (!kSpareRead)
            return reinterpret_cast<const uint4*>(half + step_off(s));
        else
            return reinterpret_cast<const uint4*>(s < (int)nst ? half + step_off(s) : spare);
    };
    uint4 gq[D], uq[D];
#pragma unroll
    for (int s = 0; s < D && s < SPU; ++s) {
        gq[s] = load16(addr(xg, s));
        uq[s] = load16(addr(xu, s));
    }
#pragma unroll
    for (int s = 0; s < SPU; ++s) {
        const uint4 g = gq[s % D], uu = uq[s % D];
        if (s + D < SPU) {
            gq[s % D] = load16(addr(xg, s + D));
            uq[s % D] = load16(addr(xu, s + D));
        }
        if (s < (int)nst)
            mbits[s] = compute_step<CLAMP, PARTIAL>(lut, g, uu, w, !PARTIAL || (step0 + s) * kWaveSize + lane < p.slots,
                                                    limit, a_limit, clamped, y[s]);
    }
}

// The addressing of one streamed unit, the same as stream_unit's (the same
// unconditional loads, spare reads past the unit's end included), for the
// first unit of a wave, whose first steps are issued before the table fill
// (streamed_rowred_loop).  stream_unit keeps its own copy: folding it into
// this one changed the register allocation of the other units' loop and cost
// up to 1.3% on large launches.
template <bool CLAMP, int SPU, bool PARTIAL>
struct StreamAddr {
    static constexpr bool kSpareRead = !CLAMP && !(PARTIAL && SPU > 12);
    uint32_t row, unit_in_row, step0, nst, lane_off, row_end;
    const char* xg;
    const char* xu;
    const char* spare;
    __device__ __forceinline__ StreamAddr(const Params& p, uint32_t u, uint32_t lane)
    {
        row = u / p.upr;
        unit_in_row = u - row * p.upr;
        step0 = unit_in_row * p.spu;
        nst = min(p.spu, p.steps_row - step0);
        xg = reinterpret_cast<const char*>(p.x) + (size_t)row * (p.slots * 32u);
        xu = xg + p.slots * 16u;
        lane_off = (step0 * kWaveSize + lane) * 16u;
        row_end = (p.slots - 1u) * 16u;
        spare = reinterpret_cast<const char*>(g_sigma_lut) + lane * 16u;
    }
    __device__ __forceinline__ const uint4* at(const char* half, int s) const
    {
        uint32_t off = lane_off + min((uint32_t)s, nst - 1u) * (kWaveSize * 16u);
        if (PARTIAL) // lanes past the row end re-read its last slot
            off = min(off, row_end);
        if constexpr (!kSpareRead)
            return reinterpret_cast<const uint4*>(half + off);
        else
            return reinterpret_cast<const uint4*>(s < (int)nst ? half + off : spare);
    }
    // the loads of steps 0 .. kStreamDepth-1
    __device__ __forceinline__ void first_loads(uint4 (&gq)[kStreamDepth], uint4 (&uq)[kStreamDepth]) const
    {
#pragma unroll
        for (int s = 0; s < kStreamDepth && s < SPU; ++s) {
            gq[s] = load16(at(xg, s));
            uq[s] = load16(at(xu, s));
        }
    }
};

// stream_unit for a unit whose first kStreamDepth steps the caller has already
// issued into gq, uq (StreamAddr::first_loads).
template <bool CLAMP, int SPU, bool PARTIAL, class CNT>
__device__ __forceinline__ void stream_unit_issued(const Params& p, const LutT* lut, uint32_t lane, uint32_t u,
                                                   float limit, float a_limit, CNT& clamped, uint32_t& row,
                                                   uint32_t& unit_in_row, uint32_t& step0, uint32_t& nst,
                                                   float (&y)[SPU][8], uint32_t (&mbits)[SPU],
                                                   uint4 (&gq)[kStreamDepth], uint4 (&uq)[kStreamDepth])
{
    constexpr int D = kStreamDepth;
    const StreamAddr<CLAMP, SPU, PARTIAL> a(p, u, lane);
    row = a.row;
    unit_in_row = a.unit_in_row;
    step0 = a.step0;
    nst = a.nst;
    const float w = p.w ? p.w[row] : 1.0f;
    auto addr = [&](const char* half, int s) { return a.at(half, s); };
    const char* xg = a.xg;
    const char* xu = a.xu;
#pragma unroll
    for (int s = 0; s < SPU; ++s) {
        const uint4 g = gq[s % D], uu = uq[s % D];
        if (s + D < SPU) {
            gq[s % D] = load16(addr(xg, s + D));
            uq[s % D] = load16(addr(xu, s + D));
        }
        if (s < (int)nst)
            mbits[s] = compute_step<CLAMP, PARTIAL>(lut, g, uu, w, !PARTIAL || (step0 + s) * kWaveSize + lane < p.slots,
                                                    limit, a_limit, clamped, y[s]);
    }
}

template <int FMT, int SFMT, bool CLAMP, int SPU, bool ROWRED, bool PARTIAL, bool WIDE, bool T16, class CNT>
__device__ __forceinline__ void process_unit(const Params& p, const LutT* lut, uint32_t lane, const Unit<SPU>& d,
                                             float limit, float a_limit, CNT& clamped)
{
    float y[SPU][8];
    uint32_t mbits[SPU];
#pragma unroll
    for (int s = 0; s < SPU; ++s)
        if (!ROWRED || s < (int)d.nst)
            mbits[s] = compute_step<CLAMP, PARTIAL, CNT, T16>(lut, d.g[s], d.u[s], d.w,
                                                    !PARTIAL || (d.step0 + s) * kWaveSize + lane < p.slots, limit,
                                                    a_limit, clamped, y[s]);
    quantize_unit<FMT, SFMT, SPU, ROWRED, PARTIAL, WIDE>(p, lane, d.row, d.unit_in_row, d.step0, d.nst, y, mbits);
}

// The persistent loop for row-reduced units of kStreamMinSteps steps or more:
// the table fill overlapping the first unit's first steps, then every unit of
// the wave streamed (stream_unit).
template <int FMT, int SFMT, bool CLAMP, int SPU, bool PARTIAL>
__device__ __forceinline__ void streamed_rowred_loop(const Params& p, LutT* lut, unsigned long long* wg_clamped,
                                                     uint32_t lane, uint32_t wave, uint32_t nwaves)
{
    if (CLAMP && threadIdx.x == 0)
        *wg_clamped = 0;
    // The table's loads first, then the first unit's first kStreamDepth
    // steps, then the table into LDS and the barrier: loads return in order,
    // so the table's wait does not wait for the unit's loads, and the unit's
    // latency overlaps the table fill instead of following it.  The unit's
    // loads are issued without a branch (a wave past the last unit reads the
    // last one and does not process it), and a scheduling barrier keeps them
    // behind the table's; named registers, as an array the table's pieces
    // were kept in scratch memory.  Interleaved A/B, outputs identical,
    // per-token rows: 256 x 7168 7.76 -> 7.33 us, 1000 x 7168 8.85 -> 8.39,
    // FP4 2000 x 8192 16.10 -> 15.08, 16384 x 4096 59.7 -> 58.6, clamp
    // 8192 x 8192 60.7 -> 59.6; clamp 4096 x 7168 29.25 -> 29.97 (+2.5%) and
    // large launches within 0.7%.
    const uint4* tsrc = reinterpret_cast<const uint4*>(g_sigma_lut) + threadIdx.x;
    static_assert(kLutSize / 2 / kThreads == 8, "eight 16-byte pieces of the table per thread");
    const uint4 t0 = tsrc[0], t1 = tsrc[kThreads], t2 = tsrc[2 * kThreads], t3 = tsrc[3 * kThreads];
    const uint4 t4 = tsrc[4 * kThreads], t5 = tsrc[5 * kThreads], t6 = tsrc[6 * kThreads], t7 = tsrc[7 * kThreads];
    __builtin_amdgcn_sched_barrier(0x0F); // arithmetic may cross, memory instructions may not
    uint4 gq[kStreamDepth], uq[kStreamDepth];
    StreamAddr<CLAMP, SPU, PARTIAL>(p, wave < p.units ? wave : p.units - 1u, lane).first_loads(gq, uq);
    uint4* tdst = reinterpret_cast<uint4*>(lut) + threadIdx.x;
    tdst[0] = t0;
    tdst[kThreads] = t1;
    tdst[2 * kThreads] = t2;
    tdst[3 * kThreads] = t3;
    tdst[4 * kThreads] = t4;
    tdst[5 * kThreads] = t5;
    tdst[6 * kThreads] = t6;
    tdst[7 * kThreads] = t7;
    __syncthreads();
    float limit = 0.0f, a_limit = 0.0f;
    if constexpr (CLAMP) {
        limit = p.clamp;
        a_limit = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                               __builtin_bit_cast(int, limit * sigmoid_rn(limit))));
    }
    WaveCount clamped;
    if (wave < p.units) {
        float y[SPU][8];
        uint32_t mbits[SPU];
        uint32_t row, unit_in_row, step0, nst;
        stream_unit_issued<CLAMP, SPU, PARTIAL>(p, lut, lane, wave, limit, a_limit, clamped, row, unit_in_row, step0,
                                                nst, y, mbits, gq, uq);
        quantize_unit<FMT, SFMT, SPU, true, PARTIAL>(p, lane, row, unit_in_row, step0, nst, y, mbits);
    }
    for (uint32_t u = wave + nwaves; u < p.units; u += nwaves) {
        float y[SPU][8];
        uint32_t mbits[SPU];
        uint32_t row, unit_in_row, step0, nst;
        stream_unit<CLAMP, SPU, PARTIAL>(p, lut, lane, u, limit, a_limit, clamped, row, unit_in_row, step0, nst, y,
                                         mbits);
        quantize_unit<FMT, SFMT, SPU, true, PARTIAL>(p, lane, row, unit_in_row, step0, nst, y, mbits);
    }
    if constexpr (CLAMP)
        flush_clamp_count(p.count, wg_clamped, clamped, lane);
}

// T16: the 16 KiB form of the table (small launches: half the fill and a
// 4-byte read per lookup, for four more VALU operations per element; interleaved
// A/B, bit-identical: 349 x 7168 ragged 5.56 -> 5.24 us replayed from a graph,
// 1000 x 7168 9.70 -> 9.03, 2400 x 2048 per-block 8.22 -> 7.98; on the large
// launches it cost 1-3%).
// TFIRST: a single-pass launch (no wave has more than one unit), which orders
// the table fill differently (below).
template <int FMT, int SFMT, bool CLAMP, int SPU, bool ROWRED, bool PARTIAL, bool WIDE = false, bool T16 = false,
          bool TFIRST = false>
__global__ __launch_bounds__(kThreads) void swiglu_cast_kernel(Params p)
{
    constexpr int kTableBytes = T16 ? kLut16LdsBytes : kLutLdsBytes;
    __shared__ __attribute__((aligned(16))) unsigned char lut_raw[kTableBytes];
    __shared__ unsigned long long wg_clamped; // the workgroup's clamp count
    LutT* lut = reinterpret_cast<LutT*>(lut_raw);

    const uint32_t lane = threadIdx.x & (kWaveSize - 1);
    const uint32_t waves_per_block = kThreads / kWaveSize;
    // Workgroup b is dispatched to XCD b % 8; renumbering it (b % 8) * (G/8) +
    // b / 8 gives each XCD a contiguous share of the grid, so in every pass of
    // the grid-stride loop each XCD (and its L2) streams one contiguous eighth
    // of the window (FP4 workload 212 -> 206 us).  A bijection whenever the
    // grid is a multiple of 8; other grids, and launches the host marks (see
    // xcd_order), keep the plain order.
    uint32_t block = blockIdx.x;
    if (p.xcd_order && (gridDim.x & 7u) == 0)
        block = (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    // wave-uniform by construction; readfirstlane lets the compiler keep all
    // unit bookkeeping (row, step, addresses) in scalar registers
    const uint32_t wave = __builtin_amdgcn_readfirstlane(block * waves_per_block + (threadIdx.x / kWaveSize));
    const uint32_t nwaves = gridDim.x * waves_per_block;
    if constexpr (ROWRED && SPU >= kStreamMinSteps) {
        static_assert(!T16, "the streamed loop reads the 32 KiB table");
        streamed_rowred_loop<FMT, SFMT, CLAMP, SPU, PARTIAL>(p, lut, &wg_clamped, lane, wave, nwaves);
        return;
    }

    // The table's global loads and the first unit's are in flight together,
    // so the unit's latency overlaps the table fill (what a launch of a few
    // hundred rows spends most of its time on).  Loads return in order, and
    // the compiler issues the unit's loads first: the table's wait then waits
    // for the unit as well, and the table reaches LDS (and the barrier
    // passes) only once both are in.
    constexpr int kLutPerThread = kTableBytes / 16 / kThreads;
    static_assert(kLutPerThread == 4 || kLutPerThread == 8, "table split");
    const uint4* table = T16 ? reinterpret_cast<const uint4*>(g_sigma_lut16) : reinterpret_cast<const uint4*>(g_sigma_lut);
    if (CLAMP && threadIdx.x == 0)
        wg_clamped = 0;
    Unit<SPU> first;
    if constexpr (TFIRST) {
        const uint4* tsrc = table + threadIdx.x;
        uint4* tdst = reinterpret_cast<uint4*>(lut_raw) + threadIdx.x;
        // A single-pass launch issues the table's loads first and the unit's
        // behind them, so the table reaches LDS and the barrier passes while
        // the unit is still in flight.  The table's wait is then a partial
        // one (vmcnt of the unit's loads): the scheduling barrier keeps the
        // unit's loads from being hoisted above the table's, and the unit's
        // loads are issued without a branch (a wave past the last unit
        // re-reads the last one and does not process it).  Interleaved A/B
        // replayed from graphs, outputs identical: ragged 349 x 7168 per-block
        // 5.23 -> 4.90 us, 17 x 7168 2.39 -> 2.21, 256 x 1024 per-token 2.72
        // -> 2.61, 2400 x 2048 per-block 8.08 -> 7.43.  In launches of several
        // passes the same order measured from 9% slower (700 x 7168) to 6%
        // faster (5000 x 2048), so they keep the compiler's order.  Named
        // registers rather than an array: with the scheduling barrier an
        // array of them was kept in scratch memory.
        const uint4 t0 = tsrc[0], t1 = tsrc[kThreads], t2 = tsrc[2 * kThreads], t3 = tsrc[3 * kThreads];
        uint4 t4{}, t5{}, t6{}, t7{};
        if constexpr (kLutPerThread == 8) {
            t4 = tsrc[4 * kThreads];
            t5 = tsrc[5 * kThreads];
            t6 = tsrc[6 * kThreads];
            t7 = tsrc[7 * kThreads];
        }
        __builtin_amdgcn_sched_barrier(0x0F); // arithmetic may cross, memory instructions may not
        load_unit<SPU, ROWRED, PARTIAL, true>(p, wave < p.units ? wave : p.units - 1u, lane, first);
        tdst[0] = t0;
        tdst[kThreads] = t1;
        tdst[2 * kThreads] = t2;
        tdst[3 * kThreads] = t3;
        if constexpr (kLutPerThread == 8) {
            tdst[4 * kThreads] = t4;
            tdst[5 * kThreads] = t5;
            tdst[6 * kThreads] = t6;
            tdst[7 * kThreads] = t7;
        }
    } else {
        uint4 lut_part[kLutPerThread];
#pragma unroll
        for (int i = 0; i < kLutPerThread; ++i)
            lut_part[i] = table[i * kThreads + threadIdx.x];
        if (wave < p.units)
            load_unit<SPU, ROWRED, PARTIAL>(p, wave, lane, first);
#pragma unroll
        for (int i = 0; i < kLutPerThread; ++i)
            reinterpret_cast<uint4*>(lut_raw)[i * kThreads + threadIdx.x] = lut_part[i];
    }
    __syncthreads();

    float limit = 0.0f, a_limit = 0.0f;
    if constexpr (CLAMP) {
        limit = p.clamp;
        a_limit = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                               __builtin_bit_cast(int, limit * sigmoid_rn(limit))));
    }
    std::conditional_t<ROWRED, WaveCount, LaneCount> clamped;

    if (wave < p.units)
        process_unit<FMT, SFMT, CLAMP, SPU, ROWRED, PARTIAL, WIDE, T16>(p, lut, lane, first, limit, a_limit, clamped);
    for (uint32_t u = wave + nwaves; u < p.units; u += nwaves) {
        Unit<SPU> d;
        load_unit<SPU, ROWRED, PARTIAL>(p, u, lane, d);
        process_unit<FMT, SFMT, CLAMP, SPU, ROWRED, PARTIAL, WIDE, T16>(p, lut, lane, d, limit, a_limit, clamped);
    }

    if constexpr (CLAMP)
        flush_clamp_count(p.count, &wg_clamped, clamped, lane);
}

// Row-reduced groups longer than one wave holds (per-token rows or 512k-column
// groups beyond 8192 columns): W waves of a workgroup share one group, each
// loading and computing ceil(k/W) of its k steps; the waves' abs-maxes meet in
// LDS (double-buffered, one barrier per pass), then every wave quantises its
// own steps and the group's first wave stores the scale.  Persistent over
// passes of 4/W groups per workgroup; every wave runs the same passes, so the
// barrier is reached by all of them.
template <int FMT, int SFMT, bool CLAMP, int SPU, bool PARTIAL, int W>
__global__ __launch_bounds__(kThreads) void swiglu_cast_xw_kernel(Params p)
{
    constexpr uint32_t kWaves = kThreads / kWaveSize;
    constexpr uint32_t kGroupsPerPass = kWaves / W;
    static_assert(kWaves % W == 0, "waves per group must divide the workgroup");
    __shared__ __attribute__((aligned(16))) unsigned char lut_raw[kLutLdsBytes];
    __shared__ uint32_t part_max[2][kWaves];
    __shared__ unsigned long long wg_clamped; // the workgroup's clamp count
    LutT* lut = reinterpret_cast<LutT*>(lut_raw);
    if (CLAMP && threadIdx.x == 0)
        wg_clamped = 0;
    load_lut_to_lds(lut);

    const uint32_t lane = threadIdx.x & (kWaveSize - 1);
    const uint32_t wib = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
    uint32_t block = blockIdx.x;
    if (p.xcd_order && (gridDim.x & 7u) == 0) // XCD-contiguous order, as in the one-wave kernel
        block = (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const uint32_t slot_in_pass = wib / W, part = wib % W;
    const uint32_t groups = p.units / W;
    const uint32_t passes = (groups + kGroupsPerPass - 1) / kGroupsPerPass;

    float limit = 0.0f, a_limit = 0.0f;
    if constexpr (CLAMP) {
        limit = p.clamp;
        a_limit = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                               __builtin_bit_cast(int, limit * sigmoid_rn(limit))));
    }
    WaveCount clamped;
    uint32_t parity = 0;
    for (uint32_t it = block; it < passes; it += gridDim.x, parity ^= 1u) {
        const uint32_t g = it * kGroupsPerPass + slot_in_pass;
        const bool valid = g < groups; // wave-uniform
        float y[SPU][8];
        uint32_t row = 0, unit_in_row = 0, step0 = 0, nst = 0, mb = 0;
        if (valid) {
            uint32_t mbits[SPU];
            stream_unit<CLAMP, SPU, PARTIAL>(p, lut, lane, g * W + part, limit, a_limit, clamped, row, unit_in_row,
                                             step0, nst, y, mbits);
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
    if constexpr (CLAMP)
        flush_clamp_count(p.count, &wg_clamped, clamped, lane);
}

// A span of `nslots` lane slots of row `row` from slot `slot0` on: lane l of
// step s holds slot slot0 + 64*s + l; lanes past the span re-read its last
// slot and give abs-max bits 0 and no clamp count.  Loads run up to
// kStreamDepth steps ahead of the arithmetic.  Used by the segmented and
// two-pass kernels, whose spans start at any slot.  NT: non-temporal loads
// (data read once); a two-pass group's first read leaves NT off so that its
// second read finds the data in the caches.
template <bool CLAMP, int SPU, class CNT, bool NT = true>
__device__ __forceinline__ void span_compute(const Params& p, const LutT* lut, uint32_t lane, uint32_t row,
                                             uint32_t slot0, uint32_t nslots, float w, float limit, float a_limit,
                                             CNT& clamped, float (&y)[SPU][8], uint32_t (&mbits)[SPU])
{
    constexpr int D = SPU < kStreamDepth ? SPU : kStreamDepth;
    const char* xg = reinterpret_cast<const char*>(p.x) + (size_t)row * (p.slots * 32u);
    const char* xu = xg + p.slots * 16u;
    const uint32_t last = slot0 + nslots - 1u;
    auto off = [&](int s) { return min(slot0 + (uint32_t)s * kWaveSize + lane, last) * 16u; };
    auto ld = [](const char* a) { return NT ? load16(reinterpret_cast<const uint4*>(a)) : *reinterpret_cast<const uint4*>(a); };
    uint4 gq[D], uq[D];
#pragma unroll
    for (int s = 0; s < D; ++s) {
        gq[s] = ld(xg + off(s));
        uq[s] = ld(xu + off(s));
    }
#pragma unroll
    for (int s = 0; s < SPU; ++s) {
        const uint4 g = gq[s % D], uu = uq[s % D];
        if (s + D < SPU) {
            gq[s % D] = ld(xg + off(s + D));
            uq[s % D] = ld(xu + off(s + D));
        }
        mbits[s] = compute_step<CLAMP, true>(lut, g, uu, w, (uint32_t)s * kWaveSize + lane < nslots, limit, a_limit,
                                             clamped, y[s]);
    }
}

// A clamp counter that counts nothing (the second pass of a two-pass group).
struct NoCount {
    __device__ __forceinline__ void add(bool) {}
};

// Groups whose width is not a power of two of lane slots up to 64 and not a
// multiple of 64, up to 8192 columns (24, 40, 48, 96, 384, 896 columns ...):
// each unit is a run of whole groups of one row (p.gpu groups of p.gslots
// slots) that one wave holds in SPU steps; the groups' abs-maxes are formed in
// the wave's own LDS buffer (quantize_seg).  Persistent like the one-wave
// kernel, with the sigmoid table in LDS.
template <int FMT, int SFMT, bool CLAMP, int SPU>
__global__ __launch_bounds__(kThreads) void swiglu_cast_seg_kernel(Params p)
{
    constexpr int kWaves = kThreads / kWaveSize;
    __shared__ __attribute__((aligned(16))) unsigned char lut_raw[kLutLdsBytes];
    __shared__ uint32_t seg_buf[kWaves][SegLds<SPU>::kSlots];
    __shared__ float seg_inv[kWaves][SegLds<SPU>::kGroups];
    __shared__ unsigned long long wg_clamped; // the workgroup's clamp count
    LutT* lut = reinterpret_cast<LutT*>(lut_raw);
    if (CLAMP && threadIdx.x == 0)
        wg_clamped = 0;
    load_lut_to_lds(lut);

    const uint32_t lane = threadIdx.x & (kWaveSize - 1);
    const uint32_t wib = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
    uint32_t block = blockIdx.x;
    if (p.xcd_order && (gridDim.x & 7u) == 0) // XCD-contiguous order, as in the one-wave kernel
        block = (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(block * kWaves + wib);
    const uint32_t nwaves = gridDim.x * kWaves;
    float limit = 0.0f, a_limit = 0.0f;
    if constexpr (CLAMP) {
        limit = p.clamp;
        a_limit = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                               __builtin_bit_cast(int, limit * sigmoid_rn(limit))));
    }
    LaneCount clamped;
    for (uint32_t u = wave; u < p.units; u += nwaves) {
        const uint32_t row = u / p.upr;
        const uint32_t g0 = (u - row * p.upr) * p.gpu;
        const uint32_t ngr = min(p.gpu, p.groups_row - g0);
        const uint32_t slot0 = g0 * p.gslots;
        const float w = p.w ? p.w[row] : 1.0f;
        float y[SPU][8];
        uint32_t mbits[SPU];
        span_compute<CLAMP, SPU>(p, lut, lane, row, slot0, ngr * p.gslots, w, limit, a_limit, clamped, y, mbits);
        quantize_seg<FMT, SFMT, SPU>(p, lane, row, g0, ngr, slot0, y, mbits, seg_buf[wib], seg_inv[wib]);
    }
    if constexpr (CLAMP)
        flush_clamp_count(p.count, &wg_clamped, clamped, lane);
}

// Groups no other kernel covers (wider than 8192 columns and not split evenly
// over 2 or 4 waves, or wider than 32768 columns): one wave per group, which
// reads the group twice, kTwoPassSteps steps at a time -- first for its
// abs-max (and the clamp count), then again for the codes with the group's
// scale.  The second read of a group is often still in the caches.
template <int FMT, int SFMT, bool CLAMP>
__global__ __launch_bounds__(kThreads) void swiglu_cast_2p_kernel(Params p)
{
    constexpr int S = kTwoPassSteps;
    constexpr uint32_t kChunk = S * kWaveSize;
    constexpr int kWaves = kThreads / kWaveSize;
    __shared__ __attribute__((aligned(16))) unsigned char lut_raw[kLutLdsBytes];
    __shared__ unsigned long long wg_clamped; // the workgroup's clamp count
    LutT* lut = reinterpret_cast<LutT*>(lut_raw);
    if (CLAMP && threadIdx.x == 0)
        wg_clamped = 0;
    load_lut_to_lds(lut);

    const uint32_t lane = threadIdx.x & (kWaveSize - 1);
    uint32_t block = blockIdx.x;
    if (p.xcd_order && (gridDim.x & 7u) == 0)
        block = (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(block * kWaves + (threadIdx.x / kWaveSize));
    const uint32_t nwaves = gridDim.x * kWaves;
    float limit = 0.0f, a_limit = 0.0f;
    if constexpr (CLAMP) {
        limit = p.clamp;
        a_limit = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                               __builtin_bit_cast(int, limit * sigmoid_rn(limit))));
    }
    WaveCount clamped;
    NoCount none;
    const uint32_t gs = p.gslots;
    for (uint32_t u = wave; u < p.units; u += nwaves) {
        const uint32_t row = u / p.upr;
        const uint32_t k = u - row * p.upr;
        const uint32_t slot0 = k * gs;
        const float w = p.w ? p.w[row] : 1.0f;
        uint32_t mb = 0;
        for (uint32_t c = 0; c < gs; c += kChunk) {
            float y[S][8];
            uint32_t mbits[S];
            span_compute<CLAMP, S, WaveCount, false>(p, lut, lane, row, slot0 + c, min(kChunk, gs - c), w, limit,
                                                     a_limit, clamped, y, mbits);
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
            span_compute<CLAMP, S>(p, lut, lane, row, slot0 + c, min(kChunk, gs - c), w, limit, a_limit, none, y,
                                   mbits);
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const uint32_t rel = c + (uint32_t)s * kWaveSize + lane;
                if (rel < gs)
                    quantize_store<FMT>(row_codes, slot0 + rel, y[s], inv);
            }
        }
    }
    if constexpr (CLAMP)
        flush_clamp_count(p.count, &wg_clamped, clamped, lane);
}

// The unfused first stage (swiglu_forward): fp32 y [n][hidden], same
// per-element arithmetic as the fused kernel.  Thread t of the grid-stride
// loop owns one 8-column lane slot of one row.
template <bool CLAMP>
__global__ __launch_bounds__(kThreads) void swiglu_forward_kernel(const uint4* __restrict__ x,
                                                                  const float* __restrict__ w,
                                                                  float4* __restrict__ y, uint32_t n,
                                                                  uint32_t slots, float limit_in,
                                                                  unsigned long long* count)
{
    __shared__ __attribute__((aligned(16))) unsigned char lut_raw[kLutLdsBytes];
    __shared__ unsigned long long wg_clamped; // the workgroup's clamp count
    LutT* lut = reinterpret_cast<LutT*>(lut_raw);
    if (CLAMP && threadIdx.x == 0)
        wg_clamped = 0;
    load_lut_to_lds(lut);
    float limit = 0.0f, a_limit = 0.0f;
    if constexpr (CLAMP) {
        limit = limit_in;
        a_limit = limit * sigmoid_rn(limit);
    }
    WaveCount clamped;
    const uint64_t total = (uint64_t)n * slots;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    // every lane runs the same trip count so that the clamp ballots see whole waves
    const uint64_t first = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t wave_first = first - (threadIdx.x & (kWaveSize - 1));
    for (uint64_t base = wave_first; base < total; base += stride) {
        const uint64_t t = base + (threadIdx.x & (kWaveSize - 1));
        const bool active = t < total;
        const uint32_t row = active ? (uint32_t)(t / slots) : 0;
        const uint32_t slot = active ? (uint32_t)(t - (uint64_t)row * slots) : 0;
        uint4 G = make_uint4(0, 0, 0, 0), U = make_uint4(0, 0, 0, 0);
        float wr = 1.0f;
        if (active) {
            G = x[(size_t)row * 2 * slots + slot];
            U = x[(size_t)row * 2 * slots + slots + slot];
            wr = w ? w[row] : 1.0f;
        }
        const uint32_t gw[4] = {G.x, G.y, G.z, G.w};
        const uint32_t uw[4] = {U.x, U.y, U.z, U.w};
        float v[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = swiglu_elem<0, CLAMP>(lut, gw[k], uw[k], wr, limit, a_limit, clamped);
            v[2 * k + 1] = swiglu_elem<16, CLAMP>(lut, gw[k], uw[k], wr, limit, a_limit, clamped);
        }
        if (active) {
            y[2 * t] = make_float4(v[0], v[1], v[2], v[3]);
            y[2 * t + 1] = make_float4(v[4], v[5], v[6], v[7]);
        }
    }
    if constexpr (CLAMP)
        flush_clamp_count(count, &wg_clamped, clamped, threadIdx.x & (kWaveSize - 1));
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
struct DeviceState {
    std::mutex mu;
    std::atomic<bool> ready{false}; // set last, after cus and the table; read without the lock
    int cus = 0;
};
DeviceState g_dev[kMaxDevices];

tk_status init_device(int dev)
{
    if (dev < 0 || dev >= kMaxDevices)
        return TK_ERR_INVALID_ARG;
    DeviceState& st = g_dev[dev];
    std::lock_guard<std::mutex> lock(st.mu);
    if (st.ready.load(std::memory_order_acquire))
        return TK_OK;
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess)
        return TK_ERR_HIP;
    if (prev != dev && hipSetDevice(dev) != hipSuccess)
        return TK_ERR_HIP;
    tk_status rc = TK_OK;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        rc = TK_ERR_HIP;
    } else {
        hipLaunchKernelGGL(sigma_lut_init_kernel, dim3((kLutSize + 255) / 256), dim3(256), 0, nullptr);
        if (hipGetLastError() != hipSuccess || hipStreamSynchronize(nullptr) != hipSuccess)
            rc = TK_ERR_HIP;
    }
    if (rc == TK_OK) {
        st.cus = cus;
        st.ready.store(true, std::memory_order_release);
    }
    if (prev != dev)
        (void)hipSetDevice(prev);
    return rc;
}

tk_status ensure_device(int& dev);

// small: a launch of at most kSmallUnitsPerCU units per CU, which takes the
// 16 KiB table (units of up to 4 steps; longer row-reduced units stream their
// loads and keep the 32 KiB table).
template <int FMT, int SFMT, bool CLAMP, int SPU, bool ROWRED, bool PARTIAL>
void launch_one(const Params& p, int blocks, bool small, hipStream_t stream)
{
    constexpr bool kCanT16 = !(ROWRED && SPU >= kStreamMinSteps);
    const bool single = p.units <= (uint32_t)blocks * (kThreads / kWaveSize); // one pass of the grid
    if constexpr (!ROWRED) {
        if (p.gl_log2 >= 5) { // per-block groups of 32 or 64 lanes
            if (small && single)
                hipLaunchKernelGGL((swiglu_cast_kernel<FMT, SFMT, CLAMP, SPU, ROWRED, PARTIAL, true, true, true>),
                                   dim3(blocks), dim3(kThreads), 0, stream, p);
            else if (small)
                hipLaunchKernelGGL((swiglu_cast_kernel<FMT, SFMT, CLAMP, SPU, ROWRED, PARTIAL, true, true>),
                                   dim3(blocks), dim3(kThreads), 0, stream, p);
            else
                hipLaunchKernelGGL((swiglu_cast_kernel<FMT, SFMT, CLAMP, SPU, ROWRED, PARTIAL, true>), dim3(blocks),
                                   dim3(kThreads), 0, stream, p);
            return;
        }
    }
    if constexpr (kCanT16) {
        if (small && single) {
            hipLaunchKernelGGL((swiglu_cast_kernel<FMT, SFMT, CLAMP, SPU, ROWRED, PARTIAL, false, true, true>),
                               dim3(blocks), dim3(kThreads), 0, stream, p);
            return;
        }
        if (small) {
            hipLaunchKernelGGL((swiglu_cast_kernel<FMT, SFMT, CLAMP, SPU, ROWRED, PARTIAL, false, true>), dim3(blocks),
                               dim3(kThreads), 0, stream, p);
            return;
        }
    }
    hipLaunchKernelGGL((swiglu_cast_kernel<FMT, SFMT, CLAMP, SPU, ROWRED, PARTIAL>), dim3(blocks), dim3(kThreads),
                       0, stream, p);
}

template <int FMT, int SFMT, bool CLAMP, bool ROWRED, bool PARTIAL>
bool launch_spu(int spu_max, const Params& p, int blocks, bool small, hipStream_t stream)
{
    switch (spu_max) {
    case 1: launch_one<FMT, SFMT, CLAMP, 1, ROWRED, PARTIAL>(p, blocks, small, stream); return true;
    case 2: launch_one<FMT, SFMT, CLAMP, 2, ROWRED, PARTIAL>(p, blocks, small, stream); return true;
    case 4: launch_one<FMT, SFMT, CLAMP, 4, ROWRED, PARTIAL>(p, blocks, small, stream); return true;
    case 8:
        if constexpr (ROWRED) { launch_one<FMT, SFMT, CLAMP, 8, ROWRED, PARTIAL>(p, blocks, small, stream); return true; }
        return false;
    case 12:
        if constexpr (ROWRED) { launch_one<FMT, SFMT, CLAMP, 12, ROWRED, PARTIAL>(p, blocks, small, stream); return true; }
        return false;
    case 16:
        if constexpr (ROWRED) { launch_one<FMT, SFMT, CLAMP, 16, ROWRED, PARTIAL>(p, blocks, small, stream); return true; }
        return false;
    default: return false;
    }
}

template <int FMT, int SFMT, bool CLAMP>
bool launch_xw(bool partial, uint32_t waves, uint32_t spu_max, const Params& p, int blocks, hipStream_t s)
{
#define TK_XW(SP, PA, WW)                                                                              \
    if (spu_max == SP && partial == PA && waves == WW) {                                                \
        hipLaunchKernelGGL((swiglu_cast_xw_kernel<FMT, SFMT, CLAMP, SP, PA, WW>), dim3(blocks), dim3(kThreads), \
                           0, s, p);                                                                    \
        return true;                                                                                    \
    }
    // a wave's share, ceil(k / W), is 9..16 steps
    TK_XW(12u, false, 2u)
    TK_XW(12u, false, 4u)
    TK_XW(12u, true, 2u)
    TK_XW(12u, true, 4u)
    TK_XW(16u, false, 2u)
    TK_XW(16u, false, 4u)
    TK_XW(16u, true, 2u)
    TK_XW(16u, true, 4u)
#undef TK_XW
    return false;
}

template <int FMT>
bool dispatch_xw(int sfmt, bool clamp, bool partial, uint32_t waves, uint32_t spu_max, const Params& p, int blocks,
                 hipStream_t s)
{
    if (sfmt == TK_SCALE_FP32)
        return clamp ? launch_xw<FMT, TK_SCALE_FP32, true>(partial, waves, spu_max, p, blocks, s)
                     : launch_xw<FMT, TK_SCALE_FP32, false>(partial, waves, spu_max, p, blocks, s);
    return clamp ? launch_xw<FMT, TK_SCALE_UE8M0, true>(partial, waves, spu_max, p, blocks, s)
                 : launch_xw<FMT, TK_SCALE_UE8M0, false>(partial, waves, spu_max, p, blocks, s);
}

template <int FMT>
bool dispatch(int sfmt, bool clamp, bool rowred, bool partial, int spu_max, const Params& p, int blocks, bool small,
              hipStream_t s)
{
#define TK_BRANCH(SF, CL, RR, PA)                                                                       \
    if (sfmt == SF && clamp == CL && rowred == RR && partial == PA)                                     \
        return launch_spu<FMT, SF, CL, RR, PA>(spu_max, p, blocks, small, s);
#define TK_BRANCH2(SF, CL, RR) TK_BRANCH(SF, CL, RR, false) TK_BRANCH(SF, CL, RR, true)
    TK_BRANCH2(TK_SCALE_FP32, false, false)
    TK_BRANCH2(TK_SCALE_FP32, false, true)
    TK_BRANCH2(TK_SCALE_FP32, true, false)
    TK_BRANCH2(TK_SCALE_FP32, true, true)
    TK_BRANCH2(TK_SCALE_UE8M0, false, false)
    TK_BRANCH2(TK_SCALE_UE8M0, false, true)
    TK_BRANCH2(TK_SCALE_UE8M0, true, false)
    TK_BRANCH2(TK_SCALE_UE8M0, true, true)
#undef TK_BRANCH2
#undef TK_BRANCH
    return false;
}


template <int FMT, int SFMT, bool CLAMP>
bool launch_seg(uint32_t spu_max, const Params& p, int blocks, hipStream_t s)
{
    switch (spu_max) {
#define TK_SEG(N)                                                                                              \
    case N:                                                                                                    \
        hipLaunchKernelGGL((swiglu_cast_seg_kernel<FMT, SFMT, CLAMP, N>), dim3(blocks), dim3(kThreads), 0, s, p); \
        return true;
        TK_SEG(1)
        TK_SEG(2)
        TK_SEG(4)
        TK_SEG(8)
        TK_SEG(12)
        TK_SEG(16)
#undef TK_SEG
    default: return false;
    }
}

template <int FMT>
bool dispatch_seg(int sfmt, bool clamp, bool twopass, uint32_t spu_max, const Params& p, int blocks, hipStream_t s)
{
    if (twopass) {
#define TK_2P(SF, CL) hipLaunchKernelGGL((swiglu_cast_2p_kernel<FMT, SF, CL>), dim3(blocks), dim3(kThreads), 0, s, p)
        if (sfmt == TK_SCALE_FP32) {
            if (clamp) TK_2P(TK_SCALE_FP32, true); else TK_2P(TK_SCALE_FP32, false);
        } else {
            if (clamp) TK_2P(TK_SCALE_UE8M0, true); else TK_2P(TK_SCALE_UE8M0, false);
        }
#undef TK_2P
        return true;
    }
    if (sfmt == TK_SCALE_FP32)
        return clamp ? launch_seg<FMT, TK_SCALE_FP32, true>(spu_max, p, blocks, s)
                     : launch_seg<FMT, TK_SCALE_FP32, false>(spu_max, p, blocks, s);
    return clamp ? launch_seg<FMT, TK_SCALE_UE8M0, true>(spu_max, p, blocks, s)
                 : launch_seg<FMT, TK_SCALE_UE8M0, false>(spu_max, p, blocks, s);
}

// Persistent grid: workgroups of 256 threads per CU.  Two measured best for
// large launches; launches of at most kSmallUnitsPerCU units per CU take four,
// so that each wave has at most four units to work through (a headline-shaped
// launch of 2400 rows: 7.7 us against 8.9; 8192 rows: 16.4 us against 18.2;
// from about 16384 units per 256 CUs the two settle level, and two win above).
constexpr int kBlocksPerCU = 2;
constexpr int kBlocksPerCUSmall = 4;
constexpr uint32_t kSmallUnitsPerCU = 64;

tk_status swiglu_cast(int fmt, const void* x, const float* w, int64_t n, int64_t hidden, int64_t group_size,
                      float clamp_limit, int scale_fmt, void* codes, void* scales, int64_t* clamped_count,
                      void* stream)
{
    // ---- validation: no HIP call before every argument is checked ----
    if (n < 0 || n >= (int64_t)INT_MAX)
        return TK_ERR_INVALID_ARG;
    if (hidden <= 0 || hidden % kSlotCols != 0 || hidden > (int64_t)INT_MAX / 4)
        return TK_ERR_INVALID_ARG;
    if (group_size < 0 || (group_size != 0 && (group_size % kSlotCols != 0 || hidden % group_size != 0)))
        return TK_ERR_INVALID_ARG;
    if (std::isnan(clamp_limit) || clamp_limit <= 0.0f)
        return TK_ERR_INVALID_ARG;
    const int64_t G = group_size ? group_size : hidden;
    const int64_t groups_row = hidden / G;
    ScaleSpec sp;
    if (!scale_spec(scale_fmt, n, groups_row, sp))
        return TK_ERR_INVALID_ARG;
    if (n > 0 && (!x || !codes || !scales))
        return TK_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(w, 4) || !aligned(codes, fmt == 8 ? 8 : 4) || !aligned(clamped_count, 8) ||
        !aligned(scales, sp.align))
        return TK_ERR_INVALID_ARG;
    const size_t x_bytes = (size_t)n * (size_t)hidden * 4u;
    const size_t w_bytes = w ? (size_t)n * 4u : 0;
    const size_t c_bytes = (size_t)n * (size_t)(fmt == 8 ? hidden : hidden / 2);
    const size_t s_bytes = sp.bytes;
    const size_t k_bytes = clamped_count ? 8u : 0u;
    if (n > 0 && (overlaps(codes, c_bytes, x, x_bytes) || overlaps(codes, c_bytes, w, w_bytes) ||
                  overlaps(scales, s_bytes, x, x_bytes) || overlaps(scales, s_bytes, w, w_bytes) ||
                  overlaps(codes, c_bytes, scales, s_bytes) || overlaps(clamped_count, k_bytes, x, x_bytes) ||
                  overlaps(clamped_count, k_bytes, w, w_bytes) || overlaps(clamped_count, k_bytes, codes, c_bytes) ||
                  overlaps(clamped_count, k_bytes, scales, s_bytes)))
        return TK_ERR_INVALID_ARG;

    // ---- shape -> kernel variant ----
    Params p{};
    UnitPlan plan;
    {
        const tk_status rc = plan_units(n, hidden, group_size, n >= 1024 ? 4u : (n >= 256 ? 2u : 1u), p, plan);
        if (rc != TK_OK)
            return rc;
    }
    if (n == 0)
        return TK_OK;

    int dev = 0;
    {
        const tk_status rc = ensure_device(dev);
        if (rc != TK_OK)
            return rc;
    }

    p.x = static_cast<const uint4*>(x);
    p.w = w;
    p.codes = static_cast<uint8_t*>(codes);
    p.scales = scales;
    p.count = reinterpret_cast<unsigned long long*>(clamped_count);
    p.scale_layout = sp.layout;
    p.scale_ld = sp.ld;
    const bool clamp = !std::isinf(clamp_limit);
    p.clamp = clamp_limit;

    const uint32_t waves_per_block = kThreads / kWaveSize;
    // one unit per wave (a group of xwaves units per xwaves waves) when the grid is not capped
    const uint32_t want = (p.units + waves_per_block - 1) / waves_per_block;
    const uint32_t cus = (uint32_t)g_dev[dev].cus;
    const bool small = (uint64_t)p.units <= (uint64_t)cus * kSmallUnitsPerCU;
    const uint32_t per_cu = small ? kBlocksPerCUSmall : kBlocksPerCU;
    const uint32_t cap = cus * per_cu;
    const int blocks = (int)(want < cap ? want : cap);
    // The XCD-contiguous block order puts the units of a partial last pass of
    // the grid-stride loop on the lowest-numbered XCDs; the plain order spreads
    // them over all eight.  That matters for a small launch of a few passes:
    // when its units do not fill the passes evenly it keeps the plain order
    // (interleaved A/B replayed from graphs, outputs identical: 1000 x 7168
    // per-block 9.18 -> 8.54 us, 2000 x 7168 15.72 -> 14.13, 600 x 7168
    // 7.07 -> 6.91; every other shape measured within 1%), while small
    // launches that fill their passes evenly, and every large one, keep the
    // XCD order, which measured up to 4% faster for them.
    p.xcd_order = (!small || p.units % ((uint32_t)blocks * waves_per_block) == 0) ? 1u : 0u;

    hipStream_t s = static_cast<hipStream_t>(stream);
    bool ok;
    if (plan.seg || plan.twopass)
        ok = fmt == 8 ? dispatch_seg<8>(sp.kind, clamp, plan.twopass, plan.spu_max, p, blocks, s)
                      : dispatch_seg<4>(sp.kind, clamp, plan.twopass, plan.spu_max, p, blocks, s);
    else if (plan.xwaves > 1)
        ok = fmt == 8 ? dispatch_xw<8>(sp.kind, clamp, plan.partial, plan.xwaves, plan.spu_max, p, blocks, s)
                      : dispatch_xw<4>(sp.kind, clamp, plan.partial, plan.xwaves, plan.spu_max, p, blocks, s);
    else
        ok = fmt == 8 ? dispatch<8>(sp.kind, clamp, plan.rowred, plan.partial, (int)plan.spu_max, p, blocks, small, s)
                      : dispatch<4>(sp.kind, clamp, plan.rowred, plan.partial, (int)plan.spu_max, p, blocks, small, s);
    if (!ok)
        return TK_ERR_UNSUPPORTED;
    if (hipGetLastError() != hipSuccess)
        return TK_ERR_HIP;
    return TK_OK;
}

tk_status ensure_device(int& dev)
{
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return TK_ERR_HIP;
    if (!g_dev[dev].ready.load(std::memory_order_acquire))
        return init_device(dev);
    return TK_OK;
}

tk_status swiglu_forward(const void* x, const float* w, int64_t n, int64_t hidden, float clamp_limit,
                         float* y, int64_t* clamped_count, void* stream)
{
    if (n < 0 || n >= (int64_t)INT_MAX)
        return TK_ERR_INVALID_ARG;
    if (hidden <= 0 || hidden % kSlotCols != 0 || hidden > (int64_t)INT_MAX / 4)
        return TK_ERR_INVALID_ARG;
    if (std::isnan(clamp_limit) || clamp_limit <= 0.0f)
        return TK_ERR_INVALID_ARG;
    if (n > 0 && (!x || !y))
        return TK_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(w, 4) || !aligned(y, 16) || !aligned(clamped_count, 8))
        return TK_ERR_INVALID_ARG;
    const size_t x_bytes = (size_t)n * (size_t)hidden * 4u;
    const size_t w_bytes = w ? (size_t)n * 4u : 0;
    const size_t y_bytes = (size_t)n * (size_t)hidden * 4u;
    const size_t k_bytes = clamped_count ? 8u : 0u;
    if (n > 0 && (overlaps(y, y_bytes, x, x_bytes) || overlaps(y, y_bytes, w, w_bytes) ||
                  overlaps(clamped_count, k_bytes, x, x_bytes) || overlaps(clamped_count, k_bytes, w, w_bytes) ||
                  overlaps(clamped_count, k_bytes, y, y_bytes)))
        return TK_ERR_INVALID_ARG;
    if (n == 0)
        return TK_OK;
    int dev = 0;
    const tk_status rc = ensure_device(dev);
    if (rc != TK_OK)
        return rc;
    const uint32_t slots = (uint32_t)(hidden / kSlotCols);
    const uint64_t total = (uint64_t)n * slots;
    const uint64_t want = (total + kThreads - 1) / kThreads;
    const uint64_t cap = (uint64_t)g_dev[dev].cus * kBlocksPerCU;
    const int blocks = (int)(want < cap ? want : cap);
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto* cnt = reinterpret_cast<unsigned long long*>(clamped_count);
    if (std::isinf(clamp_limit))
        hipLaunchKernelGGL(swiglu_forward_kernel<false>, dim3(blocks), dim3(kThreads), 0, s,
                           static_cast<const uint4*>(x), w, reinterpret_cast<float4*>(y), (uint32_t)n, slots,
                           clamp_limit, cnt);
    else
        hipLaunchKernelGGL(swiglu_forward_kernel<true>, dim3(blocks), dim3(kThreads), 0, s,
                           static_cast<const uint4*>(x), w, reinterpret_cast<float4*>(y), (uint32_t)n, slots,
                           clamp_limit, cnt);
    return hipGetLastError() == hipSuccess ? TK_OK : TK_ERR_HIP;
}

} // namespace

extern "C" {

tk_status tk_swiglu_forward(const void* x, const float* topk_weight, int64_t n, int64_t hidden,
                            float clamp_limit, float* y, int64_t* clamped_count, void* stream)
{
    return swiglu_forward(x, topk_weight, n, hidden, clamp_limit, y, clamped_count, stream);
}

tk_status tk_init(int device)
{
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess)
        return TK_ERR_HIP;
    if (device < 0 || device >= count)
        return TK_ERR_INVALID_ARG;
    return init_device(device);
}

tk_status tk_swiglu_cast_fp8(const void* x, const float* topk_weight, int64_t n, int64_t hidden,
                             int64_t group_size, float clamp_limit, tk_scale_fmt scale_fmt, void* codes,
                             void* scales, int64_t* clamped_count, void* stream)
{
    return swiglu_cast(8, x, topk_weight, n, hidden, group_size, clamp_limit, (int)scale_fmt, codes, scales,
                       clamped_count, stream);
}

tk_status tk_swiglu_cast_fp4(const void* x, const float* topk_weight, int64_t n, int64_t hidden,
                             int64_t group_size, float clamp_limit, tk_scale_fmt scale_fmt, void* codes,
                             void* scales, int64_t* clamped_count, void* stream)
{
    return swiglu_cast(4, x, topk_weight, n, hidden, group_size, clamp_limit, (int)scale_fmt, codes, scales,
                       clamped_count, stream);
}

const char* tk_status_str(tk_status status)
{
    switch (status) {
    case TK_OK: return "TK_OK";
    case TK_ERR_INVALID_ARG: return "TK_ERR_INVALID_ARG";
    case TK_ERR_UNSUPPORTED: return "TK_ERR_UNSUPPORTED";
    case TK_ERR_HIP: return "TK_ERR_HIP";
    }
    return "TK_UNKNOWN_STATUS";
}

} // extern "C"
