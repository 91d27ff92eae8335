// tk_reduce.hip -- the weighted top-k reduce of the experts' output rows for
// MI355X (gfx950), behind tk_moe_reduce in include/tk.h.
//
// The operation is the fused reduce of "【DeepSeek】TileKernels从入门到精通"
// ch.3: section "结算中心的“减法工程”" (each token's top-k expert outputs are
// weighted and summed in one pass, with the routing weights, the quantisation
// scale factors and a global scale applied in registers, so the expert outputs
// are read once and the result written once) and section "动态寻址" (the rows
// are found through a token/top-k -> position map, whatever the load across
// experts).  Per token t and column c, over the present slots j in order:
//   f = RN(w[t,j] * row_scale[p]) (or w[t,j]),  acc = RN(acc + RN(f * x[p,c]))
// from acc = +0; out = RN(acc * global_scale), rounded to bf16 (nearest, ties
// to even) or kept in fp32.
//
// gfx950 design.  The work is an HBM-bound gather: every present row is read
// once, no row is shared, so there is nothing to keep in LDS.  A unit is
// (token, SPU steps of 512 columns); one 64-lane wave owns one unit and lane
// l holds the 8 columns of 16-byte slot 64*step + l of every row it gathers.
//   1. Slot metadata in parallel: lane j < k loads pos[t,j], w[t,j] and the
//      row scale, and forms f; a ballot marks the present slots, and the wave
//      walks that mask with find-first-set to move each present slot's row and
//      f into wave-uniform registers, in slot order (dropped slots vanish, so
//      the loads below are only for rows that contribute).
//   2. All KT x SPU row loads of the unit are issued before the first use
//      (16 bytes per lane, non-temporal: nothing is re-read), row base in
//      scalar registers, lane offset in 32 bits.  Above 32 slots per token
//      (up to 64, one per lane for step 1) moe_reduce_wide_kernel takes the
//      present slots 32 at a time through steps 2 and 3, the sum carried over.
//   3. fp32 multiply and add in slot order (no contraction), the global scale,
//      then v_cvt_pk_bf16_f32 (round to nearest even) and 16-byte
//      non-temporal stores.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "tk.h"

namespace {

constexpr int kWave = 64;
constexpr uint32_t kSlotBytes = 16;   // 8 bf16 columns per lane per step
constexpr int64_t kMaxK = 64; // one slot per lane for the metadata
constexpr int kWideKT = 32;   // rows whose loads a wave holds at once above 32 slots

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct ReduceParams {
    const char* x;          // bf16 rows [n_rows, hidden]
    const float* row_scale; // [n_rows] or null
    const int32_t* pos;     // [tokens, k]
    const float* w;         // [tokens, k]
    char* out;              // [tokens, hidden] bf16 or fp32
    float gscale;
    uint32_t k;
    uint32_t n_rows;
    uint32_t slots;         // hidden / 8
    uint32_t steps_row;     // ceil(slots / 64)
    uint32_t upt;           // units per token = steps_row / SPU
    uint32_t units;         // tokens * upt
    uint32_t row_bytes;     // hidden * 2
};

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xFFFF0000u); }

template <int KT, int SPU, bool OUT_BF16, int THREADS>
__global__ __launch_bounds__(THREADS) void moe_reduce_kernel(ReduceParams p)
{
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t u = __builtin_amdgcn_readfirstlane(blockIdx.x * (THREADS / kWave) + threadIdx.x / kWave);
    if (u >= p.units)
        return;
    const uint32_t t = u / p.upt;
    const uint32_t step0 = (u - t * p.upt) * SPU;

    // ---- 1. slot metadata, one slot per lane, then compacted in slot order
    uint32_t q = 0xFFFFFFFFu;
    float f = 0.0f;
    if (lane < p.k) {
        const size_t i = (size_t)t * p.k + lane;
        q = (uint32_t)p.pos[i];
        const float wj = p.w[i];
        if (q < p.n_rows)
            f = p.row_scale ? wj * p.row_scale[q] : wj;
    }
    uint64_t mask = __builtin_amdgcn_ballot_w64(lane < p.k && q < p.n_rows);
    const uint32_t count = (uint32_t)__builtin_popcountll(mask);
    uint32_t row[KT];
    float fm[KT];
#pragma unroll
    for (int m = 0; m < KT; ++m) {
        const uint32_t l = mask ? (uint32_t)__builtin_ctzll(mask) : 0u;
        row[m] = __builtin_amdgcn_readlane(q, l);
        fm[m] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(uint32_t, f), l));
        mask &= mask - 1;
    }

    // ---- 2. every row load of the unit in flight before the first use
    const uint32_t lane_off = (step0 * kWave + lane) * kSlotBytes;
    const uint32_t last_off = (p.slots - 1u) * kSlotBytes; // lanes past the row end re-read its last slot
    u32x4 raw[KT][SPU];
#pragma unroll
    for (int m = 0; m < KT; ++m) {
        if ((uint32_t)m < count) {
            const char* xr = p.x + (size_t)row[m] * p.row_bytes;
#pragma unroll
            for (int s = 0; s < SPU; ++s) {
                const uint32_t off = min(lane_off + (uint32_t)s * (kWave * kSlotBytes), last_off);
                raw[m][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xr + off));
            }
        }
    }

    // ---- 3. weighted sum in slot order, global scale, convert, store
    float acc[SPU][8];
#pragma unroll
    for (int s = 0; s < SPU; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[s][e] = 0.0f;
#pragma unroll
    for (int m = 0; m < KT; ++m) {
        if ((uint32_t)m < count) {
#pragma unroll
            for (int s = 0; s < SPU; ++s) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[s][2 * e] = acc[s][2 * e] + fm[m] * bf16_lo(raw[m][s][e]);
                    acc[s][2 * e + 1] = acc[s][2 * e + 1] + fm[m] * bf16_hi(raw[m][s][e]);
                }
            }
        }
    }
    constexpr uint32_t kOutSlot = OUT_BF16 ? 16u : 32u;
    char* orow = p.out + (size_t)t * p.slots * kOutSlot;
#pragma unroll
    for (int s = 0; s < SPU; ++s) {
        const uint32_t slot = (step0 + (uint32_t)s) * kWave + lane;
        if (slot < p.slots) {
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o[e] = acc[s][e] * p.gscale;
            if constexpr (OUT_BF16) {
                u32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const f32x2 pr = {o[2 * e], o[2 * e + 1]};
                    v[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
                }
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(orow + (size_t)slot * kOutSlot));
            } else {
                const u32x4 a = {__builtin_bit_cast(uint32_t, o[0]), __builtin_bit_cast(uint32_t, o[1]),
                                 __builtin_bit_cast(uint32_t, o[2]), __builtin_bit_cast(uint32_t, o[3])};
                const u32x4 b = {__builtin_bit_cast(uint32_t, o[4]), __builtin_bit_cast(uint32_t, o[5]),
                                 __builtin_bit_cast(uint32_t, o[6]), __builtin_bit_cast(uint32_t, o[7])};
                u32x4* dst = reinterpret_cast<u32x4*>(orow + (size_t)slot * kOutSlot);
                __builtin_nontemporal_store(a, dst);
                __builtin_nontemporal_store(b, dst + 1);
            }
        }
    }
}

// k in 33..64: moe_reduce_kernel's steps with one 512-column step per unit,
// the present slots taken kWideKT at a time (their loads in flight together),
// the sum carried from one batch to the next in slot order.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void moe_reduce_wide_kernel(ReduceParams p)
{
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const uint32_t u = __builtin_amdgcn_readfirstlane(blockIdx.x * (256 / kWave) + threadIdx.x / kWave);
    if (u >= p.units)
        return;
    const uint32_t t = u / p.upt;
    const uint32_t step0 = u - t * p.upt;

    uint32_t q = 0xFFFFFFFFu;
    float f = 0.0f;
    if (lane < p.k) {
        const size_t i = (size_t)t * p.k + lane;
        q = (uint32_t)p.pos[i];
        const float wj = p.w[i];
        if (q < p.n_rows)
            f = p.row_scale ? wj * p.row_scale[q] : wj;
    }
    uint64_t mask = __builtin_amdgcn_ballot_w64(lane < p.k && q < p.n_rows);
    const uint32_t count = (uint32_t)__builtin_popcountll(mask);
    const uint32_t off = min((step0 * kWave + lane) * kSlotBytes, (p.slots - 1u) * kSlotBytes);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] = 0.0f;
    for (uint32_t done = 0; done < count; done += kWideKT) {
        const uint32_t n = min(count - done, (uint32_t)kWideKT);
        uint32_t row[kWideKT];
        float fm[kWideKT];
#pragma unroll
        for (int m = 0; m < kWideKT; ++m) {
            const uint32_t l = mask ? (uint32_t)__builtin_ctzll(mask) : 0u;
            row[m] = __builtin_amdgcn_readlane(q, l);
            fm[m] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(uint32_t, f), l));
            mask &= mask - 1;
        }
        u32x4 raw[kWideKT];
#pragma unroll
        for (int m = 0; m < kWideKT; ++m)
            if ((uint32_t)m < n)
                raw[m] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.x + (size_t)row[m] * p.row_bytes + off));
#pragma unroll
        for (int m = 0; m < kWideKT; ++m) {
            if ((uint32_t)m < n) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] = acc[2 * e] + fm[m] * bf16_lo(raw[m][e]);
                    acc[2 * e + 1] = acc[2 * e + 1] + fm[m] * bf16_hi(raw[m][e]);
                }
            }
        }
    }
    constexpr uint32_t kOutSlot = OUT_BF16 ? 16u : 32u;
    const uint32_t slot = step0 * kWave + lane;
    if (slot < p.slots) {
        char* dst = p.out + ((size_t)t * p.slots + slot) * kOutSlot;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            o[e] = acc[e] * p.gscale;
        if constexpr (OUT_BF16) {
            u32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const f32x2 pr = {o[2 * e], o[2 * e + 1]};
                v[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
            }
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
        } else {
            const u32x4 a = {__builtin_bit_cast(uint32_t, o[0]), __builtin_bit_cast(uint32_t, o[1]),
                             __builtin_bit_cast(uint32_t, o[2]), __builtin_bit_cast(uint32_t, o[3])};
            const u32x4 b = {__builtin_bit_cast(uint32_t, o[4]), __builtin_bit_cast(uint32_t, o[5]),
                             __builtin_bit_cast(uint32_t, o[6]), __builtin_bit_cast(uint32_t, o[7])};
            __builtin_nontemporal_store(a, reinterpret_cast<u32x4*>(dst));
            __builtin_nontemporal_store(b, reinterpret_cast<u32x4*>(dst) + 1);
        }
    }
}

bool overlaps(const void* a, size_t an, const void* b, size_t bn)
{
    if (!a || !b || an == 0 || bn == 0)
        return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

// Block size: 1024 threads (16 waves) while a unit's loads fit in the 128
// VGPRs such a block allows; measured a few per cent faster than 256 on the
// 4096 x top-8 x 7168 workload.  k > 8 keeps 256-thread blocks.
constexpr int threads_for(int kt) { return kt <= 8 ? 1024 : 256; }

template <int KT, int SPU>
void launch_out(bool bf16_out, const ReduceParams& p, hipStream_t s)
{
    constexpr int T = threads_for(KT);
    const uint32_t blocks = (p.units + (T / kWave) - 1) / (T / kWave); // one unit per wave
    if (bf16_out)
        hipLaunchKernelGGL((moe_reduce_kernel<KT, SPU, true, T>), dim3(blocks), dim3(T), 0, s, p);
    else
        hipLaunchKernelGGL((moe_reduce_kernel<KT, SPU, false, T>), dim3(blocks), dim3(T), 0, s, p);
}

// Row loads per unit: SPU steps of KT rows, SPU the largest power of two up
// to spu_max(KT) that divides the row's step count.  Eight 16-byte loads per
// lane (KT = 8, SPU = 1) measured best on the 4096 x top-8 x 7168 workload.
template <int KT>
void launch_spu(uint32_t spu, bool bf16_out, const ReduceParams& p, hipStream_t s)
{
    if constexpr (KT <= 2) {
        if (spu == 4) {
            launch_out<KT, 4>(bf16_out, p, s);
            return;
        }
    }
    if constexpr (KT <= 4) {
        if (spu == 2) {
            launch_out<KT, 2>(bf16_out, p, s);
            return;
        }
    }
    launch_out<KT, 1>(bf16_out, p, s);
}

} // namespace

extern "C" tk_status tk_moe_reduce(const void* x, const float* row_scale, const int32_t* pos,
                                   const float* topk_weight, float global_scale, int64_t tokens, int64_t k,
                                   int64_t hidden, int64_t n_rows, tk_dtype out_dtype, void* out, void* stream)
{
    // ---- validation: no HIP call before every argument is checked ----
    if (tokens < 0 || tokens >= (int64_t)INT_MAX || k <= 0 || n_rows < 0 || n_rows > (int64_t)INT_MAX)
        return TK_ERR_INVALID_ARG;
    if (hidden <= 0 || hidden % 8 != 0 || hidden > (int64_t)INT_MAX / 8)
        return TK_ERR_INVALID_ARG;
    if (out_dtype != TK_DTYPE_BF16 && out_dtype != TK_DTYPE_FP32)
        return TK_ERR_INVALID_ARG;
    if (!std::isfinite(global_scale))
        return TK_ERR_INVALID_ARG;
    if (tokens > 0 && (!pos || !topk_weight || !out || (n_rows > 0 && !x)))
        return TK_ERR_INVALID_ARG;
    if (((uintptr_t)x & 15) || ((uintptr_t)out & 15) || ((uintptr_t)pos & 3) || ((uintptr_t)topk_weight & 3) ||
        ((uintptr_t)row_scale & 3))
        return TK_ERR_INVALID_ARG;
    const size_t out_bytes = (size_t)tokens * (size_t)hidden * (out_dtype == TK_DTYPE_BF16 ? 2u : 4u);
    const size_t map_bytes = (size_t)tokens * (size_t)k * 4u;
    if (tokens > 0 && (overlaps(out, out_bytes, x, (size_t)n_rows * (size_t)hidden * 2u) ||
                       overlaps(out, out_bytes, pos, map_bytes) || overlaps(out, out_bytes, topk_weight, map_bytes) ||
                       overlaps(out, out_bytes, row_scale, (size_t)n_rows * 4u)))
        return TK_ERR_INVALID_ARG;
    if (k > kMaxK)
        return TK_ERR_UNSUPPORTED;
    const uint32_t slots = (uint32_t)(hidden / 8);
    const uint32_t steps_row = (slots + kWave - 1) / kWave;
    const uint32_t kt = k <= 1 ? 1u : k <= 2 ? 2u : k <= 4 ? 4u : k <= 8 ? 8u : k <= 16 ? 16u : k <= 32 ? 32u : 64u;
    const uint32_t spu_max = kt <= 2 ? 4u : kt <= 4 ? 2u : 1u;
    uint32_t spu = spu_max;
    while (steps_row % spu != 0)
        spu >>= 1;
    const uint32_t upt = steps_row / spu;
    if ((uint64_t)tokens * upt >= (uint64_t)UINT32_MAX - 1024u)
        return TK_ERR_UNSUPPORTED;
    if (tokens == 0)
        return TK_OK;

    ReduceParams p{};
    p.x = static_cast<const char*>(x);
    p.row_scale = row_scale;
    p.pos = pos;
    p.w = topk_weight;
    p.out = static_cast<char*>(out);
    p.gscale = global_scale;
    p.k = (uint32_t)k;
    p.n_rows = (uint32_t)n_rows;
    p.slots = slots;
    p.steps_row = steps_row;
    p.upt = upt;
    p.units = (uint32_t)tokens * upt;
    p.row_bytes = (uint32_t)(hidden * 2);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf16_out = out_dtype == TK_DTYPE_BF16;
    switch (kt) {
    case 1: launch_spu<1>(spu, bf16_out, p, s); break;
    case 2: launch_spu<2>(spu, bf16_out, p, s); break;
    case 4: launch_spu<4>(spu, bf16_out, p, s); break;
    case 8: launch_spu<8>(spu, bf16_out, p, s); break;
    case 16: launch_spu<16>(spu, bf16_out, p, s); break;
    case 32: launch_spu<32>(spu, bf16_out, p, s); break;
    default: { // k in 33..64: one step per unit (spu is 1 for kt above 4)
        const uint32_t blocks = (p.units + 3u) / 4u;
        if (bf16_out)
            hipLaunchKernelGGL(moe_reduce_wide_kernel<true>, dim3(blocks), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL(moe_reduce_wide_kernel<false>, dim3(blocks), dim3(256), 0, s, p);
        break;
    }
    }
    return hipGetLastError() == hipSuccess ? TK_OK : TK_ERR_HIP;
}
