// tk_pos.hip -- the token/top-k -> expert-row position map for MI355X
// (gfx950), behind tk_topk_to_pos in include/tk.h.
//
// The map is the one "【DeepSeek】TileKernels从入门到精通" ch.3, section "动态寻址",
// has the reduce follow to find each token's expert outputs.  Its rows are
// laid out as a grouped expert GEMM reads them: expert 0's rows first, then
// expert 1's, ...; within an expert, tokens in increasing order.  Slot (t, j)
// is present when 0 <= e = idx[t,j] < experts and no earlier slot of token t
// names e; then pos[t,j] = offsets[e] + (tokens t' < t with a present slot
// naming e), otherwise pos[t,j] = -1.  offsets[e] counts the present slots of
// the experts below e, offsets[experts] all of them.
//
// gfx950 design.  One thread per token: a token's present slots name distinct
// experts, so a token's rank within an expert is a count of tokens, kept as a
// bitmap of the block's tokens per expert (LDS atomic or), laid out word-major
// ([word][expert]) so that a wave's lanes, naming scattered experts, hit
// scattered banks.  A present slot's row is
//   offsets[e] + base[e] (the expert's tokens in earlier blocks)
//              + before[w][e] (its tokens in earlier words of this block)
//              + popcount(bits[w][e] below the token's bit).
// All tokens in one block: one launch does everything.  More: three launches
// over blocks of B tokens, with no memory beyond the two outputs:
//   1. pos_count_kernel: per block, the count of present slots per expert,
//      parked in the block's own first `experts` entries of pos (a full block
//      has B*k >= experts of them); the last block's counts in offsets.
//   2. pos_scan_kernel (one workgroup): per expert, the exclusive running sum
//      of the parked counts over the blocks, written back in place (each
//      block's base), and the totals (the last block's count included)
//      scanned into offsets[0 .. experts].
//   3. pos_write_kernel: per block, offsets and the block's bases into LDS,
//      the bitmap, the rows.  A block reads its parked bases before any of
//      its threads overwrites them (a barrier apart); no block touches
//      another's range.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "tk.h"

namespace {

constexpr int kMaxExperts = 512;
constexpr int kMaxK = 64;
constexpr int kScanThreads = 1024;

// This token's present slots: slot j is present when its expert is in range
// and no earlier slot names it.  KMAX bounds k at compile time so that the
// slot list stays in registers.
// VEC (k == 8, idx 16-byte aligned): the token's 8 slots as two 16-byte loads.
template <int KMAX, bool VEC>
__device__ __forceinline__ void load_slots(const int32_t* __restrict__ idx, uint32_t t, uint32_t k, uint32_t experts,
                                           int32_t (&e)[KMAX], bool (&present)[KMAX])
{
    if constexpr (VEC) {
        static_assert(KMAX == 8, "vector slots are 8 per token");
        const int4* p = reinterpret_cast<const int4*>(idx + (size_t)t * 8);
        const int4 a = p[0], b = p[1];
        e[0] = a.x; e[1] = a.y; e[2] = a.z; e[3] = a.w;
        e[4] = b.x; e[5] = b.y; e[6] = b.z; e[7] = b.w;
    } else {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            e[j] = (uint32_t)j < k ? idx[(size_t)t * k + j] : -1;
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        bool p = (uint32_t)j < k && e[j] >= 0 && (uint32_t)e[j] < experts;
#pragma unroll
        for (int i = 0; i < j; ++i)
            p = p && e[i] != e[j];
        present[j] = p;
    }
}

// Exclusive prefix sum of v over the workgroup's threads in thread order
// (blockDim.x = NT, a multiple of 64); *total gets the sum of all.  Wave
// scans by DPP-free shuffles, then the waves' sums through LDS.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_sums, uint32_t* total)
{
    constexpr int kWaves = NT / 64;
    const uint32_t lane = threadIdx.x & 63u, wv = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)x, d);
        if (lane >= (uint32_t)d)
            x += y;
    }
    if (lane == 63u)
        wave_sums[wv] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const uint32_t s = wave_sums[w];
        before += (uint32_t)w < wv ? s : 0u;
        all += s;
    }
    *total = all;
    __syncthreads(); // wave_sums may be reused after this
    return before + x - v;
}

// The bitmap of a block's tokens per expert and its prefix counts.  B tokens
// (one per thread, B = blockDim.x), W = B / 32 words per expert.
template <int B>
struct Bitmap {
    static constexpr int W = B / 32;
    uint32_t bits[W * kMaxExperts];   // [word][expert]
    uint16_t before[W * kMaxExperts]; // tokens of the block in earlier words naming the expert
};

template <int B, int KMAX>
__device__ __forceinline__ void bitmap_fill(Bitmap<B>& bm, uint32_t experts, uint32_t tl, bool has,
                                            const int32_t (&e)[KMAX], const bool (&present)[KMAX])
{
    if (has) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (present[j])
                atomicOr(&bm.bits[(tl >> 5) * experts + e[j]], 1u << (tl & 31u));
    }
}

// before[][x] for every expert x; returns nothing (the caller adds its own
// per-expert figures from the total it needs)
template <int B>
__device__ __forceinline__ uint32_t bitmap_prefix(Bitmap<B>& bm, uint32_t experts, uint32_t x)
{
    uint32_t run = 0;
#pragma unroll
    for (int w = 0; w < Bitmap<B>::W; ++w) {
        bm.before[w * experts + x] = (uint16_t)run;
        run += __builtin_popcount(bm.bits[w * experts + x]);
    }
    return run; // this block's count of the expert
}

// VEC (k == 8, pos 16-byte aligned): the token's 8 rows as two 16-byte stores.
template <int B, int KMAX, bool VEC>
__device__ __forceinline__ void write_rows(const Bitmap<B>& bm, uint32_t experts, uint32_t tl, size_t t, uint32_t k,
                                           const int32_t* off, const int32_t* base, const int32_t (&e)[KMAX],
                                           const bool (&present)[KMAX], int32_t* pos)
{
    int32_t p[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        p[j] = -1;
        if (present[j]) {
            const uint32_t i = (tl >> 5) * experts + e[j];
            p[j] = off[e[j]] + base[e[j]] + (int32_t)bm.before[i] +
                   (int32_t)__builtin_popcount(bm.bits[i] & ((1u << (tl & 31u)) - 1u));
        }
    }
    if constexpr (VEC) {
        int4* q = reinterpret_cast<int4*>(pos + t * 8);
        q[0] = make_int4(p[0], p[1], p[2], p[3]);
        q[1] = make_int4(p[4], p[5], p[6], p[7]);
    } else {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if ((uint32_t)j < k)
                pos[t * k + j] = p[j];
    }
}

// All tokens in one block (tokens <= B).
template <int B, int KMAX, bool VEC>
__global__ __launch_bounds__(B) void pos_single_kernel(const int32_t* __restrict__ idx, uint32_t tokens, uint32_t k,
                                                       uint32_t experts, int32_t* __restrict__ pos,
                                                       int32_t* __restrict__ offsets)
{
    __shared__ Bitmap<B> bm;
    __shared__ int32_t off[kMaxExperts + 1];
    __shared__ int32_t zero[kMaxExperts];
    __shared__ uint32_t cnt[kMaxExperts];
    __shared__ uint32_t wave_sums[B / 64];
    const uint32_t tl = threadIdx.x;
    for (uint32_t i = tl; i < Bitmap<B>::W * experts; i += B)
        bm.bits[i] = 0u;
    int32_t e[KMAX];
    bool present[KMAX];
    const bool has = tl < tokens;
    if (has)
        load_slots<KMAX, VEC>(idx, tl, k, experts, e, present);
    __syncthreads();
    bitmap_fill<B, KMAX>(bm, experts, tl, has, e, present);
    __syncthreads();
    for (uint32_t x = tl; x < experts; x += B) {
        cnt[x] = bitmap_prefix<B>(bm, experts, x);
        zero[x] = 0;
    }
    __syncthreads();
    // offsets: an exclusive scan of the counts, experts spread over the threads
    uint32_t carry = 0;
    for (uint32_t x0 = 0; x0 < experts; x0 += B) {
        const uint32_t x = x0 + tl;
        const uint32_t c = x < experts ? cnt[x] : 0u;
        uint32_t all;
        const uint32_t ex = block_exclusive_scan<B>(c, wave_sums, &all);
        if (x < experts)
            off[x] = (int32_t)(carry + ex);
        carry += all;
    }
    if (tl == 0)
        off[experts] = (int32_t)carry;
    __syncthreads();
    for (uint32_t x = tl; x <= experts; x += B)
        offsets[x] = off[x];
    if (has)
        write_rows<B, KMAX, VEC>(bm, experts, tl, tl, k, off, zero, e, present, pos);
}

template <int B, int KMAX, bool VEC>
__global__ __launch_bounds__(B) void pos_count_kernel(const int32_t* __restrict__ idx, uint32_t tokens, uint32_t k,
                                                      uint32_t experts, int32_t* pos, int32_t* offsets)
{
    __shared__ uint32_t cnt[kMaxExperts];
    for (uint32_t x = threadIdx.x; x < experts; x += B)
        cnt[x] = 0u;
    __syncthreads();
    const uint32_t t = blockIdx.x * B + threadIdx.x;
    if (t < tokens) {
        int32_t e[KMAX];
        bool present[KMAX];
        load_slots<KMAX, VEC>(idx, t, k, experts, e, present);
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
            if (present[j])
                atomicAdd(&cnt[e[j]], 1u);
    }
    __syncthreads();
    // a full block parks its counts in its own first entries of pos; the last
    // block (possibly short) in offsets
    int32_t* dst = blockIdx.x + 1 == gridDim.x ? offsets : pos + (size_t)blockIdx.x * B * k;
    for (uint32_t x = threadIdx.x; x < experts; x += B)
        dst[x] = (int32_t)cnt[x];
}

// One workgroup.  Thread (x, s) takes expert x and the s-th of `lanes`
// contiguous shares of the full blocks (`stride` entries of pos apart).  A
// share of up to kBatch blocks is read once and kept in registers; a larger
// one is read twice (its sum, then its bases).
constexpr int kBatch = 16;

__global__ __launch_bounds__(kScanThreads) void pos_scan_kernel(uint32_t blocks, size_t stride, uint32_t experts,
                                                                uint32_t lanes, int32_t* pos, int32_t* offsets)
{
    __shared__ uint32_t part[kScanThreads];
    __shared__ uint32_t total[kMaxExperts];
    __shared__ uint32_t wave_sums[kScanThreads / 64];
    const uint32_t x = threadIdx.x / lanes, s = threadIdx.x % lanes;
    const bool active = x < experts;
    const uint32_t full = blocks - 1; // blocks whose counts sit in pos
    const uint32_t per = (full + lanes - 1) / lanes;
    const uint32_t b0 = min(s * per, full), b1 = min(b0 + per, full);
    // pass 1: this share's sum (the first kBatch counts stay in c)
    uint32_t c[kBatch];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
        c[i] = active && b0 + i < b1 ? (uint32_t)pos[(b0 + i) * stride + x] : 0u;
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
        sum += c[i];
    if (active) {
        for (uint32_t b = b0 + kBatch; b < b1; b += kBatch) {
            uint32_t d[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                d[i] = b + i < b1 ? (uint32_t)pos[(b + i) * stride + x] : 0u;
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                sum += d[i];
        }
    }
    part[threadIdx.x] = sum;
    const uint32_t last = active && s == 0 ? (uint32_t)offsets[x] : 0u; // the last block's count
    __syncthreads();
    uint32_t run = 0;
    if (active) {
        for (uint32_t i = 0; i < s; ++i)
            run += part[x * lanes + i];
        if (s == 0) {
            uint32_t all = last;
            for (uint32_t i = 0; i < lanes; ++i)
                all += part[x * lanes + i];
            total[x] = all;
        }
    }
    __syncthreads(); // every read of offsets is done before it is overwritten below
    // pass 2: each full block's base within the expert, in place
    if (active) {
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            if (b0 + i < b1)
                pos[(b0 + i) * stride + x] = (int32_t)run;
            run += c[i];
        }
        for (uint32_t b = b0 + kBatch; b < b1; b += kBatch) {
            uint32_t d[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i)
                d[i] = b + i < b1 ? (uint32_t)pos[(b + i) * stride + x] : 0u;
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                if (b + i < b1)
                    pos[(b + i) * stride + x] = (int32_t)run;
                run += d[i];
            }
        }
    }
    // the experts' offsets: an exclusive scan of the totals over the threads
    const uint32_t v = threadIdx.x < experts ? total[threadIdx.x] : 0u;
    uint32_t all;
    const uint32_t ex = block_exclusive_scan<kScanThreads>(v, wave_sums, &all);
    if (threadIdx.x < experts)
        offsets[threadIdx.x] = (int32_t)ex;
    if (threadIdx.x == 0)
        offsets[experts] = (int32_t)all;
}

template <int B, int KMAX, bool VEC>
__global__ __launch_bounds__(B) void pos_write_kernel(const int32_t* __restrict__ idx, uint32_t tokens, uint32_t k,
                                                      uint32_t experts, const int32_t* __restrict__ offsets,
                                                      int32_t* pos)
{
    __shared__ Bitmap<B> bm;
    __shared__ int32_t off[kMaxExperts + 1];
    __shared__ int32_t base[kMaxExperts];
    const bool last_block = blockIdx.x + 1 == gridDim.x;
    const size_t first = (size_t)blockIdx.x * B * k;
    for (uint32_t i = threadIdx.x; i < Bitmap<B>::W * experts; i += B)
        bm.bits[i] = 0u;
    for (uint32_t x = threadIdx.x; x <= experts; x += B)
        off[x] = offsets[x];
    if (!last_block)
        for (uint32_t x = threadIdx.x; x < experts; x += B)
            base[x] = pos[first + x];
    const uint32_t tl = threadIdx.x;
    const uint32_t t = blockIdx.x * B + tl;
    int32_t e[KMAX];
    bool present[KMAX];
    const bool has = t < tokens;
    if (has)
        load_slots<KMAX, VEC>(idx, t, k, experts, e, present);
    __syncthreads();
    bitmap_fill<B, KMAX>(bm, experts, tl, has, e, present);
    __syncthreads();
    // prefix counts; the last block's base is the expert's total less this
    // block's own count
    for (uint32_t x = threadIdx.x; x < experts; x += B) {
        const uint32_t mine = bitmap_prefix<B>(bm, experts, x);
        if (last_block)
            base[x] = off[x + 1] - off[x] - (int32_t)mine;
    }
    __syncthreads();
    if (has)
        write_rows<B, KMAX, VEC>(bm, experts, tl, t, k, off, base, e, present, pos);
}

__global__ void zero_offsets_kernel(int32_t* offsets, uint32_t n)
{
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        offsets[i] = 0;
}

bool overlaps(const void* a, size_t an, const void* b, size_t bn)
{
    if (!a || !b || an == 0 || bn == 0)
        return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bn && b0 < a0 + an;
}

template <int B, int KMAX, bool VEC>
void launch_blocks(const int32_t* idx, uint32_t tokens, uint32_t k, uint32_t experts, int32_t* pos, int32_t* offsets,
                   hipStream_t s)
{
    const uint32_t blocks = (tokens + B - 1) / B;
    uint32_t lanes = 1;
    while (lanes * 2 * experts <= (uint32_t)kScanThreads)
        lanes *= 2;
    hipLaunchKernelGGL((pos_count_kernel<B, KMAX, VEC>), dim3(blocks), dim3(B), 0, s, idx, tokens, k, experts, pos,
                       offsets);
    hipLaunchKernelGGL(pos_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, blocks, (size_t)B * k, experts, lanes,
                       pos, offsets);
    hipLaunchKernelGGL((pos_write_kernel<B, KMAX, VEC>), dim3(blocks), dim3(B), 0, s, idx, tokens, k, experts,
                       offsets, pos);
}

template <int KMAX, bool VEC>
void launch_pos(const int32_t* idx, uint32_t tokens, uint32_t k, uint32_t experts, int32_t* pos, int32_t* offsets,
                hipStream_t s)
{
    // one block for up to 1024 tokens (the smallest of 256, 512, 1024 that
    // holds them); else blocks of 256 tokens, or 512 when 256 * k < experts
    // (a full block must have room for its parked counts), or 1024 from
    // 65536 tokens on (fewer blocks for the one-workgroup scan)
    if (tokens <= 256)
        hipLaunchKernelGGL((pos_single_kernel<256, KMAX, VEC>), dim3(1), dim3(256), 0, s, idx, tokens, k, experts, pos,
                           offsets);
    else if (tokens <= 512)
        hipLaunchKernelGGL((pos_single_kernel<512, KMAX, VEC>), dim3(1), dim3(512), 0, s, idx, tokens, k, experts, pos,
                           offsets);
    else if (tokens <= 1024)
        hipLaunchKernelGGL((pos_single_kernel<1024, KMAX, VEC>), dim3(1), dim3(1024), 0, s, idx, tokens, k, experts, pos,
                           offsets);
    else if (tokens >= 65536)
        launch_blocks<1024, KMAX, VEC>(idx, tokens, k, experts, pos, offsets, s);
    else if (256u * k >= experts)
        launch_blocks<256, KMAX, VEC>(idx, tokens, k, experts, pos, offsets, s);
    else
        launch_blocks<512, KMAX, VEC>(idx, tokens, k, experts, pos, offsets, s);
}

} // namespace

extern "C" tk_status tk_topk_to_pos(const int32_t* topk_idx, int64_t tokens, int64_t k, int64_t experts,
                                    int32_t* pos, int32_t* expert_offsets, void* stream)
{
    if (tokens < 0 || tokens >= (int64_t)INT_MAX || k <= 0 || experts <= 0)
        return TK_ERR_INVALID_ARG;
    if (k > kMaxK || experts > kMaxExperts)
        return TK_ERR_UNSUPPORTED;
    if (tokens * k >= (int64_t)INT_MAX)
        return TK_ERR_INVALID_ARG;
    if (!expert_offsets || (tokens > 0 && (!topk_idx || !pos)))
        return TK_ERR_INVALID_ARG;
    if (((uintptr_t)topk_idx & 3) || ((uintptr_t)pos & 3) || ((uintptr_t)expert_offsets & 3))
        return TK_ERR_INVALID_ARG;
    const size_t pairs = (size_t)tokens * (size_t)k * 4u, off_bytes = (size_t)(experts + 1) * 4u;
    if (overlaps(pos, pairs, topk_idx, pairs) || overlaps(expert_offsets, off_bytes, topk_idx, pairs) ||
        overlaps(expert_offsets, off_bytes, pos, pairs))
        return TK_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (tokens == 0) {
        hipLaunchKernelGGL(zero_offsets_kernel, dim3((uint32_t)(experts + 256) / 256), dim3(256), 0, s,
                           expert_offsets, (uint32_t)(experts + 1));
        return hipGetLastError() == hipSuccess ? TK_OK : TK_ERR_HIP;
    }
    // k == 8 with both arrays 16-byte aligned: each token's slots in two 16-byte loads and stores
    if (k == 8 && ((uintptr_t)topk_idx & 15) == 0 && ((uintptr_t)pos & 15) == 0)
        launch_pos<8, true>(topk_idx, (uint32_t)tokens, 8u, (uint32_t)experts, pos, expert_offsets, s);
    else if (k <= 8)
        launch_pos<8, false>(topk_idx, (uint32_t)tokens, (uint32_t)k, (uint32_t)experts, pos, expert_offsets, s);
    else if (k <= 32)
        launch_pos<32, false>(topk_idx, (uint32_t)tokens, (uint32_t)k, (uint32_t)experts, pos, expert_offsets, s);
    else
        launch_pos<64, false>(topk_idx, (uint32_t)tokens, (uint32_t)k, (uint32_t)experts, pos, expert_offsets, s);
    return hipGetLastError() == hipSuccess ? TK_OK : TK_ERR_HIP;
}
