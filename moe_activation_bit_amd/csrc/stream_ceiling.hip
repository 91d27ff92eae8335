// stream_ceiling.hip -- measurement kernels, not part of the fused path.
//
// Plain streaming kernels that move the same bytes as the fused step without
// any arithmetic, to measure what this GPU's HBM actually sustains for that
// traffic shape:
//   read4_write1: reads 32 bytes and writes 8 bytes per thread (the 4:1
//                 read:write ratio of bf16 -> FP8), one item per thread, a
//                 non-persistent grid, non-temporal loads and stores;
//   read_only:    reads 16 bytes per thread;
//   probe_4to1:   the fused step's own traffic without its arithmetic, over a
//                 matrix of cache policies and grid shapes: a packed
//                 [rows, 2*hidden] bf16 tensor read as gate and up halves (lane
//                 l of a wave takes the 16-byte slot 64*step + l of each half),
//                 8 bytes written per lane and step into [rows, hidden] bytes.
//                 Loads and stores are buffer instructions whose cache-policy
//                 bits are a template argument (0: none, 1: sc0, 2: nt,
//                 16: sc1, sums of these); the grid is either one unit of SPU
//                 steps per wave (non-persistent) or a persistent grid of
//                 blocks_per_cu 256-thread workgroups per CU striding over the
//                 units in the XCD-contiguous order the fused kernel uses;
//   read_n_write: another kernel's read:write mix without its arithmetic:
//                 each of n threads reads RV 16-byte vectors (vector j of
//                 thread i at j*n + i, so each load instruction of a wave is
//                 one contiguous KiB) and writes WB bytes at i*WB;
//                 non-persistent, non-temporal loads and stores.
// The benchmark times them with HIP events beside the kernels they bound.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(256) void read4_write1_kernel(const v4u* __restrict__ in, v2u* __restrict__ out,
                                                           uint64_t n_out)
{
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_out)
        return;
    const v4u a = __builtin_nontemporal_load(in + 2 * i);
    const v4u b = __builtin_nontemporal_load(in + 2 * i + 1);
    const v2u v = {a.x ^ a.y ^ b.z, a.z ^ a.w ^ b.x ^ b.y ^ b.w};
    __builtin_nontemporal_store(v, out + i);
}

__global__ __launch_bounds__(256) void read_only_kernel(const v4u* __restrict__ in, uint64_t n, uint32_t* sink)
{
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n)
        return;
    const v4u a = __builtin_nontemporal_load(in + i);
    if ((a.x ^ a.y ^ a.z ^ a.w) == 0x9E3779B9u) // practically never: keeps the load alive
        sink[0] = a.x;
}

template <int RV, int WB>
__global__ __launch_bounds__(256) void read_n_write_kernel(const v4u* __restrict__ in, char* __restrict__ out,
                                                           uint64_t n)
{
    const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n)
        return;
    v4u a[RV];
#pragma unroll
    for (int j = 0; j < RV; ++j)
        a[j] = __builtin_nontemporal_load(in + (uint64_t)j * n + i);
#pragma unroll
    for (int j = 1; j < RV; ++j)
        a[0] ^= a[j];
    if constexpr (WB == 4) {
        __builtin_nontemporal_store(a[0].x ^ a[0].y ^ a[0].z ^ a[0].w, reinterpret_cast<uint32_t*>(out) + i);
    } else if constexpr (WB == 8) {
        const v2u o = {a[0].x ^ a[0].y, a[0].z ^ a[0].w};
        __builtin_nontemporal_store(o, reinterpret_cast<v2u*>(out) + i);
    } else {
        static_assert(WB == 16, "4, 8 or 16 bytes out per thread");
        __builtin_nontemporal_store(a[0], reinterpret_cast<v4u*>(out) + i);
    }
}

template <int RV>
bool launch_read_n(uint32_t wb, dim3 grid, hipStream_t s, const v4u* in, char* out, uint64_t n)
{
    switch (wb) {
    case 4: hipLaunchKernelGGL((read_n_write_kernel<RV, 4>), grid, dim3(256), 0, s, in, out, n); return true;
    case 8: hipLaunchKernelGGL((read_n_write_kernel<RV, 8>), grid, dim3(256), 0, s, in, out, n); return true;
    case 16: hipLaunchKernelGGL((read_n_write_kernel<RV, 16>), grid, dim3(256), 0, s, in, out, n); return true;
    default: return false;
    }
}

// Word 3 of a raw buffer descriptor on gfx9-family GPUs (32-bit data format,
// no swizzle): the value AMD's composable_kernel headers use for gfx9.
constexpr int kBufWord3 = 0x00020000;

// One wave moves SPU steps of one row: per step, 16 bytes of gate and 16 of
// up per lane in, 8 bytes per lane out.  Every access is inside its row's
// buffer range (the host keeps hidden a multiple of 512, so no lane is past
// the row end), and buffer accesses outside the range would read 0 / drop
// the write rather than fault.
template <int LP, int SP, int SPU>
__global__ __launch_bounds__(256) void probe_4to1_kernel(const char* __restrict__ x, char* __restrict__ out,
                                                         uint32_t hidden, uint32_t units_per_row, uint32_t units,
                                                         uint32_t xcd_order)
{
    const uint32_t lane = threadIdx.x & 63u;
    uint32_t block = blockIdx.x;
    if (xcd_order && (gridDim.x & 7u) == 0)
        block = (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(block * 4u + (threadIdx.x >> 6));
    const uint32_t nwaves = gridDim.x * 4u;
    const uint32_t half = hidden * 2u; // bytes of one bf16 half-row
    for (uint32_t u = wave; u < units; u += nwaves) {
        const uint32_t row = u / units_per_row;
        const uint32_t step0 = (u - row * units_per_row) * SPU;
        const __amdgpu_buffer_rsrc_t rin = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(x) + (size_t)row * (2u * half), 0, 2u * half, kBufWord3);
        const __amdgpu_buffer_rsrc_t rout =
            __builtin_amdgcn_make_buffer_rsrc(out + (size_t)row * hidden, 0, hidden, kBufWord3);
        v4u g[SPU], v[SPU];
#pragma unroll
        for (int s = 0; s < SPU; ++s) {
            const uint32_t off = ((step0 + s) * 64u + lane) * 16u;
            g[s] = __builtin_amdgcn_raw_buffer_load_b128(rin, off, 0, LP);
            v[s] = __builtin_amdgcn_raw_buffer_load_b128(rin, off + half, 0, LP);
        }
#pragma unroll
        for (int s = 0; s < SPU; ++s) {
            const v2u o = {g[s].x ^ g[s].y ^ v[s].z, g[s].z ^ g[s].w ^ v[s].x ^ v[s].y ^ v[s].w};
            __builtin_amdgcn_raw_buffer_store_b64(o, rout, ((step0 + s) * 64u + lane) * 8u, 0, SP);
        }
    }
}

template <int LP, int SP>
bool launch_probe(uint32_t spu, dim3 grid, hipStream_t s, const char* x, char* out, uint32_t hidden, uint32_t upr,
                  uint32_t units, uint32_t xcd)
{
    if (spu == 1)
        hipLaunchKernelGGL((probe_4to1_kernel<LP, SP, 1>), grid, dim3(256), 0, s, x, out, hidden, upr, units, xcd);
    else if (spu == 4)
        hipLaunchKernelGGL((probe_4to1_kernel<LP, SP, 4>), grid, dim3(256), 0, s, x, out, hidden, upr, units, xcd);
    else
        return false;
    return true;
}

template <int LP>
bool probe_store(int sp, uint32_t spu, dim3 grid, hipStream_t s, const char* x, char* out, uint32_t hidden,
                 uint32_t upr, uint32_t units, uint32_t xcd)
{
    switch (sp) {
    case 0: return launch_probe<LP, 0>(spu, grid, s, x, out, hidden, upr, units, xcd);
    case 2: return launch_probe<LP, 2>(spu, grid, s, x, out, hidden, upr, units, xcd);
    case 16: return launch_probe<LP, 16>(spu, grid, s, x, out, hidden, upr, units, xcd);
    case 17: return launch_probe<LP, 17>(spu, grid, s, x, out, hidden, upr, units, xcd);
    default: return false;
    }
}

} // namespace

extern "C" {

// in: in_bytes readable bytes (16-byte aligned); out: in_bytes/4 writable bytes.
// in_bytes must be a multiple of 32.  Returns 0, or 1 on a bad argument or a
// failed launch.
int stream_read4_write1(const void* in, void* out, uint64_t in_bytes, void* stream)
{
    if (!in || !out || in_bytes == 0 || in_bytes % 32 != 0)
        return 1;
    const uint64_t n_out = in_bytes / 32;
    const uint64_t blocks = (n_out + 255) / 256;
    hipLaunchKernelGGL(read4_write1_kernel, dim3((uint32_t)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const v4u*>(in), static_cast<v2u*>(out), n_out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

// in: in_bytes readable bytes (multiple of 16); sink: 4 writable bytes.
int stream_read_only(const void* in, uint64_t in_bytes, uint32_t* sink, void* stream)
{
    if (!in || !sink || in_bytes == 0 || in_bytes % 16 != 0)
        return 1;
    const uint64_t n = in_bytes / 16;
    const uint64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(read_only_kernel, dim3((uint32_t)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const v4u*>(in), n, sink);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

// The fused step's traffic shape: x [rows, 2*hidden] bf16 (16-byte aligned),
// out [rows, hidden] bytes.  hidden must be a positive multiple of 512 * spu
// (whole steps, whole units) and at most 2^28; the unit count
// rows * hidden / (512 * spu) must be below 2^31.  load_pol / store_pol:
// 0, 2 (nt), 16 (sc1) or 17 (sc0 sc1).  spu: 1 or 4 steps per unit.
// blocks_per_cu 0: non-persistent (one unit per wave); else a persistent grid
// of blocks_per_cu * cus workgroups in the XCD-contiguous order.  Returns 0, or
// 1 on a bad argument or a failed launch.
int stream_probe_4to1(const void* x, void* out, uint64_t rows, uint32_t hidden, int load_pol, int store_pol,
                      uint32_t spu, uint32_t blocks_per_cu, uint32_t cus, void* stream)
{
    if (!x || !out || rows == 0 || (spu != 1 && spu != 4) || hidden == 0 || hidden % (512u * spu) != 0 ||
        hidden > (1u << 28))
        return 1;
    const uint64_t upr = hidden / (512u * spu);
    const uint64_t units = rows * upr;
    if (units >= (1ull << 31))
        return 1;
    const uint64_t want = (units + 3) / 4;
    const uint64_t blocks = blocks_per_cu ? (uint64_t)blocks_per_cu * cus : want;
    if (blocks == 0 || blocks >= (1ull << 31))
        return 1;
    const dim3 grid((uint32_t)(blocks < want ? blocks : want));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const char* xi = static_cast<const char*>(x);
    char* o = static_cast<char*>(out);
    const uint32_t xcd = blocks_per_cu ? 1u : 0u;
    bool ok;
    switch (load_pol) {
    case 0: ok = probe_store<0>(store_pol, spu, grid, s, xi, o, hidden, (uint32_t)upr, (uint32_t)units, xcd); break;
    case 2: ok = probe_store<2>(store_pol, spu, grid, s, xi, o, hidden, (uint32_t)upr, (uint32_t)units, xcd); break;
    case 16: ok = probe_store<16>(store_pol, spu, grid, s, xi, o, hidden, (uint32_t)upr, (uint32_t)units, xcd); break;
    case 17: ok = probe_store<17>(store_pol, spu, grid, s, xi, o, hidden, (uint32_t)upr, (uint32_t)units, xcd); break;
    default: ok = false;
    }
    if (!ok)
        return 1;
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

// Another kernel's read:write mix: in holds n * rv * 16 readable bytes, out
// n * wb writable bytes, both 16-byte aligned; rv 1, 2, 4 or 8, wb 4, 8 or 16.
// Returns 0, or 1 on a bad argument or a failed launch.
int stream_read_n_write(const void* in, void* out, uint64_t n, uint32_t rv, uint32_t wb, void* stream)
{
    if (!in || !out || n == 0 || ((uintptr_t)in & 15u) || ((uintptr_t)out & 15u))
        return 1;
    const uint64_t blocks = (n + 255) / 256;
    if (blocks >= (1ull << 31) || n > (1ull << 40))
        return 1;
    const dim3 grid((uint32_t)blocks);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const v4u* vin = static_cast<const v4u*>(in);
    char* o = static_cast<char*>(out);
    bool ok;
    switch (rv) {
    case 1: ok = launch_read_n<1>(wb, grid, s, vin, o, n); break;
    case 2: ok = launch_read_n<2>(wb, grid, s, vin, o, n); break;
    case 4: ok = launch_read_n<4>(wb, grid, s, vin, o, n); break;
    case 8: ok = launch_read_n<8>(wb, grid, s, vin, o, n); break;
    default: ok = false;
    }
    if (!ok)
        return 1;
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

} // extern "C"
