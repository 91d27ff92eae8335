// stream_ceiling.hip -- measurement kernels, not part of the fused path.
//
// Plain streaming kernels that move the same bytes as the fused step without
// any arithmetic, to measure what this GPU's HBM actually sustains for that
// traffic shape:
//   read4_write1: reads 32 bytes and writes 8 bytes per thread (the 4:1
//                 read:write ratio of bf16 -> FP8), one item per thread, a
//                 non-persistent grid, non-temporal loads and stores (the
//                 fastest form found on MI355X);
//   read_only:    reads 16 bytes per thread.
// The benchmark times them with HIP events beside the fused kernel.
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

} // extern "C"
