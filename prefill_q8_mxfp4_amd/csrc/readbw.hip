// Measurement aid, not part of the GEMM: a plain read of device memory with
// the 16-byte loads the streaming kernel uses, every load of a thread issued
// before the first is consumed.  Its rate over the same bytes (the packed
// weights, rotated the same way) is the achieved-bandwidth ceiling that the
// streaming kernel's weight stream is reported against, next to the nominal
// HBM peak.
#include "common.h"

namespace qg {

// Thread t of the grid reads 16-byte chunks t, t + T, t + 2T, ... (T threads
// in all), eight at a time, and folds them with XOR; one word per workgroup
// goes to sink so the loads are not optimised away.
__global__ __launch_bounds__(256) void read_bytes_kernel(const u32x4 *__restrict__ p, int64_t nchunks,
                                                          uint32_t *sink)
{
    const int64_t T = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4 acc = u32x4{0u, 0u, 0u, 0u};
    for (; i + 7 * T < nchunks; i += 8 * T) {
        u32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; j++)
            v[j] = __builtin_nontemporal_load(p + i + j * T);
#pragma unroll
        for (int j = 0; j < 8; j++)
            acc ^= v[j];
    }
    for (; i < nchunks; i += T)
        acc ^= __builtin_nontemporal_load(p + i);
    uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    for (int d = 32; d > 0; d >>= 1)
        r ^= __shfl_xor(r, d, 64);
    __shared__ uint32_t s[4];
    if ((threadIdx.x & 63) == 0)
        s[threadIdx.x >> 6] = r;
    __syncthreads();
    if (threadIdx.x == 0)
        sink[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

hipError_t launch_read_bytes(const void *buf, int64_t bytes, uint32_t *sink, int wgs, hipStream_t st)
{
    hipLaunchKernelGGL(read_bytes_kernel, dim3((unsigned)wgs), dim3(256), 0, st, (const u32x4 *)buf,
                       bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace qg
