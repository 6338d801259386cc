// probe.hip - the HBM read probe declared in include/rea_probe.h: a plain
// stream of the buffer with the scoring kernel's load instruction.
#include "rea_probe.h"

#include <hip/hip_runtime.h>

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Workgroup w reads KB blocks [w * per, (w + 1) * per) of the buffer (the
// last one fewer); wave v of it takes blocks v, v + 4, ... in batches of L,
// all L loads issued before any result is used.
template <int L>
__global__ __launch_bounds__(kThreads) void k_stream_read(const unsigned char *buf, int64_t kblocks,
                                                         int64_t per, uint32_t *sink) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t b1 = b0 + per < kblocks ? b0 + per : kblocks;
    uint32_t x = 0;
    for (int64_t base = b0 + wave; base < b1; base += (int64_t)kWaves * L) {
        u32x4 v[L];
#pragma unroll
        for (int i = 0; i < L; ++i) {
            int64_t blk = base + (int64_t)i * kWaves;
            blk = blk < b1 ? blk : b1 - 1;              // in range; repeats are harmless
            v[i] = __builtin_nontemporal_load(
                (const u32x4 *)(buf + blk * 1024 + lane * 16));
        }
#pragma unroll
        for (int i = 0; i < L; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    }
    for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
    __shared__ uint32_t part[kWaves];
    if (lane == 0) part[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

extern "C" int rea_probe_cu_count(void) {
    int dev = -1, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return n;
}

extern "C" int rea_probe_stream_read(const void *buf, size_t bytes, int wg_per_cu,
                                     int loads_in_flight, uint32_t *sink, void *stream) {
    if (!buf || !sink || bytes == 0 || bytes % 1024 != 0 || ((uintptr_t)buf % 16) != 0 ||
        wg_per_cu < 1 || wg_per_cu > 16)
        return 1;
    if (loads_in_flight != 4 && loads_in_flight != 8 && loads_in_flight != 16) return 1;
    const int cu = rea_probe_cu_count();
    if (cu <= 0) return 2;
    const int64_t kblocks = (int64_t)(bytes / 1024);
    const int64_t wgs = (int64_t)cu * wg_per_cu;
    const int64_t per = (kblocks + wgs - 1) / wgs;
    const hipStream_t s = (hipStream_t)stream;
    const unsigned char *p = (const unsigned char *)buf;
    if (loads_in_flight == 4)
        hipLaunchKernelGGL(k_stream_read<4>, dim3((unsigned)wgs), dim3(kThreads), 0, s, p, kblocks,
                           per, sink);
    else if (loads_in_flight == 8)
        hipLaunchKernelGGL(k_stream_read<8>, dim3((unsigned)wgs), dim3(kThreads), 0, s, p, kblocks,
                           per, sink);
    else
        hipLaunchKernelGGL(k_stream_read<16>, dim3((unsigned)wgs), dim3(kThreads), 0, s, p, kblocks,
                           per, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
