// probes.hip -- the attainable-peak probes of cakv_probes.h (measurement
// only; built into libcakv_probes.so, apart from the attention path).
#include <hip/hip_runtime.h>

#include "cakv_probes.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per thread

// Read of n 16-byte words, workgroup g taking the contiguous range
// [g * per, (g + 1) * per) in rounds of kUnroll * 256 words (every load of a
// round issued before any is used); nontemporal loads, since nothing is read
// twice.  The XOR of the workgroup's words goes to sink[blockIdx.x].  (Of
// the patterns measured on gfx950, this one reads fastest: contiguous ranges
// beat a grid-stride walk, and nontemporal loads beat ordinary ones.)
__global__ __launch_bounds__(kThreads) void probe_read_kernel(const u32x4* p, int64_t n, uint32_t* sink) {
    __shared__ uint32_t red[kThreads / 64];
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = min(n, (int64_t)blockIdx.x * per), b1 = min(n, b0 + per);
    int64_t i = b0 + threadIdx.x;
    uint32_t x = 0u;
    for (; i + (kUnroll - 1) * kThreads < b1; i += kUnroll * kThreads) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < b1; i += kThreads) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0u;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) r ^= red[w];
        sink[blockIdx.x] = r;
    }
}

// Four independent accumulation chains per wave, so that consecutive MFMAs
// never wait for each other's results.
__global__ __launch_bounds__(kThreads) void probe_mfma_kernel(int64_t iters, float* sink) {
    const uint32_t lane = threadIdx.x & 63;
    // operands 0.5 (bf16 0x3f00) and 0.5 + 2^-8 * (lane % 2): small and finite
    // for any iteration count the caller times
    const uint32_t wa = 0x3f003f00u, wb = 0x3f003f00u | (lane & 1u);
    const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{wa, wa, wa, wa});
    const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{wb, wb, wb, wb});
    f32x16 c0, c1, c2, c3;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        c0[r] = 0.0f;
        c1[r] = 0.0f;
        c2[r] = 0.0f;
        c3[r] = 0.0f;
    }
    for (int64_t it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    if (lane == 0) sink[4 * (int64_t)blockIdx.x + (threadIdx.x >> 6)] = s;
}

}  // namespace

extern "C" int cakv_probe_read(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks, hipStream_t stream) {
    if (!buf || !sink || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || blocks < 0 ||
        blocks > 65535)
        return -1;
    if (blocks == 0) blocks = 2048;
    hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       reinterpret_cast<const u32x4*>(buf), (int64_t)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" int cakv_probe_mfma_bf16(int64_t iters, int32_t blocks, float* sink, hipStream_t stream) {
    if (!sink || iters < 0 || blocks < 1 || blocks > 65535) return -1;
    hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}
