// kv_compress.hip -- softmax-weighted block compression of KV tokens.
//
// [V4 digest, CSA step 1; HCA paragraph] [V4-Pro card, Hybrid attention]:
// every m raw tokens (m = 4 for CSA, 128 for HCA; blocks do not overlap)
// become one entry, a weighted sum whose weights are a softmax over the
// block's per-token gate logits.
//
// Layout and schedule: a workgroup of 256 threads owns `epw` consecutive
// output entries; each entry is handled by D/4 threads that each own four
// consecutive channels, so every load instruction of a wave reads contiguous
// rows (coalesced streaming reduction, fp32 accumulation).  The gate softmax
// is evaluated per thread from the block's m logits (a few L1-resident
// scalars).  In fp8 mode the entry's max |c| is reduced through LDS and the
// per-entry power-of-two scale is derived exactly from the fp32 exponent.
#include "cakv_device.hpp"
#include "cakv_internal.hpp"

namespace cakv {

template <typename TIn>
__device__ __forceinline__ void load4(const TIn* p, float v[4]);

template <>
__device__ __forceinline__ void load4<float>(const float* p, float v[4]) {
    f32x4 x = *reinterpret_cast<const f32x4*>(p);
    v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
}

template <>
__device__ __forceinline__ void load4<bf16_t>(const bf16_t* p, float v[4]) {
    u32x2 x = *reinterpret_cast<const u32x2*>(p);
    v[0] = bf16_bits_to_f32(x[0] & 0xffffu);
    v[1] = bf16_bits_to_f32(x[0] >> 16);
    v[2] = bf16_bits_to_f32(x[1] & 0xffffu);
    v[3] = bf16_bits_to_f32(x[1] >> 16);
}

// OUTK: 0 = f32, 1 = bf16, 2 = fp8 E4M3 + per-entry scale
template <typename TIn, int OUTK>
__global__ __launch_bounds__(256) void kv_compress_kernel(const TIn* __restrict__ x,
                                                          const float* __restrict__ gate, int64_t T,
                                                          int D, int m, int64_t nblk,
                                                          int64_t total, int tpe, int epw,
                                                          void* __restrict__ out,
                                                          float* __restrict__ out_scale) {
    __shared__ uint32_t amax[256];
    const int tid = threadIdx.x;
    const int slot = tid / tpe;
    const int c0 = tid % tpe;
    const int64_t e = (int64_t)blockIdx.x * epw + slot;
    const bool live = slot < epw && e < total;
    if (OUTK == 2) {
        amax[tid] = 0u;
        __syncthreads();
    }
    const int nch = D / 4;  // 4-channel chunks per entry
    const int per = (nch + tpe - 1) / tpe;
    float acc[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
        acc[u][0] = acc[u][1] = acc[u][2] = acc[u][3] = 0.0f;
    float amx = 0.0f;
    if (live) {
        const int64_t b = e / nblk, j = e % nblk;
        const float* g = gate + b * T + j * m;
        float mx = -INFINITY;
        for (int i = 0; i < m; ++i) mx = fmaxf(mx, g[i]);
        float z = 0.0f;
        const TIn* xb = x + (b * T + j * m) * (int64_t)D;
        for (int i = 0; i < m; ++i) {
            float wgt = expf(g[i] - mx);
            z += wgt;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                int ch = c0 + u * tpe;
                if (u < per && ch < nch) {
                    float v[4];
                    load4<TIn>(xb + (int64_t)i * D + ch * 4, v);
                    acc[u][0] = __builtin_fmaf(wgt, v[0], acc[u][0]);
                    acc[u][1] = __builtin_fmaf(wgt, v[1], acc[u][1]);
                    acc[u][2] = __builtin_fmaf(wgt, v[2], acc[u][2]);
                    acc[u][3] = __builtin_fmaf(wgt, v[3], acc[u][3]);
                }
            }
        }
        const float rz = 1.0f / z;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                acc[u][c] *= rz;
                if (u < per && c0 + u * tpe < nch) amx = fmaxf(amx, __builtin_fabsf(acc[u][c]));
            }
    }
    if (OUTK == 2) {
        if (live) atomicMax(&amax[slot], __float_as_uint(amx));
        __syncthreads();
    }
    if (!live) return;
    if (OUTK == 0) {
        float* o = reinterpret_cast<float*>(out) + e * D;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int ch = c0 + u * tpe;
            if (u < per && ch < nch) {
                f32x4 v = {acc[u][0], acc[u][1], acc[u][2], acc[u][3]};
                *reinterpret_cast<f32x4*>(o + ch * 4) = v;
            }
        }
    } else if (OUTK == 1) {
        uint16_t* o = reinterpret_cast<uint16_t*>(out) + e * D;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int ch = c0 + u * tpe;
            if (u < per && ch < nch) {
                u32x2 v;
                v[0] = f32_to_bf16_bits(acc[u][0]) | (f32_to_bf16_bits(acc[u][1]) << 16);
                v[1] = f32_to_bf16_bits(acc[u][2]) | (f32_to_bf16_bits(acc[u][3]) << 16);
                *reinterpret_cast<u32x2*>(o + ch * 4) = v;
            }
        }
    } else {
        // s = 2^e, e the smallest integer >= -126 with A <= 448 * 2^e.
        // A = f * 2^E with f in [0.5, 1) and 448 = 0.875 * 2^9.
        const float A = __uint_as_float(amax[slot]);
        int ex = 0;
        if (A > 0.0f) {
            int E;
            float f = __builtin_frexpf(A, &E);
            ex = (f <= 0.875f) ? E - 9 : E - 8;
            ex = ex < -126 ? -126 : ex;
        }
        uint8_t* o = reinterpret_cast<uint8_t*>(out) + e * D;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int ch = c0 + u * tpe;
            if (u < per && ch < nch) {
                uint32_t w = 0;
#pragma unroll
                for (int c = 0; c < 4; ++c) w |= e4m3_encode(__builtin_ldexpf(acc[u][c], -ex)) << (8 * c);
                *reinterpret_cast<uint32_t*>(o + ch * 4) = w;
            }
        }
        if (c0 == 0) out_scale[e] = __builtin_ldexpf(1.0f, ex);
    }
}

int launch_kv_compress(const void* x, int x_dtype, const float* gate, int64_t B, int64_t T,
                       int64_t D, int32_t m, void* out, int out_dtype, float* out_scale,
                       hipStream_t stream) {
    const int64_t nblk = T / m;
    const int64_t total = B * nblk;
    if (total == 0) return 0;
    const int nch = (int)(D / 4);
    // up to four chunks per thread; threads per entry a power of two so that
    // entries never straddle a wave unevenly
    int tpe = 1;
    while (tpe * 4 < nch) tpe <<= 1;
    if (tpe > 256) return -2;
    const int epw = 256 / tpe;
    const int64_t grid = (total + epw - 1) / epw;
    if (grid > 0x7fffffffLL) return -2;
#define CAKV_KC(TIN, OK)                                                                          \
    hipLaunchKernelGGL((kv_compress_kernel<TIN, OK>), dim3((unsigned)grid), dim3(256), 0, stream, \
                       (const TIN*)x, gate, T, (int)D, m, nblk, total, tpe, epw, out, out_scale)
    prof_mark("kv_compress_kernel", false, stream);
    if (x_dtype == 0) {
        if (out_dtype == 0) CAKV_KC(float, 0);
        else if (out_dtype == 1) CAKV_KC(float, 1);
        else CAKV_KC(float, 2);
    } else {
        if (out_dtype == 0) CAKV_KC(bf16_t, 0);
        else if (out_dtype == 1) CAKV_KC(bf16_t, 1);
        else CAKV_KC(bf16_t, 2);
    }
#undef CAKV_KC
    prof_mark("kv_compress_kernel", true, stream);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace cakv
