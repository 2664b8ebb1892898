// cakv_rows.hpp -- preparation of one key (= value) row, shared by
// kv_prepare.hip and the streaming append (decode.hip) so that both write
// bitwise the same rows.
//
// [V4-Pro card, "Hybrid attention"]: RMSNorm on the single compressed KV
// head before the attention dot product, and RoPE on the last 64 dims of each
// KV entry:  y = gamma * c / sqrt(mean_d(c_d^2) + eps), then the last
// rope_dims channels, in consecutive pairs, rotated by pos * theta_i.
//
// One wave per row.  Lane l owns the 8-channel chunks l, l+64, ... of the row
// (one 16-byte load per chunk for bf16, two for f32; consecutive lanes read
// consecutive bytes), the sum of squares is an fma chain per lane reduced
// across the wave, and each lane rotates the pairs of its own chunks (pairs
// start at even channels and the rotated block starts at an even channel, so
// a pair never straddles two chunks).  Every read of a row happens before its
// writes, so in and out may be the same row.
#pragma once

#include "cakv_device.hpp"
#include "cakv_internal.hpp"

namespace cakv {

constexpr int kPrepMaxChunks = 8;  // D <= 8 * 8 * 64 = 4096

template <typename T>
struct Chunk8;

template <>
struct Chunk8<bf16_t> {
    static __device__ __forceinline__ void load(const bf16_t* p, float v[8]) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
            v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
        }
    }
    static __device__ __forceinline__ void store(bf16_t* p, const float v[8]) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16_bits(v[2 * i]) | (f32_to_bf16_bits(v[2 * i + 1]) << 16);
        *reinterpret_cast<u32x4*>(p) = w;
    }
};

template <>
struct Chunk8<float> {
    static __device__ __forceinline__ void load(const float* p, float v[8]) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(p);
        const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = a[i];
            v[4 + i] = b[i];
        }
    }
    static __device__ __forceinline__ void store(float* p, const float v[8]) {
        *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
};

// The whole wave calls this for one row (lane = lane id 0..63); `in` may
// point to LDS or HBM.
template <typename T>
__device__ __forceinline__ void prepare_row(const T* in, T* out, const float* __restrict__ gamma, int D,
                                            double pos, int rope_dims, double rope_ratio, float eps, int lane) {
    const int nch = D >> 3;
    float v[kPrepMaxChunks][8];
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < kPrepMaxChunks; ++k) {
        const int c = lane + 64 * k;
        if (c < nch) {
            Chunk8<T>::load(in + 8 * c, v[k]);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(v[k][i], v[k][i], ss);
        }
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / __builtin_sqrtf(ss / (float)D + eps);
    const int rope_lo = D - rope_dims;
#pragma unroll
    for (int k = 0; k < kPrepMaxChunks; ++k) {
        const int c = lane + 64 * k;
        if (c < nch) {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[k][i] *= inv * (gamma ? gamma[8 * c + i] : 1.0f);
            if (8 * c + 8 > rope_lo) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int d = 8 * c + 2 * p;
                    if (d < rope_lo) continue;
                    float sn, cs;
                    sincos_turns(pos * rope_turns(rope_ratio, (d - rope_lo) >> 1), &sn, &cs);
                    const float x0 = v[k][2 * p], x1 = v[k][2 * p + 1];
                    v[k][2 * p] = x0 * cs - x1 * sn;
                    v[k][2 * p + 1] = x0 * sn + x1 * cs;
                }
            }
            Chunk8<T>::store(out + 8 * c, v[k]);
        }
    }
}

}  // namespace cakv
