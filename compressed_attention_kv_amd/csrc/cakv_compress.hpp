// cakv_compress.hpp -- the arithmetic of one compressed entry, shared by the
// bulk compressor (kv_compress.hip) and the streaming append (decode.hip) so
// that both write bitwise the same entries.
//
// [V4 digest, CSA step 1 and HCA paragraph; Visualised, Dual Compression and
// Indexing] an entry is a softmax-gated (learned) weighted average of raw
// tokens.  Entry j covers the `n` tokens of its span, oldest first; the gate
// is one logit per token or one per token and channel.  Per channel d:
//     mx = max_i g_{i,d};  w_i = exp(g_{i,d} - mx);  z = sum_i w_i;
//     c_d = (sum_i w_i x_{i,d}) * (1 / z),
// the sums in token order (an fma chain for the weighted sum).  The calling
// thread owns up to four 4-channel chunks.
#pragma once

#include "cakv_device.hpp"

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

// row(i): pointer to token i's row (element 0); gate_tok(i): token i's logit
// (per-token gates); gate_row(i): pointer to token i's [D] logits
// (per-channel gates).  ch[u]: 4-channel chunk index of slot u, live[u]: the
// slot holds channels.  acc[u][c] receives channel 4 ch[u] + c.
template <typename TIn, bool PER_CHANNEL, typename RowF, typename GateTokF, typename GateRowF>
__device__ __forceinline__ void compress_entry(int n, RowF row, GateTokF gate_tok, GateRowF gate_row,
                                               const int ch[4], const bool live[4], float acc[4][4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u][0] = acc[u][1] = acc[u][2] = acc[u][3] = 0.0f;
    if constexpr (!PER_CHANNEL) {
        // (the loops are unrolled so that several tokens' loads are in flight
        // at once; the arithmetic stays one chain in token order)
        float mx = -INFINITY;
#pragma unroll 8
        for (int i = 0; i < n; ++i) mx = fmaxf(mx, gate_tok(i));
        float z = 0.0f;
#pragma unroll 8
        for (int i = 0; i < n; ++i) {
            const float wgt = expf(gate_tok(i) - mx);
            z += wgt;
            const TIn* r = row(i);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (live[u]) {
                    float v[4];
                    load4<TIn>(r + ch[u] * 4, v);
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[u][c] = __builtin_fmaf(wgt, v[c], acc[u][c]);
                }
            }
        }
        const float rz = 1.0f / z;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[u][c] *= rz;
    } else {
        float mx[4][4], z[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                mx[u][c] = -INFINITY;
                z[u][c] = 0.0f;
            }
        for (int i = 0; i < n; ++i) {
            const float* g = gate_row(i);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (live[u]) {
                    const f32x4 g4 = *reinterpret_cast<const f32x4*>(g + ch[u] * 4);
#pragma unroll
                    for (int c = 0; c < 4; ++c) mx[u][c] = fmaxf(mx[u][c], g4[c]);
                }
            }
        }
        for (int i = 0; i < n; ++i) {
            const float* g = gate_row(i);
            const TIn* r = row(i);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (live[u]) {
                    const f32x4 g4 = *reinterpret_cast<const f32x4*>(g + ch[u] * 4);
                    float v[4];
                    load4<TIn>(r + ch[u] * 4, v);
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const float wgt = expf(g4[c] - mx[u][c]);
                        z[u][c] += wgt;
                        acc[u][c] = __builtin_fmaf(wgt, v[c], acc[u][c]);
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[u][c] *= 1.0f / z[u][c];
    }
}

// fp8 E4M3 entry scale exponent: the smallest e >= -126 with A <= 448 * 2^e
// (A = max |c| of the entry; e = 0 for an all-zero entry).  A = f * 2^E with
// f in [0.5, 1) and 448 = 0.875 * 2^9.
__device__ __forceinline__ int q8_exponent(float A) {
    int ex = 0;
    if (A > 0.0f) {
        int E;
        const float f = __builtin_frexpf(A, &E);
        ex = (f <= 0.875f) ? E - 9 : E - 8;
        ex = ex < -126 ? -126 : ex;
    }
    return ex;
}

}  // namespace cakv
