// decode.hip -- the streaming side of a decode step: one new token per
// sequence enters one compressor's state.
//
// [V4-Pro card, Hybrid attention] every CSA/HCA layer keeps a window of the
// n_win most recent uncompressed tokens, because compressed keys cannot reach
// inside the block being filled; [V4 digest, CSA step 1 and HCA paragraph] a
// block of m tokens becomes one entry once all of them exist.  Per sequence b
// with its new token at position t = pos[b] (t < 0: no token this step):
//   1. the raw token and its gate logit(s) enter the raw ring at row
//      t mod Rr (the compressor's input for the blocks still being filled);
//   2. the token, prepared at position t (RMSNorm with gamma_kv, RoPE), enters
//      the window ring at row t mod Rw (the attention calls read the window
//      from it in ring mode);
//   3. if t completes block j ((t + 1) mod m == 0, j = (t + 1)/m - 1 < N),
//      entry j is compressed from the span's tokens (the ring's rows and the
//      new token) and stored: prepared at position j*m + offset for a
//      bf16/f32 cache, or as fp8 E4M3 codes with the power-of-two scale.
// The entry and the prepared rows are computed by the same device code as
// kv_compress / kv_compress_ex and kv_prepare, so streaming a sequence
// token by token leaves bitwise the cache the bulk calls would write.
//
// One workgroup of 256 threads per sequence: all threads compress the entry
// (when one completes) in 4-channel chunks; wave 0 then prepares it from LDS;
// wave 1 prepares the window row; waves 2-3 copy the raw token into the ring.
// The compressor reads ring rows of positions t-span+1 .. t-1 only, and the
// copy writes row t mod Rr, which differs from all of them since Rr >= span.
#include "cakv_compress.hpp"
#include "cakv_internal.hpp"
#include "cakv_rows.hpp"

namespace cakv {

// OUTK: 0 = f32, 1 = bf16, 2 = fp8 E4M3 + scale (the cache's type); PC:
// per-channel gates.  The workgroup's LDS: erow, 4096 elements of T (the
// completed entry, in the cache's rounding), and one word for the entry's
// absolute maximum (fp8).
template <typename T, int OUTK, bool PC>
__device__ __forceinline__ void append_body(const AppendArgs& a, T* erow, uint32_t& amax) {
    const int64_t b = blockIdx.x;
    const int32_t t = a.pos[b];
    if (t < 0) return;  // workgroup-uniform: no token for this sequence
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int D = a.D;
    const T* xt = reinterpret_cast<const T*>(a.x_tok) + b * (int64_t)D;
    const int64_t ring_row = b * a.Rr + t % a.Rr;
    const int m = a.m;
    const int64_t j = ((int64_t)t + 1) / m - 1;
    const bool complete = ((int64_t)t + 1) % m == 0 && j < a.N;  // uniform

    if (complete) {
        const int64_t hi = (int64_t)t + 1, lo = hi - a.span > 0 ? hi - a.span : 0;
        CAKV_DCHECK(hi - lo <= a.Rr && D <= 4096);  // the span fits the ring, the entry the LDS row
        const T* raw = reinterpret_cast<const T*>(a.raw_ring) + b * a.Rr * (int64_t)D;
        const float* gr = a.gate_ring + b * a.Rr * (PC ? (int64_t)D : 1);
        const float* gt = a.gate_tok + b * (PC ? (int64_t)D : 1);
        auto row = [&](int i) -> const T* {
            const int64_t p = lo + i;
            return p == t ? xt : raw + (p % a.Rr) * D;
        };
        auto gate_tok = [&](int i) -> float {
            const int64_t p = lo + i;
            return p == t ? gt[0] : gr[p % a.Rr];
        };
        auto gate_row = [&](int i) -> const float* {
            const int64_t p = lo + i;
            return p == t ? gt : gr + (p % a.Rr) * D;
        };
        // the bulk compressor's thread layout: tpe threads, up to four
        // 4-channel chunks each
        const int nch = D / 4;
        int tpe = 1;
        while (tpe * 4 < nch) tpe <<= 1;
        const int per = (nch + tpe - 1) / tpe;
        int ch[4];
        bool ok[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            ch[u] = tid + u * tpe;
            ok[u] = tid < tpe && u < per && ch[u] < nch;
        }
        if (tid == 0) amax = 0u;
        __syncthreads();
        float acc[4][4];
        float amx = 0.0f;
        if (tid < tpe) {
            compress_entry<T, PC>((int)(hi - lo), row, gate_tok, gate_row, ch, ok, acc);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (ok[u]) amx = fmaxf(amx, __builtin_fabsf(acc[u][c]));
        }
        if constexpr (OUTK == 2) {
            if (tid < tpe) atomicMax(&amax, __float_as_uint(amx));
            __syncthreads();
            const int ex = q8_exponent(__uint_as_float(amax));
            uint8_t* o = reinterpret_cast<uint8_t*>(a.cache) + (b * a.N + j) * (int64_t)D;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (ok[u]) {
                    uint32_t w = 0;
#pragma unroll
                    for (int c = 0; c < 4; ++c) w |= e4m3_encode(__builtin_ldexpf(acc[u][c], -ex)) << (8 * c);
                    *reinterpret_cast<uint32_t*>(o + ch[u] * 4) = w;
                }
            }
            if (tid == 0) a.cache_scale[b * a.N + j] = __builtin_ldexpf(1.0f, ex);
        } else {
            // round to the cache's type (what the bulk compressor stores) in LDS
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (ok[u]) {
                    if constexpr (OUTK == 0) {
                        *reinterpret_cast<f32x4*>(&erow[ch[u] * 4]) =
                            f32x4{acc[u][0], acc[u][1], acc[u][2], acc[u][3]};
                    } else {
                        u32x2 v;
                        v[0] = f32_to_bf16_bits(acc[u][0]) | (f32_to_bf16_bits(acc[u][1]) << 16);
                        v[1] = f32_to_bf16_bits(acc[u][2]) | (f32_to_bf16_bits(acc[u][3]) << 16);
                        *reinterpret_cast<u32x2*>(&erow[ch[u] * 4]) = v;
                    }
                }
            }
            __syncthreads();
            T* o = reinterpret_cast<T*>(a.cache) + (b * a.N + j) * (int64_t)D;
            if (a.prep) {
                if (wave == 0)
                    prepare_row<T>(erow, o, a.gamma_kv, D, (double)(j * m + a.pos_off), a.rope_dims, a.rope_ratio,
                                   a.eps, lane);
            } else {
                for (int c = tid; c < D / 4; c += 256) {
                    if constexpr (OUTK == 0)
                        *reinterpret_cast<f32x4*>(o + 4 * c) = *reinterpret_cast<const f32x4*>(&erow[4 * c]);
                    else
                        *reinterpret_cast<u32x2*>(o + 4 * c) = *reinterpret_cast<const u32x2*>(&erow[4 * c]);
                }
            }
        }
    }
    if (wave == 1) {
        if (a.win_ring)
            prepare_row<T>(xt, reinterpret_cast<T*>(a.win_ring) + (b * a.Rw + t % a.Rw) * (int64_t)D, a.gamma_kv, D,
                           (double)t, a.rope_dims, a.rope_ratio, a.eps, lane);
    } else if (wave >= 2) {
        // the raw token and its gate(s) into the raw ring, 16 bytes per lane
        const int l = tid - 128;
        constexpr int E16 = 16 / (int)sizeof(T);  // elements per 16 bytes
        T* dst = reinterpret_cast<T*>(a.raw_ring) + ring_row * D;
        for (int c = l; c < D / E16; c += 128)
            *reinterpret_cast<u32x4*>(dst + E16 * c) = *reinterpret_cast<const u32x4*>(xt + E16 * c);
        if constexpr (PC) {
            float* gd = a.gate_ring + ring_row * D;
            const float* gs = a.gate_tok + b * (int64_t)D;
            for (int c = l; c < D / 4; c += 128)
                *reinterpret_cast<f32x4*>(gd + 4 * c) = *reinterpret_cast<const f32x4*>(gs + 4 * c);
        } else {
            if (l == 0) a.gate_ring[ring_row] = a.gate_tok[b];
        }
    }
}

template <typename T, int OUTK, bool PC>
__global__ __launch_bounds__(256) void kv_append_kernel(const AppendArgs a) {
    __shared__ __attribute__((aligned(16))) T erow[4096];
    __shared__ uint32_t amax;
    append_body<T, OUTK, PC>(a, erow, amax);
}

// Several appends of the same tokens (the compressors of a layer or of
// several layers) in one launch: workgroup (b, y) runs append y for sequence
// b.  kind = 4 * (activations bf16) + 2 * (cache fp8) + (per-channel gates).
__global__ __launch_bounds__(256) void kv_append_batch_kernel(const AppendBatch ab) {
    __shared__ __attribute__((aligned(16))) float erow[4096];  // f32 or bf16 rows
    __shared__ uint32_t amax;
    const int y = blockIdx.y;
    CAKV_DCHECK(y < kAppendBatchMax);
    const AppendArgs& a = ab.a[y];
    bf16_t* erow_h = reinterpret_cast<bf16_t*>(erow);
    switch (ab.kind[y]) {  // workgroup-uniform
        case 0: append_body<float, 0, false>(a, erow, amax); break;
        case 1: append_body<float, 0, true>(a, erow, amax); break;
        case 2: append_body<float, 2, false>(a, erow, amax); break;
        case 3: append_body<float, 2, true>(a, erow, amax); break;
        case 4: append_body<bf16_t, 1, false>(a, erow_h, amax); break;
        case 5: append_body<bf16_t, 1, true>(a, erow_h, amax); break;
        case 6: append_body<bf16_t, 2, false>(a, erow_h, amax); break;
        case 7: append_body<bf16_t, 2, true>(a, erow_h, amax); break;
        default: break;
    }
}

int launch_kv_append_batch(const AppendBatch& ab, int32_t n, int64_t B, hipStream_t stream) {
    if (B == 0 || n == 0) return 0;
    prof_mark("kv_append_kernel", false, stream);
    hipLaunchKernelGGL(kv_append_batch_kernel, dim3((unsigned)B, (unsigned)n), dim3(256), 0, stream, ab);
    prof_mark("kv_append_kernel", true, stream);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_kv_append(const AppendArgs& a, int64_t B, int act_dtype, int cache_dtype, bool gate_per_channel,
                     hipStream_t stream) {
    if (B == 0) return 0;
#define CAKV_AP(T, OK, PC) \
    hipLaunchKernelGGL((kv_append_kernel<T, OK, PC>), dim3((unsigned)B), dim3(256), 0, stream, a)
#define CAKV_AP2(T, OK)                     \
    if (gate_per_channel) CAKV_AP(T, OK, true); \
    else CAKV_AP(T, OK, false)
    prof_mark("kv_append_kernel", false, stream);
    if (act_dtype == 0) {
        if (cache_dtype == 2) { CAKV_AP2(float, 2); }
        else { CAKV_AP2(float, 0); }
    } else {
        if (cache_dtype == 2) { CAKV_AP2(bf16_t, 2); }
        else { CAKV_AP2(bf16_t, 1); }
    }
#undef CAKV_AP2
#undef CAKV_AP
    prof_mark("kv_append_kernel", true, stream);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace cakv
