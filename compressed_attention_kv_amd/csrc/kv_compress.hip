// kv_compress.hip -- softmax-weighted block compression of KV tokens.
//
// [V4 digest, CSA step 1; HCA paragraph] [V4-Pro card, Hybrid attention]:
// every m raw tokens (m = 4 for CSA, 128 for HCA; by default blocks do not
// overlap) become one entry, a weighted sum whose weights are a softmax over
// the block's per-token gate logits.
//
// Variants (cakv_kv_compress_ex): an entry's span may reach back over earlier
// blocks (span > m; the entry still ends where its block ends), and the gate
// may be one logit per token and channel (each channel its own softmax).
//
// Layout and schedule: a workgroup of 256 threads owns `epw` consecutive
// output entries; each entry is handled by D/4 threads that each own four
// consecutive channels, so every load instruction of a wave reads contiguous
// rows (coalesced streaming reduction, fp32 accumulation).  The gate softmax
// is evaluated per thread from the block's m logits (a few L1-resident
// scalars).  In fp8 mode the entry's max |c| is reduced through LDS and the
// per-entry power-of-two scale is derived exactly from the fp32 exponent.
#include "cakv_compress.hpp"
#include "cakv_internal.hpp"

namespace cakv {

// OUTK: 0 = f32, 1 = bf16, 2 = fp8 E4M3 + per-entry scale.  PC: one gate
// logit per token and channel ([B,T,D]) instead of one per token ([B,T]).
// Entry j covers tokens [max(0, (j+1)m - span), (j+1)m).
template <typename TIn, int OUTK, bool PC>
__global__ __launch_bounds__(256) void kv_compress_kernel(const TIn* __restrict__ x,
                                                          const float* __restrict__ gate, int64_t T,
                                                          int D, int m, int span, int64_t nblk,
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
    int ch[4];
    bool ok[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        ch[u] = c0 + u * tpe;
        ok[u] = u < per && ch[u] < nch;
    }
    float acc[4][4];
    float amx = 0.0f;
    if (live) {
        const int64_t b = e / nblk, j = e % nblk;
        const int64_t hi = (j + 1) * m, lo = hi - span > 0 ? hi - span : 0;
        const TIn* xb = x + (b * T + lo) * (int64_t)D;
        const float* gb = gate + (b * T + lo) * (PC ? (int64_t)D : 1);
        compress_entry<TIn, PC>(
            (int)(hi - lo), [&](int i) { return xb + (int64_t)i * D; }, [&](int i) { return gb[i]; },
            [&](int i) { return gb + (int64_t)i * D; }, ch, ok, acc);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (ok[u]) amx = fmaxf(amx, __builtin_fabsf(acc[u][c]));
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
            if (ok[u]) {
                f32x4 v = {acc[u][0], acc[u][1], acc[u][2], acc[u][3]};
                *reinterpret_cast<f32x4*>(o + ch[u] * 4) = v;
            }
        }
    } else if (OUTK == 1) {
        uint16_t* o = reinterpret_cast<uint16_t*>(out) + e * D;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (ok[u]) {
                u32x2 v;
                v[0] = f32_to_bf16_bits(acc[u][0]) | (f32_to_bf16_bits(acc[u][1]) << 16);
                v[1] = f32_to_bf16_bits(acc[u][2]) | (f32_to_bf16_bits(acc[u][3]) << 16);
                *reinterpret_cast<u32x2*>(o + ch[u] * 4) = v;
            }
        }
    } else {
        const int ex = q8_exponent(__uint_as_float(amax[slot]));
        uint8_t* o = reinterpret_cast<uint8_t*>(out) + e * D;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (ok[u]) {
                uint32_t w = 0;
#pragma unroll
                for (int c = 0; c < 4; ++c) w |= e4m3_encode(__builtin_ldexpf(acc[u][c], -ex)) << (8 * c);
                *reinterpret_cast<uint32_t*>(o + ch[u] * 4) = w;
            }
        }
        if (c0 == 0) out_scale[e] = __builtin_ldexpf(1.0f, ex);
    }
}

int launch_kv_compress(const void* x, int x_dtype, const float* gate, bool gate_per_channel, int64_t B,
                       int64_t T, int64_t D, int32_t m, int32_t span, void* out, int out_dtype,
                       float* out_scale, hipStream_t stream) {
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
#define CAKV_KC(TIN, OK, PC)                                                                          \
    hipLaunchKernelGGL((kv_compress_kernel<TIN, OK, PC>), dim3((unsigned)grid), dim3(256), 0, stream, \
                       (const TIN*)x, gate, T, (int)D, m, span, nblk, total, tpe, epw, out, out_scale)
#define CAKV_KC2(TIN, PC)                \
    if (out_dtype == 0) CAKV_KC(TIN, 0, PC); \
    else if (out_dtype == 1) CAKV_KC(TIN, 1, PC); \
    else CAKV_KC(TIN, 2, PC)
    prof_mark("kv_compress_kernel", false, stream);
    if (x_dtype == 0) {
        if (gate_per_channel) { CAKV_KC2(float, true); }
        else { CAKV_KC2(float, false); }
    } else {
        if (gate_per_channel) { CAKV_KC2(bf16_t, true); }
        else { CAKV_KC2(bf16_t, false); }
    }
#undef CAKV_KC2
#undef CAKV_KC
    prof_mark("kv_compress_kernel", true, stream);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace cakv
