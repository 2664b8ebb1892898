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
// output entries; each entry is handled by up to D/4 threads that each own
// one to four 4-channel chunks (one for spans of 32 tokens or more), so every
// load instruction of a wave reads contiguous rows (coalesced streaming
// reduction, fp32 accumulation).  The gate softmax
// is evaluated per thread from the block's m logits (a few L1-resident
// scalars).  In fp8 mode the entry's max |c| is reduced through LDS and the
// per-entry power-of-two scale is derived exactly from the fp32 exponent.
// Short spans at m = 4 (f32/bf16 entries) take a run kernel instead, which
// loads each token once for a run of consecutive entries (below).
#include <type_traits>

#include "cakv_compress.hpp"
#include "cakv_internal.hpp"

namespace cakv {

// compress_entry with per-token gates for an entry whose threads fill whole
// waves and whose span is at most 512 tokens: lane l evaluates the weights
// of tokens l, l + 64, ... once, instead of every thread evaluating all of
// them, and each token's weight reaches the wave by v_readlane.  The same
// operations in the same order (the max; exp of each gate minus it; the
// sum and each channel's fma chain in token order; the product with 1/z),
// so the entries are bitwise those of compress_entry (and of the streaming
// append).
template <typename TIn>
__device__ __forceinline__ void compress_entry_wave(int n, const TIn* xb, const float* gb, int D, const int ch[4],
                                                    const bool live[4], float acc[4][4]) {
    constexpr int WPL = 8;  // tokens per lane (n <= 512)
    const int lane = threadIdx.x & 63;
    float g[WPL];
#pragma unroll
    for (int k = 0; k < WPL; ++k) g[k] = lane + 64 * k < n ? gb[lane + 64 * k] : -INFINITY;
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < WPL; ++k) mx = fmaxf(mx, g[k]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float w[WPL];
#pragma unroll
    for (int k = 0; k < WPL; ++k) w[k] = lane + 64 * k < n ? expf(g[k] - mx) : 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u][0] = acc[u][1] = acc[u][2] = acc[u][3] = 0.0f;
    float z = 0.0f;
#pragma unroll
    for (int k = 0; k < WPL; ++k) {
        if (64 * k >= n) break;  // uniform
        const int nt = n - 64 * k < 64 ? n - 64 * k : 64;
        const int wk = __builtin_bit_cast(int, w[k]);
#pragma unroll 8
        for (int t = 0; t < nt; ++t) {
            const float wgt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(wk, t));
            z += wgt;
            const TIn* r = xb + (int64_t)(64 * k + t) * D;
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
    }
    const float rz = 1.0f / z;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[u][c] *= rz;
}

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
        // (tpe >= 64: an entry's threads fill whole waves, so `live` and the
        // entry are uniform per wave)
        if (!PC && tpe >= 64 && hi - lo <= 512)
            compress_entry_wave<TIn>((int)(hi - lo), xb, gb, D, ch, ok, acc);
        else
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

// Short spans (m = 4, span 4 or 8; f32 or bf16 entries): thread (run r,
// 4-channel chunk c) computes chunk c of RUN consecutive entries of one
// sequence, loading every token of the run's range once: the last SPAN - M
// tokens of an entry's span stay in registers as the first ones of the next
// entry's, and the next entry's M new tokens are requested before the
// current entry is reduced (two entries ahead was slower: fewer waves fit).
// Each entry is then reduced with exactly the
// operations of compress_entry (max, exp, sum and fma chain in token order),
// so the entries are bitwise those of the general kernel.
template <typename TIn, int OUTK, bool PC, int M, int SPAN>
__global__ __launch_bounds__(256) void kv_compress_run_kernel(const TIn* __restrict__ x,
                                                              const float* __restrict__ gate, int64_t T, int D,
                                                              int64_t nblk, int64_t runs_per_seq, int64_t total_runs,
                                                              int tpr, void* __restrict__ out) {
    constexpr int RUN = 16;  // entries per run
    constexpr int OLD = SPAN - M;
    static_assert(OLD >= 0 && OLD % M == 0, "span: a multiple of m");
    const int tid = threadIdx.x;
    const int64_t r = (int64_t)blockIdx.x * (256 / tpr) + tid / tpr;
    const int c = blockIdx.y * tpr + tid % tpr;  // 4-channel chunk
    if (r >= total_runs || 4 * c >= D) return;
    const int64_t b = r / runs_per_seq;
    const int64_t j0 = (r % runs_per_seq) * RUN;
    const int64_t j1 = j0 + RUN < nblk ? j0 + RUN : nblk;
    CAKV_DCHECK(j0 < nblk);
    const TIn* xb = x + b * T * (int64_t)D + 4 * c;
    const float* gb = PC ? gate + b * T * (int64_t)D + 4 * c : gate + b * T;
    // window slot s holds token (j+1) M - SPAN + s of entry j
    float xw[SPAN][4], gw[SPAN][PC ? 4 : 1];
    auto load_tok = [&](int64_t t, float (&xv)[4], float (&gv)[PC ? 4 : 1]) __attribute__((always_inline)) {
        load4<TIn>(xb + t * D, xv);
        if constexpr (PC) {
            const f32x4 g4 = *reinterpret_cast<const f32x4*>(gb + t * D);
            gv[0] = g4[0]; gv[1] = g4[1]; gv[2] = g4[2]; gv[3] = g4[3];
        } else {
            gv[0] = gb[t];
        }
    };
#pragma unroll
    for (int s = 0; s < OLD; ++s) {
        const int64_t t = j0 * M - OLD + s;
        if (t >= 0) load_tok(t, xw[s], gw[s]);
    }
    // the M new tokens of the next PF entries, in a ring of PF register sets
    // (indexed statically: the entry loop is unrolled by PF)
    constexpr int PF = 1;
    float nx[PF][M][4], ng[PF][M][PC ? 4 : 1];
#pragma unroll
    for (int f = 0; f < PF; ++f)
        if (j0 + f < j1) {
#pragma unroll
            for (int s = 0; s < M; ++s) load_tok((j0 + f) * M + s, nx[f][s], ng[f][s]);
        }
    for (int64_t jb = j0; jb < j1; jb += PF) {
#pragma unroll
        for (int f = 0; f < PF; ++f) {
            const int64_t j = jb + f;
            if (j >= j1) break;
#pragma unroll
            for (int s = 0; s < M; ++s) {
#pragma unroll
                for (int k = 0; k < 4; ++k) xw[OLD + s][k] = nx[f][s][k];
#pragma unroll
                for (int k = 0; k < (PC ? 4 : 1); ++k) gw[OLD + s][k] = ng[f][s][k];
            }
            if (j + PF < j1) {
#pragma unroll
                for (int s = 0; s < M; ++s) load_tok((j + PF) * M + s, nx[f][s], ng[f][s]);
            }
            // tokens of the span: slots s0 .. SPAN-1 (fewer at the sequence
            // start); a full span takes an instantiation without the slot tests
            const int s0 = (j + 1) * M >= SPAN ? 0 : (int)(SPAN - (j + 1) * M);
            float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            const auto reduce = [&](auto full_span) __attribute__((always_inline)) {
                constexpr bool FULL = decltype(full_span)::value;
                if constexpr (PC) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        float mx = -INFINITY;
#pragma unroll
                        for (int s = 0; s < SPAN; ++s)
                            if (FULL || s >= s0) mx = fmaxf(mx, gw[s][k]);
                        float z = 0.0f;
#pragma unroll
                        for (int s = 0; s < SPAN; ++s) {
                            if (FULL || s >= s0) {
                                const float wgt = expf(gw[s][k] - mx);
                                z += wgt;
                                acc[k] = __builtin_fmaf(wgt, xw[s][k], acc[k]);
                            }
                        }
                        acc[k] *= 1.0f / z;
                    }
                } else {
                    float mx = -INFINITY;
#pragma unroll
                    for (int s = 0; s < SPAN; ++s)
                        if (FULL || s >= s0) mx = fmaxf(mx, gw[s][0]);
                    float z = 0.0f;
#pragma unroll
                    for (int s = 0; s < SPAN; ++s) {
                        if (FULL || s >= s0) {
                            const float wgt = expf(gw[s][0] - mx);
                            z += wgt;
#pragma unroll
                            for (int k = 0; k < 4; ++k) acc[k] = __builtin_fmaf(wgt, xw[s][k], acc[k]);
                        }
                    }
                    const float rz = 1.0f / z;
#pragma unroll
                    for (int k = 0; k < 4; ++k) acc[k] *= rz;
                }
            };
            if (s0 == 0) reduce(std::true_type{});
            else reduce(std::false_type{});
            const int64_t e = b * nblk + j;
            if constexpr (OUTK == 0) {
                *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + e * D + 4 * c) =
                    f32x4{acc[0], acc[1], acc[2], acc[3]};
            } else {
                u32x2 v;
                v[0] = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
                v[1] = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
                *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + e * D + 4 * c) = v;
            }
            // the span's newest SPAN - M tokens open the next entry's span
#pragma unroll
            for (int s = 0; s < OLD; ++s) {
#pragma unroll
                for (int k = 0; k < 4; ++k) xw[s][k] = xw[s + M][k];
#pragma unroll
                for (int k = 0; k < (PC ? 4 : 1); ++k) gw[s][k] = gw[s + M][k];
            }
        }
    }
}

template <typename TIn, int OUTK, bool PC, int M, int SPAN>
static void launch_run(const void* x, const float* gate, int64_t B, int64_t T, int64_t D, void* out,
                       hipStream_t stream) {
    const int64_t nblk = T / M;
    const int64_t runs_per_seq = (nblk + 15) / 16;
    const int64_t total_runs = B * runs_per_seq;
    const int nch = (int)(D / 4);
    int tpr = 64;  // threads per run: a power of two covering the chunks, at most 256
    while (tpr < nch && tpr < 256) tpr <<= 1;
    const dim3 grid((unsigned)((total_runs + 256 / tpr - 1) / (256 / tpr)), (unsigned)((nch + tpr - 1) / tpr));
    hipLaunchKernelGGL((kv_compress_run_kernel<TIn, OUTK, PC, M, SPAN>), grid, dim3(256), 0, stream,
                       (const TIn*)x, gate, T, (int)D, nblk, runs_per_seq, total_runs, tpr, out);
}

int launch_kv_compress(const void* x, int x_dtype, const float* gate, bool gate_per_channel, int64_t B,
                       int64_t T, int64_t D, int32_t m, int32_t span, void* out, int out_dtype,
                       float* out_scale, hipStream_t stream) {
    const int64_t nblk = T / m;
    const int64_t total = B * nblk;
    if (total == 0) return 0;
    const int nch = (int)(D / 4);
    // up to four chunks per thread (one per thread for long spans, whose
    // entries are few and each a long chain of tokens: m = 128 compresses
    // 8,192 tokens into only 64 entries); threads per entry a power of two so
    // that entries never straddle a wave unevenly
    const int cpt = span >= 32 ? 1 : 4;
    int tpe = 1;
    while (tpe * cpt < nch && tpe < 256) tpe <<= 1;
    if (nch > 4 * tpe) return -2;
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
    // short spans at m = 4 with f32/bf16 entries: the run kernel
    if (m == 4 && (span == 4 || span == 8) && out_dtype != 2 && (total + 15) / 16 <= 0x7fffffffLL) {
#define CAKV_RUN(TIN, OK, PC)                                                                       \
        if (span == 4) launch_run<TIN, OK, PC, 4, 4>(x, gate, B, T, D, out, stream);              \
        else launch_run<TIN, OK, PC, 4, 8>(x, gate, B, T, D, out, stream)
#define CAKV_RUN2(TIN, PC)                  \
        if (out_dtype == 0) { CAKV_RUN(TIN, 0, PC); } \
        else { CAKV_RUN(TIN, 1, PC); }
        if (x_dtype == 0) {
            if (gate_per_channel) { CAKV_RUN2(float, true); }
            else { CAKV_RUN2(float, false); }
        } else {
            if (gate_per_channel) { CAKV_RUN2(bf16_t, true); }
            else { CAKV_RUN2(bf16_t, false); }
        }
#undef CAKV_RUN2
#undef CAKV_RUN
        prof_mark("kv_compress_kernel", true, stream);
        return hipGetLastError() == hipSuccess ? 0 : -4;
    }
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
