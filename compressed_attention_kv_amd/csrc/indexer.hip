// indexer.hip -- Lightning-Indexer scoring and exact top-k on gfx950.
//
// [V4 digest, CSA step 2] a light indexer scores each query against every
// compressed entry and keeps the k best; [V4-Pro card, Hybrid attention] 64
// indexer heads of dim 128 keep k=1024; [Visualised, Dual Compression and
// Indexing] the pass is low precision.  Score of entry j for a query:
// S(j) = sum_h w_h * ReLU(q_h . k_j); ties go to the lower index; output
// ascending by index, -1 padded.
//
// Two kernels per call:
//   1. score: one workgroup per (query, chunk of entries).
//        fp8 mode: keys stream from HBM once, 64 bytes per lane per 32
//        entries (the next group's bytes are in flight while the current one
//        is multiplied), decoded exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8)
//        and multiplied on v_mfma_f32_32x32x16_bf16 against the bf16 query
//        heads held in VGPRs (heads x entries, fp32 accumulation); ReLU, the
//        head weights and the head reduction run on the accumulator registers
//        and one half-wave exchange.  The per-entry scale multiplies the final
//        sum (a power of two, so exact up to rounding order).
//        fp32 mode: one thread per entry runs the canonical fmaf chains.
//      Each score is written as an order-preserving 32-bit key.
//   2. top-k: one workgroup per query, no cross-workgroup hand-off.  A
//      strided sample of the keys gives a threshold (top 22 bits of the key,
//      from two 11-bit histogram levels) that a little more than k keys reach;
//      one coalesced pass collects every key at or above it into LDS; an LSD-free radix select on (key, index) finds
//      the k-th best exactly; the winners are marked in an LDS bitmap over
//      the entry range and compacted in index order.  If the guess collects
//      fewer than k or more than the LDS capacity, an exact radix select over
//      the whole key array takes over (slow, only for adversarial inputs).
#include "cakv_device.hpp"
#include "cakv_internal.hpp"

namespace cakv {

__device__ __forceinline__ int64_t query_nvis(const IndexerArgs& a, int64_t bq) {
    int32_t t = a.q_pos[bq];
    t = t < 0 ? 0 : t;
    int64_t nv = t / a.m;
    return nv < a.N ? nv : a.N;
}

// ------------------------------------------------------------------ fp8 mode
// HT: head tiles of 32 (HI = 32*HT); KS: MFMA k-steps of 16 (dI = 16*KS).
// Each wave streams its own 32-entry key groups (j0 = j_begin + 32 wave +
// 128 n) through a private ring of kSlots LDS slots filled by asynchronous
// HBM->LDS copies, kSlots - 1 groups ahead of the group it multiplies: the
// bytes in flight cost no registers and no barrier (the wave that copies a
// group is the one that reads it).  In a slot, 16-byte chunk c of row r holds
// the row's chunk c ^ (r mod chunks-per-row), which makes the per-row operand
// reads conflict-free.
constexpr int kSlots = 4;  // at most 4 (wait_groups)

template <int DI>
struct ScoreRing {
    static constexpr int GB = 32 * DI;        // key bytes of a group
    static constexpr int NDMA = GB / 1024;    // 16-byte-per-lane copies of a group
    static constexpr int CPR = DI / 16;       // 16-byte chunks per row
    static constexpr int SLOT = GB + 256;     // keys, then 64 scales (32 used)
    static constexpr int OPS = NDMA + 1;      // vector-memory operations per group
};

// Wait for a group's copies when nd later groups' copies (ops vector-memory
// operations each) and ns single stores were issued after them (wave-uniform
// nd, ns < kSlots).
template <int OPS>
__device__ __forceinline__ void wait_groups(int nd, int ns) {
    switch (nd * 4 + ns) {
#define CAKV_WAIT_CASE(d, s) \
    case (d) * 4 + (s): wait_vm<(d) * OPS + (s)>(); break;
        CAKV_WAIT_CASE(0, 0) CAKV_WAIT_CASE(0, 1) CAKV_WAIT_CASE(0, 2) CAKV_WAIT_CASE(0, 3)
        CAKV_WAIT_CASE(1, 0) CAKV_WAIT_CASE(1, 1) CAKV_WAIT_CASE(1, 2) CAKV_WAIT_CASE(1, 3)
        CAKV_WAIT_CASE(2, 0) CAKV_WAIT_CASE(2, 1) CAKV_WAIT_CASE(2, 2) CAKV_WAIT_CASE(2, 3)
        CAKV_WAIT_CASE(3, 0) CAKV_WAIT_CASE(3, 1) CAKV_WAIT_CASE(3, 2) CAKV_WAIT_CASE(3, 3)
#undef CAKV_WAIT_CASE
        default: wait_vm<0>(); break;
    }
}

template <int HT, int KS>
__global__ __launch_bounds__(256, 2) void idx_score_fp8_kernel(const IndexerArgs a) {
    constexpr int DI = 16 * KS;
    typedef ScoreRing<DI> R;
    constexpr int HALF = DI / 2;        // bytes of a key row per half-wave lane
    constexpr int NLD = HALF / 16;      // 16-byte chunks per lane
    __shared__ __attribute__((aligned(16))) uint8_t ring[4][kSlots][R::SLOT];

    const int64_t bq = blockIdx.y;
    const int64_t nvis = query_nvis(a, bq);
    const int64_t j_begin = (int64_t)blockIdx.x * a.chunk;
    if (nvis <= a.k || j_begin >= nvis) return;
    const int64_t j_end = min(nvis, j_begin + a.chunk);
    const int tid = threadIdx.x, lane = tid & 63, lrow = lane & 31, lh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: ring addresses go to M0
    const int64_t first = j_begin + 32 * wave;
    const int ng = first < j_end ? (int)((j_end - first + 127) / 128) : 0;
    if (ng == 0) return;  // nothing for this wave (no barrier below)

    const int64_t b = bq / a.Q;
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_idx) + b * a.N * DI;
    const float* sbase = a.k_scale + b * a.N;
    uint32_t* kout = a.keys + bq * a.N;
    uint8_t* slots = &ring[wave][0][0];

    // copies of group n into slot n % kSlots (rows past the cache end read
    // its last row: in bounds, never scored)
    auto issue = [&](int n) {
        const int64_t j0 = first + 128 * (int64_t)n;
        uint8_t* slot = slots + (n % kSlots) * R::SLOT;
#pragma unroll
        for (int i = 0; i < R::NDMA; ++i) {
            const int o = 1024 * i + 16 * lane;
            const int r = o / DI, c = (o % DI) / 16;
            const int64_t row = min(j0 + r, a.N - 1);
            lds_dma16(kbase + row * DI + 16 * (c ^ (r & (R::CPR - 1))), (uint32_t)(uintptr_t)(slot + 1024 * i));
        }
        lds_dma4(sbase + min(j0 + lane, a.N - 1), (uint32_t)(uintptr_t)(slot + R::GB));
    };
#pragma unroll
    for (int n = 0; n < kSlots - 1; ++n)
        if (n < ng) issue(n);

    // A operand: query heads (rows) x features, k-permutation (s, half, e) -> half*DI/2 + 8s + e
    bf16x8 qa[HT][KS];
    float wv[HT][16];
    const uint16_t* qbase = reinterpret_cast<const uint16_t*>(a.q_idx) + bq * (int64_t)(32 * HT) * DI;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
            qa[ht][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                        qbase + (32 * ht + lrow) * DI + lh * HALF + 8 * s));
#pragma unroll
        for (int r = 0; r < 16; ++r) wv[ht][r] = a.w[bq * (32 * HT) + 32 * ht + 8 * (r >> 2) + 4 * lh + (r & 3)];
    }

    for (int n = 0; n < ng; ++n) {
        // issue order: key store of group n-1, copies of group n+kSlots-1;
        // then wait for group n: after its copies came the copies of groups
        // n+1..min(n+kSlots-1, ng-1) and the stores of groups max(n-kSlots+1,0)..n-1
        const int nd = min(kSlots - 1, ng - 1 - n), ns = min(n, kSlots - 1);
        if (n + kSlots - 1 < ng) issue(n + kSlots - 1);
        wait_groups<R::OPS>(nd, ns);
        const uint8_t* slot = slots + (n % kSlots) * R::SLOT;
        u32x4 cur[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i)
            cur[i] = *reinterpret_cast<const u32x4*>(slot + lrow * DI + 16 * ((lh * NLD + i) ^ (lrow & (R::CPR - 1))));
        const float sc = *reinterpret_cast<const float*>(slot + R::GB + 4 * lrow);
        f32x16 acc[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[ht][r] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            // 8 fp8 bytes = dwords (2s, 2s+1) of this lane's half row
            const uint32_t d0 = cur[s >> 1][(s & 1) * 2], d1 = cur[s >> 1][(s & 1) * 2 + 1];
            u32x4 kb4;
            kb4[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false));
            kb4[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true));
            kb4[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false));
            kb4[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true));
            const bf16x8 kv = __builtin_bit_cast(bf16x8, kb4);
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
                acc[ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ht][s], kv, acc[ht], 0, 0, 0);
        }
        float sum = 0.0f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float v = acc[ht][r];
                sum = __builtin_fmaf(wv[ht][r], v > 0.0f ? v : 0.0f, sum);
            }
        sum += __shfl_xor(sum, 32, 64);
        sum *= sc;
        const int64_t j = first + 128 * (int64_t)n + lrow;
        if (lane < 32 && j < j_end) kout[j] = score_key(sum);
    }
}

// ------------------------------------------------------------------ fp32 mode
// Canonical order: per head an fmaf chain over d ascending from +0, ReLU as
// (s > 0 ? s : +0), then an fmaf chain over heads ascending from +0.
__global__ __launch_bounds__(256) void idx_score_f32_kernel(const IndexerArgs a) {
    __shared__ float qs[8192];
    __shared__ float ws[64];
    const int64_t bq = blockIdx.y;
    const int64_t nvis = query_nvis(a, bq);
    const int64_t j_begin = (int64_t)blockIdx.x * a.chunk;
    if (nvis <= a.k || j_begin >= nvis) return;
    const int64_t j_end = min(nvis, j_begin + a.chunk);
    const int tid = threadIdx.x;
    const int HI = a.HI, DI = a.dI;
    const float* q = reinterpret_cast<const float*>(a.q_idx) + bq * (int64_t)HI * DI;
    for (int i = tid; i < HI * DI; i += 256) qs[i] = q[i];
    for (int i = tid; i < HI; i += 256) ws[i] = a.w[bq * HI + i];
    __syncthreads();
    const int64_t b = bq / a.Q;
    const float* kb = reinterpret_cast<const float*>(a.k_idx) + b * a.N * DI;
    for (int64_t j = j_begin + tid; j < j_end; j += 256) {
        const float* kr = kb + j * DI;
        float S = 0.0f;
        for (int h = 0; h < HI; ++h) {
            float s = 0.0f;
            const float* qh = qs + h * DI;
            for (int d = 0; d < DI; d += 4) {
                const f32x4 kv = *reinterpret_cast<const f32x4*>(kr + d);
                s = __builtin_fmaf(qh[d], kv[0], s);
                s = __builtin_fmaf(qh[d + 1], kv[1], s);
                s = __builtin_fmaf(qh[d + 2], kv[2], s);
                s = __builtin_fmaf(qh[d + 3], kv[3], s);
            }
            const float rl = s > 0.0f ? s : 0.0f;
            S = __builtin_fmaf(ws[h], rl, S);
        }
        a.keys[bq * a.N + j] = score_key(S);
    }
}

// ------------------------------------------------------------------ top-k
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kBitmapWords = 8192;  // LDS bitmap covers 2^18 entries

// Workgroup-wide exclusive prefix sum of one value per thread (kSelThreads);
// every thread also receives the workgroup total.  wsum: kSelWaves + 1 words.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        uint32_t x = lane < kSelWaves ? wsum[lane] : 0u;
        uint32_t xi = x;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t t = __shfl_up(xi, o, 64);
            if (lane >= o) xi += t;
        }
        if (lane < kSelWaves) wsum[lane] = xi - x;
        if (lane == kSelWaves - 1) wsum[kSelWaves] = xi;
    }
    __syncthreads();
    const uint32_t r = wsum[wave] + incl - v;
    *total = wsum[kSelWaves];
    __syncthreads();
    return r;
}

// Wave 0 finds the digit d with below(d) < r <= below(d) + cnt[d] over 256
// counters; writes (d, below(d)) to out[0..1].
__device__ __forceinline__ void find_digit(const uint32_t* cnt, uint32_t r, uint32_t* out) {
    if (threadIdx.x >= 64) return;
    const int lane = threadIdx.x;
    const uint32_t c0 = cnt[4 * lane], c1 = cnt[4 * lane + 1], c2 = cnt[4 * lane + 2], c3 = cnt[4 * lane + 3];
    const uint32_t tot = c0 + c1 + c2 + c3;
    uint32_t incl = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    const uint32_t excl = incl - tot;
    if (excl < r && r <= incl) {
        uint32_t below = excl;
        int d = 4 * lane;
        if (r > below + c0) {
            below += c0;
            ++d;
            if (r > below + c1) {
                below += c1;
                ++d;
                if (r > below + c2) {
                    below += c2;
                    ++d;
                }
            }
        }
        out[0] = (uint32_t)d;
        out[1] = below;
    }
}

// r-th smallest (1-based) of the 64-bit values produced by get(i, &v) for
// i < n (get returns false for elements that do not take part), examining
// 8-bit digits from bit `top` down to bit `bottom`; bits above `top` are
// equal for all participants.  Whole workgroup.
template <typename Get>
__device__ uint64_t radix_select_u64(int64_t n, uint32_t r, int top, int bottom, Get get, uint32_t* cnt,
                                     uint32_t* res) {
    uint64_t prefix = 0, mask = 0;
    for (int shift = top - 7; shift >= bottom; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += blockDim.x) cnt[i] = 0u;
        __syncthreads();
        for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
            uint64_t v;
            if (get(i, &v) && (v & mask) == prefix) atomicAdd(&cnt[(v >> shift) & 255u], 1u);
        }
        __syncthreads();
        find_digit(cnt, r, res);
        __syncthreads();
        prefix |= (uint64_t)res[0] << shift;
        mask |= (uint64_t)255u << shift;
        r -= res[1];
        __syncthreads();
    }
    return prefix;
}

// ascending bitonic sort of n (power of two) 32-bit values in LDS
__device__ void bitonic_sort_u32(uint32_t* s, int n) {
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < (n >> 1); i += blockDim.x) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool asc = (lo & size) == 0;
                const uint32_t x = s[lo], y = s[hi];
                if ((x > y) == asc) {
                    s[lo] = y;
                    s[hi] = x;
                }
            }
            __syncthreads();
        }
    }
}

// rank value of entry j: ascending order = score descending, then index ascending
__device__ __forceinline__ uint64_t rank_value(uint32_t key, int64_t j) {
    return ((uint64_t)(~key) << 32) | (uint64_t)j;
}

__global__ __launch_bounds__(kSelThreads) void idx_topk_kernel(const IndexerArgs a) {
    __shared__ uint32_t hist[kHistBins];
    __shared__ uint64_t cand[kBoundaryCap];
    __shared__ uint32_t bits[kBitmapWords];
    __shared__ uint32_t wsum[kSelWaves + 1];
    __shared__ uint32_t info[16];
    const int64_t bq = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t nvis = query_nvis(a, bq);
    const int k = a.k;
    int32_t* out = a.idx + bq * k;
    if (nvis <= k) {  // every visible entry is selected
        for (int i = tid; i < k; i += kSelThreads) out[i] = i < nvis ? i : -1;
        return;
    }
    const uint32_t* keys = a.keys + bq * a.N;

    // ---- 1. threshold guess from a strided sample of the keys: the sample's
    //         want-th best key, to 22 bits (two 11-bit histogram levels)
    for (int i = tid; i < kHistBins; i += kSelThreads) hist[i] = 0u;
    if (tid < 16) info[tid] = 0u;
    __syncthreads();
    const int64_t S = nvis < 16384 ? nvis : 16384;
    // aim at ~1.5 k keys plus a margin at or above the threshold
    const uint32_t want = (uint32_t)(((1.5 * k) * (double)S) / (double)nvis) + 24u;
    uint32_t t22 = 0u;  // keys with (key >> 10) >= t22 are collected
    {
        // all of this thread's sample loads are issued before any histogram update
        uint32_t sk[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int64_t i = tid + (int64_t)u * kSelThreads;
            sk[u] = i < S ? keys[(i * nvis) / S] : 0u;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u)
            if (tid + (int64_t)u * kSelThreads < S) atomicAdd(&hist[sk[u] >> 21], 1u);
        __syncthreads();
        // bins from the top: thread t owns bins 2047-2t, 2046-2t; info[0] = the
        // bin where the running count reaches want, info[2] = samples above it
        const uint32_t h0 = hist[kHistBins - 1 - 2 * tid], h1 = hist[kHistBins - 2 - 2 * tid];
        uint32_t tot;
        const uint32_t excl = block_excl_scan(h0 + h1, wsum, &tot);
        if (excl < want && want <= excl + h0) {
            info[0] = (uint32_t)(kHistBins - 1 - 2 * tid);
            info[2] = excl;
        } else if (excl + h0 < want && want <= excl + h0 + h1) {
            info[0] = (uint32_t)(kHistBins - 2 - 2 * tid);
            info[2] = excl + h0;
        }
        __syncthreads();
        if (tot >= want) {  // else the sample is too thin: take everything (t22 = 0)
            const uint32_t tbin = info[0];
            const uint32_t want2 = want - info[2];
            for (int i = tid; i < kHistBins; i += kSelThreads) hist[i] = 0u;
            __syncthreads();
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (tid + (int64_t)u * kSelThreads < S && (sk[u] >> 21) == tbin)
                    atomicAdd(&hist[(sk[u] >> 10) & (kHistBins - 1)], 1u);
            __syncthreads();
            const uint32_t g0 = hist[kHistBins - 1 - 2 * tid], g1 = hist[kHistBins - 2 - 2 * tid];
            uint32_t tot2;
            const uint32_t ex2 = block_excl_scan(g0 + g1, wsum, &tot2);
            if (ex2 < want2 && want2 <= ex2 + g0 + g1)
                info[1] = (uint32_t)(kHistBins - 1 - 2 * tid - (ex2 + g0 >= want2 ? 0 : 1));
            __syncthreads();
            t22 = (tbin << 11) | info[1];
            __syncthreads();
            if (tid == 0) info[1] = 0u;
            __syncthreads();
        }
    }

    // ---- 2. collect every key in a bin >= tbin (coalesced pass over the keys;
    //         eight 16-byte loads per thread in flight per batch)
    constexpr int BATCH = 8;
    const bool vec_ok = (reinterpret_cast<uintptr_t>(keys) & 15u) == 0;
    for (int64_t j0 = 0; j0 < nvis; j0 += (int64_t)kSelThreads * 4 * BATCH) {
        u32x4 kv[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int64_t j = j0 + ((int64_t)u * kSelThreads + tid) * 4;
            if (vec_ok && j + 3 < nvis) {
                kv[u] = *reinterpret_cast<const u32x4*>(keys + j);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) kv[u][e] = (j + e < nvis) ? keys[j + e] : 0u;
            }
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int64_t j = j0 + ((int64_t)u * kSelThreads + tid) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (j + e < nvis && (kv[u][e] >> 10) >= t22) {
                    const uint32_t p = atomicAdd(&info[1], 1u);
                    if (p < (uint32_t)kBoundaryCap) cand[p] = rank_value(kv[u][e], j + e);
                }
            }
        }
    }
    __syncthreads();
    const uint32_t nc = info[1];
    const bool fast = nc >= (uint32_t)k && nc <= (uint32_t)kBoundaryCap;

    // ---- 3. exact k-th best in rank order
    uint64_t vth;
    if (fast) {
        vth = radix_select_u64((int64_t)nc, (uint32_t)k, 63, 0,
                               [&](int64_t i, uint64_t* v) { *v = cand[i]; return true; }, hist, info + 4);
    } else {
        vth = radix_select_u64(nvis, (uint32_t)k, 63, 0,
                               [&](int64_t i, uint64_t* v) { *v = rank_value(keys[i], i); return true; }, hist,
                               info + 4);
    }

    // ---- 4. winners (rank value <= vth), written in index order
    if (nvis <= (int64_t)kBitmapWords * 32) {
        const int words = (int)((nvis + 31) / 32);
        for (int i = tid; i < words; i += kSelThreads) bits[i] = 0u;
        __syncthreads();
        if (fast) {
            for (uint32_t i = tid; i < nc; i += kSelThreads) {
                const uint64_t v = cand[i];
                if (v <= vth) {
                    const uint32_t j = (uint32_t)(v & 0xffffffffu);
                    atomicOr(&bits[j >> 5], 1u << (j & 31));
                }
            }
        } else {
            for (int64_t j = tid; j < nvis; j += kSelThreads)
                if (rank_value(keys[j], j) <= vth) atomicOr(&bits[j >> 5], 1u << (j & 31));
        }
        __syncthreads();
        // each thread owns a contiguous run of words
        const int per = (words + kSelThreads - 1) / kSelThreads;
        const int w0 = tid * per, w1 = min(words, w0 + per);
        uint32_t c = 0;
        for (int i = w0; i < w1; ++i) c += __builtin_popcount(bits[i]);
        uint32_t tot;
        uint32_t pos = block_excl_scan(c, wsum, &tot);
        for (int i = w0; i < w1; ++i) {
            uint32_t bw = bits[i];
            while (bw) {
                const int bt = __builtin_ctz(bw);
                bw &= bw - 1u;
                out[pos++] = i * 32 + bt;
            }
        }
    } else {
        // wide entry range: gather the k winners and sort them by index
        uint32_t* srt = reinterpret_cast<uint32_t*>(bits);  // k <= 4096 <= 8192 words
        int n2 = 1;
        while (n2 < k) n2 <<= 1;
        for (int i = tid; i < n2; i += kSelThreads) srt[i] = 0xffffffffu;
        if (tid == 0) info[3] = 0u;
        __syncthreads();
        if (fast) {
            for (uint32_t i = tid; i < nc; i += kSelThreads) {
                const uint64_t v = cand[i];
                if (v <= vth) srt[atomicAdd(&info[3], 1u)] = (uint32_t)(v & 0xffffffffu);
            }
        } else {
            for (int64_t j = tid; j < nvis; j += kSelThreads)
                if (rank_value(keys[j], j) <= vth) srt[atomicAdd(&info[3], 1u)] = (uint32_t)j;
        }
        __syncthreads();
        bitonic_sort_u32(srt, n2);
        for (int i = tid; i < k; i += kSelThreads) out[i] = (int32_t)srt[i];
    }
}

size_t indexer_workspace_bytes(int64_t BQ, int64_t N, int32_t k) {
    (void)k;
    return ((size_t)BQ * (size_t)N * 4 + 255) & ~(size_t)255;  // score keys
}

int launch_indexer_topk(IndexerArgs& a, int64_t BQ, bool fp8_mode, void* ws, hipStream_t stream) {
    if (BQ == 0) return 0;
    a.keys = reinterpret_cast<uint32_t*>(ws);
    dim3 g1((unsigned)a.n_chunks, (unsigned)BQ);
    if (a.N > 0) {
        if (fp8_mode) {
            if (a.HI == 64 && a.dI == 128) hipLaunchKernelGGL((idx_score_fp8_kernel<2, 8>), g1, dim3(256), 0, stream, a);
            else if (a.HI == 32 && a.dI == 128) hipLaunchKernelGGL((idx_score_fp8_kernel<1, 8>), g1, dim3(256), 0, stream, a);
            else if (a.HI == 64 && a.dI == 64) hipLaunchKernelGGL((idx_score_fp8_kernel<2, 4>), g1, dim3(256), 0, stream, a);
            else if (a.HI == 32 && a.dI == 64) hipLaunchKernelGGL((idx_score_fp8_kernel<1, 4>), g1, dim3(256), 0, stream, a);
            else return -2;
        } else {
            hipLaunchKernelGGL(idx_score_f32_kernel, g1, dim3(256), 0, stream, a);
        }
        if (hipGetLastError() != hipSuccess) return -4;
    }
    hipLaunchKernelGGL(idx_topk_kernel, dim3((unsigned)BQ), dim3(kSelThreads), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return -4;
    return 0;
}

}  // namespace cakv
