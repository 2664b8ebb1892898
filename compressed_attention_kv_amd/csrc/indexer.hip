// indexer.hip -- Lightning-Indexer scoring and exact top-k on gfx950.
//
// [V4 digest, CSA step 2] a light indexer scores each query against every
// compressed entry and keeps the k best; [V4-Pro card, Hybrid attention] 64
// indexer heads of dim 128 keep k=1024; [Visualised, Dual Compression and
// Indexing] the pass is low precision.  Score of entry j for a query:
// S(j) = sum_h w_h * ReLU(q_h . k_j); ties go to the lower index; output
// ascending by index, -1 padded.
//
// Kernels per call:
//   0. zero: the per-query histogram blocks.
//   1. score: one workgroup per (query, chunk of entries).
//        fp8 mode: each wave streams its own 32-entry groups of keys and
//        scales straight into a ring of VGPR sets, several groups ahead of
//        the one it multiplies; keys are decoded exactly to bf16
//        (v_cvt_scalef32_pk_bf16_fp8) and multiplied on
//        v_mfma_f32_32x32x16_bf16 against the bf16 query heads held in VGPRs
//        (heads x entries, fp32 accumulation); ReLU, the head weights and the
//        head reduction run on the accumulator registers and one half-wave
//        exchange.  The per-entry scale multiplies the final sum (a power of
//        two, so exact up to rounding order).  With one query per sequence
//        (decode) the keys arrive by whole-line nontemporal loads and a
//        transpose in each quad of lanes (kLoadLines below); with several
//        (prefill) a pack pass first copies the keys into a layout where each
//        load instruction reads 1 KiB of consecutive bytes (kLoadPacked), and
//        each step issues one group's MFMAs together with the previous
//        group's reduction (software-pipelined, two accumulator sets).
//        fp32 mode: one thread per entry runs the canonical fmaf chains.
//      Each score is written as an order-preserving 32-bit key, and counted
//      in an exact histogram of the top 11 key bits (LDS, then HBM atomics).
//   2. refine (same grid): lists the entries above the threshold bin and in
//      it; histograms the next 11 bits of the ones in it (see top-k below).
//      When the fp8 score grid has one workgroup per query (many queries, as
//      in a prefill chunk), that workgroup does this work itself after its
//      score loop, and neither 0 nor 2 is launched.
//   3. select: one workgroup per query ranks the threshold bin's entries and
//      writes the k winners in index order.
#include "cakv_device.hpp"
#include "cakv_internal.hpp"

namespace cakv {

__device__ __forceinline__ int64_t query_nvis(const IndexerArgs& a, int64_t bq) {
    int32_t t = a.q_pos[bq];
    t = t < 0 ? 0 : t;
    int64_t nv = t / a.m;
    return nv < a.N ? nv : a.N;
}

// Add a workgroup's LDS histogram into the query's histogram in HBM
// (nonzero bins only; the HBM copy was zeroed before the score pass).
__device__ __forceinline__ void flush_hist(const uint32_t* h, uint32_t* g, int nthreads) {
    for (int i = threadIdx.x; i < kHistBins; i += nthreads) {
        const uint32_t c = h[i];
        if (c) __hip_atomic_fetch_add(g + i, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// the refine pass's work done by the score workgroup itself when it is the
// only one of its query (defined with the top-k below)
__device__ __forceinline__ void fused_refine(const IndexerArgs& a, int64_t bq, int64_t nvis, const uint32_t* h1);

// ------------------------------------------------------------------ fp8 mode
// HT: head tiles of 32 (HI = 32*HT); KS: MFMA k-steps of 16 (dI = 16*KS).
// Each wave streams its own 32-entry key groups (entries first + 128 n +
// lrow) straight into VGPRs with ordinary vector loads, kPD groups ahead of
// the group it multiplies (a ring of kPD + 1 register sets, indexed
// statically by unrolling): lane (entry lrow, half lh) loads the half row it
// multiplies and the entry's scale.
constexpr int kPD = 3;  // groups in flight ahead of the one multiplied

// DPP partner in a quad of lanes: lane ^ D (quad_perm [1,0,3,2] or [2,3,0,1])
template <int D>
__device__ __forceinline__ uint32_t quad_xor(uint32_t x) {
    static_assert(D == 1 || D == 2, "quad partner");
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, D == 1 ? 0xB1 : 0x4E, 0xF, 0xF, true);
}

// In every quad of lanes, the 4 x 4 transpose of (lane, register) over the
// four 16-byte registers v[0..3]: afterwards lane 4q + a holds in v[i] what
// lane 4q + i held in v[a].  Two butterfly stages per dword: partner lane ^ 1
// on the register pairs (0, 1) and (2, 3), then lane ^ 2 on (0, 2) and (1, 3).
__device__ __forceinline__ void quad_transpose4(u32x4 (&v)[4], int lane) {
    const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
    auto stage = [](uint32_t& x, uint32_t& y, bool bit, auto xr) __attribute__((always_inline)) {
        const uint32_t sy = xr(y), sx = xr(x);
        const uint32_t nx = bit ? sy : x, ny = bit ? y : sx;
        x = nx;
        y = ny;
    };
    auto x1 = [](uint32_t t) __attribute__((always_inline)) { return quad_xor<1>(t); };
    auto x2 = [](uint32_t t) __attribute__((always_inline)) { return quad_xor<2>(t); };
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t r0 = v[0][d], r1 = v[1][d], r2 = v[2][d], r3 = v[3][d];
        stage(r0, r1, b0, x1);
        stage(r2, r3, b0, x1);
        stage(r0, r2, b1, x2);
        stage(r1, r3, b1, x2);
        v[0][d] = r0;
        v[1][d] = r1;
        v[2][d] = r2;
        v[3][d] = r3;
    }
}

// How a lane gets the NLD 16-byte chunks of the half row it multiplies (lane
// (entry lrow, half lh) of a 32-entry group):
//   kLoadDirect: loads them from the row; each load instruction covers a
//     quarter of 32 cache lines and the other instructions find the lines
//     in cache.
//   kLoadLines (128-dim keys, one query per sequence): instruction j of lane
//     4q + s loads chunk s of the half row that lane 4q + j multiplies, so
//     each instruction reads eight whole rows (both halves: quads q and
//     q + 8), the loads are nontemporal (nothing is read twice when each
//     sequence has one query), and a transpose in each quad of lanes hands
//     every lane its own chunks.
//   kLoadPacked (several queries per sequence): the pack pass has stored
//     chunk i of every lane of group g at 16-byte slot (g NLD + i) 64 + lane
//     of the sequence's packed keys, so instruction i of the wave reads 1 KiB
//     of consecutive bytes; the keys are then read by every query of the
//     sequence, and packed once per call.
constexpr int kLoadDirect = 0, kLoadLines = 1, kLoadPacked = 2;

// The pack pass: for sequence b and 32-entry group g, slot (g NLD + i) 64 + l
// holds bytes [(l >> 5) DI/2 + 16 i, + 16) of row min(32 g + (l & 31), N - 1).
// One thread per slot; G = ceil(N / 32) groups per sequence.
template <int NLD>
__global__ __launch_bounds__(256) void idx_pack_keys_kernel(const IndexerArgs a, int64_t B, int64_t G) {
    constexpr int DI = 32 * NLD, HALF = DI / 2;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= B * G * NLD * 64) return;
    const int l = (int)(t & 63);
    const int64_t gi = t >> 6;
    const int i = (int)(gi % NLD);
    const int64_t bg = gi / NLD, b = bg / G, g = bg % G;
    const int64_t row = min(32 * g + (l & 31), a.N - 1);
    CAKV_DCHECK(b < B && row >= 0);
    const uint8_t* src = reinterpret_cast<const uint8_t*>(a.k_idx) + (b * a.N + row) * DI + (l >> 5) * HALF + 16 * i;
    reinterpret_cast<u32x4*>(const_cast<void*>(a.kpack))[t] = *reinterpret_cast<const u32x4*>(src);
}

template <int HT, int KS, int LOAD>
__global__ __launch_bounds__(256, 2) void idx_score_fp8_kernel(const IndexerArgs a) {
    constexpr bool COAL = LOAD == kLoadLines, PACKED = LOAD == kLoadPacked;
    // software-pipelined steps for packed loads (several queries per
    // sequence, bound by instruction issue) at 64 heads of 128 dims; the
    // second accumulator set takes the registers of two of the three groups
    // in flight (the packed keys mostly come from L2).  (At other shapes it
    // would cost a wave per SIMD; the decode kernel, bound by its key
    // stream, was slower with it: 32-34 -> 35-36 us at 128K, 53-56 -> 59-63
    // us at 1M.)
    constexpr bool PIPE = PACKED && HT == 2 && KS == 8;
    constexpr int kPD = PIPE ? 1 : cakv::kPD;  // groups in flight ahead of the one multiplied
    constexpr int DI = 16 * KS;
    constexpr int HALF = DI / 2;        // bytes of a key row per half-wave lane
    constexpr int NLD = HALF / 16;      // 16-byte chunks per lane
    constexpr int RS = kPD + 1;         // register sets in the ring
    __shared__ uint32_t hist[kHistBins];

    const int64_t bq = blockIdx.y;
    const int64_t nvis = query_nvis(a, bq);
    const int64_t j_begin = (int64_t)blockIdx.x * a.chunk;
    if (nvis <= a.k || j_begin >= nvis) return;
    const int64_t j_end = min(nvis, j_begin + a.chunk);
    const int tid = threadIdx.x, lane = tid & 63, lrow = lane & 31, lh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t first = j_begin + 32 * wave;
    const int ng = first < j_end ? (int)((j_end - first + 127) / 128) : 0;

    const int64_t b = bq / a.Q;
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_idx) + b * a.N * DI;
    const float* sbase = a.k_scale + b * a.N;
    uint32_t* kout = a.keys + bq * a.N;
    const int64_t G = (a.N + 31) / 32;  // packed groups per sequence
    const u32x4* pbase = PACKED ? reinterpret_cast<const u32x4*>(a.kpack) + b * G * NLD * 64 : nullptr;

    // group n's half rows and scales (rows past the cache end read its last
    // row: in bounds, never scored)
    struct Grp {
        u32x4 c[NLD];
        float sc;
    };
    // (a group past the wave's last one reloads the last one's rows, usually
    // still in cache, instead of fetching rows of other waves' ranges)
    static_assert(!COAL || NLD == 4, "whole-line loads: four chunks per lane");
    auto load_group = [&](int n, Grp& g) __attribute__((always_inline)) {
        const int nn = n < ng ? n : (ng > 0 ? ng - 1 : 0);
        const int64_t row = min(first + 128 * (int64_t)nn + lrow, a.N - 1);
        if constexpr (COAL) {
            // the target lane 4q + j is in this lane's half (same quad): its
            // row is (lane & 28) + j of the group, its half lh
            const int q4 = lrow & ~3, ch = lane & 3;
#pragma unroll
            for (int j = 0; j < NLD; ++j) {
                const int64_t rj = min(first + 128 * (int64_t)nn + q4 + j, a.N - 1);
                g.c[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + rj * DI + lh * HALF) + ch);
            }
            g.sc = __builtin_nontemporal_load(sbase + row);
        } else if constexpr (PACKED) {
            // (a wave with no group reads the sequence's last group)
            const int64_t gi = min((first + 128 * (int64_t)nn) / 32, G - 1);
            CAKV_DCHECK(gi >= 0 && (first + 128 * (int64_t)nn) % 32 == 0);
#pragma unroll
            for (int i = 0; i < NLD; ++i) g.c[i] = pbase[(gi * NLD + i) * 64 + lane];
            g.sc = sbase[row];
        } else {
            const u32x4* src = reinterpret_cast<const u32x4*>(kbase + row * DI + lh * HALF);
#pragma unroll
            for (int i = 0; i < NLD; ++i) g.c[i] = src[i];
            g.sc = sbase[row];
        }
    };

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
    // The first groups are requested after the query operand and weights,
    // which are then awaited explicitly: had any of those loads still been
    // pending at the loop, the compiler would wait for them inside it on
    // every turn, draining the groups in flight.  Groups past the last one
    // load (clamped) rows too, for the same reason: a load under a condition
    // leaves the count of loads in flight unknown.
    Grp ring[RS];
#pragma unroll
    for (int n = 0; n < kPD; ++n) load_group(n, ring[n]);
    for (int i = tid; i < kHistBins; i += 256) hist[i] = 0u;
    wait_vm<kPD * (NLD + 1)>();
    __syncthreads();  // the histogram is clear

    // group g's dot products: acc[ht] = heads of tile ht x the group's entries
    auto mfma_group = [&](const Grp& g, f32x16 (&acc)[HT]) __attribute__((always_inline)) {
        u32x4 c[NLD];  // chunk i of this lane's half row
#pragma unroll
        for (int i = 0; i < NLD; ++i) c[i] = g.c[i];
        if constexpr (COAL) quad_transpose4(c, lane);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[ht][r] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            // 8 fp8 bytes = dwords (2s, 2s+1) of this lane's half row
            const uint32_t d0 = c[s >> 1][(s & 1) * 2], d1 = c[s >> 1][(s & 1) * 2 + 1];
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
    };
    // the weighted head sum of ReLU'd accumulators, times the entries' scales
    auto reduce_group = [&](const f32x16 (&acc)[HT], float sc) __attribute__((always_inline)) -> float {
        float sum = 0.0f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sum = __builtin_fmaf(wv[ht][r], relu_bits(acc[ht][r]), sum);
        return xor32_sum(sum) * sc;
    };
    // group n's scores into the key array and the LDS histogram
    auto put_group = [&](int n, float sum) __attribute__((always_inline)) {
        const int64_t j = first + 128 * (int64_t)n + lrow;
        if (lane < 32 && j < j_end) {
            const uint32_t key = score_key(sum);
            kout[j] = key;
            atomicAdd(&hist[key >> 21], 1u);
        }
    };
    auto score_group = [&](int n, const Grp& g) __attribute__((always_inline)) {
        f32x16 acc[HT];
        mfma_group(g, acc);
        put_group(n, reduce_group(acc, g.sc));
    };
    if constexpr (PIPE) {
        // Software-pipelined: a step issues group n's conversions and MFMAs
        // and the reduction of group n - 1 (from the other accumulator set;
        // the sets alternate with the group's parity, which the ring's even
        // length keeps across turns), with no dependence between them, so the
        // VALU work rides under the MFMAs; then it stores group n - 1's scores.
        static_assert(RS % 2 == 0, "accumulator sets alternate by group parity");
        f32x16 accb[2][HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int r = 0; r < 16; ++r) accb[1][ht][r] = 0.0f;
        float scp = 0.0f;
        for (int n0 = 0; n0 < ng; n0 += RS) {
#pragma unroll
            for (int u = 0; u < RS; ++u) {
                const int n = n0 + u;
                if (n >= ng) break;  // uniform
                load_group(n + kPD, ring[(u + kPD) % RS]);
                __builtin_amdgcn_sched_barrier(0);
                mfma_group(ring[u], accb[u & 1]);
                const float sp = reduce_group(accb[(u + 1) & 1], scp);  // (group n - 1; unused at n = 0)
                scp = ring[u].sc;
                __builtin_amdgcn_sched_barrier(0);
                if (n > 0) put_group(n - 1, sp);
            }
        }
        if (ng > 0) {  // the last group (a uniform branch keeps both sets in registers)
            float sl;
            if ((ng - 1) & 1) sl = reduce_group(accb[1], scp);
            else sl = reduce_group(accb[0], scp);
            put_group(ng - 1, sl);
        }
    } else {
        for (int n0 = 0; n0 < ng; n0 += RS) {
#pragma unroll
            for (int u = 0; u < RS; ++u) {
                const int n = n0 + u;
                if (n >= ng) break;  // uniform
                load_group(n + kPD, ring[(u + kPD) % RS]);
                // the next group's loads go out before this group's work, and
                // each group's work stays in its own step
                __builtin_amdgcn_sched_barrier(0);
                score_group(n, ring[u]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    __syncthreads();
    if (a.n_chunks == 1) {  // (uniform) the query's only workgroup: its histogram is the query's
        fused_refine(a, bq, nvis, hist);
        return;
    }
    flush_hist(hist, a.hist + bq * kHistStride, 256);
}

// ------------------------------------------------------------------ fp32 mode
// Canonical order: per head an fmaf chain over d ascending from +0, ReLU as
// (s > 0 ? s : +0), then an fmaf chain over heads ascending from +0.
__global__ __launch_bounds__(256) void idx_score_f32_kernel(const IndexerArgs a) {
    __shared__ float qs[8192];
    __shared__ float ws[64];
    __shared__ uint32_t hist[kHistBins];
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
    for (int i = tid; i < kHistBins; i += 256) hist[i] = 0u;
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
        const uint32_t key = score_key(S);
        a.keys[bq * a.N + j] = key;
        atomicAdd(&hist[key >> 21], 1u);
    }
    __syncthreads();
    flush_hist(hist, a.hist + bq * kHistStride, 256);
}

// ------------------------------------------------------------------ top-k
// The score pass leaves an exact histogram of the top 11 key bits per query
// (level 1).  Its threshold bin b1 is where the running count from the top
// reaches k: the keys above it are fewer than k, with it at least k.  A
// refine pass on the score grid lists the entries above b1 (all winners) and
// those in b1, and, unless b1 holds only a few keys (kSmallBin), histograms
// the next 11 key bits of the ones in b1 (level 2).  One workgroup per query
// then takes the entries of b1 above the level-2 threshold bin (found the
// same way), ranks the ones in that bin (or, at level 1, all of b1) by (key,
// lower index first), and writes the winners in index order.  If b1 holds
// more than kCandCap keys, a radix select over the whole key array is used.
constexpr int kBitmapWords = 8192;  // LDS bitmap covers 2^18 entries
constexpr uint32_t kSmallBin = 64;  // a threshold bin this small is ranked whole

// Workgroup-wide exclusive prefix sum of one value per thread (NT threads);
// every thread also receives the workgroup total.  wsum: NT/64 + 1 words.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    constexpr int NW = NT / 64;
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
        uint32_t x = lane < NW ? wsum[lane] : 0u;
        uint32_t xi = x;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t t = __shfl_up(xi, o, 64);
            if (lane >= o) xi += t;
        }
        if (lane < NW) wsum[lane] = xi - x;
        if (lane == NW - 1) wsum[NW] = xi;
    }
    __syncthreads();
    const uint32_t r = wsum[wave] + incl - v;
    *total = wsum[NW];
    __syncthreads();
    return r;
}

// Bin b of an 11-bit histogram h with (count above b) < want <= (count at
// or above b), scanning from the top bin down; want >= 1 and at most the
// histogram total (otherwise the result is bin 0 with 0 above: still a valid
// index).  Whole workgroup (NT threads); every thread gets the bin and the
// count above it.  info: 2 words, wsum: NT/64 + 1 words.
template <int NT>
__device__ void find_bin(const uint32_t* h, uint32_t want, uint32_t* wsum, uint32_t* info, uint32_t* bin,
                         uint32_t* above) {
    constexpr int BPT = kHistBins / NT;  // bins per thread, descending from the top
    const int t = threadIdx.x;
    if (t == 0) {  // (the scan's barriers order this before the finder's write)
        info[0] = 0u;
        info[1] = 0u;
    }
    uint32_t c[BPT];
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        c[i] = h[kHistBins - 1 - BPT * t - i];
        local += c[i];
    }
    uint32_t tot;
    const uint32_t excl = block_excl_scan<NT>(local, wsum, &tot);
    if (excl < want && want <= excl + local) {
        uint32_t cum = excl;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            if (cum < want && want <= cum + c[i]) {
                info[0] = (uint32_t)(kHistBins - 1 - BPT * t - i);
                info[1] = cum;
            }
            cum += c[i];
        }
    }
    __syncthreads();
    *bin = info[0];
    *above = info[1];
    __syncthreads();
}

// The same search by one wave over an LDS histogram: lane l owns the 32
// bins just below 2048 - 32 l; no barrier.  Writes (bin, above) to out when
// the histogram holds at least want (the caller zeroes out beforehand).
__device__ void find_bin_wave(const uint32_t* h, uint32_t want, uint32_t* out) {
    const int lane = threadIdx.x & 63;
    const u32x4* hb = reinterpret_cast<const u32x4*>(h + kHistBins - 32 * (lane + 1));
    uint32_t c[32];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const u32x4 v = hb[q];
        c[4 * q] = v[0];
        c[4 * q + 1] = v[1];
        c[4 * q + 2] = v[2];
        c[4 * q + 3] = v[3];
    }
    uint32_t local = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) local += c[i];
    uint32_t incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    const uint32_t excl = incl - local;
    if (excl < want && want <= incl) {
        uint32_t cum = excl;
#pragma unroll
        for (int i = 31; i >= 0; --i) {  // bin 2048 - 32 lane - 32 + i, from the top down
            if (cum < want && want <= cum + c[i]) {
                out[0] = (uint32_t)(kHistBins - 32 * (lane + 1) + i);
                out[1] = cum;
            }
            cum += c[i];
        }
    }
}

// One workgroup per query's histogram block.
__global__ __launch_bounds__(256) void idx_zero_kernel(u32x4* p) {
    u32x4* q = p + (int64_t)blockIdx.x * (kHistStride / 4);
    for (int i = threadIdx.x; i < kHistStride / 4; i += 256) q[i] = u32x4{0u, 0u, 0u, 0u};
}

// Append the values of the whole workgroup (NT threads, KPT per thread)
// whose flag is set to two lists at once: the waves' counts meet in LDS and
// one returning atomic per list and workgroup reserves the space (the lists'
// counters are shared by all workgroups of a query).  Every thread calls it;
// sh: 2 NT/64 + 2 words of LDS.
template <int NT, int KPT, typename TA, typename TB>
__device__ __forceinline__ void block_append2(TA* la, uint32_t* ca, const bool (&sa)[KPT], const TA (&va)[KPT],
                                              bool use_b, TB* lb, uint32_t* cb, const bool (&sb)[KPT],
                                              const TB (&vb)[KPT], uint32_t* sh) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t c_a = 0, c_b = 0;
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        c_a += sa[u] ? 1u : 0u;
        c_b += (use_b && sb[u]) ? 1u : 0u;
    }
    uint32_t inc_a = c_a, inc_b = c_b;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t ta = __shfl_up(inc_a, o, 64), tb = __shfl_up(inc_b, o, 64);
        if (lane >= o) {
            inc_a += ta;
            inc_b += tb;
        }
    }
    if (lane == 63) {
        sh[wave] = inc_a;
        sh[NW + wave] = inc_b;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t ta = 0, tb = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            ta += sh[w];
            tb += sh[NW + w];
        }
        sh[2 * NW] = ta ? atomicAdd(ca, ta) : 0u;
        sh[2 * NW + 1] = tb ? atomicAdd(cb, tb) : 0u;
    }
    __syncthreads();
    uint32_t pa = sh[2 * NW] + inc_a - c_a, pb = sh[2 * NW + 1] + inc_b - c_b;
    for (int w = 0; w < wave; ++w) {
        pa += sh[w];
        pb += sh[NW + w];
    }
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        if (sa[u]) la[pa++] = va[u];
        if (use_b && sb[u]) lb[pb++] = vb[u];
    }
    __syncthreads();  // sh is reused by the next call
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

// Keys [j0, j0 + NT KPT) of a query that lie below j_end (others read as 0),
// one per thread and u, all requested before any is used.
template <int NT, int KPT>
__device__ __forceinline__ void load_key_batch(const uint32_t* keys, int64_t j0, int64_t j_end, uint32_t (&dst)[KPT]) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        const int64_t j = j0 + (int64_t)u * NT + threadIdx.x;
        dst[u] = j < j_end ? keys[j] : 0u;
    }
}

// The refine work on entries [j_begin, j_end) of a query: lists the ones
// above the level-1 threshold bin b1 (list A) and in it (list B, if it fits),
// and counts the next 11 key bits of b1's entries into h2 (if level2).
// cnt_a and cnt_b are the lists' append counters; kv holds the first batch
// of keys, already requested (each batch requests the next before it is
// classified).  Every thread of the workgroup (256) calls it.
template <int KPT>
__device__ __forceinline__ void refine_entries(const uint32_t* keys, int64_t j_begin, int64_t j_end, uint32_t b1,
                                               bool fits, bool level2, uint32_t (&kv)[KPT], uint32_t* h2,
                                               uint32_t* list_a, uint32_t* cnt_a, uint64_t* list_b,
                                               uint32_t* cnt_b, uint32_t* ash) {
    constexpr int NT = 256;
    constexpr int64_t STEP = (int64_t)NT * KPT;
    const int tid = threadIdx.x;
    for (int64_t j0 = j_begin; j0 < j_end; j0 += STEP) {  // uniform trip count
        uint32_t jv[KPT], kn[KPT];
        uint64_t rv[KPT];
        bool sa[KPT], sb[KPT];
        const bool more = j0 + STEP < j_end;  // uniform
        if (more) load_key_batch<NT, KPT>(keys, j0 + STEP, j_end, kn);
#pragma unroll
        for (int u = 0; u < KPT; ++u) jv[u] = (uint32_t)(j0 + (int64_t)u * NT + tid);
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const bool in = (int64_t)j0 + (int64_t)u * NT + tid < j_end;
            const uint32_t top = kv[u] >> 21;
            sa[u] = in && top > b1;
            sb[u] = in && top == b1;
            rv[u] = rank_value(kv[u], jv[u]);
            if (level2 && sb[u]) atomicAdd(&h2[(kv[u] >> 10) & (kHistBins - 1)], 1u);
        }
        block_append2<NT, KPT>(list_a, cnt_a, sa, jv, fits, list_b, cnt_b, sb, rv, ash);
        if (more) {
#pragma unroll
            for (int u = 0; u < KPT; ++u) kv[u] = kn[u];
        }
    }
}

// Refine, on the score grid: every workgroup of a query lists its entries
// above the level-1 threshold bin b1 (list A) and in it (list B) and adds
// the level-2 histogram of b1.  (Handing the lists to one workgroup inside
// this kernel would need device-scope release fences, which write back the
// L2 of the issuing XCD: the kernel boundary does that once.)
__global__ __launch_bounds__(256) void idx_refine_kernel(const IndexerArgs a) {
    __shared__ uint32_t h2[kHistBins];
    __shared__ uint32_t wsum[5];
    __shared__ uint32_t info[2];
    __shared__ uint32_t ash[2 * 4 + 2];
    constexpr int NT = 256, KPT = 8;
    const int64_t bq = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t nvis = query_nvis(a, bq);
    const int k = a.k;
    const int64_t j_begin = (int64_t)blockIdx.x * a.chunk;
    if (nvis <= k || j_begin >= nvis) return;
    const int64_t j_end = min(nvis, j_begin + a.chunk);
    const uint32_t* keys = a.keys + bq * a.N;
    uint32_t* qh = a.hist + bq * kHistStride;
    uint32_t* cnt = qh + 2 * kHistBins;  // [0] list A, [1] list B, [2] b1, [3] count above b1
    // keys are requested one round ahead; the first round before the
    // threshold search, so that its latency overlaps the search
    uint32_t kv[KPT];
    load_key_batch<NT, KPT>(keys, j_begin, j_end, kv);
    for (int i = tid; i < kHistBins; i += NT) h2[i] = 0u;
    uint32_t b1, a1;
    find_bin<NT>(qh, (uint32_t)k, wsum, info, &b1, &a1);  // (syncs, so h2 is clear)
    const uint32_t nb1 = qh[b1];
    const bool fits = nb1 <= (uint32_t)kCandCap, level2 = nb1 > kSmallBin;  // uniform
    if (blockIdx.x == 0 && tid == 0) {  // for the select pass
        cnt[2] = b1;
        cnt[3] = a1;
    }
    refine_entries<KPT>(keys, j_begin, j_end, b1, fits, level2, kv, h2, a.cand_a + bq * kTopkCap, cnt,
                        a.cand_b + bq * kCandCap, cnt + 1, ash);
    if (level2) {
        __syncthreads();
        flush_hist(h2, qh + kHistBins, NT);
    }
}

// The refine work done by a query's only score workgroup, after its score
// loop: h1 (LDS) is then the query's whole level-1 histogram, so the
// threshold comes from it, the list counters live in LDS, and both
// histogram levels and the threshold are written out for the select pass
// without atomics.  The workgroup reads back the keys it wrote (its own
// stores, ordered before the loads by the barrier after the score loop).
// Nothing here needs the histogram block cleared beforehand, so calls whose
// score grid has one workgroup per query launch neither the clearing nor the
// refine kernel.  (The read-back is not hidden: the workgroups of a round,
// whose queries see nearly equal entry counts, reach it together.)
__device__ __forceinline__ void fused_refine(const IndexerArgs& a, int64_t bq, int64_t nvis, const uint32_t* h1) {
    __shared__ uint32_t h2[kHistBins];
    __shared__ uint32_t wsum[5];
    __shared__ uint32_t info[2];
    __shared__ uint32_t ash[2 * 4 + 2];
    __shared__ uint32_t lcnt[2];
    constexpr int NT = 256, KPT = 8;
    const int tid = threadIdx.x;
    const uint32_t* keys = a.keys + bq * a.N;
    uint32_t* qh = a.hist + bq * kHistStride;
    uint32_t kv[KPT];
    load_key_batch<NT, KPT>(keys, 0, nvis, kv);
    for (int i = tid; i < kHistBins; i += NT) h2[i] = 0u;
    if (tid < 2) lcnt[tid] = 0u;
    uint32_t b1, a1;
    find_bin<NT>(h1, (uint32_t)a.k, wsum, info, &b1, &a1);  // (syncs, so h2 and lcnt are clear)
    const uint32_t nb1 = h1[b1];
    const bool fits = nb1 <= (uint32_t)kCandCap, level2 = nb1 > kSmallBin;  // uniform
    refine_entries<KPT>(keys, 0, nvis, b1, fits, level2, kv, h2, a.cand_a + bq * kTopkCap, lcnt,
                        a.cand_b + bq * kCandCap, lcnt + 1, ash);  // (ends with a barrier)
    static_assert(kHistBins % (4 * NT) == 0, "histogram copy in whole rounds");
    for (int i = tid; i < kHistBins / 4; i += NT) {
        reinterpret_cast<u32x4*>(qh)[i] = reinterpret_cast<const u32x4*>(h1)[i];
        reinterpret_cast<u32x4*>(qh + kHistBins)[i] = reinterpret_cast<const u32x4*>(h2)[i];
    }
    if (tid == 0) {
        qh[2 * kHistBins + 2] = b1;
        qh[2 * kHistBins + 3] = a1;
    }
}

// Select: one workgroup per query takes list A, the entries of B above the
// level-2 threshold bin, and the best of the ones in that bin (or, at level
// 1, of all of B) by (key, lower index first), then writes the k winners in
// index order.  If b1 holds more than kCandCap keys, a radix select over the
// whole key array replaces the lists.
constexpr int kSelThreads = 1024;
constexpr int kBndCap = 4096;  // boundary entries ranked in LDS

__global__ __launch_bounds__(kSelThreads) void idx_select_kernel(const IndexerArgs a) {
    __shared__ uint32_t hs[2 * kHistBins];
    // the ranked boundary entries and the winners' bitmap are never live at
    // once (a barrier separates the ranking from the bitmap), so they share
    // LDS: two select workgroups then fit on a CU
    __shared__ __attribute__((aligned(16))) uint64_t bnd_bits[kBndCap];
    static_assert(kBitmapWords * 4 <= kBndCap * 8, "the bitmap fits the boundary entries' space");
    uint64_t* const bnd = bnd_bits;
    uint32_t* const bits = reinterpret_cast<uint32_t*>(bnd_bits);
    __shared__ uint32_t win[kTopkCap];
    __shared__ uint32_t cnt256[256];
    __shared__ uint32_t wsum[kSelThreads / 64 + 1];
    __shared__ uint32_t info[16];
    constexpr int NT = kSelThreads, KPT = kCandCap / kSelThreads;
    const int64_t bq = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t nvis = query_nvis(a, bq);
    const int k = a.k;
    int32_t* out = a.idx + bq * k;
    if (nvis <= k) {  // every visible entry is selected
        for (int i = tid; i < k; i += NT) out[i] = i < nvis ? i : -1;
        return;
    }
    const uint32_t* keys = a.keys + bq * a.N;
    const uint32_t* qh = a.hist + bq * kHistStride;
    const uint32_t* list_a = a.cand_a + bq * kTopkCap;
    const uint64_t* list_b = a.cand_b + bq * kCandCap;
    // both histogram levels into LDS with one batch of loads
    static_assert(2 * kHistBins == 4 * NT, "histogram staging: one u32x4 per thread");
    reinterpret_cast<u32x4*>(hs)[tid] = reinterpret_cast<const u32x4*>(qh)[tid];
    // the level-1 threshold bin and the count above it come from the refine
    // pass (clamped, so that any word there gives in-bounds indices); other
    // bins default to 0
    if (tid < 16) {
        uint32_t v = 0u;
        if (tid == 8) v = qh[2 * kHistBins + 2] & (kHistBins - 1);
        if (tid == 9) v = min(qh[2 * kHistBins + 3], (uint32_t)k);
        info[tid] = v;
    }
    __syncthreads();
    // wave 0 finds the level-2 threshold bin where it was built
    if (tid < 64) {
        const uint32_t b = info[8], ab = info[9];
        if (hs[b] > kSmallBin && hs[b] <= (uint32_t)kCandCap) find_bin_wave(hs + kHistBins, (uint32_t)k - ab, info + 10);
    }
    __syncthreads();
    const uint32_t b1 = info[8], a1 = info[9];
    const uint32_t nb1 = hs[b1];
    const bool fits = nb1 <= (uint32_t)kCandCap, level2 = nb1 > kSmallBin;

    // winners' entry indices go to win[0..k)
    if (fits) {
        const uint32_t b2 = level2 ? info[10] : 0u, a2 = level2 ? info[11] : 0u;
        for (uint32_t i = tid; i < a1; i += NT) win[i] = list_a[i];
        for (uint32_t i0 = 0; i0 < nb1; i0 += NT * KPT) {
            uint64_t rv[KPT];
#pragma unroll
            for (int u = 0; u < KPT; ++u) {
                const uint32_t i = i0 + u * NT + tid;
                rv[u] = i < nb1 ? list_b[i] : 0u;
            }
#pragma unroll
            for (int u = 0; u < KPT; ++u) {
                if (i0 + u * NT + tid >= nb1) continue;
                const uint32_t key = ~(uint32_t)(rv[u] >> 32), j = (uint32_t)(rv[u] & 0xffffffffu);
                const uint32_t lo = (key >> 10) & (kHistBins - 1);
                if (level2 && lo > b2) {
                    win[a1 + atomicAdd(&info[0], 1u)] = j;
                } else if (!level2 || lo == b2) {
                    const uint32_t p = atomicAdd(&info[1], 1u);
                    if (p < (uint32_t)kBndCap) bnd[p] = rv[u];
                }
            }
        }
        __syncthreads();
        const uint32_t above = a1 + a2, nb = info[1];
        const uint32_t need = (uint32_t)k - above;  // 1 .. nb
        if (need >= nb) {  // (then nb <= k <= kBndCap... or all of them win)
            if (nb <= (uint32_t)kBndCap) {
                for (uint32_t i = tid; i < nb; i += NT) win[above + i] = (uint32_t)(bnd[i] & 0xffffffffu);
            } else {
                for (uint32_t i = tid; i < nb1; i += NT) {
                    const uint64_t v = list_b[i];
                    const uint32_t lo = (~(uint32_t)(v >> 32) >> 10) & (kHistBins - 1);
                    if (!level2 || lo == b2) win[above + atomicAdd(&info[2], 1u)] = (uint32_t)(v & 0xffffffffu);
                }
            }
        } else if (nb <= (uint32_t)kBndCap) {
            for (uint32_t i = tid; i < nb; i += NT) {
                const uint64_t v = bnd[i];
                uint32_t r = 0;
                // eight independent LDS reads per round, so their latencies overlap
                uint32_t l = 0;
                for (; l + 8 <= nb; l += 8) {
                    const u32x4* p = reinterpret_cast<const u32x4*>(bnd + l);
                    u32x4 w[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) w[u] = p[u];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint64_t x0 = (uint64_t)w[u][0] | ((uint64_t)w[u][1] << 32);
                        const uint64_t x1 = (uint64_t)w[u][2] | ((uint64_t)w[u][3] << 32);
                        r += (x0 < v ? 1u : 0u) + (x1 < v ? 1u : 0u);
                    }
                }
                for (; l < nb; ++l) r += bnd[l] < v ? 1u : 0u;
                if (r < need) win[above + r] = (uint32_t)(v & 0xffffffffu);  // ranks are distinct
            }
        } else {  // a crowded bin: radix select straight from list B
            auto get = [&](int64_t i, uint64_t* v) {
                *v = list_b[i];
                return !level2 || ((~(uint32_t)(*v >> 32) >> 10) & (kHistBins - 1)) == b2;
            };
            const uint64_t vth = radix_select_u64((int64_t)nb1, need, 63, 0, get, cnt256, info + 4);
            for (uint32_t i = tid; i < nb1; i += NT) {
                uint64_t v;
                if (get(i, &v) && v <= vth) win[above + atomicAdd(&info[2], 1u)] = (uint32_t)(v & 0xffffffffu);
            }
        }
    } else {
        const uint64_t vth = radix_select_u64(nvis, (uint32_t)k, 63, 0,
                                              [&](int64_t i, uint64_t* v) { *v = rank_value(keys[i], i); return true; },
                                              cnt256, info + 4);
        for (int64_t j = tid; j < nvis; j += NT)
            if (rank_value(keys[j], j) <= vth) win[atomicAdd(&info[2], 1u)] = (uint32_t)j;
    }
    __syncthreads();

    // winners in index order
    if (nvis <= (int64_t)kBitmapWords * 32) {
        const int words = (int)((nvis + 31) / 32);
        for (int i = tid; i < words; i += NT) bits[i] = 0u;
        __syncthreads();
        for (int i = tid; i < k; i += NT) {
            CAKV_DCHECK(win[i] < (uint32_t)nvis);
            atomicOr(&bits[win[i] >> 5], 1u << (win[i] & 31));
        }
        __syncthreads();
        // each thread owns a contiguous run of words
        const int per = (words + NT - 1) / NT;
        const int w0 = tid * per, w1 = min(words, w0 + per);
        uint32_t c = 0;
        for (int i = w0; i < w1; ++i) c += __builtin_popcount(bits[i]);
        uint32_t tot;
        uint32_t pos = block_excl_scan<NT>(c, wsum, &tot);
        CAKV_DCHECK(tot == (uint32_t)k);  // k distinct winners
        for (int i = w0; i < w1; ++i) {
            uint32_t bw = bits[i];
            while (bw) {
                const int bt = __builtin_ctz(bw);
                bw &= bw - 1u;
                out[pos++] = i * 32 + bt;
            }
        }
    } else {
        // wide entry range: sort the k winners by index (k <= 4096 <= 8192 words)
        uint32_t* srt = bits;
        int n2 = 1;
        while (n2 < k) n2 <<= 1;
        for (int i = tid; i < n2; i += NT) srt[i] = i < k ? win[i] : 0xffffffffu;
        __syncthreads();
        bitonic_sort_u32(srt, n2);
        for (int i = tid; i < k; i += NT) out[i] = (int32_t)srt[i];
    }
}

// Workspace: score keys [BQ][N], histograms [BQ][kHistStride], lists A
// [BQ][kTopkCap] (entry indices) and B [BQ][kCandCap] (rank values), and,
// with several queries per sequence, the packed keys [B][ceil(N/32)][32 *
// 128 bytes] (sized for the largest fp8 key width); each region 256-byte
// aligned.
static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

static size_t packed_key_bytes(int64_t B, int64_t Q, int64_t N) {
    return Q > 1 ? (size_t)B * (size_t)((N + 31) / 32) * 32 * 128 : 0;
}

size_t indexer_workspace_bytes(int64_t B, int64_t Q, int64_t N, int32_t k) {
    (void)k;
    const int64_t BQ = B * Q;
    return al256((size_t)BQ * (size_t)N * 4) + al256((size_t)BQ * kHistStride * 4) +
           al256((size_t)BQ * kTopkCap * 4) + al256((size_t)BQ * kCandCap * 8) + al256(packed_key_bytes(B, Q, N));
}

int launch_indexer_topk(IndexerArgs& a, int64_t BQ, bool fp8_mode, void* ws, hipStream_t stream) {
    if (BQ == 0) return 0;
    uint8_t* w = reinterpret_cast<uint8_t*>(ws);
    a.keys = reinterpret_cast<uint32_t*>(w);
    w += al256((size_t)BQ * (size_t)a.N * 4);
    a.hist = reinterpret_cast<uint32_t*>(w);
    w += al256((size_t)BQ * kHistStride * 4);
    a.cand_a = reinterpret_cast<uint32_t*>(w);
    w += al256((size_t)BQ * kTopkCap * 4);
    a.cand_b = reinterpret_cast<uint64_t*>(w);
    w += al256((size_t)BQ * kCandCap * 8);
    const int64_t B = BQ / a.Q;
    // several queries per sequence: the fp8 score kernel reads packed keys
    const bool packed = fp8_mode && a.Q > 1 && a.N > 0;
    a.kpack = packed ? w : nullptr;
    dim3 g1((unsigned)a.n_chunks, (unsigned)BQ);
    // one fp8 score workgroup per query: it does the refine work itself
    const bool fused = fp8_mode && a.n_chunks == 1;
    if (a.N > 0) {
        static_assert(kHistStride % 4 == 0, "histogram block in 16-byte units");
        if (!fused) {
            prof_mark("idx_zero_kernel", false, stream);
            hipLaunchKernelGGL(idx_zero_kernel, dim3((unsigned)BQ), dim3(256), 0, stream,
                               reinterpret_cast<u32x4*>(a.hist));
            prof_mark("idx_zero_kernel", true, stream);
        }
        if (fp8_mode) {
            if (!((a.HI == 32 || a.HI == 64) && (a.dI == 64 || a.dI == 128))) return -2;
            if (packed) {
                const int64_t G = (a.N + 31) / 32, n = B * G * 2 * a.dI;  // 16-byte slots
                if ((size_t)n * 16 > packed_key_bytes(B, a.Q, a.N)) return -2;  // (dI <= 128 keeps this false)
                prof_mark("idx_pack_keys_kernel", false, stream);
                if (a.dI == 128)
                    hipLaunchKernelGGL(idx_pack_keys_kernel<4>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                                       a, B, G);
                else
                    hipLaunchKernelGGL(idx_pack_keys_kernel<2>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                                       a, B, G);
                prof_mark("idx_pack_keys_kernel", true, stream);
            }
            prof_mark("idx_score_fp8_kernel", false, stream);
            // one query per sequence: whole-line nontemporal loads (128-dim
            // keys) or direct loads; several: the packed keys
            const bool lines = a.Q == 1;
            if (a.HI == 64 && a.dI == 128) {
                if (lines) hipLaunchKernelGGL((idx_score_fp8_kernel<2, 8, kLoadLines>), g1, dim3(256), 0, stream, a);
                else hipLaunchKernelGGL((idx_score_fp8_kernel<2, 8, kLoadPacked>), g1, dim3(256), 0, stream, a);
            } else if (a.HI == 32 && a.dI == 128) {
                if (lines) hipLaunchKernelGGL((idx_score_fp8_kernel<1, 8, kLoadLines>), g1, dim3(256), 0, stream, a);
                else hipLaunchKernelGGL((idx_score_fp8_kernel<1, 8, kLoadPacked>), g1, dim3(256), 0, stream, a);
            } else if (a.HI == 64 && a.dI == 64) {
                if (lines) hipLaunchKernelGGL((idx_score_fp8_kernel<2, 4, kLoadDirect>), g1, dim3(256), 0, stream, a);
                else hipLaunchKernelGGL((idx_score_fp8_kernel<2, 4, kLoadPacked>), g1, dim3(256), 0, stream, a);
            } else {
                if (lines) hipLaunchKernelGGL((idx_score_fp8_kernel<1, 4, kLoadDirect>), g1, dim3(256), 0, stream, a);
                else hipLaunchKernelGGL((idx_score_fp8_kernel<1, 4, kLoadPacked>), g1, dim3(256), 0, stream, a);
            }
            prof_mark("idx_score_fp8_kernel", true, stream);
        } else {
            prof_mark("idx_score_f32_kernel", false, stream);
            hipLaunchKernelGGL(idx_score_f32_kernel, g1, dim3(256), 0, stream, a);
            prof_mark("idx_score_f32_kernel", true, stream);
        }
        if (!fused) {
            prof_mark("idx_refine_kernel", false, stream);
            hipLaunchKernelGGL(idx_refine_kernel, g1, dim3(256), 0, stream, a);
            prof_mark("idx_refine_kernel", true, stream);
        }
    }
    prof_mark("idx_select_kernel", false, stream);
    hipLaunchKernelGGL(idx_select_kernel, dim3((unsigned)BQ), dim3(kSelThreads), 0, stream, a);
    prof_mark("idx_select_kernel", true, stream);
    if (hipGetLastError() != hipSuccess) return -4;
    return 0;
}

}  // namespace cakv
