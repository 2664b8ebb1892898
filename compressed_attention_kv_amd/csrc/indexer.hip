// indexer.hip -- Lightning-Indexer scoring and exact top-k on gfx950.
//
// [V4 digest, CSA step 2] a light indexer scores each query against every
// compressed entry and keeps the k best; [V4-Pro card, Hybrid attention] 64
// indexer heads of dim 128 keep k=1024; [Visualised, Dual Compression and
// Indexing] the pass is low precision.  Score of entry j for a query:
// S(j) = sum_h w_h * ReLU(q_h . k_j); ties go to the lower index; output
// ascending by index, -1 padded.
//
// Three kernels per call:
//   1. score: one workgroup per (query, chunk of entries).
//        fp8 mode: keys stream from HBM once, 64 bytes per lane per 32
//        entries, decoded exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8) and
//        multiplied on v_mfma_f32_32x32x16_bf16 against the bf16 query heads
//        held in VGPRs (heads x entries, fp32 accumulation); ReLU, the head
//        weights and the head reduction run on the accumulator registers and
//        one half-wave exchange.  The per-entry scale multiplies the final
//        sum (it is a power of two, so this is exact up to rounding order).
//        fp32 mode: one thread per entry runs the canonical fmaf chains.
//      Each score becomes an order-preserving 32-bit key, written to the
//      workspace, and a 2048-bin histogram of its top 11 bits is built in
//      LDS and added to the query's global histogram.
//   2. select: one workgroup per (query, chunk).  Every workgroup finds from
//      the histogram the bin holding the k-th best key; entries in higher
//      bins are certainly selected and entries in that bin are candidates.
//      The last workgroup of a query (ticket counter) selects exactly among
//      the candidates with a radix select on (key, index) in LDS -- or over
//      the whole key array if the candidates overflow -- and sorts the k
//      winners by index with a bitonic sort in LDS.
#include "cakv_device.hpp"
#include "cakv_internal.hpp"

namespace cakv {

__global__ void idx_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

__device__ __forceinline__ int64_t query_nvis(const IndexerArgs& a, int64_t bq) {
    int32_t t = a.q_pos[bq];
    t = t < 0 ? 0 : t;
    int64_t nv = t / a.m;
    return nv < a.N ? nv : a.N;
}

__device__ __forceinline__ void flush_hist(const uint32_t* lds, uint32_t* g) {
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) {
        const uint32_t h = lds[i];
        if (h) atomicAdd(g + i, h);
    }
}

// ------------------------------------------------------------------ fp8 mode
// HT: head tiles of 32 (HI = 32*HT); KS: MFMA k-steps of 16 (dI = 16*KS)
template <int HT, int KS>
__global__ __launch_bounds__(256) void idx_score_fp8_kernel(const IndexerArgs a) {
    __shared__ uint32_t hist[kHistBins];
    const int64_t bq = blockIdx.y;
    const int64_t nvis = query_nvis(a, bq);
    const int64_t j_begin = (int64_t)blockIdx.x * a.chunk;
    if (nvis <= a.k || j_begin >= nvis) return;
    const int64_t j_end = min(nvis, j_begin + a.chunk);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lrow = lane & 31, lh = lane >> 5;
    constexpr int DI = 16 * KS;
    constexpr int HALF = DI / 2;        // bytes of a key row per half-wave lane
    constexpr int NLD = HALF / 16;      // 16-byte loads per lane
    for (int i = tid; i < kHistBins; i += 256) hist[i] = 0u;

    // A operand: query heads (rows) x features, k-permutation (s, half, e) -> half*DI/2 + 8s + e
    bf16x8 qa[HT][KS];
    float wv[HT][16];
    const int64_t b = bq / a.Q;
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
    __syncthreads();

    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_idx) + b * a.N * DI;
    const float* sbase = a.k_scale + b * a.N;
    for (int64_t j0 = j_begin + 32 * wave; j0 < j_end; j0 += 128) {
        const int64_t j = j0 + lrow;
        const int64_t jj = j < a.N ? j : a.N - 1;
        u32x4 raw[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i)
            raw[i] = *reinterpret_cast<const u32x4*>(kbase + jj * DI + lh * HALF + 16 * i);
        const float sc = sbase[jj];
        f32x16 acc[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[ht][r] = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            // 8 fp8 bytes = dwords (2s, 2s+1) of this lane's half row
            const uint32_t d0 = raw[s >> 1][(s & 1) * 2], d1 = raw[s >> 1][(s & 1) * 2 + 1];
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
        if (lane < 32 && j < j_end) {
            const uint32_t key = score_key(sum);
            a.keys[bq * a.N + j] = key;
            atomicAdd(&hist[key >> 21], 1u);
        }
    }
    __syncthreads();
    flush_hist(hist, a.hist + bq * kHistBins);
}

// ------------------------------------------------------------------ fp32 mode
// Canonical order: per head an fmaf chain over d ascending from +0, ReLU as
// (s > 0 ? s : +0), then an fmaf chain over heads ascending from +0.
__global__ __launch_bounds__(256) void idx_score_f32_kernel(const IndexerArgs a) {
    __shared__ uint32_t hist[kHistBins];
    __shared__ float qs[8192];
    __shared__ float ws[64];
    const int64_t bq = blockIdx.y;
    const int64_t nvis = query_nvis(a, bq);
    const int64_t j_begin = (int64_t)blockIdx.x * a.chunk;
    if (nvis <= a.k || j_begin >= nvis) return;
    const int64_t j_end = min(nvis, j_begin + a.chunk);
    const int tid = threadIdx.x;
    const int HI = a.HI, DI = a.dI;
    for (int i = tid; i < kHistBins; i += 256) hist[i] = 0u;
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
        const uint32_t key = score_key(S);
        a.keys[bq * a.N + j] = key;
        atomicAdd(&hist[key >> 21], 1u);
    }
    __syncthreads();
    flush_hist(hist, a.hist + bq * kHistBins);
}

// ------------------------------------------------------------------ selection
// Wave-aggregated append: returns this lane's slot (valid only where pred).
__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t* counter) {
    const uint64_t m = __ballot(pred);
    if (m == 0) return 0;
    const int lane = threadIdx.x & 63;
    const int leader = __builtin_ctzll(m);
    uint32_t base = 0;
    if (lane == leader) base = atomicAdd(counter, (uint32_t)__builtin_popcountll(m));
    base = __shfl(base, leader, 64);
    return base + (uint32_t)__builtin_popcountll(m & ((1ull << lane) - 1ull));
}

// Wave 0 finds the digit d with below(d) < r <= below(d) + cnt[d] over 256
// counters; writes (d, below(d)) to out[0..1].  Other waves do nothing.
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

// r-th smallest (1-based) of the values produced by get(i) for i < n, where
// get returns false for elements that do not take part.  Whole workgroup.
template <typename Get>
__device__ uint64_t radix_select_u64(int64_t n, uint32_t r, Get get, uint32_t* cnt, uint32_t* res) {
    uint64_t prefix = 0, mask = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
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

__global__ __launch_bounds__(256) void idx_select_kernel(const IndexerArgs a) {
    __shared__ uint32_t hist[kHistBins];
    __shared__ uint32_t part[256];
    __shared__ uint32_t cnt[256];
    __shared__ uint32_t info[8];
    __shared__ uint64_t cand[kBoundaryCap];
    __shared__ uint32_t sorted[kTopkCap];
    const int64_t bq = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t nvis = query_nvis(a, bq);
    const int k = a.k;
    int32_t* out = a.idx + bq * k;
    if (nvis <= k) {  // every visible entry is selected
        if (blockIdx.x == 0)
            for (int i = tid; i < k; i += 256) out[i] = i < nvis ? i : -1;
        return;
    }
    // ---- threshold bin: walk bins from the top; thread t owns bins 2047-8t .. 2040-8t
    const uint32_t* gh = a.hist + bq * kHistBins;
    uint32_t loc = 0;
    uint32_t hb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        hb[i] = gh[kHistBins - 1 - (8 * tid + i)];
        loc += hb[i];
    }
    part[tid] = loc;
    __syncthreads();
    // inclusive scan of part[] (Hillis-Steele)
    for (int o = 1; o < 256; o <<= 1) {
        const uint32_t v = tid >= o ? part[tid - o] : 0u;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    const uint32_t incl = part[tid], excl = incl - loc;
    if (excl < (uint32_t)k && (uint32_t)k <= incl) {
        uint32_t above = excl;
        int i = 0;
        while (above + hb[i] < (uint32_t)k) {
            above += hb[i];
            ++i;
        }
        info[0] = (uint32_t)(kHistBins - 1 - (8 * tid + i));  // threshold bin
        info[1] = above;                                       // keys in higher bins
    }
    __syncthreads();
    const uint32_t tbin = info[0];
    const uint32_t n_above = info[1];
    uint32_t* ctr = a.counters + bq * 4;
    int32_t* sel = a.sel + bq * k;
    uint64_t* bnd = a.bnd + bq * kBoundaryCap;
    const uint32_t* keys = a.keys + bq * a.N;

    // ---- classify this chunk
    const int64_t j_begin = (int64_t)blockIdx.x * a.sel_chunk;
    const int64_t j_end = min(nvis, j_begin + a.sel_chunk);
    for (int64_t j0 = j_begin; j0 < j_end; j0 += 256) {
        const int64_t j = j0 + tid;
        uint32_t key = 0, bin = 0;
        const bool in = j < j_end;
        if (in) {
            key = keys[j];
            bin = key >> 21;
        }
        const bool hi = in && bin > tbin;
        const bool eq = in && bin == tbin;
        const uint32_t ph = wave_append(hi, ctr + 0);
        if (hi) sel[ph] = (int32_t)j;
        const uint32_t pe = wave_append(eq, ctr + 1);
        if (eq && pe < (uint32_t)kBoundaryCap) bnd[pe] = ((uint64_t)(~key) << 32) | (uint64_t)j;
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) info[2] = atomicAdd(ctr + 2, 1u);
    __syncthreads();
    if (info[2] != (uint32_t)(gridDim.x - 1)) return;
    __threadfence();

    // ---- last workgroup of this query: exact choice inside the threshold bin
    const uint32_t need = (uint32_t)k - n_above;  // >= 1
    const uint32_t nb = __atomic_load_n(ctr + 1, __ATOMIC_RELAXED);
    uint64_t vth;
    if (nb <= (uint32_t)kBoundaryCap) {
        for (uint32_t i = tid; i < nb; i += 256) cand[i] = __atomic_load_n(bnd + i, __ATOMIC_RELAXED);
        __syncthreads();
        vth = radix_select_u64(
            (int64_t)nb, need, [&](int64_t i, uint64_t* v) { *v = cand[i]; return true; }, cnt, info + 4);
    } else {
        vth = radix_select_u64(
            nvis, need,
            [&](int64_t i, uint64_t* v) {
                const uint32_t key = __atomic_load_n(keys + i, __ATOMIC_RELAXED);
                *v = ((uint64_t)(~key) << 32) | (uint64_t)i;
                return (key >> 21) == tbin;
            },
            cnt, info + 4);
    }
    // gather: the n_above certain winners, then candidates with value <= vth
    int n2 = 1;
    while (n2 < k) n2 <<= 1;
    for (int i = tid; i < n2; i += 256)
        sorted[i] = i < (int)n_above ? (uint32_t)__atomic_load_n(sel + i, __ATOMIC_RELAXED) : 0xffffffffu;
    if (tid == 0) info[3] = n_above;
    __syncthreads();
    if (nb <= (uint32_t)kBoundaryCap) {
        for (uint32_t i = tid; i < nb; i += 256) {
            const uint64_t v = cand[i];
            if (v <= vth) sorted[atomicAdd(&info[3], 1u)] = (uint32_t)(v & 0xffffffffu);
        }
    } else {
        for (int64_t i = tid; i < nvis; i += 256) {
            const uint32_t key = __atomic_load_n(keys + i, __ATOMIC_RELAXED);
            const uint64_t v = ((uint64_t)(~key) << 32) | (uint64_t)i;
            if ((key >> 21) == tbin && v <= vth) sorted[atomicAdd(&info[3], 1u)] = (uint32_t)i;
        }
    }
    __syncthreads();
    bitonic_sort_u32(sorted, n2);
    for (int i = tid; i < k; i += 256) out[i] = (int32_t)sorted[i];
}

size_t indexer_workspace_bytes(int64_t BQ, int64_t N, int32_t k) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    size_t s = 0;
    s += al((size_t)BQ * (size_t)N * 4);             // keys
    s += al((size_t)BQ * (kHistBins + 4) * 4);       // hist + counters (zeroed together)
    s += al((size_t)BQ * (size_t)k * 4);             // sel
    s += al((size_t)BQ * kBoundaryCap * 8);          // bnd
    return s;
}

int launch_indexer_topk(IndexerArgs& a, int64_t BQ, bool fp8_mode, void* ws, hipStream_t stream) {
    if (BQ == 0) return 0;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    uint8_t* p = reinterpret_cast<uint8_t*>(ws);
    a.keys = reinterpret_cast<uint32_t*>(p);
    p += al((size_t)BQ * (size_t)a.N * 4);
    a.hist = reinterpret_cast<uint32_t*>(p);
    a.counters = a.hist + BQ * kHistBins;
    p += al((size_t)BQ * (kHistBins + 4) * 4);
    a.sel = reinterpret_cast<int32_t*>(p);
    p += al((size_t)BQ * (size_t)a.k * 4);
    a.bnd = reinterpret_cast<uint64_t*>(p);

    const int64_t nzero = BQ * (kHistBins + 4);
    const int64_t zblocks = (nzero + 255) / 256;
    const unsigned zgrid = (unsigned)(zblocks < 4096 ? zblocks : 4096);
    hipLaunchKernelGGL(idx_zero_kernel, dim3(zgrid), dim3(256), 0, stream, a.hist, nzero);
    if (hipGetLastError() != hipSuccess) return -4;

    dim3 g1((unsigned)a.n_chunks, (unsigned)BQ);
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
    dim3 g2((unsigned)a.n_sel_chunks, (unsigned)BQ);
    hipLaunchKernelGGL(idx_select_kernel, g2, dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return -4;
    return 0;
}

}  // namespace cakv
