// backward.hip -- gradients of the hot path for training, on gfx950.
//
// [V4-Pro card, section 5 "1M context, gradually"] sparse attention is
// trained from 64K context on, after a short warm-up of the Lightning
// Indexer.  This file computes the gradients of the forward steps:
//
//   * core attention (sparse or dense, window, sink), per query and head,
//     with do = RoPE_t(dout) (the transpose of the output's rotation by -t),
//     P = exp(l - lse) from the forward's lse, delta = do . o:
//         dl = P (do . k - delta),  dsink = -P_sink delta,
//         dq_hat = tau dl K,        dK += tau dl^T Q_hat + P^T dO,
//     then dq through RoPE_t's transpose and q's RMSNorm.  Four launches:
//       prep    (one wave per query and head, 16 heads per workgroup):
//               q_hat and do (bf16, rows and, through LDS, transposed),
//               delta, the sink gradient;
//       logits  (one workgroup per query and key split, 4 waves of 32
//               heads): S^T = K Q_hat^T and dP^T = K dO^T on
//               v_mfma_f32_32x32x16_bf16 (one K read feeds both), then P
//               and dl, stored bf16 key-major and head-major;
//       dkeys   (same grid, 8 waves of 64 output dims): dK = [tau dl^T |
//               P^T] [Q_hat ; dO] on MFMA, the [Q_hat ; dO] operand held in
//               VGPRs for the split, added into the key rows' gradient with
//               float atomics (rows can be shared by the queries of one
//               sequence), or plain adds with one query per sequence, where
//               no two workgroups touch the same row;
//       dquery  (one workgroup per query and block of 32 heads, over all
//               of the query's keys: no split partials): dq_hat = dl K as the
//               forward's P V product (dl in the A-operand layout, K read
//               transposed from LDS), then from LDS the rotation's transpose
//               and the RMSNorm gradient.
//   * kv_prepare: one wave per row (rotation by -position, RMSNorm).
//   * the compressor (spans, per-channel gates): entry statistics, then one
//     workgroup per token summing over the entries whose span holds it.
//   * the indexer score over the selected entries: one workgroup per query
//     and 128 selected slots; the ReLU decisions use the forward's canonical
//     fp32 dot product (register-tiled fmaf chains), the two products that
//     follow (dq, dk) run on fp32 MFMA.
//
// Key rows are staged in LDS exactly as the forward stages them (1 KiB
// rows padded to 1,088 bytes, 16-byte granule g of row r at g ^ ((r >> 2) & 3)),
// so the same operand reads apply; tiles are double-buffered.
#include <algorithm>
#include <type_traits>

#include "cakv_attn_common.hpp"
#include "cakv_rows.hpp"

namespace cakv {

namespace {

constexpr int kBD = 512;            // head dim of the attention backward
constexpr int kRS = 1088;           // LDS row stride of a key tile
constexpr int kBuf = TK * kRS;      // one tile
constexpr int kKS = kBD / 16;       // QK k-steps
constexpr int kDT = kBD / 32;       // output dim tiles

typedef __fp16 f16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) f16x4_t lds_f16x4_t;

__device__ __forceinline__ int gperm(int row) { return (row >> 2) & 3; }

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t bf16_of(float f) { return (uint16_t)f32_to_bf16_bits(f); }

// gradient row of key slot `slot` (mirrors slot_row): dkv_c row of a
// visible compressed entry, dkv_raw row of a window position, or nullptr
__device__ __forceinline__ float* slot_grad_row(const AttnArgs& a, const QueryGeom& g, int slot, int32_t j,
                                                float* dkv_c, float* dkv_raw) {
    if (slot < g.n_c) {
        if (j < 0 || j >= g.n_vis) return nullptr;
        return dkv_c + (g.b * a.N + j) * (int64_t)kBD;
    }
    const int s = slot - g.n_c;
    if (s >= g.n_w) return nullptr;
    const int32_t p = g.p_lo + s;
    int64_t row = (int64_t)p - g.raw0;
    if (a.raw_ring && row < 0) row += a.R;
    if (row < 0 || row >= a.R) return nullptr;
    return dkv_raw + (g.b * a.R + row) * (int64_t)kBD;
}

// The tile's 32 key rows into LDS buffer `dst` (wave w copies rows 8w .. 8w+7,
// one 1 KiB row per instruction; an empty slot copies `spare` so that every
// wave always has 8 copies in flight), and the tile's validity mask.
template <bool SPARSE>
__device__ __forceinline__ uint32_t load_tile(const AttnArgs& a, const QueryGeom& g, int64_t bq, int tile,
                                              uint8_t* dst, const uint8_t* spare, int wave, int lane) {
    const int slot = tile * TK + (lane & 31);
    const bf16_t* row = nullptr;
    if (lane < TK && slot < g.n_c + g.n_w) row = slot_row<bf16_t>(a, g, slot, slot_entry<SPARSE>(a, g, bq, slot), kBD);
    const uint32_t mask = (uint32_t)__ballot(row != nullptr);
    const uint64_t rp = reinterpret_cast<uint64_t>(row);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int r = 8 * wave + k;
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(rp >> 32), r);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)rp, r);
        const uint64_t p = ((uint64_t)hi << 32) | lo;
        const uint8_t* src = p ? reinterpret_cast<const uint8_t*>(p) : spare;
        lds_dma16(src + 16 * (lane ^ gperm(r)), (uint32_t)(uintptr_t)(dst + r * kRS));
    }
    return mask;
}

}  // namespace

// ---------------------------------------------------------------- prep
// One workgroup of 16 waves per (query, block of 16 heads), one head per
// wave, lane l owning channels 8l .. 8l+7 of the head's rows.  The bf16 q_hat
// and do rows are also staged in LDS, so that the transposed copies
// ([D][HP]) leave as pairs of adjacent 16-byte stores (16 heads of one dim).
constexpr int kPrepHeads = 16;
__global__ __launch_bounds__(64 * kPrepHeads) void bwd_prep_kernel(const BwdArgs w) {
    constexpr int RW = kBD + 8;  // LDS row stride (elements): 16-byte rows
    __shared__ __attribute__((aligned(16))) uint16_t sq[kPrepHeads * RW];
    __shared__ __attribute__((aligned(16))) uint16_t sd[kPrepHeads * RW];
    const AttnArgs& a = w.f;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t bq = blockIdx.x;
    const int h0 = kPrepHeads * blockIdx.y;  // grid.y = HP / 16
    const int H = a.H;
    int32_t t = a.q_pos[bq];
    t = t < 0 ? 0 : t;
    const int rope_lo = kBD - a.rope_dims;
    {
        const int hl = wave, h = h0 + hl;
        u32x4* lq = reinterpret_cast<u32x4*>(sq + hl * RW + 8 * lane);
        u32x4* ld = reinterpret_cast<u32x4*>(sd + hl * RW + 8 * lane);
        const int64_t orow = (bq * w.HP + h) * (int64_t)kBD + 8 * lane;
        if (h >= H) {  // padding head (wave-uniform): zero rows and transposed columns
            *lq = u32x4{0u, 0u, 0u, 0u};
            *ld = u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(w.qh + orow) = u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(w.doh + orow) = u32x4{0u, 0u, 0u, 0u};
        } else {
            const int64_t row = (bq * H + h) * (int64_t)kBD + 8 * lane;
            float x[8], g8[8], d8[8], o8[8];
            Chunk8<bf16_t>::load(reinterpret_cast<const bf16_t*>(a.q) + row, x);
            Chunk8<float>::load(w.dout + row, d8);
            if (w.out_f32) Chunk8<float>::load(reinterpret_cast<const float*>(w.out) + row, o8);
            else Chunk8<bf16_t>::load(reinterpret_cast<const bf16_t*>(w.out) + row, o8);
            float ss = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) ss = __builtin_fmaf(x[k], x[k], ss);
            ss = wave_sum(ss);
            const float inv = 1.0f / __builtin_sqrtf(ss / (float)kBD + a.rms_eps);
#pragma unroll
            for (int k = 0; k < 8; ++k) g8[k] = x[k] * inv * (a.gamma_q ? a.gamma_q[8 * lane + k] : 1.0f);
            // q_hat = RoPE_t(q_n), do = RoPE_t(dout), o = RoPE_t(out): every rotated
            // pair of this lane's chunk turns by +t
#pragma unroll
            for (int pi = 0; pi < 4; ++pi) {
                const int d = 8 * lane + 2 * pi;
                if (d < rope_lo) continue;
                float sn, cs;
                sincos_turns((double)t * rope_turns(a.rope_ratio, (d - rope_lo) >> 1), &sn, &cs);
                float* v3[3] = {g8, d8, o8};
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    const float x0 = v3[k][2 * pi], x1 = v3[k][2 * pi + 1];
                    v3[k][2 * pi] = x0 * cs - x1 * sn;
                    v3[k][2 * pi + 1] = x0 * sn + x1 * cs;
                }
            }
            float dl = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) dl = __builtin_fmaf(d8[k], o8[k], dl);
            dl = wave_sum(dl);
            u32x4 qw, dw4;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                qw[k] = pack_bf16x2(g8[2 * k], g8[2 * k + 1]);
                dw4[k] = pack_bf16x2(d8[2 * k], d8[2 * k + 1]);
            }
            *reinterpret_cast<u32x4*>(w.qh + orow) = qw;
            *reinterpret_cast<u32x4*>(w.doh + orow) = dw4;
            *lq = qw;
            *ld = dw4;
            if (lane == 0) {
                w.delta[bq * H + h] = dl;
                const float z = a.sinks[h], lse = w.lse[bq * H + h];
                if (z != -INFINITY && lse != -INFINITY && w.dsinks) unsafeAtomicAdd(w.dsinks + h, -expf(z - lse) * dl);
            }
        }
    }
    __syncthreads();
    // transposed copies: thread (dim d, part p) stores heads 8p .. 8p+7 of the
    // block for dim d, 16 bytes (the two parts of a dim are adjacent threads)
    uint16_t* qt = w.qt + bq * (int64_t)kBD * w.HP + h0;
    uint16_t* dt = w.dot + bq * (int64_t)kBD * w.HP + h0;
    const int part = threadIdx.x & 1;
    static_assert(64 * kPrepHeads == 2 * kBD, "one thread per (dim, 8 heads)");
    {
        const int d = threadIdx.x >> 1;
        u32x4 vq, vd;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int h = 8 * part + 2 * k;
            vq[k] = (uint32_t)sq[h * RW + d] | ((uint32_t)sq[(h + 1) * RW + d] << 16);
            vd[k] = (uint32_t)sd[h * RW + d] | ((uint32_t)sd[(h + 1) * RW + d] << 16);
        }
        *reinterpret_cast<u32x4*>(qt + d * (int64_t)w.HP + 8 * part) = vq;
        *reinterpret_cast<u32x4*>(dt + d * (int64_t)w.HP + 8 * part) = vd;
    }
}

// ---------------------------------------------------------------- logits
// S^T = K Q_hat^T and dP^T = K dO^T for each tile of the split; P and dl.
template <bool SPARSE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_logits_kernel(const BwdArgs w) {
    const AttnArgs& a = w.f;
    __shared__ __attribute__((aligned(16))) uint8_t ring[2][kBuf];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lrow = lane & 31, lh = lane >> 5;
    const int64_t wg = xcd_order(blockIdx.x + (int64_t)gridDim.x * blockIdx.y, (int64_t)gridDim.x * gridDim.y);
    const int64_t bq = wg / a.n_splits;
    const int split = (int)(wg % a.n_splits);
    const int H = a.H;
    const QueryGeom g = query_geom<SPARSE>(a, bq);
    const int L = g.n_c + g.n_w;
    const int n_tiles = (L + TK - 1) / TK;
    const int tps = (n_tiles + a.n_splits - 1) / a.n_splits;
    const int tile0 = split * tps, tile1 = min(n_tiles, tile0 + tps);
    const uint8_t* spare = reinterpret_cast<const uint8_t*>(a.q) + bq * (int64_t)H * kBD * 2;
    const bool has_heads = 32 * wave < w.HP;
    const int head = 32 * wave + lrow;
    bf16x8 qf[kKS], df[kKS];
    {
        const int hh = head < H ? head : 0;
        const uint16_t* qr = w.qh + (bq * w.HP + hh) * (int64_t)kBD + 8 * lh;
        const uint16_t* dr = w.doh + (bq * w.HP + hh) * (int64_t)kBD + 8 * lh;
#pragma unroll
        for (int s = 0; s < kKS; ++s) {
            qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qr + 16 * s));
            df[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(dr + 16 * s));
        }
    }
    const float LOG2E = 1.4426950408889634f;
    const float sc = a.scale_log2;  // tau * log2 e
    const float mlse = head < H ? w.lse[bq * H + head] * LOG2E : 0.0f;
    const float dlta = head < H ? w.delta[bq * H + head] : 0.0f;
    const bool hlive = head < H && mlse != -INFINITY;
    const int64_t S = w.S;
    uint32_t masks[2] = {0u, 0u};
    if (tile0 < tile1) masks[0] = load_tile<SPARSE>(a, g, bq, tile0, ring[0], spare, wave, lane);
    for (int T = tile0; T < tile1; ++T) {
        const int cur = (T - tile0) & 1;
        if (T + 1 < tile1) {
            masks[cur ^ 1] = load_tile<SPARSE>(a, g, bq, T + 1, ring[cur ^ 1], spare, wave, lane);
            wait_vm<8>();
        } else {
            wait_vm<0>();
        }
        barrier_lds();
        const uint32_t mask = masks[cur];
        if (has_heads) {
            const uint8_t* kh = ring[cur];
            const int ga = gperm(lrow);
            const uint8_t* kq0 = kh + lrow * kRS + 16 * (lh ^ (ga & 1)) + 32 * (ga >> 1);
            const uint8_t* kq1 = kh + lrow * kRS + 16 * (lh ^ (ga & 1)) + 32 * ((ga >> 1) ^ 1);
            f32x16 st, dpt;
#pragma unroll
            for (int r = 0; r < 16; ++r) st[r] = dpt[r] = 0.0f;
#pragma unroll
            for (int s = 0; s < kKS; ++s) {
                const bf16x8 kv = *reinterpret_cast<const bf16x8*>(((s & 1) ? kq1 : kq0) + 64 * (s >> 1));
                st = mfma_bf16(kv, qf[s], st);
                dpt = mfma_bf16(kv, df[s], dpt);
            }
            // element r: key 8 (r/4) + 4 lh + r%4 of the tile, head `head`
            uint16_t* ptp = w.pt + (bq * S + (int64_t)T * TK) * w.HP + head;
            uint16_t* dtp = w.dlt + (bq * S + (int64_t)T * TK) * w.HP + head;
            uint16_t* dlp = w.dl + (bq * w.HP + head) * S + (int64_t)T * TK;
#pragma unroll
            for (int r0 = 0; r0 < 16; r0 += 4) {
                uint16_t dv[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int r = r0 + k;
                    const int key = 8 * (r >> 2) + 4 * lh + (r & 3);
                    const bool live = hlive && ((mask >> key) & 1u);
                    const float p = live ? __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], sc, -mlse)) : 0.0f;
                    const float dlv = p * (dpt[r] - dlta);
                    ptp[key * (int64_t)w.HP] = bf16_of(p);
                    dtp[key * (int64_t)w.HP] = bf16_of(w.tau * dlv);
                    dv[k] = bf16_of(dlv);
                }
                const int key0 = 8 * (r0 >> 2) + 4 * lh;
                *reinterpret_cast<u32x2*>(dlp + key0) =
                    u32x2{(uint32_t)dv[0] | ((uint32_t)dv[1] << 16), (uint32_t)dv[2] | ((uint32_t)dv[3] << 16)};
            }
        }
        barrier_lds();  // every wave is done with this buffer before it is refilled
    }
}

// ---------------------------------------------------------------- dkeys
// dK = [tau dl^T | P^T] [Q_hat ; dO]: 8 waves, wave w owns output dims
// 64 w .. +64 (two 32-dim tiles); the [Q_hat ; dO] operand (k = 2 HP stacked
// heads) stays in VGPRs for the whole split (2 x 16 k-steps x 4 VGPRs).
template <bool SPARSE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkeys_kernel(const BwdArgs w) {
    const AttnArgs& a = w.f;
    constexpr int MAXK = 16;  // k-steps of 16 stacked heads: 2 HP / 16 for HP <= 128
    constexpr int NT = 2;     // dim tiles per wave
    __shared__ uint64_t gptr[TK];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lrow = lane & 31, lh = lane >> 5;
    const int64_t wg = xcd_order(blockIdx.x + (int64_t)gridDim.x * blockIdx.y, (int64_t)gridDim.x * gridDim.y);
    const int64_t bq = wg / a.n_splits;
    const int split = (int)(wg % a.n_splits);
    const QueryGeom g = query_geom<SPARSE>(a, bq);
    const int L = g.n_c + g.n_w;
    const int n_tiles = (L + TK - 1) / TK;
    const int tps = (n_tiles + a.n_splits - 1) / a.n_splits;
    const int tile0 = split * tps, tile1 = min(n_tiles, tile0 + tps);
    const int nks = 2 * w.HP / 16;  // uniform, <= MAXK
    const int ksq = w.HP / 16;      // k-steps from Q_hat (the rest from dO)
    const int64_t S = w.S;
    // B operand of dim tile dt, k-step ks: lane (dim column lrow, half lh)
    // holds stacked heads 16 ks + 8 lh .. +7 of that dim
    bf16x8 bop[NT][MAXK];
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
        const int dim = 64 * wave + 32 * dt + lrow;
        const uint16_t* qc = w.qt + (bq * kBD + dim) * (int64_t)w.HP + 8 * lh;
        const uint16_t* dc = w.dot + (bq * kBD + dim) * (int64_t)w.HP + 8 * lh;
#pragma unroll
        for (int ks = 0; ks < MAXK; ++ks) {
            const uint16_t* src = ks < ksq ? qc + 16 * ks : dc + 16 * (ks - ksq);
            bop[dt][ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
            if (ks < nks) bop[dt][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src));
        }
    }
    for (int T = tile0; T < tile1; ++T) {
        // the tile's gradient rows
        if (wave == 0 && lane < TK) {
            const int slot = T * TK + lane;
            float* gr = nullptr;
            if (slot < L) gr = slot_grad_row(a, g, slot, slot_entry<SPARSE>(a, g, bq, slot), w.dkv_c, w.dkv_raw);
            gptr[lane] = reinterpret_cast<uint64_t>(gr);
        }
        barrier_lds();
        // A operand, k-step ks: lane (key lrow, half lh) holds stacked heads
        // 16 ks + 8 lh .. +7 of that key (tau dl^T, then P^T)
        const uint16_t* ad = w.dlt + (bq * S + (int64_t)T * TK + lrow) * w.HP + 8 * lh;
        const uint16_t* ap = w.pt + (bq * S + (int64_t)T * TK + lrow) * w.HP + 8 * lh;
        f32x16 acc[NT];
#pragma unroll
        for (int dt = 0; dt < NT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < MAXK; ++ks) {
            if (ks < nks) {  // uniform
                const uint16_t* src = ks < ksq ? ad + 16 * ks : ap + 16 * (ks - ksq);
                const bf16x8 av = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src));
#pragma unroll
                for (int dt = 0; dt < NT; ++dt) acc[dt] = mfma_bf16(av, bop[dt][ks], acc[dt]);
            }
        }
        // element r of tile dt: key 8 (r/4) + 4 lh + r%4, dim 64 w + 32 dt + lrow
        if (w.unique_rows) {
            // no other workgroup touches these rows: a plain read-modify-write,
            // every load issued before the first add (empty slots skipped)
            float old[16][NT];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float* gr = reinterpret_cast<float*>(gptr[8 * (r >> 2) + 4 * lh + (r & 3)]);
#pragma unroll
                for (int dt = 0; dt < NT; ++dt) old[r][dt] = gr ? gr[64 * wave + 32 * dt + lrow] : 0.0f;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float* gr = reinterpret_cast<float*>(gptr[8 * (r >> 2) + 4 * lh + (r & 3)]);
                if (gr) {
#pragma unroll
                    for (int dt = 0; dt < NT; ++dt) gr[64 * wave + 32 * dt + lrow] = old[r][dt] + acc[dt][r];
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float* gr = reinterpret_cast<float*>(gptr[8 * (r >> 2) + 4 * lh + (r & 3)]);
                if (gr) {
#pragma unroll
                    for (int dt = 0; dt < NT; ++dt) unsafeAtomicAdd(gr + 64 * wave + 32 * dt + lrow, acc[dt][r]);
                }
            }
        }
        barrier_lds();  // gptr is rewritten for the next tile
    }
}

// ---------------------------------------------------------------- dquery
// dq: one workgroup per (query, block of 32 heads) over all of the query's key
// tiles (no key splits, so no partials).  Wave w forms dims 128 w .. +127 of
// dq_hat / tau = dl K for the block's heads: the forward's P V product with dl
// in the A-operand layout and K read transposed from the LDS tile.  Tiles
// land in a ring of four LDS buffers, three in flight: each holds the tile's
// rows and its dl block (32 heads x 32 keys), all copied asynchronously, nine
// copies per wave per tile (so a count of copies in flight says which tiles
// have landed).  A query's selected entry indices are staged in LDS once
// (when there are at most kDqIdxCap), so that building a tile's row pointers
// waits on no load.  The block's dq_hat then goes through LDS (over the ring)
// to the finish, one wave per head in turn: tau, the rotation's transpose and
// the RMSNorm gradient
//     dq = gamma du / r - x sum(gamma du x) / (D r^3),  du = RoPE_-t(dq_hat).
constexpr int kDqRow = kBD + 4;   // LDS row stride (floats) of the dq_hat block
constexpr int kDqBuf = kBuf + 3072;  // a tile's rows, its dl block (2 KiB), the idle waves' copy (1 KiB)
constexpr int kDqIdxCap = 2048;   // selected slots whose entry indices are staged in LDS
// IDX_LDS (sparse, K <= kDqIdxCap): the indices come from LDS; otherwise from
// memory (each tile's row pointers then wait for that load, and with it for
// the copies in flight: correct, with a shallower pipeline).  A compile-time
// choice: with both paths in one kernel the compiler waits for the union of
// their loads where they join, on every tile.
// HB: heads per workgroup, 32 or 16 (16 when 32-head blocks would leave CUs
// idle: the MFMA rows of the other 16 heads then hold zeros).
template <bool SPARSE, bool IDX_LDS, int HB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dquery_kernel(const BwdArgs w) {
    static_assert(SPARSE || !IDX_LDS, "indices exist only for the sparse call");
    static_assert(HB == 16 || HB == 32, "head blocks of 16 or 32");
    const AttnArgs& a = w.f;
    __shared__ __attribute__((aligned(16))) uint8_t ring[4][kDqBuf];
    __shared__ int32_t sidx[IDX_LDS ? kDqIdxCap : 1];
    static_assert(32 * kDqRow * 4 <= 4 * kDqBuf, "the dq_hat block fits over the ring");
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lrow = lane & 31, lh = lane >> 5;
    const int nhb = w.HP / HB;
    const int64_t wg = xcd_order(blockIdx.x + (int64_t)gridDim.x * blockIdx.y, (int64_t)gridDim.x * gridDim.y);
    const int64_t bq = wg / nhb;
    const int h0 = HB * (int)(wg % nhb);
    const int H = a.H;
    const QueryGeom g = query_geom<SPARSE>(a, bq);
    const int L = g.n_c + g.n_w;
    const int n_tiles = (L + TK - 1) / TK;
    const uint8_t* spare = reinterpret_cast<const uint8_t*>(a.q) + bq * (int64_t)H * kBD * 2;
    const int64_t S = w.S;
    if constexpr (IDX_LDS) {
        for (int i = tid; i < g.n_c; i += 256) sidx[i] = a.idx[bq * a.K + i];
        __syncthreads();
    }
    // copies of tile T into buf: rows (8 per wave, as load_tile) and the dl
    // block (waves 0-1: 16 heads each; waves 2-3 copy wave 0's rows into the
    // idle kilobyte, so that every wave has nine copies per tile)
    auto issue = [&](int T, uint8_t* buf) __attribute__((always_inline)) {
        const int slot = T * TK + (lane & 31);
        const bf16_t* row = nullptr;
        if (lane < TK && slot < L) {
            int32_t j = slot;
            if constexpr (IDX_LDS) j = slot < g.n_c ? sidx[slot] : 0;
            else if constexpr (SPARSE) j = slot < g.n_c ? a.idx[bq * a.K + slot] : 0;
            row = slot_row<bf16_t>(a, g, slot, j, kBD);
        }
        const uint64_t rp = reinterpret_cast<uint64_t>(row);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int r = 8 * wave + k;
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(rp >> 32), r);
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)rp, r);
            const uint64_t p = ((uint64_t)hi << 32) | lo;
            const uint8_t* src = p ? reinterpret_cast<const uint8_t*>(p) : spare;
            lds_dma16(src + 16 * (lane ^ gperm(r)), (uint32_t)(uintptr_t)(buf + r * kRS));
        }
        const int dr = (HB == 32 ? 16 * (wave & 1) : 0) + (lane >> 2);  // dl row (head of the block)
        const uint16_t* dsrc = w.dl + (bq * w.HP + h0 + dr) * S + (int64_t)T * TK + 8 * (lane & 3);
        lds_dma16(dsrc, (uint32_t)(uintptr_t)(buf + kBuf + (wave < 2 ? 1024 * wave : 2048)));
    };
    constexpr int WDT = kDT / 4;  // output dim tiles of a wave
    f32x16 acc[WDT];
#pragma unroll
    for (int i = 0; i < WDT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
#pragma unroll
    for (int T = 0; T < 3; ++T)
        if (T < n_tiles) issue(T, ring[T]);
    for (int T = 0; T < n_tiles; ++T) {
        if (T + 3 < n_tiles) {
            issue(T + 3, ring[(T + 3) & 3]);
            wait_vm<27>();
        } else if (T + 2 < n_tiles) {
            wait_vm<18>();
        } else if (T + 1 < n_tiles) {
            wait_vm<9>();
        } else {
            wait_vm<0>();
        }
        barrier_lds();
        const uint8_t* kh = ring[T & 3];
        // A operand (dl, heads x keys): lane (head lrow, half lh) holds keys
        // 16 ks + {4 lh + j, 8 + 4 lh + j}, j < 4 (the order the V reads use)
        const uint8_t* dlr = kh + kBuf + 64 * lrow;
        bf16x8 pa[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const u32x2 plo = *reinterpret_cast<const u32x2*>(dlr + 2 * (16 * ks + 4 * lh));
            const u32x2 phi = *reinterpret_cast<const u32x2*>(dlr + 2 * (16 * ks + 8 + 4 * lh));
            pa[ks] = (HB == 32 || lrow < HB) ? __builtin_bit_cast(bf16x8, u32x4{plo[0], plo[1], phi[0], phi[1]})
                                             : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        }
        const int q = lane >> 4, i16 = lane & 15;
        const uint8_t* vrow[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int rr = 8 * hf + 4 * (q >> 1) + (i16 >> 2);
            vrow[hf] = kh + rr * kRS + 16 * ((2 * (q & 1) + ((i16 & 3) >> 1)) ^ gperm(rr)) + 8 * (i16 & 1);
        }
#pragma unroll
        for (int i = 0; i < WDT; ++i) {
            const int dt = WDT * wave + i;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int off = ks * 16 * kRS + 64 * dt;
                const f16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_f16x4_t*)const_cast<uint8_t*>(vrow[0] + off));
                const f16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_f16x4_t*)const_cast<uint8_t*>(vrow[1] + off));
                const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
                const bf16x8 vb = __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
                acc[i] = mfma_bf16(pa[ks], vb, acc[i]);
            }
        }
        barrier_lds();  // before the buffer takes tile T + 4
    }
    // the dq_hat block over the ring (every tile has been consumed): element r
    // of tile i is head 8 (r/4) + 4 lh + r%4 of the block, dim 32 (WDT wave + i) + lrow
    float* dqs = reinterpret_cast<float*>(&ring[0][0]);
#pragma unroll
    for (int i = 0; i < WDT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dqs[(8 * (r >> 2) + 4 * lh + (r & 3)) * kDqRow + 32 * (WDT * wave + i) + lrow] = acc[i][r];
    __syncthreads();
    int32_t t = a.q_pos[bq];
    t = t < 0 ? 0 : t;
    const int rope_lo = kBD - a.rope_dims;
    for (int hl = wave; hl < HB; hl += 4) {
        const int h = h0 + hl;
        if (h >= H) break;  // wave-uniform
        float du[8];
        {
            const f32x4 v0 = *reinterpret_cast<const f32x4*>(&dqs[hl * kDqRow + 8 * lane]);
            const f32x4 v1 = *reinterpret_cast<const f32x4*>(&dqs[hl * kDqRow + 8 * lane + 4]);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                du[k] = v0[k] * w.tau;
                du[4 + k] = v1[k] * w.tau;
            }
        }
#pragma unroll
        for (int pi = 0; pi < 4; ++pi) {
            const int d = 8 * lane + 2 * pi;
            if (d < rope_lo) continue;
            float sn, cs;
            sincos_turns(-(double)t * rope_turns(a.rope_ratio, (d - rope_lo) >> 1), &sn, &cs);
            const float x0 = du[2 * pi], x1 = du[2 * pi + 1];
            du[2 * pi] = x0 * cs - x1 * sn;
            du[2 * pi + 1] = x0 * sn + x1 * cs;
        }
        const int64_t row = (bq * H + h) * (int64_t)kBD + 8 * lane;
        float x[8];
        Chunk8<bf16_t>::load(reinterpret_cast<const bf16_t*>(a.q) + row, x);
        float ss = 0.0f, dot = 0.0f;
        float gm[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            gm[k] = a.gamma_q ? a.gamma_q[8 * lane + k] : 1.0f;
            ss = __builtin_fmaf(x[k], x[k], ss);
            dot = __builtin_fmaf(gm[k] * du[k], x[k], dot);
        }
        ss = wave_sum(ss);
        dot = wave_sum(dot);
        const float rr = __builtin_sqrtf(ss / (float)kBD + a.rms_eps);
        const float ir = 1.0f / rr, c3 = dot / ((float)kBD * rr * rr * rr);
        float dq[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            dq[k] = gm[k] * du[k] * ir - x[k] * c3;
            if (w.dgamma_q) unsafeAtomicAdd(w.dgamma_q + 8 * lane + k, du[k] * x[k] * ir);
        }
        Chunk8<float>::store(w.dq + row, dq);
    }
}

// ---------------------------------------------------------------- kv_prepare
template <typename T>
__global__ __launch_bounds__(256) void kv_prepare_bwd_kernel(const T* in, const float* dy, float* dx,
                                                             const float* __restrict__ gamma, float* dgamma,
                                                             int64_t N, int D, int64_t j0, int64_t n, int64_t rows,
                                                             int m, int rope_dims, double rope_ratio, int pos_off,
                                                             float eps) {
    const int64_t rw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (rw >= rows) return;
    const int lane = threadIdx.x & 63;
    const int64_t b = rw / n, j = j0 + rw % n;
    const int64_t off = (b * N + j) * (int64_t)D;
    const int nch = D >> 3;
    const double pos = (double)(j * m + pos_off);
    const int rope_lo = D - rope_dims;
    float x[kPrepMaxChunks][8], u[kPrepMaxChunks][8];
    float ss = 0.0f, dot = 0.0f;
#pragma unroll
    for (int k = 0; k < kPrepMaxChunks; ++k) {
        const int c = lane + 64 * k;
        if (c < nch) {
            Chunk8<T>::load(in + off + 8 * c, x[k]);
            Chunk8<float>::load(dy + off + 8 * c, u[k]);
            if (8 * c + 8 > rope_lo) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int d = 8 * c + 2 * p;
                    if (d < rope_lo) continue;
                    float sn, cs;
                    sincos_turns(-pos * rope_turns(rope_ratio, (d - rope_lo) >> 1), &sn, &cs);
                    const float x0 = u[k][2 * p], x1 = u[k][2 * p + 1];
                    u[k][2 * p] = x0 * cs - x1 * sn;
                    u[k][2 * p + 1] = x0 * sn + x1 * cs;
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                ss = __builtin_fmaf(x[k][i], x[k][i], ss);
                dot = __builtin_fmaf((gamma ? gamma[8 * c + i] : 1.0f) * u[k][i], x[k][i], dot);
            }
        }
    }
    ss = wave_sum(ss);
    dot = wave_sum(dot);
    const float r = __builtin_sqrtf(ss / (float)D + eps);
    const float ir = 1.0f / r, c3 = dot / ((float)D * r * r * r);
#pragma unroll
    for (int k = 0; k < kPrepMaxChunks; ++k) {
        const int c = lane + 64 * k;
        if (c < nch) {
            float o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float gm = gamma ? gamma[8 * c + i] : 1.0f;
                o[i] = gm * u[k][i] * ir - x[k][i] * c3;
                if (dgamma) unsafeAtomicAdd(dgamma + 8 * c + i, u[k][i] * x[k][i] * ir);
            }
            Chunk8<float>::store(dx + off + 8 * c, o);
        }
    }
}

// ---------------------------------------------------------------- kv_compress
// Entry statistics per (entry, channel): mx, 1/z and c (the forward value in fp32).
template <typename TIn, bool PC>
__global__ __launch_bounds__(256) void kv_compress_stats_kernel(const TIn* x, const float* gate, int64_t T, int D,
                                                                int m, int span, int64_t nblk, float* st) {
    const int64_t e = blockIdx.x;  // b * nblk + j
    const int64_t b = e / nblk, j = e % nblk;
    const int64_t hi = (j + 1) * m, lo = hi - span > 0 ? hi - span : 0;
    const int n = (int)(hi - lo);
    for (int d = threadIdx.x; d < D; d += 256) {
        float mx = -INFINITY;
        for (int i = 0; i < n; ++i) {
            const float gi = PC ? gate[(b * T + lo + i) * D + d] : gate[b * T + lo + i];
            mx = fmaxf(mx, gi);
        }
        float z = 0.0f, c = 0.0f;
        for (int i = 0; i < n; ++i) {
            const float gi = PC ? gate[(b * T + lo + i) * D + d] : gate[b * T + lo + i];
            const float wgt = expf(gi - mx);
            z += wgt;
            float xv;
            if constexpr (sizeof(TIn) == 4) xv = reinterpret_cast<const float*>(x)[(b * T + lo + i) * D + d];
            else xv = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[(b * T + lo + i) * D + d]);
            c = __builtin_fmaf(wgt, xv, c);
        }
        const float rz = 1.0f / z;
        float* o = st + (e * (int64_t)D + d) * 3;
        o[0] = mx;
        o[1] = rz;
        o[2] = c * rz;
    }
}

// One workgroup per token i: the entries whose span holds i are
// j = ceil((i+1)/m) - 1 .. floor((i + span)/m) - 1 (below nblk).
template <typename TIn, bool PC>
__global__ __launch_bounds__(256) void kv_compress_bwd_kernel(const TIn* x, const float* gate, const float* dc,
                                                              const float* st, int64_t T, int D, int m, int span,
                                                              int64_t nblk, float* dx, float* dgate) {
    __shared__ float red[4];
    const int64_t bi = blockIdx.x;  // b * T + i
    const int64_t b = bi / T, i = bi % T;
    int64_t jlo = (i + m) / m - 1;  // ceil((i+1)/m) - 1
    int64_t jhi = (i + span) / m - 1;
    if (jhi > nblk - 1) jhi = nblk - 1;
    float gsum = 0.0f;
    for (int d = threadIdx.x; d < D; d += 256) {
        float xv;
        if constexpr (sizeof(TIn) == 4) xv = reinterpret_cast<const float*>(x)[bi * D + d];
        else xv = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[bi * D + d]);
        const float gi = PC ? gate[bi * D + d] : gate[bi];
        float ax = 0.0f, ag = 0.0f;
        for (int64_t j = jlo; j <= jhi; ++j) {
            const float* s = st + ((b * nblk + j) * (int64_t)D + d) * 3;
            const float a = expf(gi - s[0]) * s[1];
            const float g = dc[(b * nblk + j) * (int64_t)D + d];
            ax = __builtin_fmaf(a, g, ax);
            ag = __builtin_fmaf(a * (xv - s[2]), g, ag);
        }
        dx[bi * D + d] = ax;
        if (PC) dgate[bi * D + d] = ag;
        else gsum += ag;
    }
    if (!PC) {
        gsum = wave_sum(gsum);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = gsum;
        __syncthreads();
        if (threadIdx.x == 0) dgate[bi] = (red[0] + red[1]) + (red[2] + red[3]);
    }
}

// ---------------------------------------------------------------- indexer
// Workgroup = (query, 128 selected slots), four waves; q (64 x 128), the 128
// key rows and the coefficients coef[j][h] = dS_j w_h [s_jh > 0] sit in LDS
// as fp32 (zero beyond HI, dI and for empty slots).
//  1. scores: thread (slot group sg = lane % 32, head group hg = 2 wave +
//     lane / 32) holds the 4 x 8 scores of slots sg + 32 i and heads hg + 8 u,
//     each an fmaf chain in the canonical order (head dim ascending from +0),
//     16-byte LDS reads reused across the tile; decisions, coef and the dw
//     partials (summed over the 32 lanes of a head group) follow.
//  2. dq (heads x dims) = coef^T K and 3. dk (slots x dims) = coef Q are dense
//     fp32 contractions on v_mfma_f32_32x32x2f32: wave w owns dims 32 w .. +31
//     of dq and slots 32 w .. +31 of dk.
// dq and dw are sums over the workgroups of a query (float atomics into
// zeroed outputs), dk over queries (float atomics, accumulated); each atomic
// instruction covers 32 consecutive floats of two rows.
constexpr int kIBS = 128;  // slots per workgroup

__global__ __launch_bounds__(256) void indexer_bwd_zero_kernel(float* dq, int64_t nq, float* dw, int64_t nw) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nq; i += (int64_t)gridDim.x * 256) {
        dq[i] = 0.0f;
        if (i < nw) dw[i] = 0.0f;
    }
}

template <typename TQ, bool FP8>
__global__ __launch_bounds__(256) void indexer_bwd_kernel(const IndexerBwdArgs a) {
    constexpr int QST = 128;  // q[h][d] row stride (floats)
    constexpr int KST = 132;  // k[slot][d] row stride: 16-byte rows, 4-bank shift per row
    constexpr int CST = 65;   // coef[slot][h] row stride: 1-bank shift per row
    __shared__ __attribute__((aligned(16))) float qs[64 * QST];
    __shared__ __attribute__((aligned(16))) float ks[kIBS * KST];
    __shared__ float coef[kIBS * CST];
    __shared__ float dsv[kIBS];
    __shared__ float wsv[64];
    __shared__ float dwsum[64];
    __shared__ int32_t ents[kIBS];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, lh = lane >> 5;
    const int64_t bq = blockIdx.x;
    const int64_t b = bq / a.Q;
    const int HI = a.HI, dI = a.dI, NE = HI * dI;
    const int s0 = blockIdx.y * kIBS;
    const int32_t t = a.q_pos[bq];
    const int64_t nv = t < 0 ? 0 : ((int64_t)t / a.m < a.N ? (int64_t)t / a.m : a.N);
    // staging, every global load of a round issued before its first LDS store:
    // round 1 the selection, dS, w and q (16-byte chunks, each inside one head
    // row since dI is a multiple of 8); round 2 the key rows
    {
        constexpr int QE = 16 / sizeof(TQ);          // q elements per chunk
        constexpr int QCH = 64 * 128 / QE / 256;     // chunks per thread at HI = 64, dI = 128
        const int nch = NE / QE;
        u32x4 qc[QCH];
#pragma unroll
        for (int i = 0; i < QCH; ++i) {
            const int c = tid + 256 * i;
            qc[i] = c < nch ? reinterpret_cast<const u32x4*>(a.q_idx)[(bq * NE) / QE + c] : u32x4{0u, 0u, 0u, 0u};
        }
        int32_t e = -1;
        float g = 0.0f, wv = 0.0f;
        const int s = s0 + tid;
        if (tid < kIBS && s < a.K) {
            e = a.idx[bq * a.K + s];
            g = a.dS[bq * a.K + s];
        }
        if (tid >= kIBS && tid < kIBS + 64 && tid - kIBS < HI) wv = a.w[bq * HI + tid - kIBS];
        if (tid < kIBS) {
            if (e < 0 || e >= nv) e = -1;
            ents[tid] = e;
            dsv[tid] = e >= 0 ? g : 0.0f;
        } else if (tid < kIBS + 64) {
            wsv[tid - kIBS] = wv;
        }
#pragma unroll
        for (int i = 0; i < QCH; ++i) {
            const int c = tid + 256 * i;
            if (c < nch) {
                const int h = (c * QE) / dI, d = (c * QE) % dI;
                float* dst = &qs[h * QST + d];
                if constexpr (QE == 4) {
                    *reinterpret_cast<f32x4*>(dst) = __builtin_bit_cast(f32x4, qc[i]);
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        dst[2 * k] = __builtin_bit_cast(float, qc[i][k] << 16);
                        dst[2 * k + 1] = __builtin_bit_cast(float, qc[i][k] & 0xffff0000u);
                    }
                }
            }
        }
        // zero padding (disjoint from the chunks above)
        if (HI < 64 || dI < 128) {
            for (int x = tid; x < 64 * QST; x += 256)
                if (x / QST >= HI || x % QST >= dI) qs[x] = 0.0f;
        }
    }
    __syncthreads();
    {
        constexpr int KCH = kIBS * 16 / 256;  // 8-element chunks of the 128 (padded) dims per thread
        using KV = typename std::conditional<FP8, u32x2, u32x4>::type;
        KV lo[KCH], hi[KCH];
        float sc[KCH];
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int c = tid + 256 * i, r = c >> 4, d = (c & 15) * 8;
            const int32_t e = ents[r];
            lo[i] = KV{};
            hi[i] = KV{};
            sc[i] = 0.0f;
            if (d < dI && e >= 0) {
                const int64_t row = b * a.N + e;
                if constexpr (FP8) {
                    lo[i] = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(a.k_idx) + row * dI + d);
                    sc[i] = a.k_scale[row];
                } else {
                    const u32x4* src = reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(a.k_idx) + row * dI + d);
                    lo[i] = src[0];
                    hi[i] = src[1];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int c = tid + 256 * i, r = c >> 4, d = (c & 15) * 8;
            float v[8];
            if constexpr (FP8) {
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] = e4m3_decode_f32((lo[i][k >> 2] >> (8 * (k & 3))) & 0xffu) * sc[i];
            } else {  // whole-vector casts (a cast of one vector element would read element 0)
                const f32x4 fl = __builtin_bit_cast(f32x4, lo[i]), fh = __builtin_bit_cast(f32x4, hi[i]);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v[k] = fl[k];
                    v[4 + k] = fh[k];
                }
            }
            *reinterpret_cast<f32x4*>(&ks[r * KST + d]) = f32x4{v[0], v[1], v[2], v[3]};
            *reinterpret_cast<f32x4*>(&ks[r * KST + d + 4]) = f32x4{v[4], v[5], v[6], v[7]};
        }
    }
    __syncthreads();
    // 1. scores, decisions, coef, dw
    {
        const int sg = l32, hg = 2 * wave + lh;
        float acc[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int u = 0; u < 8; ++u) acc[i][u] = 0.0f;
        for (int d = 0; d < dI; d += 4) {
            f32x4 k4[4], q4[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) k4[i] = *reinterpret_cast<const f32x4*>(&ks[(sg + 32 * i) * KST + d]);
#pragma unroll
            for (int u = 0; u < 8; ++u) q4[u] = *reinterpret_cast<const f32x4*>(&qs[(hg + 8 * u) * QST + d]);
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int u = 0; u < 8; ++u) acc[i][u] = __builtin_fmaf(q4[u][c], k4[i][c], acc[i][u]);
        }
        float dwp[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) dwp[u] = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = sg + 32 * i;
            const float g = dsv[r];
            const bool live = ents[r] >= 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int h = hg + 8 * u;
                const bool pos = live && h < HI && acc[i][u] > 0.0f;
                coef[r * CST + h] = pos ? g * wsv[h] : 0.0f;
                dwp[u] += pos ? g * acc[i][u] : 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float v = group_sum<32>(dwp[u]);
            if (l32 == 0) dwsum[hg + 8 * u] = v;
        }
    }
    __syncthreads();
    // 2. dq[h][d] = sum_j coef[j][h] k[j][d]: A = coef^T (heads x slots), B = K;
    // operands of 16 k-steps read into registers ahead of their MFMAs
    const auto dq_tiles = [&](auto two_tiles) {
        constexpr bool TWO = decltype(two_tiles)::value;
        constexpr int BS = 16;
        f32x16 c0 = {}, c1 = {};
#pragma unroll
        for (int blk = 0; blk < kIBS / (2 * BS); ++blk) {
            float av0[BS], av1[BS], bv[BS];
#pragma unroll
            for (int u = 0; u < BS; ++u) {
                const int r = 2 * (blk * BS + u) + lh;
                bv[u] = ks[r * KST + 32 * wave + l32];
                av0[u] = coef[r * CST + l32];
                if constexpr (TWO) av1[u] = coef[r * CST + 32 + l32];
            }
#pragma unroll
            for (int u = 0; u < BS; ++u) {
                c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av0[u], bv[u], c0, 0, 0, 0);
                if constexpr (TWO) c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av1[u], bv[u], c1, 0, 0, 0);
            }
        }
        const int d = 32 * wave + l32;
        if (d < dI) {
            float* dq = a.dq + bq * NE + d;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int h = 8 * (i >> 2) + 4 * lh + (i & 3);
                if (h < HI && c0[i] != 0.0f) unsafeAtomicAdd(dq + h * dI, c0[i]);
                if constexpr (TWO)
                    if (h + 32 < HI && c1[i] != 0.0f) unsafeAtomicAdd(dq + (h + 32) * dI, c1[i]);
            }
        }
    };
    if (32 * wave < dI) {
        if (HI > 32) dq_tiles(std::true_type{});
        else dq_tiles(std::false_type{});
    }
    // 3. dk[j][d] = sum_h coef[j][h] q[h][d]: A = coef (slots x heads), B = Q;
    // blocks of 16 heads (zero beyond HI), all four 32-dim tiles (zero beyond dI)
    {
        f32x16 c[4] = {};
        const int nblk = (HI + 15) / 16;
        for (int blk = 0; blk < nblk; ++blk) {
            float av[8], bv[8][4];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int h = 16 * blk + 2 * u + lh;
                av[u] = coef[(32 * wave + l32) * CST + h];
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) bv[u][dt] = qs[h * QST + 32 * dt + l32];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) c[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[u], bv[u][dt], c[dt], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int32_t e = ents[32 * wave + 8 * (i >> 2) + 4 * lh + (i & 3)];
            if (e < 0) continue;
            float* dk = a.dk + (b * a.N + e) * dI + l32;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                if (32 * dt + l32 < dI && c[dt][i] != 0.0f) unsafeAtomicAdd(dk + 32 * dt, c[dt][i]);
        }
    }
    if (tid < HI && dwsum[tid] != 0.0f) unsafeAtomicAdd(a.dw + bq * HI + tid, dwsum[tid]);
}

// ---------------------------------------------------------------- launchers
size_t mqa_bwd_workspace_bytes(int64_t BQ, int32_t H, int64_t max_slots, int n_splits) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const int64_t HP = (H + 31) / 32 * 32;
    const int64_t S = (max_slots + TK - 1) / TK * TK;
    size_t n = 0;
    n += 4 * al((size_t)BQ * HP * kBD * 2);  // qh, doh, qt, dot
    n += al((size_t)BQ * H * 4);             // delta
    n += 3 * al((size_t)BQ * (S > 0 ? S : TK) * HP * 2);  // pt, dlt, dl
    (void)n_splits;  // the dq kernel runs over all of a query's keys: no split partials
    return n;
}

int launch_mqa_bwd(BwdArgs& w, int64_t BQ, int64_t max_slots, void* ws, hipStream_t stream) {
    if (BQ == 0) return 0;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const int64_t HP = (w.f.H + 31) / 32 * 32;
    const int64_t S = (max_slots + TK - 1) / TK * TK;
    w.HP = (int32_t)HP;
    w.S = (int32_t)(S > 0 ? S : TK);
    uint8_t* p = reinterpret_cast<uint8_t*>(ws);
    auto take = [&](size_t bytes) {
        uint8_t* r = p;
        p += al(bytes);
        return r;
    };
    w.qh = reinterpret_cast<uint16_t*>(take((size_t)BQ * HP * kBD * 2));
    w.doh = reinterpret_cast<uint16_t*>(take((size_t)BQ * HP * kBD * 2));
    w.qt = reinterpret_cast<uint16_t*>(take((size_t)BQ * HP * kBD * 2));
    w.dot = reinterpret_cast<uint16_t*>(take((size_t)BQ * HP * kBD * 2));
    w.delta = reinterpret_cast<float*>(take((size_t)BQ * w.f.H * 4));
    w.pt = reinterpret_cast<uint16_t*>(take((size_t)BQ * w.S * HP * 2));
    w.dlt = reinterpret_cast<uint16_t*>(take((size_t)BQ * w.S * HP * 2));
    w.dl = reinterpret_cast<uint16_t*>(take((size_t)BQ * w.S * HP * 2));
    const bool sparse = w.f.idx != nullptr;
    const dim3 gp((unsigned)BQ, (unsigned)(HP / kPrepHeads));
    const dim3 gs((unsigned)w.f.n_splits, (unsigned)BQ);
    prof_mark("bwd_prep_kernel", false, stream);
    hipLaunchKernelGGL(bwd_prep_kernel, gp, dim3(64 * kPrepHeads), 0, stream, w);
    prof_mark("bwd_prep_kernel", true, stream);
    prof_mark("bwd_logits_kernel", false, stream);
    if (sparse) hipLaunchKernelGGL(bwd_logits_kernel<true>, gs, dim3(256), 0, stream, w);
    else hipLaunchKernelGGL(bwd_logits_kernel<false>, gs, dim3(256), 0, stream, w);
    prof_mark("bwd_logits_kernel", true, stream);
    prof_mark("bwd_dkeys_kernel", false, stream);
    if (sparse) hipLaunchKernelGGL(bwd_dkeys_kernel<true>, gs, dim3(512), 0, stream, w);
    else hipLaunchKernelGGL(bwd_dkeys_kernel<false>, gs, dim3(512), 0, stream, w);
    prof_mark("bwd_dkeys_kernel", true, stream);
    // 16-head blocks while 32-head ones would give fewer workgroups than CUs
    const bool hb16 = BQ * (HP / 32) < 256;
    const dim3 gq((unsigned)(HP / (hb16 ? 16 : 32)), (unsigned)BQ);
#define CAKV_DQ(SP, IL)                                                                                  \
    if (hb16) hipLaunchKernelGGL((bwd_dquery_kernel<SP, IL, 16>), gq, dim3(256), 0, stream, w);        \
    else hipLaunchKernelGGL((bwd_dquery_kernel<SP, IL, 32>), gq, dim3(256), 0, stream, w)
    prof_mark("bwd_dquery_kernel", false, stream);
    if (sparse && w.f.K <= kDqIdxCap) { CAKV_DQ(true, true); }
    else if (sparse) { CAKV_DQ(true, false); }
    else { CAKV_DQ(false, false); }
#undef CAKV_DQ
    prof_mark("bwd_dquery_kernel", true, stream);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_kv_prepare_bwd(const void* in, const float* dy, float* dx, float* dgamma, int dtype, int64_t B, int64_t N,
                          int64_t D, int64_t j0, int64_t n, const float* gamma, int32_t m, int32_t rope_dims,
                          double rope_ratio, int32_t pos_off, float eps, hipStream_t stream) {
    const int64_t rows = B * n;
    if (rows == 0) return 0;
    if (D > 64 * 8 * kPrepMaxChunks) return -2;
    const int64_t grid = (rows + 3) / 4;
    if (grid > 0x7fffffffLL) return -2;
    prof_mark("kv_prepare_bwd_kernel", false, stream);
    if (dtype == 0)
        hipLaunchKernelGGL((kv_prepare_bwd_kernel<float>), dim3((unsigned)grid), dim3(256), 0, stream,
                           (const float*)in, dy, dx, gamma, dgamma, N, (int)D, j0, n, rows, m, rope_dims, rope_ratio,
                           pos_off, eps);
    else
        hipLaunchKernelGGL((kv_prepare_bwd_kernel<bf16_t>), dim3((unsigned)grid), dim3(256), 0, stream,
                           (const bf16_t*)in, dy, dx, gamma, dgamma, N, (int)D, j0, n, rows, m, rope_dims, rope_ratio,
                           pos_off, eps);
    prof_mark("kv_prepare_bwd_kernel", true, stream);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

size_t kv_compress_bwd_workspace_bytes(int64_t B, int64_t T, int64_t D, int32_t m) {
    return (size_t)B * (size_t)(T / m) * (size_t)D * 3 * 4;
}

int launch_kv_compress_bwd(const void* x, int x_dtype, const float* gate, bool pc, int64_t B, int64_t T, int64_t D,
                           int32_t m, int32_t span, const float* dc, float* dx, float* dgate, void* ws,
                           hipStream_t stream) {
    const int64_t nblk = T / m;
    if (B * T == 0) return 0;
    if (B * nblk > 0x7fffffffLL || B * T > 0x7fffffffLL) return -2;
    float* st = reinterpret_cast<float*>(ws);
#define CAKV_CB(TIN, PC)                                                                                          \
    do {                                                                                                         \
        if (nblk > 0)                                                                                            \
            hipLaunchKernelGGL((kv_compress_stats_kernel<TIN, PC>), dim3((unsigned)(B * nblk)), dim3(256), 0,   \
                               stream, (const TIN*)x, gate, T, (int)D, m, span, nblk, st);                       \
        hipLaunchKernelGGL((kv_compress_bwd_kernel<TIN, PC>), dim3((unsigned)(B * T)), dim3(256), 0, stream,    \
                           (const TIN*)x, gate, dc, st, T, (int)D, m, span, nblk, dx, dgate);                    \
    } while (0)
    prof_mark("kv_compress_bwd_kernel", false, stream);
    if (x_dtype == 0) {
        if (pc) CAKV_CB(float, true);
        else CAKV_CB(float, false);
    } else {
        if (pc) CAKV_CB(bf16_t, true);
        else CAKV_CB(bf16_t, false);
    }
#undef CAKV_CB
    prof_mark("kv_compress_bwd_kernel", true, stream);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int launch_indexer_bwd(const IndexerBwdArgs& a, int64_t BQ, bool q_f32, bool fp8, hipStream_t stream) {
    if (BQ == 0) return 0;
    if (a.dI > 128 || a.HI > 64) return -2;
    const int64_t nq = BQ * a.HI * a.dI, nw = BQ * a.HI;
    // nw <= nq: the zero kernel's loop covers both
    hipLaunchKernelGGL(indexer_bwd_zero_kernel, dim3((unsigned)std::min<int64_t>((nq + 255) / 256, 8192)), dim3(256),
                       0, stream, a.dq, nq, a.dw, nw);
    if (a.K == 0) return hipGetLastError() == hipSuccess ? 0 : -4;
    const dim3 grid((unsigned)BQ, (unsigned)((a.K + kIBS - 1) / kIBS));
    prof_mark("indexer_bwd_kernel", false, stream);
    if (q_f32) {
        if (fp8) hipLaunchKernelGGL((indexer_bwd_kernel<float, true>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((indexer_bwd_kernel<float, false>), grid, dim3(256), 0, stream, a);
    } else {
        if (fp8) hipLaunchKernelGGL((indexer_bwd_kernel<bf16_t, true>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((indexer_bwd_kernel<bf16_t, false>), grid, dim3(256), 0, stream, a);
    }
    prof_mark("indexer_bwd_kernel", true, stream);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace cakv
